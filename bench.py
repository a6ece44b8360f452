"""Benchmark: AutoRound per-Linear tuning throughput on one MI355X.

One bench step = the whole hot path for one Linear: ar_tune_linear (staging,
cfg.iters SignSGD iterations, best-state restore and final quantization) and
ar_pack, on inputs already resident in HBM. Workload: Llama-7B-shaped q_proj
4096->4096, bf16, W4 asym g128, 128 samples x 2048 tokens, minibatch 8 x 2048,
200 iterations, synthetic seeded data (synth module).

Prints one JSON line. `value` is tuning iterations per second for the whole
job; `roofline` reports the dominant kernel against the bf16 MFMA peak with its
average duration measured by HIP events on the launch stream during the timed
steps; `cpu_baseline` is the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 3] [--warmup 1] [--workload llama7b_q_proj]

detail.gram reports the same job in the Gram form (ar_tune_linear_gram);
detail.dequant_gemm the tuned codes through the packed-format product;
detail.block sequential block-wise tuning of a Llama-7B-shaped decoder block.
"""
import argparse
import json
import os
import platform
import sys
import time
import types

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COPY_BYTES = 1 << 30
TIME_EVERY = 8              # HIP events around the kernels of every 8th SignSGD step
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_gemm_llama7b_q_proj.txt")
GEMM_SOURCE = os.path.join(ROOT, "autoround_signsgd_rounding_amd", "csrc", "ar_gemm.hip")


def gemm_code_hash(path=GEMM_SOURCE):
    """sha256 of the GEMM source's code: comments removed and whitespace
    collapsed, so that an edit of comments alone keeps the counters valid."""
    import hashlib
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode("utf-8")).hexdigest()


def _measured_traffic(workload):
    """HBM bytes per launch of the forward GEMM from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs, or None when they were taken on another
    workload or the GEMM code has changed since."""
    if workload != "llama7b_q_proj" or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("gemm_code_sha256") != gemm_code_hash():
        return None
    return int(float(kv["traffic_bytes"]))


def _cpu_baseline(case, Yd, w, steps=8):
    """The CPU oracle as it stands on the same workload. A launch-bound layer
    (under 1 GFLOP per iteration) is timed on its whole tuning run
    (oracle.tune_linear, all w.iters iterations, restore and quantization);
    a larger one on `steps` SignSGD steps of the full problem, minibatch
    i mod nb for step i as in the tuning loop."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    cfg = O.Config(bits=w.bits, group_size=w.group_size, sym=w.sym, nsamples=w.nsamples,
                   seqlen=w.seqlen, batch_samples=w.batch_samples, iters=w.iters, lr=w.lr,
                   minmax_lr=w.minmax_lr, minmax_shrink=w.minmax_shrink)
    Tb = w.Tb
    nb = w.nsamples // w.batch_samples
    host = {"host_cpus": os.cpu_count(), "affinity_cpus": _affinity(),
            "blas_threads": int(threads), "cpu_model": _cpu_model(),
            "host": platform.processor() or platform.machine()}
    batches = []
    for b in range(min(steps, nb) if w.flop_per_iter >= 1e9 else nb):
        xb = synth.bf16_bits_to_f32(case.X_bits[b * Tb:(b + 1) * Tb])
        yb = Yd[b * Tb:(b + 1) * Tb].float().cpu().numpy()
        batches.append((xb, yb))
    if w.flop_per_iter < 1e9:
        t0 = time.perf_counter()
        O.tune_linear(case.W, lambda b: batches[b], nb, cfg)
        el = time.perf_counter() - t0
        return {"value": w.iters / el, "unit": "iters/s", "cores": int(threads),
                "kind": "oracle",
                "sample": f"the whole {w.iters}-iteration tuning run of the {w.N}x{w.K} layer "
                          f"(staging, every SignSGD step, best-state restore, final "
                          f"quantization) in {el:.3f} s", **host}
    V = np.zeros((w.N, w.K), np.float32)
    wmin, wmax = O.group_minmax(case.W, w.group_size)
    a = np.full(wmin.shape, np.float32(w.minmax_shrink))
    b = a.copy()
    t0 = time.perf_counter()
    for i in range(steps):
        xb, yb = batches[i % len(batches)]
        r = O.tune_step(case.W, V, a, b, wmin, wmax, xb, yb, cfg)
        V, a, b = r.V, r.alpha, r.beta
    el = time.perf_counter() - t0
    return {"value": steps / el, "unit": "iters/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} SignSGD steps (fwd+wgrad contractions, STE fold, update) of the "
                      f"full {w.N}x{w.K} problem on {Tb}-token minibatches; "
                      f"{el / steps:.2f} s/step; a {w.iters}-iteration run extrapolates to "
                      f"{w.iters * el / steps / 60:.1f} min", **host}


def _affinity():
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        return None


def _cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return platform.processor() or None


def _dequant_run(ar, torch, X, out, w, reps=20):
    """The tuned layer's packed codes through ar_dequant_gemm: decode sizes
    (M = 1, 16; bound by reading the packed weight, reported as GB/s of
    algorithmic bytes against 8 TB/s) and one minibatch of prefill (M = Tb;
    TFLOP/s against the bf16 peak). Buffers are allocated once; the decode
    calls are captured `reps` at a time in a HIP graph and the replays timed
    with HIP events, so host call overhead is not in the figure."""
    qw, qz = ar.pack(out.codes, out.zp, w.bits)
    G = w.K // w.group_size
    res = {}
    stream = torch.cuda.current_stream()
    for M in (1, 16, w.Tb):
        Xm = X[:M]
        Yo = torch.empty((M, w.N), dtype=torch.float32, device=X.device)
        need = ar.dequant_gemm_workspace_size(w.bits, w.group_size, M, w.N, w.K)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=X.device)

        def call():
            ar.dequant_gemm(Xm, qw, qz, out.scale, w.bits, w.group_size, w.N, out=Yo,
                            workspace=ws)
        call()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        if M <= 16:
            g = torch.cuda.CUDAGraph()
            s2 = torch.cuda.Stream()
            with torch.cuda.stream(s2):
                with torch.cuda.graph(g, stream=s2):
                    for _ in range(reps):
                        call()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            n_rep = 5
            e0.record(stream)
            for _ in range(n_rep):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / (n_rep * reps)
        else:
            n = 5
            e0.record(stream)
            for _ in range(n):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n
        if M <= 16:
            nbytes = (w.N * w.K * w.bits // 8 + w.N * G * 4 + G * w.N * w.bits // 8
                      + M * w.K * 2 + M * w.N * 4)
            gbs = nbytes / (ms * 1e-3) / 1e9
            res[f"M{M}"] = {"us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes}
        else:
            tf = 2.0 * M * w.N * w.K / (ms * 1e-3) / 1e12
            res[f"M{M}"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
                            "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        del Yo, ws
    res["config"] = f"W{w.bits} g{w.group_size} {w.N}x{w.K}, tuned codes, float32 output"
    res["M1_large"] = _decode_large(ar, torch, reps)
    return res


def _decode_large(ar, torch, reps, N=29568, K=8192, bits=4, g=128):
    """One-token product on a Qwen2.5-72B up_proj-sized layer, W`bits` g`g`
    (random codes: the speed does not depend on their values), graph-timed like
    the decode sizes above; at 4 bits, 121 MB of packed weight make the HBM
    roofline the honest bound."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    G = K // g
    qw = torch.randint(-2 ** 31, 2 ** 31 - 1, (K * bits // 32, N), dtype=torch.int32, device=dev,
                       generator=gen)
    qz = torch.randint(-2 ** 31, 2 ** 31 - 1, (G, N * bits // 32), dtype=torch.int32, device=dev,
                       generator=gen)
    sc = torch.rand((N, G), device=dev, generator=gen) * 0.01
    X = torch.randn((1, K), device=dev, generator=gen).to(torch.bfloat16)
    Y = torch.empty((1, N), device=dev)
    ws = torch.empty(max(ar.dequant_gemm_workspace_size(bits, g, 1, N, K), 256), dtype=torch.uint8,
                     device=dev)

    def call():
        ar.dequant_gemm(X, qw, qz, sc, bits, g, N, out=Y, workspace=ws)
    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        with torch.cuda.graph(graph, stream=s2):
            for _ in range(reps):
                call()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    for _ in range(5):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (5 * reps)
    nbytes = N * K * bits // 8 + N * G * 4 + G * N * bits // 8 + K * 2 + N * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"shape": f"W{bits} g{g} {N}x{K}", "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes}


def _step_run(ar, torch, W, X, Y, cfg, w, warm=10, timed=30):
    """ar_tune_step, one SignSGD iteration from caller-owned state per call on
    the workload's minibatches in turn (each call stages its own minibatch):
    HIP events around each call on the launch stream, median over `timed`
    calls after `warm` untimed ones."""
    dev = W.device
    G = w.K // w.group_size
    V = torch.zeros((w.N, w.K), dtype=torch.float32, device=dev)
    a = torch.full((w.N, G), float(w.minmax_shrink), dtype=torch.float32, device=dev)
    b = a.clone()
    best = (torch.empty_like(V), torch.empty_like(a), torch.empty_like(b),
            torch.full((1,), float("inf"), dtype=torch.float32, device=dev))
    ydt = ar.AR_BF16 if Y.dtype == torch.bfloat16 else ar.AR_F32
    ws = torch.empty(ar.step_workspace_size(cfg, w.N, w.K, w.Tb, ydt), dtype=torch.uint8,
                     device=dev)
    nb = w.nsamples // w.batch_samples
    stream = torch.cuda.current_stream()
    ms = []
    for i in range(warm + timed):
        j = i % nb
        Xb, Yb = X[j * w.Tb:(j + 1) * w.Tb], Y[j * w.Tb:(j + 1) * w.Tb]
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ar.tune_step(W, V, a, b, Xb, Yb, cfg, best=best, want_grads=False, workspace=ws)
        e1.record(stream)
        if i >= warm:
            ms.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in ms)
    med = t[len(t) // 2]
    return {"ms_median": round(med, 4), "iters_per_s": round(1e3 / med, 1),
            "note": "per call, including the call's own transposition of its minibatch"}


def _pack_time(ar, torch, out, bits, reps=20):
    """GPU time of one ar_pack of the tuned codes and zero-points: a HIP graph
    of `reps` calls into preallocated outputs, replayed between two events (the
    tuning call returns after synchronizing, so timing one call from the host
    would include its launch latency)."""
    qw, qz = ar.pack(out.codes, out.zp, bits)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        with torch.cuda.graph(g, stream=s2):
            for _ in range(reps):
                ar.pack(out.codes, out.zp, bits, out=(qw, qz))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    for _ in range(5):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (5 * reps)


def _pack_large(ar, torch, N=29568, K=8192, bits=4, g=128):
    """ar_pack on a Qwen2.5-72B up_proj-sized layer (random codes and
    zero-points of the grid; the speed does not depend on their values),
    graph-timed as above: N·K code bytes in, N·K·bits/8 packed bytes out, plus
    the zero-points."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    G = K // g
    hi = 1 << bits
    codes = torch.randint(0, hi, (N, K), dtype=torch.uint8, device=dev, generator=gen)
    zp = torch.randint(0, hi, (N, G), dtype=torch.uint8, device=dev, generator=gen)
    ms = _pack_time(ar, torch, types.SimpleNamespace(codes=codes, zp=zp), bits)
    nbytes = N * K + N * K * bits // 8 + N * G * (1 + bits / 8)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"shape": f"W{bits} g{g} {N}x{K}", "ms": round(ms, 4), "GB/s": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": int(nbytes)}


def _block_run(ar, torch, iters=200):
    """Sequential block-wise tuning with quantized inputs (ar_tune_block) of a
    Llama-7B-shaped decoder block (D 4096, 32 heads, F 11008) on 16 synthetic
    sequences of 2048 tokens, W4 g128, 200 iterations per Linear on minibatches
    of 8 sequences: wall time for the whole block (both pipelines' forwards and
    the seven tuning loops) after one untimed single-iteration call."""
    dims = synth.BLOCKS["llama7b_block"]
    c = synth.make_block_case(dims)
    dev = torch.device("cuda:0")

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    W = {n: bf(c.W_bits[n]) for n in ar.BLOCK_LINEARS}
    norms = tuple(bf(x) for x in c.norm_bits)
    h = bf(c.H_bits)
    bd = ar.block_dims(dims.D, dims.H, dims.F, dims.seqlen, dims.nsamples, dims.rms_eps,
                       dims.rope_theta)
    res = {}
    for it in (1, iters):
        cfg = ar.Config(bits=4, group_size=128, nsamples=dims.nsamples, seqlen=dims.seqlen,
                        batch_samples=8, iters=it)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out, out_fp, out_q = ar.tune_block(h, W, norms, bd, cfg, quanted_input=True)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        res[it] = (el, out, out_fp, out_q)
    el, out, out_fp, out_q = res[iters]
    mse = float(((out_q.float() - out_fp.float()) ** 2).mean())
    return {"workload": f"{dims.name}: D {dims.D}, H {dims.H}, F {dims.F}, {dims.nsamples}x"
                        f"{dims.seqlen} tokens, W4 g128, {iters} iters per Linear, quantized inputs",
            "seconds": round(el, 3), "seconds_1_iter": round(res[1][0], 3),
            "tune_iters_per_s": round(7 * iters / el, 1),
            "best_loss": {n: float(out[n][4].min()) for n in ar.BLOCK_LINEARS},
            "block_out_mse": mse}


def _graph_steps(ar, torch, W, X, Y, cfg, w, ws, args, step):
    """Steps of a launch-bound layer: ar_tune_linear + ar_pack captured once in
    a HIP graph (no allocation or memset inside: the buffers come from the
    capture's pool, the library clears with fill kernels), one replay per
    step. Every replay recomputes the whole job from the same inputs; the
    last replay's outputs must equal an eager call's bit for bit. Per-kernel
    times come from `args.steps` eager calls with HIP events around every
    step's kernels. Returns (eager records, seconds for the timed replays,
    check record)."""
    recs = []
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        with torch.cuda.graph(g, stream=s2):
            gout = ar.tune_linear(W, X, Y, cfg, want_state=False, workspace=ws)
            gqw, gqz = ar.pack(gout.codes, gout.zp, w.bits)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ref = recs[-1][1]
    rqw, rqz = ar.pack(ref.codes, ref.zp, w.bits)
    same = (torch.equal(gout.codes, ref.codes) and torch.equal(gout.scale, ref.scale)
            and torch.equal(gout.zp, ref.zp) and torch.equal(gqw, rqw) and torch.equal(gqz, rqz)
            and torch.equal(gout.losses, ref.losses))
    if not same:
        raise RuntimeError("graph replay differs from the eager call")
    return recs, el, {"replays": args.warmup + args.steps, "equal_to_eager": same}


def _yardstick(torch, w, reps=50):
    """The vendor library's GEMM (torch -> hipBLASLt, run as a black box) on the
    step's two contraction shapes, bf16 operands with float32 accumulation:
    forward Y' = X_b·Ŵᵀ (F.linear, [Tb, K] x [N, K]) and gradient G = dYᵀ·X_b
    (torch.mm on the transposed view, [Tb, N]ᵀ x [Tb, K]), on random operands.
    HIP events around `reps` calls on the current stream, after 5 untimed."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    X = torch.randn((w.Tb, w.K), device=dev, generator=gen).to(torch.bfloat16)
    W = (torch.randn((w.N, w.K), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    dY = (torch.randn((w.Tb, w.N), device=dev, generator=gen) * 0.01).to(torch.bfloat16)
    flop = 2.0 * w.Tb * w.K * w.N
    calls = {"forward": lambda: torch.nn.functional.linear(X, W),
             "gradient": lambda: torch.mm(dY.t(), X)}
    out = {"workload": w.name, "shapes": {"forward": [w.Tb, w.K, w.N],
                                          "gradient": [w.N, w.Tb, w.K]}}
    stream = torch.cuda.current_stream()
    for name, fn in calls.items():
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = flop / (ms * 1e-3) / 1e12
        out[name] = {"us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1),
                     "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    return out


def _gram_run(ar, torch, W, X, Y, cfg, w, args):
    """The same job in the Gram form (ar_tune_linear_gram + ar_pack): per-minibatch
    statistics staged inside the call, then one D·H product (2·N·K·3K FLOP on a
    hi/lo bf16 split) and one update kernel per iteration."""
    ws = torch.empty(ar.gram_workspace_size(cfg, ar.AR_BF16 if W.dtype == torch.bfloat16
                                            else ar.AR_F32, w.N, w.K,
                                            ar.AR_BF16 if Y.dtype == torch.bfloat16
                                            else ar.AR_F32), dtype=torch.uint8, device=W.device)
    recs = []

    def step(keep):
        out = ar.tune_linear(W, X, Y, cfg, want_state=False, timed=True, time_every=TIME_EVERY,
                             workspace=ws, gram=True)
        ar.pack(out.codes, out.zp, w.bits)
        if keep:
            recs.append(out)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    iters_total = w.iters * args.steps
    timed = sum(r.times.steps for r in recs)
    prod_ms = sum(r.times.fwd_gemm_ms for r in recs) / timed
    upd_ms = sum(r.times.ste_update_ms for r in recs) / timed
    prod_flop = 2.0 * w.N * w.K * 3 * w.K
    achieved = prod_flop / (prod_ms * 1e-3) / 1e12
    del ws
    torch.cuda.empty_cache()
    return {
        "value": round(iters_total / el, 3), "unit": "iters/s",
        "ms_per_step": round(el / args.steps * 1e3, 3),
        "ms_per_iter": round(el / iters_total * 1e3, 4),
        "kernel_ms_per_iter": {"gram_product": round(prod_ms, 4), "update": round(upd_ms, 4)},
        "roofline": {"kernel": "gram_product", "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4)},
        "first_loss": float(recs[-1].losses[0]), "best_loss": float(recs[-1].losses.min()),
        "note": "same loss with the residual unrounded; per-minibatch H, Cn, e2 staged "
                "inside each timed call",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama7b_q_proj")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", choices=("auto", "on", "off"), default="auto",
                    help="time steps as replays of one HIP graph holding the whole call "
                         "(auto: for launch-bound layers under 1 GFLOP per iteration)")
    ap.add_argument("--no-gram", action="store_true",
                    help="skip the Gram-form run reported under detail.gram")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the block-wise tuning run reported under detail.block")
    ap.add_argument("--block-only", action="store_true",
                    help="only run the block-wise tuning measurement and print its record "
                         "(for a kernel-trace profile of that workload alone)")
    ap.add_argument("--dequant-only", action="store_true",
                    help="only run the one-token packed-format product on the 29568x8192 W4 "
                         "layer at every bit width and print its record (for profiles of that "
                         "kernel alone)")
    ap.add_argument("--yardstick", action="store_true",
                    help="only time the black-box library GEMM (torch: hipBLASLt) on the two "
                         "contraction shapes of the workload's step and print its record "
                         "(for counter profiles of that GEMM beside the library's)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the per-Linear tuning path runs on a single "
              "MI355X (multi-GPU sharding by output rows is a design note, not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import autoround_signsgd_rounding_amd as ar

    if args.block_only:
        print(json.dumps({"block": _block_run(ar, torch)}), flush=True)
        return
    if args.yardstick:
        print(json.dumps({"yardstick": _yardstick(torch, synth.WORKLOADS[args.workload])}),
              flush=True)
        return
    if args.dequant_only:
        print(json.dumps({"dequant_decode": [_decode_large(ar, torch, 20, bits=b)
                                             for b in (4, 2, 3, 8)]}), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    t_gen = time.time()
    case = synth.make_workload_case(w)
    X = torch.from_numpy(case.X_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    Y = synth.reference_outputs_torch(case, dev)
    if w.wdtype == "bf16":
        W = torch.from_numpy(case.W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        W = torch.from_numpy(case.W).to(dev)
    cfg = ar.Config(bits=w.bits, group_size=w.group_size, sym=w.sym, nsamples=w.nsamples,
                    seqlen=w.seqlen, batch_samples=w.batch_samples, iters=w.iters, lr=w.lr,
                    minmax_lr=w.minmax_lr, minmax_shrink=w.minmax_shrink)
    ws = torch.empty(ar.workspace_size(cfg, w.N, w.K, ar.AR_BF16 if Y.dtype == torch.bfloat16
                                       else ar.AR_F32), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    graph = args.graph == "on" or (args.graph == "auto" and w.flop_per_iter < 1e9)

    def step(times):
        out = ar.tune_linear(W, X, Y, cfg, want_state=False, timed=True,
                             time_every=1 if graph else TIME_EVERY, workspace=ws)
        ar.pack(out.codes, out.zp, w.bits)
        times.append((out.times, out))

    if graph:
        recs, el, graph_check = _graph_steps(ar, torch, W, X, Y, cfg, w, ws, args, step)
    else:
        for _ in range(args.warmup):
            step([])
        torch.cuda.synchronize()
        recs = []
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(recs)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0

    iters_total = w.iters * args.steps
    value = iters_total / el
    timed_steps = sum(r[0].steps for r in recs)
    fwd_ms = sum(r[0].fwd_gemm_ms for r in recs) / timed_steps
    wgrad_ms = sum(r[0].wgrad_gemm_ms for r in recs) / timed_steps
    ste_ms = sum(r[0].ste_update_ms for r in recs) / timed_steps
    pack_ms = _pack_time(ar, torch, recs[-1][1], w.bits)
    gemm_flop = 2.0 * w.Tb * w.K * w.N
    kern = {"fwd_gemm": fwd_ms, "wgrad_gemm": wgrad_ms}
    dom = max(kern, key=kern.get)
    achieved = gemm_flop / (kern[dom] * 1e-3) / 1e12
    step_tflops = w.flop_per_iter * iters_total / el / 1e12
    G = w.K // w.group_size
    pack_bytes = w.N * w.K + w.N * w.K * w.bits // 8 + w.N * G * (1 + w.bits / 8)
    final_loss = float(recs[-1][1].losses.min())

    line = {
        "metric": "AutoRound tune iters/sec per Linear (TFLOP/s, % MFMA peak) + pack GB/s",
        "value": round(value, 3),
        "unit": "iters/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(el / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian W/X with outlier columns/channels; Y = X·Wᵀ)",
        "config": {
            "workload": f"{w.name}: Linear {w.K}->{w.N} {w.wdtype}, W{w.bits} "
                        f"{'sym' if w.sym else 'asym'} g{w.group_size}, "
                        f"{w.nsamples}x{w.seqlen} calibration tokens, minibatch "
                        f"{w.batch_samples}x{w.seqlen}, {w.iters} iters, lr {w.lr}",
            "step": f"ar_tune_linear ({w.iters} SignSGD iterations incl. staging and final "
                    f"quantization) + ar_pack" + (", captured once in a HIP graph and replayed "
                                                  "(one replay per step)" if graph else ""),
            "N": w.N, "K": w.K, "Tb": w.Tb, "M": w.M, "iters": w.iters,
        },
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": _measured_traffic(w.name) if dom == "fwd_gemm" else None,
        },
        "detail": {
            "tflops_per_iter_effective": round(step_tflops, 1),
            "mfma_peak_frac_effective": round(step_tflops / PEAK_BF16_TFLOPS, 4),
            "ms_per_iter": round(el / iters_total * 1e3, 4),
            "kernel_ms_per_iter": {"fwd_gemm": round(fwd_ms, 4), "wgrad_gemm": round(wgrad_ms, 4),
                                   "ste_update": round(ste_ms, 4)},
            "kernel_timing": (f"HIP events around the kernels of every step of "
                              f"{len(recs)} eager calls ({timed_steps} steps timed)" if graph else
                              f"HIP events around the kernels of every {TIME_EVERY}th step "
                              f"({timed_steps} steps timed)"),
            "fwd_gemm_tflops": round(gemm_flop / (fwd_ms * 1e-3) / 1e12, 1),
            "wgrad_gemm_tflops": round(gemm_flop / (wgrad_ms * 1e-3) / 1e12, 1),
            "pack_ms": round(pack_ms, 4),
            "pack_timing": "HIP graph of 20 ar_pack calls on the tuned codes, replayed",
            "pack_gbps": round(pack_bytes / (pack_ms * 1e-3) / 1e9, 1),
            "pack_hbm_frac": round(pack_bytes / (pack_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "pack_large": _pack_large(ar, torch),
            "best_loss": final_loss,
            "input_gen_s": round(t_gen, 1),
        },
    }
    if graph:
        line["detail"]["graph_check"] = graph_check
    line["detail"]["tune_step"] = _step_run(ar, torch, W, X, Y, cfg, w)
    if not graph:
        line["detail"]["dequant_gemm"] = _dequant_run(ar, torch, X, recs[-1][1], w)
    if not args.no_block and not graph:
        line["detail"]["block"] = _block_run(ar, torch)
    if not args.no_gram:
        line["detail"]["gram"] = _gram_run(ar, torch, W, X, Y, cfg, w, args)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline(case, Y, w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
