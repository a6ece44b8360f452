"""Write oracle-computed expected values for the long-loop GPU parity test.

Calls only ``oracle`` and ``synth`` (never the HIP library). Runs the full
200-iteration tuning loop of a named workload on the CPU and stores, for a
fixed sample of output rows, the final codes / scales / zero-points / clip
factors, plus the whole loss trajectory and the best step.

    python tests/golden/make_golden.py llama7b_q_proj          # ~15 min on 8 cores
    python tests/golden/make_golden.py llama7b_q_proj --gram   # the oracle's Gram mode
    python tests/golden/make_golden.py --block                 # Llama-7B-shaped block, see below
    python tests/golden/make_golden.py qwen72b_up_proj --short # 8 iterations on 4 minibatches
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

N_ROWS = 128
ROW_SEED = 123


def sample_rows(N):
    return np.sort(np.random.default_rng(ROW_SEED).choice(N, size=min(N_ROWS, N), replace=False))


# A short run of a layer too large for the oracle's 200 iterations: the first
# SHORT_NSAMPLES samples (SHORT_NSAMPLES / batch_samples minibatches), cycled
# for SHORT_ITERS iterations.
SHORT_NSAMPLES, SHORT_ITERS = 32, 8


def main(name, gram=False, short=False):
    w = synth.WORKLOADS[name]
    if short:
        w = synth.Workload(**{**w.__dict__, "nsamples": SHORT_NSAMPLES, "iters": SHORT_ITERS})
    t0 = time.time()
    case = synth.make_workload_case(w)
    Y = synth.reference_outputs(case)
    print(f"inputs ready {time.time() - t0:.1f}s", flush=True)
    cfg = O.Config(bits=w.bits, group_size=w.group_size, sym=w.sym, nsamples=w.nsamples,
                   seqlen=w.seqlen, batch_samples=w.batch_samples, iters=w.iters, lr=w.lr,
                   minmax_lr=w.minmax_lr, minmax_shrink=w.minmax_shrink)
    Tb = w.Tb
    nb = w.nsamples // w.batch_samples

    def minibatch(b):
        xb = synth.bf16_bits_to_f32(case.X_bits[b * Tb:(b + 1) * Tb])
        yb = Y[b * Tb:(b + 1) * Tb]
        yb = synth.bf16_bits_to_f32(yb) if w.wdtype == "bf16" else yb
        return xb, yb

    def on_step(i, r):
        print(f"step {i} loss {r.loss:.9e} t={time.time() - t0:.0f}s", flush=True)

    res = O.tune_linear(case.W, minibatch, nb, cfg, on_step=on_step, gram=gram)
    rtn_codes, _, _, _ = O.rtn_quant(case.W, cfg)
    rows = sample_rows(w.N)
    tag = "tune_gram_" if gram else ("tune_short_" if short else "tune_")
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"{tag}{name}.npz")
    np.savez_compressed(
        out, rows=rows, losses=np.array(res.losses, np.float64),
        best_step=np.int64(res.best_step), best_loss=np.float64(res.best_loss),
        codes=res.codes[rows], scale=res.scale[rows], zp=res.zp[rows],
        alpha=res.alpha[rows], beta=res.beta[rows],
        changed_vs_rtn=np.float64((res.codes != rtn_codes).mean()))
    print(f"wrote {out}; best step {res.best_step} loss {res.best_loss:.6e}; "
          f"codes changed vs RTN {(res.codes != rtn_codes).mean():.4f}", flush=True)


# Block-wise tuning at the Llama-7B block shape (D 4096, 32 heads, F 11008), kept
# small enough for the oracle: 2 sequences of 2048 tokens, minibatches of one
# sequence, 2 iterations per Linear, W4 g128 asym, quantized inputs.
BLOCK_NSAMPLES, BLOCK_ITERS = 2, 2
N_BLOCK_ROWS = 32


def main_block():
    from oracle import block_ref as B
    dims = synth.BLOCKS["llama7b_block"]
    t0 = time.time()
    c = synth.make_block_case(dims, nsamples=BLOCK_NSAMPLES)
    od = synth.BlockDims(dims.name, dims.D, dims.H, dims.F, dims.seqlen, BLOCK_NSAMPLES,
                         dims.rms_eps, dims.rope_theta)
    W = {n: synth.bf16_bits_to_f32(c.W_bits[n]) for n in B.LINEARS}
    norms = tuple(synth.bf16_bits_to_f32(x) for x in c.norm_bits)
    h = synth.bf16_bits_to_f32(c.H_bits)
    cfg = O.Config(bits=4, group_size=128, nsamples=BLOCK_NSAMPLES, seqlen=dims.seqlen,
                   batch_samples=1, iters=BLOCK_ITERS)
    print(f"inputs ready {time.time() - t0:.1f}s", flush=True)
    r = B.tune_block(h, W, norms, od, cfg, quanted_input=True)
    rng = np.random.default_rng(ROW_SEED)
    out = {"err": np.float64(r.err)}
    for n in B.LINEARS:
        res = r.results[n]
        rows = np.sort(rng.choice(res.codes.shape[0], size=N_BLOCK_ROWS, replace=False))
        out[f"{n}_losses"] = np.array(res.losses, np.float64)
        out[f"{n}_rows"] = rows
        out[f"{n}_codes"] = res.codes[rows]
    trows = np.sort(rng.choice(r.out_q.shape[0], size=64, replace=False))
    out["token_rows"] = trows
    out["out_fp"] = r.out_fp[trows]
    out["out_q"] = r.out_q[trows]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tune_block_llama7b.npz")
    np.savez_compressed(path, **out)
    print(f"wrote {path}; block output mse {r.err:.6e}; t={time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    if "--block" in sys.argv:
        main_block()
    else:
        main(args[0] if args else "llama7b_q_proj", gram="--gram" in sys.argv,
             short="--short" in sys.argv)
