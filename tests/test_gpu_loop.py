"""GPU parity of the whole per-Linear tuning loop (ar_tune_linear): final
codes at least 99.9% identical to the oracle's, final loss within 1%."""
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_common import F32, bf16_dev, dev, log, oracle_cfg, to_np, weight_dev

pytestmark = pytest.mark.gpu
ar = pytest.importorskip("autoround_signsgd_rounding_amd")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(w, **kw):
    d = dict(bits=w.bits, group_size=w.group_size, sym=w.sym, nsamples=w.nsamples,
             seqlen=w.seqlen, batch_samples=w.batch_samples, iters=w.iters, lr=w.lr,
             minmax_lr=w.minmax_lr, minmax_shrink=w.minmax_shrink)
    d.update(kw)
    return ar.Config(**d)


def _targets(case):
    Y = synth.reference_outputs(case)
    if case.wdtype == "bf16":
        return synth.bf16_bits_to_f32(Y), bf16_dev(Y)
    return Y, torch.from_numpy(Y).to(dev())


def _oracle_loop(case, Yf, cfg, Tb, nb):
    Xf = synth.bf16_bits_to_f32(case.X_bits)
    return O.tune_linear(case.W, lambda b: (Xf[b * Tb:(b + 1) * Tb], Yf[b * Tb:(b + 1) * Tb]),
                         nb, oracle_cfg(cfg))


def test_toy_full_run():
    """256->256 fp32 layer, W4 asym g64, 20 iterations on all 256 tokens."""
    w = synth.WORKLOADS["toy_256"]
    log("tune_linear toy_256")
    case = synth.make_workload_case(w)
    Yf, Yd = _targets(case)
    cfg = _cfg(w)
    out = ar.tune_linear(weight_dev(case), bf16_dev(case.X_bits), Yd, cfg, want_wq=True)
    torch.cuda.synchronize()
    r = _oracle_loop(case, Yf, cfg, w.Tb, 1)
    losses = to_np(out.losses).astype(np.float64)
    ol = np.array(r.losses)
    log(f"  gpu losses {losses[:3]} ... best {losses.min():.6e}; oracle best {r.best_loss:.6e}")
    assert np.all(np.abs(losses - ol) <= 1e-3 * ol)
    agree = np.mean(to_np(out.codes) == r.codes)
    log(f"  final codes agree {agree:.6f}")
    assert agree >= 0.999
    assert abs(losses.min() - r.best_loss) <= 0.01 * r.best_loss
    assert losses.min() <= losses[0]               # the RTN state was a candidate
    np.testing.assert_array_equal(to_np(out.zp), r.zp)
    assert np.mean(to_np(out.scale) == r.scale) >= 0.99


def test_iters_zero_is_rtn():
    w = synth.WORKLOADS["toy_256"]
    case = synth.make_workload_case(w)
    _, Yd = _targets(case)
    cfg = _cfg(w, iters=0)
    out = ar.tune_linear(weight_dev(case), bf16_dev(case.X_bits), Yd, cfg, want_wq=True)
    codes, scale, zp, Wq = ar.rtn_quant(weight_dev(case), cfg)
    torch.cuda.synchronize()
    for x, y in ((out.codes, codes), (out.scale, scale), (out.zp, zp), (out.Wq, Wq)):
        assert torch.equal(x, y)
    oc, os_, oz, _ = O.rtn_quant(case.W, oracle_cfg(cfg))
    np.testing.assert_array_equal(to_np(codes), oc)
    assert not out.V.any() and torch.all(out.alpha == 1.0)


@pytest.mark.parametrize("K,gs", [(256, 64), (520, 40)])
def test_loop_equals_repeated_steps(K, gs):
    """ar_tune_linear runs the same kernels as ar_tune_step: 7 steps over 3
    minibatches give the bit-identical best state and loss sequence. K = 520
    spans three 256-wide tiles of the staged input, the last one partial."""
    N, seqlen, nsamples = 192, 40, 3
    case = synth.make_case(N, K, nsamples * seqlen, wdtype="bf16", seed=21)
    Yf, Yd = _targets(case)
    cfg = ar.Config(bits=3, group_size=gs, nsamples=nsamples, seqlen=seqlen, batch_samples=1,
                    iters=7)
    Wd, Xd = weight_dev(case), bf16_dev(case.X_bits)
    out = ar.tune_linear(Wd, Xd, Yd, cfg)
    G = K // gs
    V = torch.zeros((N, K), device=dev())
    a = torch.ones((N, G), device=dev())
    b = torch.ones((N, G), device=dev())
    bV, bA, bB = V.clone(), a.clone(), b.clone()
    bL = torch.full((1,), float("inf"), device=dev())
    losses = []
    for i in range(cfg.iters):
        s = i % nsamples
        loss, _, _, _ = ar.tune_step(Wd, V, a, b, Xd[s * seqlen:(s + 1) * seqlen],
                                     Yd[s * seqlen:(s + 1) * seqlen], cfg,
                                     best=(bV, bA, bB, bL), want_grads=False)
        losses.append(loss)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(out.losses), to_np(torch.cat(losses)))
    assert torch.equal(out.V, bV) and torch.equal(out.alpha, bA) and torch.equal(out.beta, bB)
    _, codes, _, _ = ar.fakequant_fwd(Wd, bV, bA, bB, cfg)
    assert torch.equal(codes, out.codes)


def test_loop_is_deterministic():
    w = synth.WORKLOADS["toy_256"]
    case = synth.make_workload_case(w)
    _, Yd = _targets(case)
    cfg = _cfg(w)
    runs = []
    for _ in range(2):
        o = ar.tune_linear(weight_dev(case), bf16_dev(case.X_bits), Yd, cfg)
        torch.cuda.synchronize()
        runs.append((to_np(o.codes), to_np(o.V), to_np(o.losses)))
    for x, y in zip(*runs):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("name", ["llama7b_q_proj", "llama7b_down_proj", "llama7b_gate_proj"])
def test_200_iters_against_oracle_golden(name):
    """A Llama-7B linear (q_proj 4096->4096 W4 g128 asym; down_proj
    11008->4096 W2 g128 asym; gate_proj 4096->11008 W3 g128 sym), 200
    iterations over 16 minibatches of 8x2048 tokens, against the oracle's own
    200-iteration run stored by tests/golden/make_golden.py (codes of 128
    sampled rows, loss trajectory)."""
    path = os.path.join(GOLDEN, f"tune_{name}.npz")
    if not os.path.exists(path):
        pytest.skip("golden file not generated")
    gold = np.load(path)
    w = synth.WORKLOADS[name]
    log(f"tune_linear {name} 200 iters: generating inputs")
    case = synth.make_workload_case(w)
    Xd = bf16_dev(case.X_bits)
    Yd = synth.reference_outputs_torch(case, dev())
    del case.X_bits
    log("  running")
    out = ar.tune_linear(weight_dev(case), Xd, Yd, _cfg(w))
    torch.cuda.synchronize()
    losses = to_np(out.losses).astype(np.float64)
    gl = gold["losses"]
    rows = torch.from_numpy(gold["rows"]).to(dev())
    agree = np.mean(to_np(out.codes[rows]) == gold["codes"])
    log(f"  first loss {losses[0]:.6e} vs {gl[0]:.6e}; best {losses.min():.6e} "
        f"(step {losses.argmin()}) vs {float(gold['best_loss']):.6e} (step {int(gold['best_step'])})"
        f"; sampled-row codes agree {agree:.6f}")
    assert abs(losses[0] - gl[0]) <= 1e-3 * gl[0]
    assert abs(losses.min() - float(gold["best_loss"])) <= 0.01 * float(gold["best_loss"])
    assert agree >= 0.999


def test_short_loop_72b_against_oracle_golden():
    """The Qwen2.5-72B up_proj layer (8192->29568 W4 g128 asym), too large for
    the oracle's 200 iterations: its first 32 samples (4 minibatches of 8x2048
    tokens), 8 iterations (each minibatch twice), against the oracle's run of
    the same problem stored by tests/golden/make_golden.py --short. Every step's
    loss within 1e-3, the same best step, and the codes of 128 sampled rows at
    least 99.9% identical."""
    path = os.path.join(GOLDEN, "tune_short_qwen72b_up_proj.npz")
    if not os.path.exists(path):
        pytest.skip("golden file not generated")
    gold = np.load(path)
    w0 = synth.WORKLOADS["qwen72b_up_proj"]
    w = synth.Workload(**{**w0.__dict__, "nsamples": 32, "iters": 8})
    log("tune_linear qwen72b_up_proj, 32 samples, 8 iters: generating inputs")
    case = synth.make_workload_case(w)
    Xd = bf16_dev(case.X_bits)
    Yd = synth.reference_outputs_torch(case, dev())
    del case.X_bits
    out = ar.tune_linear(weight_dev(case), Xd, Yd, _cfg(w))
    torch.cuda.synchronize()
    losses = to_np(out.losses).astype(np.float64)
    gl = gold["losses"]
    rows = torch.from_numpy(gold["rows"]).to(dev())
    agree = np.mean(to_np(out.codes[rows]) == gold["codes"])
    log(f"  losses {losses}\n  oracle {gl}\n  best step {int(losses.argmin())} vs "
        f"{int(gold['best_step'])}; sampled-row codes agree {agree:.6f}")
    assert np.all(np.abs(losses - gl) <= 1e-3 * gl)
    assert int(losses.argmin()) == int(gold["best_step"])
    assert agree >= 0.999


@pytest.mark.parametrize("every", [1, 3, 40])
def test_timed_mode_samples_steps_and_changes_nothing(every):
    """Event timing on every `every`-th step: the step count is ceil(iters /
    every), every kernel time is positive, and the results are bit-identical to
    an untimed run."""
    w = synth.WORKLOADS["toy_256"]
    case = synth.make_workload_case(w)
    _, Yd = _targets(case)
    cfg = _cfg(w)
    Wd, Xd = weight_dev(case), bf16_dev(case.X_bits)
    plain = ar.tune_linear(Wd, Xd, Yd, cfg)
    timed = ar.tune_linear(Wd, Xd, Yd, cfg, timed=True, time_every=every)
    torch.cuda.synchronize()
    t = timed.times
    assert t.steps == -(-cfg.iters // every) and t.sample_every == every
    assert min(t.fwd_gemm_ms, t.wgrad_gemm_ms, t.ste_update_ms) > 0
    for x, y in ((plain.codes, timed.codes), (plain.V, timed.V), (plain.losses, timed.losses)):
        assert torch.equal(x, y)
