"""GPU parity of one SignSGD step (ar_tune_step) from an identical state:
loss and the V / alpha / beta gradients within 1e-3 relative (norm-wise for
the gradients), the updated state, and the best-loss snapshot."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_common import F32, bf16_dev, dev, log, oracle_cfg, rel_norm, to_np, weight_dev

pytestmark = pytest.mark.gpu
ar = pytest.importorskip("autoround_signsgd_rounding_amd")

TOL = 1e-3


def _inputs(N, K, Tb, wdtype, ydtype, seed, sigma_w=0.02, outliers=True):
    case = synth.make_case(N, K, Tb, wdtype=wdtype, sigma_w=sigma_w, outliers=outliers, seed=seed)
    Y = synth.reference_outputs(case)
    Yf = synth.bf16_bits_to_f32(Y) if wdtype == "bf16" else Y
    if ydtype == "bf16":
        Yf = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(Yf))
        Yd = bf16_dev(synth.f32_to_bf16_bits(Yf))
    else:
        Yd = torch.from_numpy(np.ascontiguousarray(Yf)).to(dev())
    return case, Yf, Yd


def _state(N, K, G, seed, random=True, shrink=1.0):
    rng = np.random.default_rng(seed)
    if random:
        V = rng.uniform(-0.5, 0.5, (N, K)).astype(F32)
        a = rng.uniform(0.5, 1.0, (N, G)).astype(F32)
        b = rng.uniform(0.5, 1.0, (N, G)).astype(F32)
    else:
        V = np.zeros((N, K), F32)
        a = np.full((N, G), F32(shrink))
        b = a.copy()
    return V, a, b


def _gpu(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(x)).to(dev()) for x in arrs]


STEP_CASES = [
    # N, K, Tb, wdtype, ydtype, bits, group, sym, minmax_lr
    (300, 384, 520, "bf16", "bf16", 4, 128, False, None),   # ragged N and Tb, 2x3 fwd tiles
    (257, 256, 264, "f32", "f32", 3, 64, True, None),
    (64, 512, 256, "bf16", "bf16", 2, -1, False, 0.01),
    (520, 200, 136, "bf16", "f32", 8, 40, False, None),     # ragged K and Tb reductions
    (100, 1024, 1032, "bf16", "bf16", 4, 1024, False, 0.0), # frozen clip factors
    (1, 64, 8, "f32", "f32", 4, 64, True, None),            # one row, one 8-token batch
    # ragged N and Tb over 17 x 17 = 289 forward tiles: with one workgroup per CU some run a
    # second tile; K = 640 is the shortest reduction the streamed forward takes (20 steps)
    (4100, 640, 4104, "bf16", "bf16", 4, 128, False, None),
    # float32 targets take the one-tile forward (EpiFwdF32): long reductions, ragged tiles
    (300, 1024, 520, "f32", "f32", 4, 128, False, None),
    (260, 768, 264, "bf16", "f32", 3, 128, True, None),
]


@pytest.mark.parametrize("N,K,Tb,wdtype,ydtype,bits,g,sym,mlr", STEP_CASES)
def test_tune_step_parity(N, K, Tb, wdtype, ydtype, bits, g, sym, mlr):
    log(f"tune_step N={N} K={K} Tb={Tb} {wdtype}/{ydtype} b{bits} g{g} sym={sym}")
    case, Yf, Yd = _inputs(N, K, Tb, wdtype, ydtype, seed=N * 7 + K)
    G = 1 if g == -1 else K // g
    V, a, b = _state(N, K, G, seed=N + K + Tb)
    cfg = ar.Config(bits=bits, group_size=g, sym=sym, minmax_lr=mlr)
    Vd, ad, bd = _gpu(V, a, b)
    bV, bA, bB = (torch.full_like(Vd, 7.0), torch.full_like(ad, 7.0), torch.full_like(bd, 7.0))
    bL = torch.full((1,), float("inf"), device=dev())
    Xd = bf16_dev(case.X_bits)
    loss, gV, ga, gb = ar.tune_step(weight_dev(case), Vd, ad, bd, Xd, Yd, cfg,
                                    best=(bV, bA, bB, bL))
    torch.cuda.synchronize()

    oc = oracle_cfg(cfg)
    wmin, wmax = O.group_minmax(case.W, g)
    Xf = synth.bf16_bits_to_f32(case.X_bits)
    r = O.tune_step(case.W, V, a, b, wmin, wmax, Xf, Yf, oc)

    L = float(to_np(loss)[0])
    assert abs(L - r.loss) <= TOL * r.loss, (L, r.loss)
    assert rel_norm(to_np(gV), r.gV) <= TOL
    if np.linalg.norm(r.galpha) > 0:
        assert rel_norm(to_np(ga), r.galpha) <= TOL
    if np.linalg.norm(r.gbeta) > 0:
        assert rel_norm(to_np(gb), r.gbeta) <= TOL
    agree_V = np.mean(to_np(Vd) == r.V)
    agree_a = np.mean(to_np(ad) == r.alpha)
    agree_b = np.mean(to_np(bd) == r.beta)
    log(f"  loss {L:.6e} vs {r.loss:.6e}; updated V agree {agree_V:.6f}, "
        f"alpha {agree_a:.4f}, beta {agree_b:.4f}")
    assert agree_V >= 0.999 and agree_a >= 0.99 and agree_b >= 0.99
    # first evaluation always improves on +inf: the pre-update state is snapshotted
    assert float(to_np(bL)[0]) == L
    np.testing.assert_array_equal(to_np(bV), V)
    np.testing.assert_array_equal(to_np(bA), a)
    np.testing.assert_array_equal(to_np(bB), b)


def test_snapshot_only_on_strict_improvement():
    N, K, Tb = 64, 128, 64
    case, Yf, Yd = _inputs(N, K, Tb, "bf16", "bf16", seed=3)
    V, a, b = _state(N, K, 1, seed=4)
    cfg = ar.Config(bits=4, group_size=128)
    Vd, ad, bd = _gpu(V, a, b)
    bV, bA, bB = torch.zeros_like(Vd), torch.zeros_like(ad), torch.zeros_like(bd)
    bL = torch.full((1,), -1.0, device=dev())            # nothing beats a negative loss
    loss, _, _, _ = ar.tune_step(weight_dev(case), Vd, ad, bd, bf16_dev(case.X_bits), Yd, cfg,
                                 best=(bV, bA, bB, bL), want_grads=False)
    torch.cuda.synchronize()
    assert float(to_np(bL)[0]) == -1.0 and float(to_np(loss)[0]) > 0
    assert not bV.any() and not bA.any()
    # apply_update = 0 leaves the state alone
    V2 = Vd.clone()
    ar.tune_step(weight_dev(case), Vd, ad, bd, bf16_dev(case.X_bits), Yd, cfg,
                 apply_update=False, want_grads=False)
    torch.cuda.synchronize()
    assert torch.equal(V2, Vd)


def test_step_is_deterministic():
    N, K, Tb = 300, 384, 520
    case, Yf, Yd = _inputs(N, K, Tb, "bf16", "bf16", seed=5)
    V, a, b = _state(N, K, 3, seed=6)
    cfg = ar.Config(bits=4, group_size=128)
    outs = []
    for _ in range(2):
        Vd, ad, bd = _gpu(V, a, b)
        loss, gV, ga, gb = ar.tune_step(weight_dev(case), Vd, ad, bd, bf16_dev(case.X_bits), Yd,
                                        cfg)
        torch.cuda.synchronize()
        outs.append([to_np(t) for t in (loss, gV, ga, gb, Vd, ad, bd)])
    for x, y in zip(*outs):
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))


BIG = ["llama7b_q_proj", "llama7b_down_proj", "llama7b_gate_proj", "qwen72b_up_proj"]


@pytest.mark.parametrize("name", BIG)
def test_tune_step_full_size(name):
    """One step at the workload's full shape and minibatch (Tb = 16384 tokens),
    launched as the tuning loop launches it. Rows of the problem are independent
    apart from the loss normalisation, so the oracle checks the gradients and
    updated state of 32 sampled rows, and the loss of the whole problem."""
    w = synth.WORKLOADS[name]
    log(f"tune_step full size {name}")
    case = synth.make_case(w.N, w.K, w.Tb, wdtype=w.wdtype, sigma_w=w.sigma_w,
                           outliers=w.outliers, seed=w.seed)
    Yd = synth.reference_outputs_torch(case, dev())
    G = w.K // w.group_size
    V, a, b = _state(w.N, w.K, G, seed=11)
    cfg = ar.Config(bits=w.bits, group_size=w.group_size, sym=w.sym, minmax_lr=w.minmax_lr,
                    minmax_shrink=w.minmax_shrink)
    Vd, ad, bd = _gpu(V, a, b)
    loss, gV, ga, gb = ar.tune_step(weight_dev(case), Vd, ad, bd, bf16_dev(case.X_bits), Yd, cfg)
    torch.cuda.synchronize()
    L = float(to_np(loss)[0])
    log(f"  gpu loss {L:.6e}")
    rows = np.sort(np.random.default_rng(1).choice(w.N, 32, replace=False))
    rt = torch.from_numpy(rows).to(dev())
    Xf = synth.bf16_bits_to_f32(case.X_bits)
    Yr = to_np(Yd[:, rt]).astype(F32)
    oc = oracle_cfg(cfg)
    wmin, wmax = O.group_minmax(case.W[rows], w.group_size)
    r = O.tune_step(case.W[rows], V[rows], a[rows], b[rows], wmin, wmax, Xf, Yr, oc,
                    n_scale=w.N)
    assert rel_norm(to_np(gV[rt]), r.gV) <= TOL
    assert rel_norm(to_np(ga[rt]), r.galpha) <= TOL
    assert rel_norm(to_np(gb[rt]), r.gbeta) <= TOL
    agree = np.mean(to_np(Vd[rt]) == r.V)
    log(f"  sampled rows: updated V agree {agree:.6f}")
    assert agree >= 0.999
    Lo = _oracle_loss(case.W, V, a, b, Xf, to_np(Yd), w.group_size, w.bits, w.sym)
    log(f"  oracle loss {Lo:.6e}")
    assert abs(L - Lo) <= TOL * Lo


def _oracle_loss(W, V, a, b, Xf, Y, g, bits, sym, chunk=4096):
    """The oracle's loss of the whole problem, summed over row chunks (rows are
    independent apart from the normalisation, which n_scale carries)."""
    N = W.shape[0]
    total = 0.0
    for r0 in range(0, N, chunk):
        sl = slice(r0, min(N, r0 + chunk))
        wmin, wmax = O.group_minmax(W[sl], g)
        qp = O.qparams(wmin, wmax, a[sl], b[sl], bits, sym)
        fq = O.fake_quant(W[sl], V[sl], qp, bits, g)
        _, _, ls = O.forward_backward(Xf, Y[:, sl], fq.what, n_scale=N)
        total += ls
    return total / (Xf.shape[0] * N)


def test_tune_step_partial_last_wave():
    """A shape whose products have a partial last wave (17 x 17 = 289 gradient
    tiles and 8 x 17 forward tiles for 256 compute units): the loss of the
    whole problem, the gradients and updated state of 64 sampled rows (every
    tile column), and two runs bit for bit."""
    N = K = 4352
    Tb = 2048
    log(f"tune_step partial last wave N={N} K={K} Tb={Tb}")
    case, Yf, Yd = _inputs(N, K, Tb, "bf16", "bf16", seed=21)
    G = K // 128
    V, a, b = _state(N, K, G, seed=22)
    cfg = ar.Config(bits=4, group_size=128)
    outs = []
    for _ in range(2):
        Vd, ad, bd = _gpu(V, a, b)
        loss, gV, ga, gb = ar.tune_step(weight_dev(case), Vd, ad, bd, bf16_dev(case.X_bits), Yd,
                                        cfg)
        torch.cuda.synchronize()
        outs.append([to_np(t) for t in (loss, gV, ga, gb, Vd, ad, bd)])
    for x, y in zip(*outs):
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))
    L, gV, ga, gb, Vn = outs[0][0][0], outs[0][1], outs[0][2], outs[0][3], outs[0][4]
    rows = np.sort(np.random.default_rng(2).choice(N, 64, replace=False))
    Xf = synth.bf16_bits_to_f32(case.X_bits)
    wmin, wmax = O.group_minmax(case.W[rows], 128)
    r = O.tune_step(case.W[rows], V[rows], a[rows], b[rows], wmin, wmax, Xf, Yf[:, rows],
                    oracle_cfg(cfg), n_scale=N)
    assert rel_norm(gV[rows], r.gV) <= TOL
    assert rel_norm(ga[rows], r.galpha) <= TOL and rel_norm(gb[rows], r.gbeta) <= TOL
    assert np.mean(Vn[rows] == r.V) >= 0.999
    Lo = _oracle_loss(case.W, V, a, b, Xf, Yf, 128, 4, False)
    log(f"  loss {L:.6e} vs oracle {Lo:.6e}")
    assert abs(L - Lo) <= TOL * Lo
