"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names the part of the oracle it pins and what it is pinned to:
hand-derived vectors (tests/golden/), a nearest-grid search, an exhaustive
search, torch autograd, the Gram (H = XᵀX) identity, a library bf16 cast and
big-integer packing.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _cfg(**kw):
    return O.Config(**kw)


# ------------------------------------------------------------------ bf16
def test_bf16_matches_library_cast():
    """bf16() against torch's float32 -> bfloat16 cast (round to nearest even)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000).astype(F32) * F32(3.0)
    # exact ties and edge values
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7FFFFF, 0x00008000,
                     0x00018000, 0x7F800000, 0xFF800000, 0x80000000, 0x00000001],
                    dtype=np.uint32).view(F32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = O.bf16(x)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(O.bf16(np.array([np.nan], F32)))[0]


# ------------------------------------------------------------------ S1
def test_group_minmax_against_loops():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((3, 24)).astype(F32)
    mn, mx = O.group_minmax(W, 8)
    for n in range(3):
        for j in range(3):
            vals = [float(W[n, j * 8 + i]) for i in range(8)]
            assert mn[n, j] == min(vals) and mx[n, j] == max(vals)
    mn, mx = O.group_minmax(W, -1)
    assert mn.shape == (3, 1) and mx[1, 0] == W[1].max()


# ------------------------------------------------------------------ S2, S3
def _hand_cases():
    with open(os.path.join(GOLDEN, "hand_vectors.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_hand_vectors(case):
    """qparams + fake_quant against hand-derived vectors (tests/golden)."""
    W = np.array([case["W"]], F32)
    V = np.array([case["V"]], F32)
    g = case["group_size"]
    wmin, wmax = O.group_minmax(W, g)
    a = np.full(wmin.shape, F32(case["alpha"]))
    b = np.full(wmin.shape, F32(case["beta"]))
    qp = O.qparams(wmin, wmax, a, b, case["bits"], case["sym"])
    assert qp.s[0, 0] == F32(case["s"])
    assert qp.zp[0, 0] == case["zp"]
    fq = O.fake_quant(W, V, qp, case["bits"], g)
    np.testing.assert_array_equal(fq.q[0].astype(int), case["codes"])
    np.testing.assert_array_equal(fq.m[0].astype(int), case["mask"])
    np.testing.assert_array_equal(fq.what[0], np.array(case["what"], F32))


@pytest.mark.parametrize("bits,sym", [(2, False), (3, False), (4, False), (8, False),
                                      (2, True), (3, True), (4, True), (8, True)])
def test_rtn_is_nearest_grid_point(bits, sym):
    """With V = 0 and alpha = beta = 1 each code is the grid point nearest to
    W (the RTN equation), found here by searching every code q in [0, maxq]."""
    rng = np.random.default_rng(bits * 10 + sym)
    N, K, g = 16, 64, 16
    W = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    W[3, :16] = np.abs(W[3, :16])          # an all-positive group
    W[5, 16:32] = -np.abs(W[5, 16:32])     # an all-negative group
    cfg = _cfg(bits=bits, sym=sym, group_size=g)
    codes, s, zp, what = O.rtn_quant(W, cfg)
    maxq = 2 ** bits - 1
    assert codes.max() <= maxq and zp.max() <= maxq
    s_e = np.repeat(s, g, axis=1).astype(np.float64)
    zp_e = np.repeat(zp, g, axis=1).astype(np.float64)
    grid = s_e[..., None] * (np.arange(maxq + 1)[None, None, :] - zp_e[..., None])
    dist = np.abs(grid - W.astype(np.float64)[..., None])
    nearest = dist.argmin(axis=2)
    t64 = W.astype(np.float64) / s_e
    frac = np.abs(t64 - np.floor(t64) - 0.5)
    clear = frac > 1e-5                   # away from exact halves
    np.testing.assert_array_equal(codes[clear], nearest[clear])
    # |what - W| <= s/2 in range
    err = np.abs(what.astype(np.float64) - W.astype(np.float64))
    inrange = (np.abs(t64 + zp_e - np.clip(t64 + zp_e, 0, maxq)) == 0) & clear
    assert np.all(err[inrange] <= s_e[inrange] * 0.5 * (1 + 1e-6))


def test_codes_and_offsets_stay_in_range():
    rng = np.random.default_rng(3)
    N, K, g = 8, 128, 32
    W = (rng.standard_normal((N, K)) * 0.05).astype(F32)
    V = rng.uniform(-0.5, 0.5, (N, K)).astype(F32)
    for bits in O.SUPPORTED_BITS:
        for sym in (False, True):
            wmin, wmax = O.group_minmax(W, g)
            a = rng.uniform(0.5, 1.0, wmin.shape).astype(F32)
            b = rng.uniform(0.5, 1.0, wmin.shape).astype(F32)
            qp = O.qparams(wmin, wmax, a, b, bits, sym)
            fq = O.fake_quant(W, V, qp, bits, g)
            assert fq.q.min() >= 0 and fq.q.max() <= 2 ** bits - 1
            assert qp.zp.min() >= 0 and qp.zp.max() <= 2 ** bits - 1
            assert np.all(qp.s > 0)


def test_offset_zero_reproduces_rint():
    """V = 0 turns the offset equation into the RTN equation."""
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((4, 64)) * 0.02).astype(F32)
    wmin, wmax = O.group_minmax(W, 16)
    one = np.ones_like(wmin)
    qp = O.qparams(wmin, wmax, one, one, 4, False)
    fq = O.fake_quant(W, np.zeros_like(W), qp, 4, 16)
    s_e = np.repeat(qp.s, 16, axis=1)
    zp_e = np.repeat(qp.zp, 16, axis=1)
    np.testing.assert_array_equal(fq.q, np.clip(np.rint(W / s_e) + zp_e, 0, 15))


# ------------------------------------------------------------------ S4-S7
def _problem(N=6, K=32, T=40, seed=5, sym=False, bits=3, g=8):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    W[0, :g] = np.abs(W[0, :g]) + F32(0.001)   # all-positive group
    X = rng.standard_normal((T, K))
    Y = X @ W.astype(np.float64).T
    wmin, wmax = O.group_minmax(W, g)
    a = rng.uniform(0.6, 1.0, wmin.shape).astype(F32)
    b = rng.uniform(0.6, 1.0, wmin.shape).astype(F32)
    V = rng.uniform(-0.5, 0.5, (N, K)).astype(F32)
    return W, X, Y, wmin, wmax, a, b, V


def test_loss_and_grad_gram_identity():
    """Exact mode: L = Tr(ΔW·H·ΔWᵀ)/(T·N) and G = 2·ΔW·H/(T·N) with H = XᵀX
    (the Hessian form of the layer objective on the ADMM-Q page)."""
    W, X, Y, wmin, wmax, a, b, V = _problem()
    qp = O.qparams(wmin, wmax, a, b, 3, False)
    fq = O.fake_quant(W, V, qp, 3, 8)
    L, G, _ = O.forward_backward(X, Y, fq.what, amp=False)
    T, N = X.shape[0], W.shape[0]
    dW = fq.what.astype(np.float64) - W.astype(np.float64)
    H = X.T @ X
    np.testing.assert_allclose(L, np.trace(dW @ H @ dW.T) / (T * N), rtol=1e-10)
    np.testing.assert_allclose(G, 2.0 * dW @ H / (T * N), rtol=1e-9, atol=1e-15)


def _gram_problem(seed=5, N=20, K=48, T=64, wdt="f32"):
    """bf16 tokens, a target that the unquantized layer does not reproduce
    exactly (bf16-rounded product plus noise), and an arbitrary state."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.03).astype(F32)
    if wdt == "bf16":
        W = O.bf16(W)
    X = O.bf16(rng.standard_normal((T, K)).astype(F32))
    Y = O.bf16((X.astype(np.float64) @ W.astype(np.float64).T
                + 0.01 * rng.standard_normal((T, N))).astype(F32))
    wmin, wmax = O.group_minmax(W, 8)
    a = rng.uniform(0.6, 1.0, wmin.shape).astype(F32)
    b = rng.uniform(0.6, 1.0, wmin.shape).astype(F32)
    V = rng.uniform(-0.5, 0.5, (N, K)).astype(F32)
    qp = O.qparams(wmin, wmax, a, b, 4, False)
    fq = O.fake_quant(W, V, qp, 4, 8)
    return W, X, Y, fq


@pytest.mark.parametrize("wdt", ["f32", "bf16"])
def test_gram_form_equals_token_form(wdt):
    """The Gram form reproduces the token form of the same loss: with the bf16
    operand Ŵ, R = Xb·bf16(Ŵ)ᵀ − Yb summed over tokens in float64 gives
    sum(R²) and the gradient (2/(T·N))·Rᵀ·Xb."""
    W, X, Y, fq = _gram_problem(wdt=wdt)
    T, N = X.shape[0], W.shape[0]
    R = X.astype(np.float64) @ O.bf16(fq.what).astype(np.float64).T - Y.astype(np.float64)
    st = O.gram_stats(X, Y, W)
    L, G, loss_sum = O.forward_backward_gram(st, W, fq.what)
    np.testing.assert_allclose(loss_sum, np.sum(R * R), rtol=1e-10)
    np.testing.assert_allclose(L, np.sum(R * R) / (T * N), rtol=1e-10)
    Gt = 2.0 * R.T @ X.astype(np.float64) / (T * N)
    assert np.abs(G - Gt).max() <= 1e-10 * np.abs(Gt).max()
    # and the same loss as the token-form oracle (whose loss also keeps R unrounded)
    L_tok, _, _ = O.forward_backward(X, Y, fq.what, amp=True)
    np.testing.assert_allclose(L, L_tok, rtol=1e-10)


def test_gram_stats_vanish_for_exact_targets():
    """Yb = Xb·Wᵀ exactly: the target terms vanish and the loss is the
    Hessian-weighted form Tr(D·H·Dᵀ)/(T·N) of the ADMM-Q page."""
    W, X, _, fq = _gram_problem(seed=6)
    Y = X.astype(np.float64) @ W.astype(np.float64).T
    st = O.gram_stats(X, Y, W)
    assert st.e2 == 0.0 and not st.Cn.any()
    D = O.bf16(fq.what).astype(np.float64) - W.astype(np.float64)
    T, N = X.shape[0], W.shape[0]
    L, G, _ = O.forward_backward_gram(st, W, fq.what)
    np.testing.assert_allclose(L, np.trace(D @ st.H @ D.T) / (T * N), rtol=1e-12)
    np.testing.assert_allclose(st.H, st.H.T, rtol=0, atol=0)


def test_gram_loop_first_loss_matches_token_loop():
    """Both loop modes evaluate the same RTN state first, with the same
    unrounded residual, so the first losses agree; every Gram-mode loss is
    the token-form loss of the state it was taken at."""
    W, X, Y = _full_batch_problem()
    cfg = _cfg(bits=4, group_size=16, iters=12)
    seen = []
    r_g = O.tune_linear(W, lambda b: (X, Y), 1, cfg, gram=True,
                        on_step=lambda i, r: seen.append(r.what))
    r_t = O.tune_linear(W, lambda b: (X, Y), 1, cfg)
    np.testing.assert_allclose(r_g.losses[0], r_t.losses[0], rtol=1e-10)
    for L, what in zip(r_g.losses, seen):
        Lt, _, _ = O.forward_backward(X, Y, what, amp=True)
        np.testing.assert_allclose(L, Lt, rtol=1e-9)
    assert r_g.best_loss == min(r_g.losses) and r_g.best_loss <= r_g.losses[0]


def test_amp_rounds_dy_to_bf16_hand_value():
    """amp=True ([LLMC] parameter table: mixed precision) rounds the residual to
    bf16 before the gradient product, while the loss keeps it unrounded. One
    token, one output, K = 2: X = [1, 0.5], Ŵ = [1, 0], Y = 2^-9, so
    R = 1 - 2^-9 = 0.111111111b needs 9 significant bits; bf16 keeps 8, the
    dropped bit is exactly half an ulp and the tie goes to the even neighbour
    1.0. By hand: L = (1 - 2^-9)^2, G = (2/(T·N))·bf16(R)·X = 2·[1, 0.5] = [2, 1]
    (unrounded it would be [1.99609375, 0.998046875])."""
    X = np.array([[1.0, 0.5]], F32)
    Wq = np.array([[1.0, 0.0]], F32)
    Y = np.array([[2.0 ** -9]], F32)
    L, G, loss_sum = O.forward_backward(X, Y, Wq, amp=True)
    assert L == (1.0 - 2.0 ** -9) ** 2 and loss_sum == L
    np.testing.assert_array_equal(G, np.array([[2.0, 1.0]]))
    # amp=False keeps the residual exact
    _, G2, _ = O.forward_backward(X, Y, Wq, amp=False)
    np.testing.assert_array_equal(G2, np.array([[1.99609375, 0.998046875]]))


def test_empty_minibatch_is_rejected():
    """The loss is a mean over the minibatch ([LLMC] tuning loop, ``.mean()``):
    an empty minibatch has none, and the oracle refuses it instead of
    dividing by zero."""
    with pytest.raises(ValueError):
        O.forward_backward(np.zeros((0, 8), F32), np.zeros((0, 4), F32), np.zeros((4, 8), F32))


def test_amp_close_to_exact():
    W, X, Y, wmin, wmax, a, b, V = _problem(K=64, T=64)
    qp = O.qparams(wmin, wmax, a, b, 3, False)
    fq = O.fake_quant(W, V, qp, 3, 8)
    Xb = O.bf16(X.astype(F32))
    L1, G1, _ = O.forward_backward(Xb, Y, fq.what, amp=True)
    L2, G2, _ = O.forward_backward(Xb, Y, fq.what, amp=False)
    assert abs(L1 - L2) / L2 < 2e-2
    assert np.linalg.norm(G1 - G2) / np.linalg.norm(G2) < 5e-2


# ------------------------------------------------------------------ S8
def _autograd_grads(W, X, Y, wmin, wmax, a, b, V, bits, sym, g):
    """The same forward in torch float64 with a straight-through rint
    (x + (round(x) - x).detach()); gradients by autograd."""
    d = torch.float64
    Wt = torch.tensor(W, dtype=d)
    Vt = torch.tensor(V, dtype=d, requires_grad=True)
    at = torch.tensor(a, dtype=d, requires_grad=True)
    bt = torch.tensor(b, dtype=d, requires_grad=True)
    mn = torch.tensor(wmin, dtype=d)
    mx = torch.tensor(wmax, dtype=d)
    maxq = 2 ** bits - 1

    def rint_ste(x):
        return x + (torch.round(x) - x).detach()

    if sym:
        amax = torch.maximum((at * mn).abs(), (bt * mx).abs())
        s = 2 * amax / maxq
        s = torch.where(s == 0, torch.ones_like(s), s)
        zp = torch.full_like(s, 2 ** (bits - 1))
    else:
        lo = torch.minimum(at * mn, torch.zeros_like(mn))
        hi = torch.maximum(bt * mx, torch.zeros_like(mx))
        s = (hi - lo) / maxq
        s = torch.where(s == 0, torch.ones_like(s), s)
        zp = torch.clamp(rint_ste(-lo / s), 0, maxq)
    s_e = s.repeat_interleave(g, dim=1)
    zp_e = zp.repeat_interleave(g, dim=1)
    q = torch.clamp(rint_ste(Wt / s_e + Vt) + zp_e, 0, maxq)
    what = s_e * (q - zp_e)
    Yp = torch.tensor(X, dtype=d) @ what.T
    L = ((Yp - torch.tensor(Y, dtype=d)) ** 2).mean()
    L.backward()
    return Vt.grad.numpy(), at.grad.numpy(), bt.grad.numpy()


@pytest.mark.parametrize("sym,bits", [(False, 2), (False, 3), (False, 4), (True, 3), (True, 4)])
def test_ste_grads_match_autograd(sym, bits):
    W, X, Y, wmin, wmax, a, b, V = _problem(seed=10 + bits, sym=sym, bits=bits)
    g = 8
    qp = O.qparams(wmin, wmax, a, b, bits, sym)
    fq = O.fake_quant(W, V, qp, bits, g)
    L, G, _ = O.forward_backward(X, Y, fq.what, amp=False)
    gV, ga, gb = O.ste_grads(G, W, fq, qp, wmin, wmax, a, b, bits, sym, g)
    rV, ra, rb = _autograd_grads(W, X, Y, wmin, wmax, a, b, V, bits, sym, g)
    # float32 (oracle) vs float64 (autograd) forward: agreement to ~1e-5; a
    # wrong sign or a dropped term would be an O(1) difference.
    np.testing.assert_allclose(gV, rV, rtol=1e-4, atol=1e-6 * np.abs(rV).max())
    np.testing.assert_allclose(ga, ra, rtol=1e-4, atol=1e-6 * np.abs(ra).max())
    np.testing.assert_allclose(gb, rb, rtol=1e-4, atol=1e-6 * np.abs(rb).max())
    assert np.abs(ga).max() > 0 and np.abs(gb).max() > 0


def test_ste_sym_tie_goes_to_beta_hand_value():
    """Symmetric grid with |alpha·wmin| = |beta·wmax|: the clip-factor gradient
    goes to beta alone (the pages are silent; max() has no unique derivative
    at a tie, and the reading taken is that the max side wins). 2-bit sym,
    one group W = [-0.5, 0, 0.25, 0.5], alpha = beta = 1: amax = 0.5,
    s = 2·0.5/3 (float32 0.33333334), zp = 2; t = W/s = [-1.5, 0, 0.75, 1.5];
    rint = [-2, 0, 1, 2]; c = [0, 2, 3, 4]; q = [0, 2, 3, 3]; m = [1, 1, 1, 0].
    With G = 1 everywhere: A = Σ G·((q - zp) - m·t) = (-2 + 1.5) + 0 +
    (1 - 0.75) + 1 = 0.75; dL/damax = 2A/maxq = 0.5; so dL/dbeta = 0.5·|wmax| =
    0.25 and dL/dalpha = 0; dL/dV = G·s·m."""
    W = np.array([[-0.5, 0.0, 0.25, 0.5]], F32)
    V = np.zeros_like(W)
    a = np.ones((1, 1), F32)
    b = np.ones((1, 1), F32)
    wmin, wmax = O.group_minmax(W, 4)
    qp = O.qparams(wmin, wmax, a, b, 2, True)
    fq = O.fake_quant(W, V, qp, 2, 4)
    np.testing.assert_array_equal(fq.q[0], [0, 2, 3, 3])
    np.testing.assert_array_equal(fq.m[0], [True, True, True, False])
    G = np.ones((1, 4))
    gV, ga, gb = O.ste_grads(G, W, fq, qp, wmin, wmax, a, b, 2, True, 4)
    assert ga[0, 0] == 0.0
    assert abs(gb[0, 0] - 0.25) < 1e-7
    s = float(F32(1.0) / F32(3.0))
    np.testing.assert_allclose(gV[0], [s, s, s, 0.0], rtol=1e-7)


# ------------------------------------------------------------------ S9
def test_signsgd_update_invariants():
    rng = np.random.default_rng(7)
    cfg = _cfg(lr=0.005, minmax_lr=0.01)
    V = rng.uniform(-0.5, 0.5, (4, 64)).astype(F32)
    V[0, :4] = [0.5, -0.5, 0.498, 0.0]
    gV = rng.standard_normal((4, 64))
    gV[0, :4] = [-1.0, 1.0, -1.0, 0.0]
    a = np.array([[1.0, 0.5, 0.75, 0.7]], F32)
    ga = np.array([[-1.0, 1.0, 0.0, 2.0]])
    Vn, an, bn = O.signsgd_update(V, a, a, gV, ga, -ga, cfg)
    assert Vn.min() >= -0.5 and Vn.max() <= 0.5
    np.testing.assert_array_equal(Vn[0, :4], np.array([0.5, -0.5, 0.5, 0.0], F32))
    dV = Vn.astype(np.float64) - V
    assert np.all(dV * gV <= 0)                       # against the gradient
    assert np.all(np.abs(dV) <= 0.005 * (1 + 1e-6))
    np.testing.assert_array_equal(an[0], np.array([1.0, 0.5, 0.75, F32(0.7) - F32(0.01)], F32))
    np.testing.assert_array_equal(bn[0], np.array([F32(1.0) - F32(0.01), F32(0.5) + F32(0.01),
                                                   0.75, F32(0.7) + F32(0.01)], F32))


# ------------------------------------------------------------------ whole loop
def _full_batch_problem(N=4, K=32, T=64, g=16, seed=11):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    X = O.bf16(rng.standard_normal((T, K)).astype(F32))
    Y = (X.astype(np.float64) @ W.astype(np.float64).T).astype(F32)
    return W, X, Y


def test_iters_zero_is_rtn():
    """Zero iterations give the RTN result (Introducing AutoRound page,
    section 4)."""
    W, X, Y = _full_batch_problem()
    cfg = _cfg(bits=4, group_size=16, iters=0)
    r = O.tune_linear(W, lambda b: (X, Y), 1, cfg)
    codes, s, zp, what = O.rtn_quant(W, cfg)
    np.testing.assert_array_equal(r.codes, codes)
    np.testing.assert_array_equal(r.zp, zp)
    np.testing.assert_array_equal(r.scale, s)
    assert r.losses == [] and r.best_step == -1


def test_best_snapshot_not_worse_than_rtn():
    """Full batch: the returned state is the best evaluated one, so its loss
    equals best_loss and is not above the RTN loss (the first evaluated)."""
    W, X, Y = _full_batch_problem()
    for bits in (2, 3, 4):
        cfg = _cfg(bits=bits, group_size=16, iters=25)
        r = O.tune_linear(W, lambda b: (X, Y), 1, cfg)
        assert r.best_loss <= r.losses[0]
        assert r.best_loss == min(r.losses)
        wmin, wmax = O.group_minmax(W, 16)
        qp = O.qparams(wmin, wmax, r.alpha, r.beta, bits, False)
        fq = O.fake_quant(W, r.V, qp, bits, 16)
        L, _, _ = O.forward_backward(X, Y, fq.what)
        assert L == r.best_loss
        assert r.V.min() >= -0.5 and r.V.max() <= 0.5
        assert r.alpha.min() >= 0.5 and r.beta.max() <= 1.0


def test_snapshot_keeps_the_first_of_equal_losses():
    """The snapshot takes a state only when its loss is strictly below every
    earlier one (llm-compressor AutoRound page, the tuning loop's best-loss
    bookkeeping). With both step sizes zero the state never moves, every step
    has the same loss, and the first step stays the best."""
    W, X, Y = _full_batch_problem()
    cfg = _cfg(bits=4, group_size=16, iters=6, lr=0.0, minmax_lr=0.0)
    r = O.tune_linear(W, lambda b: (X, Y), 1, cfg)
    assert len(set(r.losses)) == 1
    assert r.best_step == 0 and r.best_loss == r.losses[0]


def test_steps_cycle_through_minibatches():
    """Step i draws minibatch i mod nb (the tuning loop walks the calibration
    batches in turn); the same three minibatches are requested in order."""
    W, X, Y = _full_batch_problem()
    seen = []

    def minibatch(b):
        seen.append(b)
        return X, Y
    O.tune_linear(W, minibatch, 3, _cfg(bits=4, group_size=16, iters=8))
    assert seen == [0, 1, 2, 0, 1, 2, 0, 1]


def test_nan_target_never_snapshotted_and_moves_nothing():
    """A NaN in one minibatch's targets: every step on that minibatch has a NaN
    loss, which the strict < of the best-state snapshot never takes, and the
    NaN reaches only the gradient row of the NaN's output, whose sign is taken
    as 0, so that row does not move on those steps while the other rows do.
    The returned state is finite. (The pages' loop reads each batch loss on the
    host and leaves non-finite data open; these are the readings the loop
    follows: sgn(NaN) = 0, snapshot on a strictly lower loss.)"""
    rng = np.random.default_rng(3)
    N, K, T, nb = 4, 16, 12, 3
    W = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    Xs = [rng.standard_normal((T, K)).astype(F32) for _ in range(nb)]
    Ys = [(x.astype(np.float64) @ W.astype(np.float64).T).astype(F32) for x in Xs]
    Ys[1] = Ys[1].copy()
    Ys[1][5, 2] = np.nan                      # output row 2, minibatch 1
    cfg = _cfg(bits=3, group_size=8, iters=7, minmax_lr=0.01)
    rows = []

    def on_step(i, r):
        rows.append(r)
    res = O.tune_linear(W, lambda b: (Xs[b], Ys[b]), nb, cfg, on_step=on_step)
    losses = np.array(res.losses)
    nan_steps = [i for i in range(cfg.iters) if i % nb == 1]
    assert np.all(np.isnan(losses[nan_steps]))
    assert np.all(np.isfinite(np.delete(losses, nan_steps)))
    assert res.best_step not in nan_steps and res.best_loss == np.nanmin(losses)
    for arr in (res.V, res.alpha, res.beta, res.what, res.scale):
        assert np.all(np.isfinite(arr))
    V = np.zeros((N, K), F32)
    for i, r in enumerate(rows):
        if i in nan_steps:
            assert np.all(np.isnan(r.gV[2])) and np.all(np.isfinite(np.delete(r.gV, 2, 0)))
            np.testing.assert_array_equal(r.V[2], V[2])
            assert not np.array_equal(np.delete(r.V, 2, 0), np.delete(V, 2, 0))
        V = r.V


def test_brute_force_2x4():
    """2x4 weight, 2-bit asym, one group per row, s and zp frozen
    (minmax_lr = 0), exact arithmetic: neither RTN nor 200 SignSGD steps can
    beat the exhaustive optimum over all 2^8 up/down roundings."""
    rng = np.random.default_rng(0)
    W = (rng.normal(0.0, 0.02, (2, 4))).astype(F32)
    X = rng.standard_normal((16, 4))
    Y = X @ W.astype(np.float64).T
    cfg = _cfg(bits=2, group_size=4, iters=200, minmax_lr=0.0)
    wmin, wmax = O.group_minmax(W, 4)
    one = np.ones_like(wmin)
    qp = O.qparams(wmin, wmax, one, one, 2, False)
    t = W / np.repeat(qp.s, 4, axis=1)
    assert np.all(np.abs(t - np.floor(t) - 0.5) > 1e-3)   # generic t
    best_rows, best_codes = O.brute_force_rounding(W, X, Y, qp, 2, 4)

    def row_losses(codes):
        w_hat = np.repeat(qp.s, 4, axis=1).astype(np.float64) * \
            (codes.astype(np.float64) - np.repeat(qp.zp, 4, axis=1))
        return np.sum((X @ w_hat.T - Y) ** 2, axis=0)

    rtn_codes, _, _, _ = O.rtn_quant(W, cfg)
    r = O.tune_linear(W, lambda b: (X, Y), 1, cfg, amp=False)
    np.testing.assert_array_equal(r.scale, qp.s)
    assert np.all(row_losses(rtn_codes) >= best_rows - 1e-12)
    assert np.all(row_losses(r.codes) >= best_rows - 1e-12)
    assert row_losses(r.codes).sum() <= row_losses(rtn_codes).sum() + 1e-15


# ------------------------------------------------------------------ S11
def _pack_cases():
    with open(os.path.join(GOLDEN, "pack_vectors.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _pack_cases(), ids=lambda c: f"b{c['bits']}")
def test_pack_hand_words(case):
    bits = case["bits"]
    if "codes" in case:
        codes = np.array(case["codes"], np.uint8)
    else:
        codes = np.full(case["length"], case.get("codes_fill", 0), np.uint8)
        for k, v in case.get("codes_sparse", {}).items():
            codes[int(k)] = v
    qw = O._pack_axis0(codes[:, None], bits)
    assert [int(w) for w in qw[:, 0]] == [int(w, 16) for w in case["words"]]
    np.testing.assert_array_equal(O._unpack_axis0(qw, bits, len(codes))[:, 0], codes)


@pytest.mark.parametrize("bits", O.SUPPORTED_BITS)
def test_pack_matches_bigint_and_roundtrips(bits):
    """Packing against a Python big-integer bit string built per column."""
    rng = np.random.default_rng(bits)
    N, K, g = 32, 96, 32
    codes = rng.integers(0, 2 ** bits, (N, K), dtype=np.uint8)
    zp = rng.integers(0, 2 ** bits, (N, K // g), dtype=np.uint8)
    qw, qz = O.pack(codes, zp, bits)
    assert qw.shape == (K * bits // 32, N) and qz.shape == (K // g, N * bits // 32)
    for n in range(N):
        acc = 0
        for k in range(K):
            acc |= int(codes[n, k]) << (k * bits)
        words = [(acc >> (32 * w)) & 0xFFFFFFFF for w in range(K * bits // 32)]
        assert [int(x) for x in qw[:, n]] == words
    for j in range(K // g):
        acc = 0
        for n in range(N):
            acc |= int(zp[n, j]) << (n * bits)
        assert [int(x) for x in qz[j]] == [(acc >> (32 * w)) & 0xFFFFFFFF
                                           for w in range(N * bits // 32)]
    c2, z2 = O.unpack(qw, qz, bits, N, K)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(z2, zp)


# ------------------------------------------------------------------ initial scale (MSE)
def _mse_err(W, p, cfg):
    """Squared RTN error of every group at shrink p (alpha = beta = p)."""
    N, K = W.shape
    g = cfg.g(K)
    wmin, wmax = O.group_minmax(W, cfg.group_size)
    a = np.full(wmin.shape, F32(p))
    qp = O.qparams(wmin, wmax, a, a, cfg.bits, cfg.sym)
    fq = O.fake_quant(W, np.zeros_like(W), qp, cfg.bits, cfg.group_size)
    d = (W - fq.what).astype(np.float64)
    return (d * d).reshape(N, K // g, g).sum(axis=2)


def test_minmax_shrink_sets_the_initial_clip_factors():
    """With the Min-Max initial scale, alpha = beta = minmax_shrink in every
    group (llm-compressor AutoRound page, constructor parameter table), so a
    group whose range straddles zero gets 0.8 times the unshrunk scale."""
    rng = np.random.default_rng(7)
    W = rng.standard_normal((4, 32)).astype(F32)
    cfg = _cfg(bits=4, group_size=16, minmax_shrink=0.8, clip_lo=0.5)
    a, b = O.init_clip(W, cfg)
    assert a.shape == (4, 2) and np.all(a == F32(0.8)) and np.all(b == F32(0.8))
    wmin, wmax = O.group_minmax(W, 16)
    assert np.all(wmin < 0) and np.all(wmax > 0)
    s08 = O.rtn_quant(W, cfg)[1]
    s10 = O.rtn_quant(W, _cfg(bits=4, group_size=16))[1]
    np.testing.assert_allclose(s08, 0.8 * s10, rtol=1e-6)


def test_mse_grid_points():
    pts = O.mse_grid_points(O.Config())
    assert len(pts) == 51 and pts[0] == 1.0 and pts[-1] == F32(0.5)
    assert np.all(np.diff(pts) < 0)
    assert len(O.mse_grid_points(O.Config(clip_lo=0.8, mse_grid=20))) == 5
    np.testing.assert_array_equal(O.mse_grid_points(O.Config(clip_lo=0.7, clip_hi=0.9,
                                                             mse_grid=10)),
                                  np.array([0.9, 0.8, 0.7], F32))
    with pytest.raises(ValueError):
        O.mse_grid_points(O.Config(clip_lo=0.91, clip_hi=0.99, mse_grid=10))


@pytest.mark.parametrize("sym,bits", [(False, 2), (False, 4), (True, 3)])
def test_mse_shrink_never_worse_than_minmax(sym, bits):
    rng = np.random.default_rng(40 + bits)
    W = (rng.standard_normal((24, 64)) * 0.02).astype(F32)
    W[:, 5] *= 12.0                                         # an outlier column
    cfg = O.Config(bits=bits, group_size=16, sym=sym, init="mse")
    p = O.mse_shrink(W, cfg)
    assert p.min() >= F32(0.5) and p.max() <= 1.0
    e_best = np.minimum.reduce([_mse_err(W, q, cfg) for q in O.mse_grid_points(cfg)])
    np.testing.assert_allclose(np.array([[_mse_err(W[n:n + 1], p[n, j], cfg)[0, j]
                                          for j in range(p.shape[1])] for n in range(24)]),
                               e_best, rtol=1e-12)
    assert np.all(e_best <= _mse_err(W, 1.0, cfg))
    assert (p < 1.0).any()                                  # outlier groups get clipped


def test_mse_shrink_keeps_an_exact_grid():
    """Values exactly on the min-max grid quantize with zero error at p = 1, so
    p = 1 (the first candidate) is kept."""
    s, zp = F32(0.125), 1
    row = (s * (np.arange(4, dtype=F32) - zp)).astype(F32)  # [-0.125, 0, 0.125, 0.25], 2 bits
    W = np.tile(row, (3, 2))
    p = O.mse_shrink(W, O.Config(bits=2, group_size=4, init="mse"))
    np.testing.assert_array_equal(p, np.ones_like(p))


def test_mse_shrink_single_outlier_prefers_clipping():
    """Seven small values and one large one at 2 bits: shrinking the range
    trades a larger error on the outlier for a finer grid on the rest."""
    W = np.array([[0.011, -0.02, 0.017, -0.005, 0.013, -0.019, 0.008, 0.2]], F32)
    cfg = O.Config(bits=2, group_size=8, init="mse")
    p = O.mse_shrink(W, cfg)
    assert p[0, 0] < 1.0
    assert _mse_err(W, p[0, 0], cfg)[0, 0] < _mse_err(W, 1.0, cfg)[0, 0]


def test_mse_shrink_power_of_two_scaling():
    rng = np.random.default_rng(44)
    W = (rng.standard_normal((16, 128)) * 0.03).astype(F32)
    cfg = O.Config(bits=3, group_size=32, init="mse")
    np.testing.assert_array_equal(O.mse_shrink(W, cfg), O.mse_shrink(W * F32(8.0), cfg))


def test_mse_init_feeds_rtn_and_loop():
    W, X, Y = _full_batch_problem()
    cfg = _cfg(bits=2, group_size=16, iters=0)
    cfg.init = "mse"
    a, b = O.init_clip(W, cfg)
    np.testing.assert_array_equal(a, O.mse_shrink(W, cfg))
    codes, s, zp, what = O.rtn_quant(W, cfg)
    r = O.tune_linear(W, lambda i: (X, Y), 1, cfg)
    np.testing.assert_array_equal(r.codes, codes)
    np.testing.assert_array_equal(r.alpha, a)
    cfg_mm = _cfg(bits=2, group_size=16, iters=0)
    e_mse = float(((W - what) ** 2).sum())
    e_mm = float(((W - O.rtn_quant(W, cfg_mm)[3]) ** 2).sum())
    assert e_mse <= e_mm


# ------------------------------------------------------------------ per-layer config
DEF = (4, 128, False)


def test_layer_config_without_rules():
    assert O.resolve_layer_config([], DEF, True, "model.layers.0.mlp.up_proj") == (4, 128, False)
    assert O.resolve_layer_config([], DEF, False, "lm_head") == (16, -1, True)


def test_layer_config_exact_then_regex():
    rules = [
        (r"model\.layers\.\d+\.mlp\..*", {"bits": 8}),
        ("model.layers.0.mlp.down_proj", {"bits": 2, "group_size": 64}),
        (r"model\.layers\.1\..*", {"bits": 3, "sym": True}),
        ("lm_head", {"bits": 16}),
    ]
    # an exact key wins over an earlier pattern
    assert O.resolve_layer_config(rules, DEF, True, "model.layers.0.mlp.down_proj") == (2, 64, False)
    # the first pattern that fully matches wins
    assert O.resolve_layer_config(rules, DEF, True, "model.layers.1.mlp.up_proj") == (8, 128, False)
    assert O.resolve_layer_config(rules, DEF, True, "model.layers.1.self_attn.q_proj") == (3, 128, True)
    # full match only
    assert O.resolve_layer_config(rules, DEF, True, "x.model.layers.1.self_attn.q_proj") == DEF
    assert O.resolve_layer_config(rules, DEF, True, "lm_head") == (16, 128, False)
    assert O.resolve_layer_config(rules, DEF, True, "model.layers.2.self_attn.o_proj") == DEF


def test_layer_config_patterns_match_whole_names():
    """A pattern must match the whole layer name, not a prefix of it."""
    rules = [(r"model\.layers\.2", {"bits": 4, "sym": True})]
    assert O.resolve_layer_config(rules, DEF, True, "model.layers.2.self_attn.o_proj") == DEF
    assert O.resolve_layer_config(rules, DEF, True, "model.layers.2") == (4, 128, True)


def test_layer_config_plain_keys_are_not_patterns():
    """'.' is not in the special set: a dotted key is only an exact name."""
    rules = [("model.layers.0.mlp", {"bits": 8})]
    assert O.resolve_layer_config(rules, DEF, True, "modelXlayersX0Xmlp") == DEF
    assert O.resolve_layer_config(rules, DEF, True, "model.layers.0.mlp") == (8, 128, False)


def test_layer_config_bad_pattern_skipped():
    rules = [("layers.(", {"bits": 2}), (r"layers\.\d", {"bits": 3})]
    assert O.resolve_layer_config(rules, DEF, True, "layers.7") == (3, 128, False)


def test_layer_config_outside_quantized_set():
    """Exact keys fill missing fields from (16, -1, True) outside the quantized
    set; pattern matches fill them from the defaults."""
    rules = [("lm_head", {"group_size": 32}), (r"embed.*", {"sym": True})]
    assert O.resolve_layer_config(rules, DEF, False, "lm_head") == (16, 32, True)
    assert O.resolve_layer_config(rules, DEF, False, "embed_tokens") == (4, 128, True)
    assert O.resolve_layer_config(rules, DEF, False, "norm") == (16, -1, True)


def test_fused_configs():
    rules = [("m.q_proj", {"bits": 8}), ("m.k_proj", {"bits": 8}), ("m.v_proj", {"bits": 4}),
             ("e.experts.0.w1", {"bits": 3}), ("e.experts.1.w1", {"bits": 3})]
    with pytest.raises(ValueError):
        O.resolve_fused_config(rules, DEF, True, "m.qkv_proj", ["m.q_proj", "m.k_proj", "m.v_proj"])
    assert O.resolve_fused_config(rules, DEF, True, "m.qk", ["m.q_proj", "m.k_proj"]) == (8, 128, False)
    assert O.resolve_fused_config(rules, DEF, True, "e.experts") == (3, 128, False)
    assert O.resolve_fused_config(rules, DEF, True, "f.experts") == DEF
    with pytest.raises(ValueError):
        O.resolve_fused_config(rules + [("e.experts.2.w1", {"bits": 2})], DEF, True, "e.experts")


# ------------------------------------------------------------------ dequantisation
@pytest.mark.parametrize("bits,sym", [(2, False), (3, False), (4, True), (8, False)])
def test_dequantize_inverts_the_quantizer(bits, sym):
    """Packing the codes and zero-points of a state and dequantizing gives back
    the quantizer's own Ŵ bit for bit."""
    rng = np.random.default_rng(60 + bits)
    N, K, g = 32, 256, 64
    W = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    cfg = O.Config(bits=bits, group_size=g, sym=sym)
    codes, s, zp, what = O.rtn_quant(W, cfg)
    qw, qz = O.pack(codes, zp, bits)
    got = O.dequantize(qw, None if sym else qz, s, bits, g, N, K)
    np.testing.assert_array_equal(got, what)


def test_dequant_matmul_hand_example():
    """4-bit, one group of 8 per row, written out by hand (rows 2..7 have zero
    scale; zero-points pack 8 rows to a word)."""
    codes = np.zeros((8, 8), np.uint8)
    codes[0] = [0, 1, 2, 3, 4, 5, 6, 7]
    codes[1] = [15, 14, 13, 12, 11, 10, 9, 8]
    zp = np.zeros((8, 1), np.uint8)
    zp[0, 0], zp[1, 0] = 3, 8
    scale = np.zeros((8, 1), F32)
    scale[0, 0], scale[1, 0] = 0.5, 0.25
    qw, qz = O.pack(codes, zp, 4)
    # word of row 0: codes 0..7 LSB first -> 0x76543210; row 1 -> 0x89ABCDEF
    assert qw[0, 0] == 0x76543210 and qw[0, 1] == 0x89ABCDEF
    assert qz[0, 0] == 0x83                                  # zp 3 then 8, LSB first
    X = np.array([[1, 0, 0, 0, 0, 0, 0, 2]], F32)
    # row 0: 0.5*(0-3) + 2*0.5*(7-3) = -1.5 + 4 = 2.5; row 1: 0.25*(15-8) + 2*0.25*(8-8) = 1.75
    Y = O.dequant_matmul(X, qw, qz, scale, 4, 8, 8, 8)
    np.testing.assert_allclose(Y[0, :2], [2.5, 1.75])
    assert not Y[0, 2:].any()


def test_dequant_product_uses_the_bf16_weight():
    """The product's weight operand is bf16(Ŵ), the operand of the tuning
    loop's forward product: scale float32(0.1), code 3, zero-point 0 give
    Ŵ = 0.3000000119 in float32, whose bf16 value is 0.30078125 (0x3E9A)."""
    codes = np.zeros((8, 8), np.uint8)
    codes[0, 0] = 3
    zp = np.zeros((8, 1), np.uint8)
    scale = np.zeros((8, 1), F32)
    scale[0, 0] = F32(0.1)
    qw, qz = O.pack(codes, zp, 4)
    X = np.zeros((1, 8), F32)
    X[0, 0] = 1.0
    Y = O.dequant_matmul(X, qw, qz, scale, 4, 8, 8, 8)
    assert Y[0, 0] == 0.30078125


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_aligned_column_block_is_a_packed_layer(bits):
    """32 adjacent columns starting at a multiple of 32 are a packed layer of
    their own: their qweight columns, the qzeros words that hold their
    zero-points and their scale rows dequantize to the same Ŵ rows as the whole
    layer (the large-shape GPU tests compare such blocks)."""
    rng = np.random.default_rng(70 + bits)
    N, K, g = 96, 256, 64
    codes = rng.integers(0, 2 ** bits, (N, K), dtype=np.uint8)
    zp = rng.integers(0, 2 ** bits, (N, K // g), dtype=np.uint8)
    scale = rng.uniform(0.5, 2.0, (N, K // g)).astype(F32)
    qw, qz = O.pack(codes, zp, bits)
    full = O.dequantize(qw, qz, scale, bits, g, N, K)
    for c0 in (0, 32, 64):
        zc = slice(c0 * bits // 32, (c0 + 32) * bits // 32)
        sub = O.dequantize(qw[:, c0:c0 + 32], qz[:, zc], scale[c0:c0 + 32], bits, g, 32, K)
        np.testing.assert_array_equal(sub, full[c0:c0 + 32])
