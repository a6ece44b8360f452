"""Pins of the decoder-block oracle (oracle/block_ref.py) against things
other than itself: brute-force loops, causality, rotary invariances, scale
invariance, zero-weight identities, and the sequential tuning's consistency
with per-Linear tuning."""
import numpy as np
import pytest

import oracle as O
from oracle import block_ref as B
import synth

F32 = np.float32


def test_attention_matches_loops():
    rng = np.random.default_rng(1)
    S, H, Dh = 5, 2, 4
    q, k, v = (B.b16(rng.standard_normal((2 * S, H * Dh)).astype(F32)) for _ in range(3))
    got = B.attention(q, k, v, S, H)
    want = np.zeros((2 * S, H * Dh))
    for s0 in (0, S):
        for h in range(H):
            for i in range(S):
                sc = [sum(float(q[s0 + i, h * Dh + d]) * float(k[s0 + j, h * Dh + d])
                          for d in range(Dh)) / np.sqrt(Dh) for j in range(i + 1)]
                mx = max(sc)
                e = [np.exp(x - mx) for x in sc]
                for d in range(Dh):
                    want[s0 + i, h * Dh + d] = sum(e[j] * float(v[s0 + j, h * Dh + d])
                                                   for j in range(i + 1)) / sum(e)
    np.testing.assert_allclose(got, B.b16(want.astype(F32)), rtol=2 ** -8, atol=1e-6)


def test_attention_is_causal_and_per_sequence():
    rng = np.random.default_rng(2)
    S, H, D = 8, 2, 16
    q, k, v = (B.b16(rng.standard_normal((2 * S, D)).astype(F32)) for _ in range(3))
    base = B.attention(q, k, v, S, H)
    k2, v2 = k.copy(), v.copy()
    k2[5], v2[5] = k2[5] * 3, -v2[5]                      # a later token of sequence 0
    k2[S + 1] += 1.0                                     # a token of sequence 1
    out = B.attention(q, k2, v2, S, H)
    np.testing.assert_array_equal(out[:5], base[:5])
    np.testing.assert_array_equal(out[S:S + 1], base[S:S + 1])


def test_rope_properties():
    rng = np.random.default_rng(3)
    S, H, Dh = 16, 2, 8
    x = B.b16(rng.standard_normal((S, H * Dh)).astype(F32))
    y = B.rope(x, S, H, 10000.0)
    np.testing.assert_array_equal(y[0], x[0])             # position 0: identity
    xa, ya = x.reshape(S, H, 2, Dh // 2), y.reshape(S, H, 2, Dh // 2)
    n0 = np.hypot(xa[:, :, 0], xa[:, :, 1])
    n1 = np.hypot(ya[:, :, 0], ya[:, :, 1])
    np.testing.assert_allclose(n1, n0, rtol=2 ** -7, atol=1e-6)   # rotations keep pair norms
    # relative positions: <rope(q, p), rope(k, p')> depends on p - p' only
    q = np.tile(B.b16(rng.standard_normal(H * Dh).astype(F32)), (S, 1))
    k = np.tile(B.b16(rng.standard_normal(H * Dh).astype(F32)), (S, 1))
    rq, rk = B.rope(q, S, H, 10000.0), B.rope(k, S, H, 10000.0)
    d1 = float(rq[3, :Dh] @ rk[1, :Dh])
    d2 = float(rq[10, :Dh] @ rk[8, :Dh])
    assert abs(d1 - d2) <= 2e-2 * (abs(d1) + 1e-3)


def test_rmsnorm_scale_invariance_and_unit_rows():
    rng = np.random.default_rng(4)
    x = B.b16(rng.standard_normal((6, 32)).astype(F32))
    w = B.b16((1 + 0.1 * rng.standard_normal(32)).astype(F32))
    np.testing.assert_array_equal(B.rmsnorm(x, w, 1e-6), B.rmsnorm(x * F32(4.0), w, 1e-6 * 16))
    ones = np.ones((2, 32), F32)
    np.testing.assert_array_equal(B.rmsnorm(ones, np.ones(32, F32), 0.0), ones)


def test_rmsnorm_applies_the_weight_per_channel():
    """Power-of-two channel weights scale each output column exactly (the
    products and the bf16 rounding commute with them)."""
    rng = np.random.default_rng(5)
    x = B.b16(rng.standard_normal((6, 32)).astype(F32))
    w = (2.0 ** (np.arange(32) % 5 - 2)).astype(F32)
    base = B.rmsnorm(x, np.ones(32, F32), 1e-6)
    np.testing.assert_array_equal(B.rmsnorm(x, w, 1e-6), base * w)


def test_rope_rotates_by_the_closed_form_angles():
    """A head vector with ones in its first half and zeros in its second half
    turns, pair j at position p, into (cos a, sin a) with a = p·theta^(−2j/Dh)."""
    S, H, Dh, theta = 12, 1, 8, 10000.0
    x = np.zeros((S, Dh), F32)
    x[:, :Dh // 2] = 1.0
    y = B.rope(x, S, H, theta)
    for p in range(S):
        for j in range(Dh // 2):
            a = p * theta ** (-2.0 * j / Dh)
            assert abs(y[p, j] - np.cos(a)) <= 4e-3 and abs(y[p, Dh // 2 + j] - np.sin(a)) <= 4e-3


def test_silu_values():
    """SiLU(g)·u against g/(1 + e^−g) at a few points."""
    g = np.array([[0.0, 1.0, -1.0, 4.0, -4.0, 0.5]], F32)
    u = np.array([[1.0, 1.0, 1.0, 1.0, 2.0, -3.0]], F32)
    want = [float(a) / (1.0 + np.exp(-float(a))) * float(b) for a, b in zip(g[0], u[0])]
    np.testing.assert_allclose(B.silu_mul(g, u)[0], want, rtol=2 ** -8, atol=1e-7)


def test_mlp_sees_the_attention_output():
    """The MLP normalises the residual stream after attention: with the
    attention output projection zeroed it sees RMSNorm(h), and any other
    output projection changes what it sees."""
    dims, W, norms, h = _toy(1)
    Z = dict(W, o_proj=np.zeros_like(W["o_proj"]))
    t0 = B.block_forward(h, Z, norms, dims)
    np.testing.assert_array_equal(t0["m"], B.rmsnorm(h, norms[1], dims.rms_eps))
    t1 = B.block_forward(h, W, norms, dims)
    assert not np.array_equal(t1["m"], t0["m"])


def _toy(nsamples=4):
    dims = synth.BLOCKS["toy_block"]
    c = synth.make_block_case(dims, nsamples=nsamples)
    W = {n: synth.bf16_bits_to_f32(c.W_bits[n]) for n in B.LINEARS}
    norms = tuple(synth.bf16_bits_to_f32(x) for x in c.norm_bits)
    h = synth.bf16_bits_to_f32(c.H_bits)
    return dims, W, norms, h


def test_zero_weights_give_the_identity():
    dims, W, norms, h = _toy(1)
    Z = {n: np.zeros_like(w) for n, w in W.items()}
    np.testing.assert_array_equal(B.block_forward(h, Z, norms, dims)["out"], h)


def _cfg(dims, iters, ns=4):
    return O.Config(bits=4, group_size=64, nsamples=ns, seqlen=dims.seqlen, batch_samples=2,
                    iters=iters)


def test_sequential_tuning_without_quantized_inputs_is_per_linear():
    dims, W, norms, h = _toy()
    cfg = _cfg(dims, 4)
    r = B.tune_block(h, W, norms, dims, cfg, quanted_input=False)
    fp = B.block_forward(h, W, norms, dims)
    Tb = cfg.batch_samples * cfg.seqlen
    for name in ("o_proj", "down_proj"):
        X, Y = fp[B.LINEAR_INPUT[name]], fp[name]
        alone = O.tune_linear(W[name], lambda b: (X[b * Tb:(b + 1) * Tb], Y[b * Tb:(b + 1) * Tb]),
                              2, cfg)
        np.testing.assert_array_equal(r.results[name].codes, alone.codes)
        assert r.results[name].losses == alone.losses


def test_quantized_inputs_change_only_later_linears():
    """q/k/v see the same input either way; o_proj onwards see the quantized
    pipeline's activations; both runs quantize every Linear."""
    dims, W, norms, h = _toy()
    cfg = _cfg(dims, 4)
    a = B.tune_block(h, W, norms, dims, cfg, quanted_input=True)
    b = B.tune_block(h, W, norms, dims, cfg, quanted_input=False)
    for name in ("q_proj", "k_proj", "v_proj"):
        np.testing.assert_array_equal(a.results[name].codes, b.results[name].codes)
    assert a.results["o_proj"].losses != b.results["o_proj"].losses
    assert a.err > 0 and b.err > 0


def test_iters_zero_is_rtn_per_linear():
    dims, W, norms, h = _toy(2)
    cfg = _cfg(dims, 0, ns=2)
    r = B.tune_block(h, W, norms, dims, cfg)
    for name in B.LINEARS:
        codes, _, _, what = O.rtn_quant(W[name], cfg)
        np.testing.assert_array_equal(r.results[name].codes, codes)
        np.testing.assert_array_equal(r.Wq[name], B.b16(what))
