"""GPU parity of the W{2,3,4,8} x bf16 product on the packed format
(ar_dequant_gemm) against the oracle's dequant_matmul (float64 on the same
bf16 Ŵ), on both paths (M <= 16 split-K reading the packed words; larger M
through the blocked MFMA product), and end to end: a tuned layer's packed
output reproduces the product with its own Ŵ."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_common import F32, bf16_dev, dev, log, rel_norm, to_np, weight_dev

pytestmark = pytest.mark.gpu
ar = pytest.importorskip("autoround_signsgd_rounding_amd")


def _packed(N, K, bits, g, sym, seed):
    """Random codes / zero-points / scales of a plausible layer, packed."""
    rng = np.random.default_rng(seed)
    G = 1 if g == -1 else K // g
    codes = rng.integers(0, 2 ** bits, (N, K), dtype=np.uint8)
    zp = rng.integers(0, 2 ** bits, (N, G), dtype=np.uint8)
    scale = (rng.uniform(0.5, 2.0, (N, G)) * 0.01).astype(F32)
    if sym:   # no zero-points: pack placeholder ones for a whole number of words
        qw, _ = O.pack(codes, np.zeros((-(-N // 32) * 32, G), np.uint8), bits)
        return qw, None, scale
    qw, qz = O.pack(codes, zp, bits)
    return qw, qz, scale


def _gpu_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev())


CASES = [
    # M, N, K, bits, g, sym, out
    (1, 4096, 4096, 4, 128, False, "f32"),
    (5, 256, 512, 2, 32, False, "f32"),
    (16, 96, 384, 3, 128, False, "bf16"),
    (3, 64, 256, 8, -1, True, "f32"),
    (17, 256, 512, 4, 64, True, "f32"),       # smallest M on the MFMA path
    (300, 520, 200, 8, 40, False, "f32"),     # ragged tiles and reduction
    (257, 128, 768, 3, 96, False, "bf16"),
    (64, 160, 256, 2, -1, False, "f32"),
    # small-M path: columns not a multiple of 4 (per-column loads), groups of
    # 24 and 8 (several groups per 32-wide step), a K tail past the last step
    (2, 90, 256, 4, 64, True, "f32"),
    (4, 128, 384, 3, 24, False, "f32"),
    (1, 256, 256, 2, 8, False, "f32"),
    (7, 520, 200, 8, 40, False, "f32"),
    (16, 300, 1024, 4, -1, True, "bf16"),
    # wider layers: a K tail past the last whole step (K = 1000), each width,
    # bf16 output, a column count that is not a multiple of 4 (per-column
    # loads), one group per row
    (1, 2048, 1000, 4, 40, False, "f32"),
    (3, 2304, 512, 2, 64, False, "bf16"),
    (2, 2049, 768, 3, 128, True, "f32"),
    (1, 4096, 2048, 8, -1, True, "f32"),
    (8, 2048, 1024, 4, 128, True, "bf16"),
]


@pytest.mark.parametrize("M,N,K,bits,g,sym,out", CASES)
def test_dequant_gemm_parity(M, N, K, bits, g, sym, out):
    log(f"dequant_gemm M={M} N={N} K={K} b{bits} g{g} sym={sym} out={out}")
    qw, qz, scale = _packed(N, K, bits, g, sym, seed=M + N + K + bits)
    rng = np.random.default_rng(M * 3 + K)
    Xb = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(F32))
    Xf = synth.bf16_bits_to_f32(Xb)
    Y = ar.dequant_gemm(bf16_dev(Xb), _gpu_i32(qw), None if qz is None else _gpu_i32(qz),
                        torch.from_numpy(scale).to(dev()), bits, g, N,
                        out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    ref = O.dequant_matmul(Xf, qw, qz, scale, bits, g, N, K)
    got = to_np(Y).astype(np.float64)
    err = rel_norm(got, ref)
    log(f"  rel err {err:.2e}")
    if out == "f32":
        assert err <= 1e-5
        assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()
    else:
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())


@pytest.mark.parametrize("N,K", [(256, 512), (320, 520)])
def test_prefill_with_a_dirty_workspace(N, K):
    """The MFMA path (M > 16) in a workspace whose every byte is 0xFF (NaN as
    bf16): with whole tiles (N % 256 == 0, K % 32 == 0) the dequantization
    writes every element of the blocked operand; with ragged ones its padding
    is cleared first. Either way the product equals the oracle's."""
    M, bits, g = 40, 4, 40 if K % 40 == 0 else 128
    if K % g:
        g = 8
    qw, qz, scale = _packed(N, K, bits, g, False, seed=N + K)
    rng = np.random.default_rng(K)
    Xb = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(F32))
    ws = torch.full((ar.dequant_gemm_workspace_size(bits, g, M, N, K),), 255, dtype=torch.uint8,
                    device=dev())
    Y = ar.dequant_gemm(bf16_dev(Xb), _gpu_i32(qw), _gpu_i32(qz),
                        torch.from_numpy(scale).to(dev()), bits, g, N, workspace=ws)
    torch.cuda.synchronize()
    ref = O.dequant_matmul(synth.bf16_bits_to_f32(Xb), qw, qz, scale, bits, g, N, K)
    got = to_np(Y).astype(np.float64)
    assert np.all(np.isfinite(got))
    assert rel_norm(got, ref) <= 1e-5


def test_tuned_layer_round_trip():
    """Tune (toy 256->256, W4 g64), pack, and multiply through the packed format:
    the product equals X·bf16(Ŵ)ᵀ with the tuning loop's own Ŵ."""
    w = synth.WORKLOADS["toy_256"]
    case = synth.make_workload_case(w)
    Y = synth.reference_outputs(case)
    cfg = ar.Config(bits=w.bits, group_size=w.group_size, nsamples=w.nsamples, seqlen=w.seqlen,
                    batch_samples=w.batch_samples, iters=w.iters)
    Xd = bf16_dev(case.X_bits)
    out = ar.tune_linear(weight_dev(case), Xd, torch.from_numpy(Y).to(dev()), cfg, want_wq=True)
    qw, qz = ar.pack(out.codes, out.zp, w.bits)
    for M in (4, 256):
        Yq = ar.dequant_gemm(Xd[:M], qw, qz, out.scale, w.bits, w.group_size, w.N)
        torch.cuda.synchronize()
        Wq = O.bf16(to_np(out.Wq)).astype(np.float64)
        ref = synth.bf16_bits_to_f32(case.X_bits[:M]).astype(np.float64) @ Wq.T
        log(f"  M={M}: rel err {rel_norm(to_np(Yq), ref):.2e}")
        assert rel_norm(to_np(Yq), ref) <= 1e-5


@pytest.mark.parametrize("M", [1, 16, 2048])
def test_dequant_gemm_q_proj_shape(M):
    """Llama-7B q_proj 4096->4096, W4 g128 asym: the decode sizes in full, the
    prefill size on 64 sampled rows of X."""
    N = K = 4096
    qw, qz, scale = _packed(N, K, 4, 128, False, seed=M)
    rng = np.random.default_rng(M)
    Xb = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(F32))
    Y = ar.dequant_gemm(bf16_dev(Xb), _gpu_i32(qw), _gpu_i32(qz),
                        torch.from_numpy(scale).to(dev()), 4, 128, N)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 16 else np.sort(rng.choice(M, 64, replace=False))
    ref = O.dequant_matmul(synth.bf16_bits_to_f32(Xb[rows]), qw, qz, scale, 4, 128, N, K)
    err = rel_norm(to_np(Y)[rows], ref)
    log(f"  M={M}: rel err {err:.2e}")
    assert err <= 1e-5


@pytest.mark.parametrize("N", [512, 4096])
def test_decode_product_under_graph_capture(N):
    """The small-M path (split-K slices, then their sum in a second launch)
    captured in a HIP graph, at two widths: every replay (with eager work and
    synchronizations between replays) equals the eager result bit for bit."""
    K, M = 1024, 8
    qw, qz, scale = _packed(N, K, 4, 128, False, seed=99)
    rng = np.random.default_rng(5)
    Xd = bf16_dev(synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(F32)))
    args = (_gpu_i32(qw), _gpu_i32(qz), torch.from_numpy(scale).to(dev()), 4, 128, N)
    eager = ar.dequant_gemm(Xd, *args)
    Y = torch.empty_like(eager)
    ws = torch.empty(max(ar.dequant_gemm_workspace_size(4, 128, M, N, K), 256), dtype=torch.uint8,
                     device=dev())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ar.dequant_gemm(Xd, *args, out=Y, workspace=ws)
    torch.cuda.synchronize()
    for i in range(4):
        Y.fill_(float(i + 7))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager), i
        junk = ar.dequant_gemm(Xd[:1], *args)          # eager work between replays
        torch.cuda.synchronize()
        del junk


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("M", [1, 16])
def test_decode_full_size_sampled_columns(bits, M):
    """The decode sizes on a Qwen2.5-72B up_proj-shaped layer (8192 -> 29568,
    g128 asym, random packed words: every word is a valid packing), in the
    launch configuration the product uses at this size (several 32-wide steps
    per slice, a half-filled last column block). Aligned blocks of 32 columns
    are sampled: their qweight columns, qzeros words and scale rows form a
    32-column layer of their own, which the oracle multiplies."""
    N, K, g = 29568, 8192, 128
    G = K // g
    log(f"dequant_gemm full size M={M} b{bits}: generating")
    gen = torch.Generator(device=dev())
    gen.manual_seed(bits * 100 + M)
    qw = torch.randint(-2 ** 31, 2 ** 31 - 1, (K * bits // 32, N), dtype=torch.int32,
                       device=dev(), generator=gen)
    qz = torch.randint(-2 ** 31, 2 ** 31 - 1, (G, N * bits // 32), dtype=torch.int32,
                       device=dev(), generator=gen)
    scale = (torch.rand((N, G), device=dev(), generator=gen) + 0.5) * 0.01
    X = torch.randn((M, K), device=dev(), generator=gen).to(torch.bfloat16)
    Y = ar.dequant_gemm(X, qw, qz, scale, bits, g, N)
    torch.cuda.synchronize()
    Xf = X.float().cpu().numpy()
    got = to_np(Y).astype(np.float64)
    qw_h, qz_h, sc_h = (to_np(t) for t in (qw, qz, scale))
    for c0 in (0, 256 * 57 + 96, N - 256 - 32, N - 32):
        zc = slice(c0 * bits // 32, (c0 + 32) * bits // 32)
        ref = O.dequant_matmul(Xf, qw_h[:, c0:c0 + 32].view(np.uint32),
                               qz_h[:, zc].view(np.uint32), sc_h[c0:c0 + 32], bits, g, 32, K)
        err = rel_norm(got[:, c0:c0 + 32], ref)
        log(f"  columns {c0}..{c0 + 31}: rel err {err:.2e}")
        assert err <= 1e-5
        assert np.abs(got[:, c0:c0 + 32] - ref).max() <= 1e-5 * np.abs(ref).max()
