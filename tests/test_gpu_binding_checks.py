"""The binding refuses tensors whose shape or dtype does not match the call
(ValueError before anything reaches the library): the kernels index every
buffer by the shapes they are given, so a mismatch would otherwise read or
write out of bounds. Each case perturbs one argument of an otherwise valid
call; the valid call itself runs once to show the arguments are right."""
import pytest
import torch

from gpu_common import dev

pytestmark = pytest.mark.gpu
ar = pytest.importorskip("autoround_signsgd_rounding_amd")

N, K, G, TB = 64, 256, 2, 64
F32, BF16, U8, I32 = torch.float32, torch.bfloat16, torch.uint8, torch.int32


def t(shape, dtype=F32):
    return torch.zeros(shape, dtype=dtype, device=dev())


def cfg(**kw):
    return ar.Config(bits=4, group_size=128, nsamples=2, seqlen=32, batch_samples=1, iters=1,
                     **kw)


def step_args():
    return dict(W=t((N, K), BF16), V=t((N, K)), alpha=torch.ones((N, G), device=dev()),
                beta=torch.ones((N, G), device=dev()), Xb=t((TB, K), BF16), Yb=t((TB, N), BF16))


def call_step(a, best=None):
    return ar.tune_step(a["W"], a["V"], a["alpha"], a["beta"], a["Xb"], a["Yb"], cfg(),
                        best=best)


def test_tune_step_checks():
    a = step_args()
    call_step(a)
    torch.cuda.synchronize()
    bad = {"V": [t((N, K + 8)), t((N, K), BF16), t((N, K))[:, :K // 2]],
           "alpha": [t((N, G + 1)), t((N, G), BF16)],
           "beta": [t((N - 1, G))],
           "Xb": [t((TB, K)), t((TB, K - 8), BF16)],
           "Yb": [t((TB + 8, N), BF16), t((TB, N), U8)],
           "W": [t((N, K), U8), t((N * K,), BF16)]}
    for name, vals in bad.items():
        for v in vals:
            b = dict(a, **{name: v})
            with pytest.raises(ValueError):
                call_step(b)
    good_best = (t((N, K)), t((N, G)), t((N, G)), torch.full((1,), float("inf"), device=dev()))
    call_step(a, best=good_best)
    for i, v in enumerate((t((N, K + 8)), t((N, G), BF16), t((N, 1)), t((2,)))):
        best = list(good_best)
        best[i] = v
        with pytest.raises(ValueError):
            call_step(a, best=tuple(best))


def test_tune_linear_checks():
    c = cfg()
    M = c.nsamples * c.seqlen
    W, X, Y = t((N, K), BF16), t((M, K), BF16), t((M, N), BF16)
    ar.tune_linear(W, X, Y, c)
    for args in ((W, t((M + 8, K), BF16), Y), (W, t((M, K)), Y), (W, X, t((M, N + 1), BF16)),
                 (W, X, t((M - 8, N), BF16)), (t((N, K), I32), X, Y)):
        with pytest.raises(ValueError):
            ar.tune_linear(*args, c)
    with pytest.raises(ValueError):
        ar.tune_linear(W, X, Y, c, workspace=t((4096,)))


def test_fakequant_and_rtn_checks():
    c = cfg()
    W = t((N, K), BF16)
    ar.fakequant_fwd(W, t((N, K)), t((N, G)), t((N, G)), c)
    with pytest.raises(ValueError):
        ar.fakequant_fwd(W, t((N, K - 8)), t((N, G)), t((N, G)), c)
    with pytest.raises(ValueError):
        ar.fakequant_fwd(W, t((N, K)), t((N, G), BF16), t((N, G)), c)
    with pytest.raises(ValueError):
        ar.rtn_quant(t((K,), BF16), c)
    with pytest.raises(ValueError):
        ar.init_clip(t((N, K), U8), c)


def test_pack_and_product_checks():
    codes, zp = t((N, K), U8), t((N, G), U8)
    qw, qz = ar.pack(codes, zp, 4)
    for cz in ((t((N, K), I32), zp), (codes, t((N - 1, G), U8)), (codes, t((N, G), I32))):
        with pytest.raises(ValueError):
            ar.pack(*cz, 4)
    ar.unpack(qw, qz, 4, N, K, G)
    with pytest.raises(ValueError):
        ar.unpack(qw, qz, 4, N, K + 8, G)
    with pytest.raises(ValueError):
        ar.unpack(qw.float(), qz, 4, N, K, G)
    X = t((3, K), BF16)
    sc = t((N, G))
    ar.dequant_gemm(X, qw, qz, sc, 4, 128, N)
    for args in ((X, qw[:-1], qz, sc), (X, qw, qz[:, :-1], sc), (X, qw, qz, t((N, G + 1))),
                 (X.float(), qw, qz, sc), (X, qw.float(), qz, sc)):
        with pytest.raises(ValueError):
            ar.dequant_gemm(*args, 4, 128, N)
    with pytest.raises(ValueError):
        ar.dequant_gemm(X, qw, qz, sc, 4, 128, N, out=t((3, N + 1)))
    with pytest.raises(ValueError):
        ar.dequant_gemm(X, qw, qz, sc, 5, 128, N)


def test_block_checks():
    D, H, F, S, B = 128, 2, 256, 32, 2
    dims = ar.block_dims(D, H, F, S, B)
    shapes = {"q_proj": (D, D), "k_proj": (D, D), "v_proj": (D, D), "o_proj": (D, D),
              "gate_proj": (F, D), "up_proj": (F, D), "down_proj": (D, F)}
    W = {n: t(s, BF16) for n, s in shapes.items()}
    norms = (t((D,), BF16), t((D,), BF16))
    h = t((S * B, D), BF16)
    ar.block_forward(h, W, norms, dims)
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        ar.block_forward(t((S * B + 8, D), BF16), W, norms, dims)
    with pytest.raises(ValueError):
        ar.block_forward(h, dict(W, down_proj=t((F, D), BF16)), norms, dims)
    with pytest.raises(ValueError):
        ar.block_forward(h, W, (norms[0], t((D + 8,), BF16)), dims)
    with pytest.raises(ValueError):
        ar.attention(h, h, t((S * B, D)), dims)
