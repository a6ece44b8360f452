"""Products of at most four 256 x 256 tiles run on the one-wave small-product
kernel; larger ones on the 256 x 256 kernels. Both give every output element
the same MFMA sequence, so a layer's rows come out the same whichever kernel
computes them. Checked by embedding a 256-row layer (every product one tile:
the small kernel) as the first rows of a 2048-row layer (8 tiles: the large
kernels), same K, same minibatch. The gradient scale 2/(T_b N) is a power of
two at both N, so the large layer's gradients are the small one's times
exactly 1/8, bit for bit; the updated state agrees exactly. Token and Gram
form, bf16 and float32 operands."""
import pytest
import torch

from gpu_common import dev, log

pytestmark = pytest.mark.gpu
ar = pytest.importorskip("autoround_signsgd_rounding_amd")

NS, NL, K, TB = 256, 2048, 256, 256     # 2/(TB*NS) = 2^-15, 2/(TB*NL) = 2^-18


def _bits(t):
    return t.contiguous().view(torch.int32)


@pytest.mark.parametrize("gram", [False, True])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_small_kernel_rows_equal_large_kernel_rows(gram, dt):
    log(f"small vs large products, gram={gram} dtype={dt}")
    gen = torch.Generator().manual_seed(7 + int(gram))
    W = (torch.randn(NL, K, generator=gen) * 0.02).to(dt)
    X = torch.randn(TB, K, generator=gen).to(torch.bfloat16)
    Y = (X.float() @ W.float().t() + 0.01 * torch.randn(TB, NL, generator=gen)).to(dt)
    g = 64
    G = K // g
    V0 = (torch.rand(NL, K, generator=gen) - 0.5) * 0.2
    a0 = 0.7 + 0.3 * torch.rand(NL, G, generator=gen)
    b0 = 0.7 + 0.3 * torch.rand(NL, G, generator=gen)
    cfg = ar.Config(bits=4, group_size=g, sym=False)
    out = {}
    for n in (NS, NL):
        Wd = W[:n].contiguous().to(dev())
        Yd = Y[:, :n].contiguous().to(dev())
        V, a, b = (t[:n].contiguous().to(dev()) for t in (V0, a0, b0))
        _, gV, ga, gb = ar.tune_step(Wd, V, a, b, X.to(dev()), Yd, cfg, gram=gram)
        torch.cuda.synchronize()
        out[n] = [t[:NS].cpu() for t in (gV, ga, gb, V, a, b)]
    names = ("gV", "galpha", "gbeta", "V", "alpha", "beta")
    for i, name in enumerate(names):
        small, large = out[NS][i], out[NL][i]
        if i < 3:
            small = small * 0.125          # exact: a power of two on normal float32 values
        assert bool(torch.isfinite(small).all())
        same = torch.equal(_bits(small), _bits(large))
        if not same:
            d = (small - large).abs().max().item()
            log(f"  {name}: max |diff| {d:.3e}")
        assert same, name
    assert float(out[NS][0].abs().max()) > 0 and float(out[NS][1].abs().max()) > 0
