"""ar_tune_step_noalloc (the step without a workspace argument, for callers
that cannot allocate) against ar_tune_step with a caller workspace: identical
loss, gradients, updated state and best-loss snapshot, on two calls in a row
whose second problem is smaller than the first (the fixed scratch keeps the
first call's contents), plus the oracle's step on the same inputs. The size
limit is checked on the host: a problem beyond the fixed scratch is refused
before anything is enqueued."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_common import F32, bf16_dev, dev, log, oracle_cfg, rel_norm, to_np, weight_dev

ar = pytest.importorskip("autoround_signsgd_rounding_amd")

TOL = 1e-3

# N, K, Tb, wdtype, ydtype, bits, group, sym: the first is the larger problem
# (ragged N and Tb, several forward tiles), the second a smaller one
CALLS = [
    (300, 832, 520, "bf16", "bf16", 4, 64, False),
    (256, 256, 256, "f32", "f32", 3, 64, True),
]


def _problem(N, K, Tb, wdtype, ydtype, g, seed):
    case = synth.make_case(N, K, Tb, wdtype=wdtype, sigma_w=0.02, outliers=True, seed=seed)
    Y = synth.reference_outputs(case)
    Yf = synth.bf16_bits_to_f32(Y) if wdtype == "bf16" else Y
    if ydtype == "bf16":
        Yf = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(Yf))
        Yd = bf16_dev(synth.f32_to_bf16_bits(Yf))
    else:
        Yd = torch.from_numpy(np.ascontiguousarray(Yf)).to(dev())
    G = K // g
    rng = np.random.default_rng(seed + 1)
    V = rng.uniform(-0.5, 0.5, (N, K)).astype(F32)
    a = rng.uniform(0.5, 1.0, (N, G)).astype(F32)
    b = rng.uniform(0.5, 1.0, (N, G)).astype(F32)
    return case, Yf, Yd, V, a, b


def _run(case, Yd, V, a, b, cfg, noalloc):
    t = [torch.from_numpy(x.copy()).to(dev()) for x in (V, a, b)]
    best = (torch.full_like(t[0], 7.0), torch.full_like(t[1], 7.0), torch.full_like(t[2], 7.0),
            torch.full((1,), float("inf"), device=dev()))
    loss, gV, ga, gb = ar.tune_step(weight_dev(case), *t, bf16_dev(case.X_bits), Yd, cfg,
                                    best=best, noalloc=noalloc)
    torch.cuda.synchronize()
    return [to_np(x) for x in (loss, gV, ga, gb, *t, *best)]


@pytest.mark.gpu
def test_noalloc_step_matches_workspace_step_twice():
    for i, (N, K, Tb, wdtype, ydtype, bits, g, sym) in enumerate(CALLS):
        log(f"noalloc call {i}: N={N} K={K} Tb={Tb} {wdtype}/{ydtype} b{bits} g{g} sym={sym}")
        case, Yf, Yd, V, a, b = _problem(N, K, Tb, wdtype, ydtype, g, seed=17 + i)
        cfg = ar.Config(bits=bits, group_size=g, sym=sym)
        assert ar.step_workspace_size(cfg, N, K, Tb, ar._dt(Yd)) <= ar.NOALLOC_SCRATCH_BYTES
        got = _run(case, Yd, V, a, b, cfg, noalloc=True)
        ref = _run(case, Yd, V, a, b, cfg, noalloc=False)
        names = ("loss", "gV", "galpha", "gbeta", "V", "alpha", "beta",
                 "best_V", "best_alpha", "best_beta", "best_loss")
        for nm, x, y in zip(names, got, ref):
            np.testing.assert_array_equal(x, y, err_msg=nm)
        # and the oracle's step on the same state, to the step parity bar
        wmin, wmax = O.group_minmax(case.W, g)
        r = O.tune_step(case.W, V, a, b, wmin, wmax, synth.bf16_bits_to_f32(case.X_bits), Yf,
                        oracle_cfg(cfg))
        L = float(got[0][0])
        assert abs(L - r.loss) <= TOL * r.loss, (L, r.loss)
        assert rel_norm(got[1], r.gV) <= TOL
        assert rel_norm(got[2], r.galpha) <= TOL and rel_norm(got[3], r.gbeta) <= TOL
        log(f"  bit-identical to ar_tune_step; loss {L:.6e} vs oracle {r.loss:.6e}")


@pytest.mark.gpu
def test_noalloc_refuses_problems_beyond_its_scratch():
    N = K = 4096
    Tb = 16384
    cfg = ar.Config(bits=4, group_size=128)
    need = ar.step_workspace_size(cfg, N, K, Tb, ar.AR_BF16)
    assert need > ar.NOALLOC_SCRATCH_BYTES
    W = torch.zeros((N, K), dtype=torch.bfloat16, device=dev())
    V = torch.zeros((N, K), dtype=torch.float32, device=dev())
    a = torch.ones((N, 32), dtype=torch.float32, device=dev())
    X = torch.zeros((Tb, K), dtype=torch.bfloat16, device=dev())
    Y = torch.zeros((Tb, N), dtype=torch.bfloat16, device=dev())
    with pytest.raises(ar.ArError) as e:
        ar.tune_step(W, V, a, a.clone(), X, Y, cfg, noalloc=True)
    assert e.value.status == 4
    # nothing was enqueued: the state is untouched
    assert int(torch.count_nonzero(V)) == 0
