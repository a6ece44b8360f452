"""Non-finite data on the GPU. Without check_finite, one NaN in one minibatch's
targets makes the loss of every step on that minibatch NaN; such a step is
never the best and moves only the rows its NaN does not reach (sgn(NaN) = 0),
exactly as in the oracle's loop on the same data. With check_finite the tuning
entry points refuse the data (AR_ERR_NONFINITE) before writing any output."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_common import bf16_dev, dev, log, oracle_cfg, to_np, weight_dev

pytestmark = pytest.mark.gpu
ar = pytest.importorskip("autoround_signsgd_rounding_amd")

N, K, NS, SEQ = 256, 256, 4, 64          # 4 minibatches of 64 tokens


def _case():
    case = synth.make_case(N, K, NS * SEQ, wdtype="f32", sigma_w=0.02, outliers=False, seed=11)
    Y = np.ascontiguousarray(synth.reference_outputs(case)).copy()
    Y[2 * SEQ + 5, 17] = np.nan               # minibatch 2, output row 17
    return case, Y


def _cfg(**kw):
    return ar.Config(bits=4, group_size=64, nsamples=NS, seqlen=SEQ, batch_samples=1, iters=12,
                     minmax_lr=0.01, **kw)


def test_nan_target_matches_oracle_loop():
    case, Y = _case()
    cfg = _cfg()
    out = ar.tune_linear(weight_dev(case), bf16_dev(case.X_bits), torch.from_numpy(Y).to(dev()),
                         cfg)
    torch.cuda.synchronize()
    Xf = synth.bf16_bits_to_f32(case.X_bits)
    r = O.tune_linear(case.W, lambda b: (Xf[b * SEQ:(b + 1) * SEQ], Y[b * SEQ:(b + 1) * SEQ]),
                      NS, oracle_cfg(cfg))
    losses = to_np(out.losses).astype(np.float64)
    ref = np.array(r.losses)
    nan_steps = [i for i in range(cfg.iters) if i % NS == 2]
    log(f"losses {losses}; oracle best step {r.best_step}")
    assert np.all(np.isnan(losses[nan_steps])) and np.all(np.isnan(ref[nan_steps]))
    fin = np.delete(np.arange(cfg.iters), nan_steps)
    assert np.all(np.abs(losses[fin] - ref[fin]) <= 1e-3 * ref[fin])
    assert int(np.nanargmin(losses)) == r.best_step and r.best_step not in nan_steps
    for t in (out.V, out.alpha, out.beta, out.scale):
        assert bool(torch.isfinite(t).all())
    agree = float(np.mean(to_np(out.codes) == r.codes))
    assert agree >= 0.999, agree
    # row 17 never moved on the NaN steps: its offsets are those of the steps before
    assert np.array_equal(np.isfinite(to_np(out.V)), np.ones((N, K), bool))


def test_check_finite_refuses_nan_inputs():
    case, Y = _case()
    cfg = _cfg(check_finite=True)
    W, X, Yd = weight_dev(case), bf16_dev(case.X_bits), torch.from_numpy(Y).to(dev())
    with pytest.raises(ar.ArError) as e:
        ar.tune_linear(W, X, Yd, cfg)
    assert e.value.status == 5
    with pytest.raises(ar.ArError) as e:
        ar.tune_linear(W, X, Yd, cfg, gram=True)
    assert e.value.status == 5
    # finite data passes the scan and gives the unchecked call's result
    Yok = torch.nan_to_num(Yd, nan=0.0)
    a = ar.tune_linear(W, X, Yok, cfg)
    b = ar.tune_linear(W, X, Yok, _cfg())
    assert torch.equal(a.codes, b.codes) and torch.equal(a.losses, b.losses)
    # the step: a NaN in the state or the minibatch is refused, nothing is updated
    G = K // 64
    V = torch.zeros((N, K), device=dev())
    al = torch.ones((N, G), device=dev())
    be = torch.ones((N, G), device=dev())
    Xb, Yb = X[:SEQ], Yok[:SEQ]
    V[3, 4] = float("inf")
    for noalloc in (False, True):
        with pytest.raises(ar.ArError) as e:
            ar.tune_step(W, V, al, be, Xb, Yb, cfg, noalloc=noalloc)
        assert e.value.status == 5
    with pytest.raises(ar.ArError) as e:
        ar.tune_step(W, V, al, be, Xb, Yb, cfg, gram=True)
    assert e.value.status == 5
    assert float(V[3, 4]) == float("inf") and int(torch.count_nonzero(V)) == 1
    V[3, 4] = 0.0
    Yb2 = Yb.clone()
    Yb2[7, 9] = float("nan")
    with pytest.raises(ar.ArError) as e:
        ar.tune_step(W, V, al, be, Xb, Yb2, cfg)
    assert e.value.status == 5
    ar.tune_step(W, V, al, be, Xb, Yb, cfg)      # finite: runs
    torch.cuda.synchronize()
    assert bool(torch.isfinite(V).all())
