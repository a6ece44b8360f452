"""The seeded input generator: deterministic, and the two Y_true evaluations
(numpy float64 and torch float64) give identical bytes."""
import numpy as np
import torch

import synth


def test_deterministic_and_prefix():
    a = synth.make_case(64, 128, 300, wdtype="bf16", seed=3)
    b = synth.make_case(64, 128, 300, wdtype="bf16", seed=3)
    np.testing.assert_array_equal(a.W_bits, b.W_bits)
    np.testing.assert_array_equal(a.X_bits, b.X_bits)
    assert a.W.dtype == np.float32 and a.X_bits.dtype == np.uint16
    # outlier columns/channels present with the stated counts
    w_big = np.abs(a.W).max(axis=0) > 0.02 * 10 * 1.5
    assert 1 <= w_big.sum() <= int(np.rint(0.005 * 128)) + 2


def test_bf16_cast_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(ref),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_reference_outputs_numpy_equals_torch():
    for wd in ("bf16", "f32"):
        c = synth.make_case(96, 256, 512, wdtype=wd, seed=1)
        y_np = synth.reference_outputs(c)
        y_t = synth.reference_outputs_torch(c, "cpu")
        if wd == "bf16":
            np.testing.assert_array_equal(y_np, y_t.view(torch.int16).numpy().view(np.uint16))
        else:
            np.testing.assert_array_equal(y_np, y_t.numpy())


def test_workload_table():
    w = synth.WORKLOADS["llama7b_q_proj"]
    assert (w.N, w.K, w.M, w.Tb) == (4096, 4096, 262144, 16384)
    assert w.flop_per_iter == 4 * 16384 * 4096 * 4096
    t = synth.WORKLOADS["toy_256"]
    assert (t.M, t.Tb, t.iters) == (256, 256, 20)
