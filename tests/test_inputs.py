"""Host checks of the seeded input generator (no method arithmetic there)."""
import numpy as np
import torch

import kata_inputs as ki


def test_bf16_rounding_matches_torch_rne():
    g = np.random.Generator(np.random.PCG64(0))
    x = np.concatenate([g.standard_normal(100_000) * 10.0 ** g.integers(-8, 8, 100_000),
                        [0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.0e38]])
    f32 = x.astype(np.float32)
    want = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ki.bf16_bits(x), want)
    back = ki.bf16_to_f64(want)
    np.testing.assert_array_equal(back, torch.from_numpy(f32).to(torch.bfloat16).double().numpy())


def test_forward_inputs_shapes_norms_and_determinism():
    a = ki.forward_inputs(2, 3, 17, 16, 8, ki.BF16, seed=5)
    b = ki.forward_inputs(2, 3, 17, 16, 8, ki.BF16, seed=5)
    assert a.q.shape == (2, 3, 17, 16) and a.q.dtype == np.uint16
    assert a.v.shape == (2, 3, 17, 8)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.v64, b.v64)
    n = np.linalg.norm(a.q64, axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)  # unit rows up to bf16 rounding
    f = ki.forward_inputs(1, 1, 9, 16, 16, ki.F32, seed=0)
    assert f.q.dtype == np.float32
    np.testing.assert_array_equal(f.q.astype(np.float64), f.q64)


def test_decode_head_streams_are_independent_of_subset():
    full = ki.decode_inputs(4, heads=6, prefill=5, steps=3, d=4, dv=2)
    sub = ki.decode_inputs(4, heads=6, prefill=5, steps=3, d=4, dv=2, head_ids=[2, 5])
    np.testing.assert_array_equal(sub.pk, full.pk[[2, 5]])
    np.testing.assert_array_equal(sub.sv, full.sv[:, [2, 5]])


def test_workloads_describe_the_measured_shapes():
    assert (ki.LONG.B, ki.LONG.H, ki.LONG.T, ki.LONG.d, ki.LONG.dv, ki.LONG.chunk) == (1, 8, 131072, 16, 64, 128)
    assert ki.DECODE.heads == 4096
    assert ki.TINY.dtype == ki.F32 and ki.TINY.seed == 0
