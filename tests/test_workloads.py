"""The shared input generator: determinism, bf16 rounding, shapes (no GPU)."""
import numpy as np
import torch

import workloads as wl


def test_bf16_rounding_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # exact ties
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(wl.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_seeded_draws_are_reproducible_and_independent():
    w = wl.FORTY_PAGE
    a = wl.step_qkv(w, 17)
    b = wl.step_qkv(w, 17)
    c = wl.step_qkv(w, 18)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    assert a[0].shape == (32, 16, 128) and a[0].dtype == np.uint16
    s = wl.steps_qkv(w, 17, 18)
    np.testing.assert_array_equal(s[1][1], c[1])


def test_workload_shapes():
    assert wl.FORTY_PAGE.ref_len == 10272 and wl.ONE_PAGE.ref_len == 288
    assert wl.PACKED_32K.ref_len == 4128
    r = wl.ragged_lengths(wl.RAGGED_64)
    assert r.ref_len.min() >= 288 and r.ref_len.max() <= 50 * 256 + 32
    assert 1 <= r.t_now.min() and r.t_now.max() <= 8192
    q = wl.draw("fp32", 1.0, (2, 3), 1, 2)
    assert q.dtype == np.float32
