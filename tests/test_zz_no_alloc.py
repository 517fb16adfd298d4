"""rswa_decode_attn_noalloc (the decode call on the library's static device
buffer) against rswa_decode_attn with a caller workspace, through the C ABI:
two identical caches driven step by step must give the same output bits, step
counters and cache images; then a second, smaller input on the same buffer."""
import numpy as np
import pytest
import torch

import reference_sliding_window_amd as rs
import workloads as wl
from gpu_util import DecodeRun, bits, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _pair_run(w, num_splits, steps):
    print(f"\n[case] noalloc vs workspace: {w.name} B={w.batch} H={w.heads} d={w.head_dim} L={w.ref_len} "
          f"n={w.window} splits={num_splits}", flush=True)
    a = DecodeRun(w, num_splits=num_splits)
    b = DecodeRun(w, num_splits=num_splits, ref=(a.kref, a.vref))
    for T in range(1, steps + 1):
        q, k, v = (to_dev(x[0], w.dtype) for x in wl.steps_qkv(w, T, T))
        rs.rswa_decode_attn(a.cache.desc, q, a.out, k, v, 0.0, num_splits, a.ws)
        rs.rswa_decode_attn_noalloc(b.cache.desc, q, b.out, k, v, 0.0, num_splits)
        torch.cuda.synchronize()
        assert np.array_equal(bits(a.out), bits(b.out)), f"step {T}: outputs differ"
    assert a.cache.step.cpu().tolist() == b.cache.step.cpu().tolist() == [steps] * w.batch
    assert np.array_equal(bits(a.cache.k), bits(b.cache.k))
    assert np.array_equal(bits(a.cache.v), bits(b.cache.v))
    assert rs.rswa_check_device_error(b.cache.desc) == 0
    # attend only (no append) on the same state
    q = torch.randn((w.batch, w.heads, w.head_dim), device="cuda").to(a.out.dtype)
    rs.rswa_decode_attn(a.cache.desc, q, a.out, None, None, 0.0, num_splits, a.ws)
    rs.rswa_decode_attn_noalloc(b.cache.desc, q, b.out, None, None, 0.0, num_splits)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a.out), bits(b.out)), "attend-only outputs differ"


def test_noalloc_matches_workspace_call_then_smaller_input():
    big = wl.DecodeWorkload("noalloc-big", batch=4, heads=16, head_dim=128, ref_len=3000, window=128,
                            steps=140, dtype="bf16", sigma_q=1.0, sigma_kv=1.0, base_seed=8101)
    _pair_run(big, 0, 140)        # split chunks and the merge launch, through the ring's wrap
    small = wl.DecodeWorkload("noalloc-small", batch=2, heads=2, head_dim=64, ref_len=40, window=8,
                              steps=20, dtype="fp32", sigma_q=1.0, sigma_kv=1.0, base_seed=8102)
    _pair_run(small, 3, 20)


def test_noalloc_one_launch_batch():
    """A full batch decoded in one launch per step (arrival counters), as the 40-page shape."""
    w = wl.DecodeWorkload("noalloc-one-launch", batch=32, heads=16, head_dim=128, ref_len=500, window=16,
                          steps=20, dtype="bf16", sigma_q=1.0, sigma_kv=1.0, base_seed=8103)
    _pair_run(w, 0, 20)


def test_noalloc_rejects_more_than_its_buffer():
    cache = rs.KVCache.allocate([10272] * 32, 16, 128, 128)
    need = rs.rswa_decode_workspace_size(cache.desc, 64)
    assert need > 8 << 20
    q = torch.zeros((32, 16, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    st = rs.rswa_decode_attn_noalloc(cache.desc, q, out, None, None, 0.0, 64, check=False)
    assert st == rs.RSWA_ERR_WORKSPACE
