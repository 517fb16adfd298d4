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


def test_noalloc_under_graph_capture():
    """The caller it is for: a decode step captured into a HIP graph (torch.cuda.graph), so
    the call may not allocate. Every replay, with the program's own eager work between
    replays, gives the bits of the eager no-alloc call on an identical cache; both run on
    one stream, so they never overlap on the shared buffer."""
    w = wl.DecodeWorkload("noalloc-graph", batch=4, heads=16, head_dim=128, ref_len=3000, window=128,
                          steps=12, dtype="bf16", sigma_q=1.0, sigma_kv=1.0, base_seed=8104)
    print("\n[case] noalloc under graph capture", flush=True)
    eager = DecodeRun(w)
    graphed = DecodeRun(w, ref=(eager.kref, eager.vref))
    sq, sk, sv = (torch.zeros((w.batch, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
                  for _ in range(3))
    sout = torch.zeros_like(sq)
    out_e = torch.empty_like(sq)
    q, k, v = wl.steps_qkv(w, 1, w.steps)
    # step 1 eagerly on both caches (also the library's first call on this device, outside capture)
    for r in (eager, graphed):
        rs.rswa_decode_attn_noalloc(r.cache.desc, to_dev(q[0], "bf16"), r.out, to_dev(k[0], "bf16"),
                                    to_dev(v[0], "bf16"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rs.rswa_decode_attn_noalloc(graphed.cache.desc, sq, sout, sk, sv)
    other = torch.randn(1 << 20, device="cuda")
    for T in range(2, w.steps + 1):
        qd, kd, vd = (to_dev(x[T - 1], "bf16") for x in (q, k, v))
        rs.rswa_decode_attn_noalloc(eager.cache.desc, qd, out_e, kd, vd)
        sq.copy_(qd); sk.copy_(kd); sv.copy_(vd)
        g.replay()
        other.mul_(1.0001)                  # the program's own eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(bits(sout), bits(out_e)), f"step {T}"
    assert eager.cache.step.cpu().tolist() == graphed.cache.step.cpu().tolist() == [w.steps] * w.batch
    assert np.array_equal(bits(eager.cache.k), bits(graphed.cache.k))
    assert np.array_equal(bits(eager.cache.v), bits(graphed.cache.v))
    assert rs.rswa_check_device_error(graphed.cache.desc) == 0
