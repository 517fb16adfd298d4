"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Decode: every step of the tiny fp32 and one-page workloads, a spread of steps
(both sides of the window filling and wrapping) of the 40-page workload at
full size, the full-attention contrast, and the ragged batch; cache images are
compared bit for bit against the ring rule. Packed form: every row of small
cases (both prefix modes, ragged tails) and sampled rows of the 32K workload.
"""
import math

import numpy as np
import pytest
import torch

import oracle.rswa as orc
import reference_sliding_window_amd as rs
import workloads as wl
import oracle.pool as opool
from gpu_util import (DecodeRun, bits, check_close, oracle_decode_all_pairs, score_range_qkv,
                      shared_decode_inputs, storage_bits, to_dev, to_f64)

DTYPE = {"bf16": rs.RSWA_BF16, "fp32": rs.RSWA_FP32}

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


# ------------------------------------------------------------------ decode
def test_tiny_fp32_every_step_fused_and_unfused():
    w = wl.TINY_FP32
    banner("tiny fp32 decode, all 40 steps, fused append+attend")
    run = DecodeRun(w)
    got = run.run(w.steps, keep=range(1, w.steps + 1))
    steps = wl.steps_qkv(w, 1, w.steps)
    for T in range(1, w.steps + 1):
        check_close(got[T][0], run.oracle(T, steps=steps), "fp32", f"tiny T={T}")
    run.check_cache_image()
    banner("tiny fp32 decode, separate append then attend")
    run2 = DecodeRun(w, ref=(run.kref, run.vref))
    got2 = run2.run(w.steps, keep=range(1, w.steps + 1), fused=False)
    for T in range(1, w.steps + 1):
        np.testing.assert_array_equal(got2[T], got[T])   # same arithmetic, same order
    run2.check_cache_image()
    assert rs.rswa_check_device_error(run.cache.desc) == 0


def test_tiny_fp32_step_by_step_cache_images():
    w = wl.TINY_FP32
    banner("tiny fp32 cache image after every step")
    run = DecodeRun(w)
    for T in range(1, w.steps + 1):
        run.run(T)
        run.check_cache_image()
        assert int(run.cache.step[0].item()) == T


def test_one_page_bf16_every_step():
    w = wl.ONE_PAGE
    banner("one-page bf16 decode, all 2048 steps")
    run = DecodeRun(w)
    got = run.run(w.steps, keep=range(1, w.steps + 1), chunk=512)
    steps = wl.steps_qkv(w, 1, w.steps)
    worst = (0.0, 0.0)
    for T in range(1, w.steps + 1):
        ma, rel = check_close(got[T][0], run.oracle(T, steps=steps), "bf16", f"one-page T={T}")
        worst = (max(worst[0], ma), max(worst[1], rel))
    print(f"one-page worst max|d|={worst[0]:.3e} rel={worst[1]:.3e}")
    run.check_cache_image()


FORTY_CHECK = [1, 2, 127, 128, 129, 130, 256, 1024, 3072, 6143, 6144]


@pytest.mark.slow
def test_forty_page_full_size():
    """Every (sequence, head) at the listed steps and 5 seeded random ones, against
    the oracle on all host cores; window-slot images bit for bit."""
    w = wl.FORTY_PAGE
    rng = np.random.default_rng(3)
    extra = sorted(set(rng.integers(3, w.steps, size=5).tolist()) - set(FORTY_CHECK))
    checks = sorted(set(FORTY_CHECK) | set(extra))
    banner(f"40-page bf16 decode, full size, {w.steps} steps; every (b,h) at {checks}")
    with opool.SharedArrays() as arrays:
        kref, vref, steps = shared_decode_inputs(w, arrays, w.steps)
        run = DecodeRun(w, ref=(kref, vref))
        got = run.run(w.steps, keep=checks, chunk=512, steps=steps)
        # every window slot of every (sequence, head) after all 6144 steps, and reference rows
        run.check_cache_image(ref_rows=[0, 1, 127, 128, 5000, 10270, 10271])
        assert rs.rswa_check_device_error(run.cache.desc) == 0
        del run
        print(f"oracle: {len(checks)} steps x {w.batch * w.heads} (b,h) on {opool.workers()} processes",
              flush=True)
        ref = oracle_decode_all_pairs(w, w.window, arrays, checks)
    for T in checks:
        ma, rel = check_close(got[T], ref[T], "bf16", f"40-page T={T}")
        print(f"T={T}: all {w.batch * w.heads} (b,h) max|d|={ma:.3e} worst (b,h) rel={rel:.3e}", flush=True)


@pytest.mark.slow
def test_forty_page_full_attention_contrast():
    """Same kernels with the window >= all outputs: the cache grows as L_m + T (Eq. 5).
    Every (sequence, head) at each checked step."""
    w = wl.FORTY_PAGE
    checks = [1, 129, 2048, 6144]
    banner("40-page full-attention contrast (window = 6144), every (b,h)")
    with opool.SharedArrays() as arrays:
        kref, vref, steps = shared_decode_inputs(w, arrays, w.steps)
        run = DecodeRun(w, window=w.steps, ref=(kref, vref))
        got = run.run(w.steps, keep=checks, chunk=512, steps=steps)
        assert rs.rswa_check_device_error(run.cache.desc) == 0
        del run
        ref = oracle_decode_all_pairs(w, w.steps, arrays, checks)
    for T in checks:
        ma, rel = check_close(got[T], ref[T], "bf16", f"contrast T={T}")
        print(f"contrast T={T}: max|d|={ma:.3e} worst (b,h) rel={rel:.3e}", flush=True)


def _flat_workspace_bytes(B, H, d):
    r256 = lambda x: (x + 255) // 256 * 256
    return r256((512 + B * H) * d * 4) + r256((512 + B * H) * 8) + r256(B * 4) + r256((B + 1) * 8)


@pytest.mark.parametrize("dtype,d,B,H,max_L,n,fused,seed", [
    ("bf16", 128, 70, 4, 15000, 128, True, 31),
    ("fp32", 64, 130, 3, 11000, 16, True, 32),
    ("bf16", 128, 3, 16, 90000, 128, False, 33),
    ("bf16", 64, 200, 2, 11000, 8, True, 34),
])
def test_flat_work_list_ragged_batches(dtype, d, B, H, max_L, n, fused, seed):
    """The flat work list (the library's plan for large steps not decoded in one launch):
    sequences of very different lengths -- empty references, a window not yet full,
    wrapped rings -- and one sequence flagged invalid; every (sequence, head) of the
    step against the oracle, the new token's slot bit for bit, the step counters."""
    rng = np.random.default_rng(seed)
    L = rng.integers(0, max_L + 1, size=B)
    L[0], L[-1] = 0, max_L
    T_now = rng.integers(1, 3 * n, size=B)          # the step's output index (1-based)
    bad = B // 2
    banner(f"flat work list {dtype} d={d} B={B} H={H} L {L.min()}..{L.max()} n={n} fused={fused}")
    cache = rs.KVCache.allocate(L.tolist(), H, d, n, dtype=DTYPE[dtype])
    assert rs.rswa_decode_workspace_size(cache.desc, 0) == _flat_workspace_bytes(B, H, d)
    dt = np.uint16 if dtype == "bf16" else np.float32
    host_k = np.zeros(cache.k.numel(), dtype=dt)
    host_v = np.zeros(cache.v.numel(), dtype=dt)
    bases = cache.seq_base.cpu().numpy()
    draw = lambda *words, shape: wl.draw(dtype, 1.0, shape, 20269000 + seed, *words)
    q = draw(0, shape=(B, H, d))
    k_new = draw(1, shape=(B, H, d))
    v_new = draw(2, shape=(B, H, d))
    refs, wins = [], []
    for b in range(B):
        Lb, T = int(L[b]), int(T_now[b])
        kr, vr = draw(3, b, shape=(H, Lb, d)), draw(4, b, shape=(H, Lb, d))
        blk_k = host_k[bases[b]:bases[b] + H * (Lb + n) * d].reshape(H, Lb + n, d)
        blk_v = host_v[bases[b]:bases[b] + H * (Lb + n) * d].reshape(H, Lb + n, d)
        blk_k[:, :Lb], blk_v[:, :Lb] = kr, vr
        win = {t: (draw(5, b, t, shape=(H, d)), draw(6, b, t, shape=(H, d))) for t in range(max(1, T - n), T)}
        win[T] = (k_new[b], v_new[b])
        last = T if not fused else T - 1          # outputs already in the cache before the call
        for t in range(max(1, last - n + 1), last + 1):
            blk_k[:, orc.ring_slot(Lb, n, t)], blk_v[:, orc.ring_slot(Lb, n, t)] = win[t]
        refs.append((kr, vr))
        wins.append(win)
    cache.k.copy_(to_dev(host_k, dtype))
    cache.v.copy_(to_dev(host_v, dtype))
    steps0 = (T_now - 1 if fused else T_now).astype(np.int32)
    cache.step.copy_(torch.from_numpy(steps0))
    cache.ref_len[bad] = max_L + 1                    # above max_ref_len: flagged and skipped
    ws = cache.workspace()
    out = torch.full((B, H, d), float("nan"), dtype=cache.k.dtype, device="cuda")
    kd, vd = (to_dev(k_new, dtype), to_dev(v_new, dtype)) if fused else (None, None)
    rs.rswa_decode_attn(cache.desc, to_dev(q, dtype), out, kd, vd, 0.0, 0, ws)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert rs.rswa_check_device_error(cache.desc) == rs.RSWA_DEVERR_REF_LEN
    steps = cache.step.cpu().numpy()
    expect_steps = T_now.astype(np.int32).copy()
    expect_steps[bad] = steps0[bad]
    assert np.array_equal(steps, expect_steps)
    assert np.all(got[bad] == 0)
    good = [b for b in range(B) if b != bad]
    ref = np.zeros((len(good), H, d))
    for i, b in enumerate(good):
        Lb, T = int(L[b]), int(T_now[b])
        first = max(1, T - n + 1)
        ko = np.stack([wins[b][t][0] for t in range(first, T + 1)], axis=1)
        vo = np.stack([wins[b][t][1] for t in range(first, T + 1)], axis=1)
        kr, vr = refs[b]
        for h in range(H):
            ref[i, h] = orc.decode_output(wl.to_f64(q[b, h], dtype), wl.to_f64(kr[h], dtype),
                                          wl.to_f64(vr[h], dtype), wl.to_f64(ko[h], dtype),
                                          wl.to_f64(vo[h], dtype), first, Lb, n, T, 1.0 / math.sqrt(d))
    ma, rel = check_close(got[good], ref, dtype, "flat work list")
    print(f"flat work list: max|d|={ma:.3e} worst (b,h) rel={rel:.3e}")
    if fused:   # the new token sits in its ring slot, bit for bit (flagged sequence untouched)
        kb_all = bits(cache.k)
        for b in good:
            Lb, T = int(L[b]), int(T_now[b])
            blk = kb_all[bases[b]:bases[b] + H * (Lb + n) * d].reshape(H, Lb + n, d)
            assert np.array_equal(blk[:, orc.ring_slot(Lb, n, T)], storage_bits(k_new[b]))


def test_ragged_batch_one_fused_step():
    """64 sequences with their own L_m and decode position; the caller writes the
    cache state directly by the ABI's slot rule, then one fused append+attend."""
    w = wl.RAGGED_64
    r = wl.ragged_lengths(w)
    banner(f"ragged 64 sequences, L_m {r.ref_len.min()}..{r.ref_len.max()}, T {r.t_now.min()}..{r.t_now.max()}")
    n, H, d = w.window, w.heads, w.head_dim
    cache = rs.KVCache.allocate(r.ref_len.tolist(), H, d, n, dtype=rs.RSWA_BF16)
    host_k = np.zeros(cache.k.numel(), dtype=np.uint16)
    host_v = np.zeros(cache.v.numel(), dtype=np.uint16)
    bases = cache.seq_base.cpu().numpy()
    refs, wins = [], []
    q_new = np.zeros((w.batch, H, d), np.uint16)
    k_new = np.zeros((w.batch, H, d), np.uint16)
    v_new = np.zeros((w.batch, H, d), np.uint16)
    for b in range(w.batch):
        L, T = int(r.ref_len[b]), int(r.t_now[b])
        kr, vr = wl.ragged_ref_kv(w, b, L)
        blk_k = host_k[bases[b]:bases[b] + H * (L + n) * d].reshape(H, L + n, d)
        blk_v = host_v[bases[b]:bases[b] + H * (L + n) * d].reshape(H, L + n, d)
        blk_k[:, :L] = kr
        blk_v[:, :L] = vr
        first = max(1, T - n + 1)
        win = {}
        for t_out in range(first, T + 1):
            win[t_out] = wl.ragged_token_kv(w, b, t_out)
        for t_out in range(max(1, T - n), T):     # outputs already in the cache before the step
            kt, vt = win[t_out] if t_out in win else wl.ragged_token_kv(w, b, t_out)
            blk_k[:, orc.ring_slot(L, n, t_out)] = kt
            blk_v[:, orc.ring_slot(L, n, t_out)] = vt
        k_new[b], v_new[b] = win[T]
        q_new[b] = wl.ragged_query(w, b, T)
        refs.append((kr, vr))
        wins.append(win)
    cache.k.copy_(to_dev(host_k, "bf16"))
    cache.v.copy_(to_dev(host_v, "bf16"))
    cache.step.copy_(torch.from_numpy((r.t_now - 1).astype(np.int32)))
    ws = cache.workspace()
    out = torch.empty((w.batch, H, d), dtype=torch.bfloat16, device="cuda")
    rs.rswa_decode_attn(cache.desc, to_dev(q_new, "bf16"), out, to_dev(k_new, "bf16"), to_dev(v_new, "bf16"),
                        0.0, 0, ws)
    got = to_f64(out)
    assert np.array_equal(cache.step.cpu().numpy(), r.t_now.astype(np.int32))
    ref = np.zeros_like(got)
    for b in range(w.batch):
        L, T = int(r.ref_len[b]), int(r.t_now[b])
        first = max(1, T - n + 1)
        kr, vr = refs[b]
        ko = np.stack([wins[b][t][0] for t in range(first, T + 1)], axis=1)   # [H][S][d]
        vo = np.stack([wins[b][t][1] for t in range(first, T + 1)], axis=1)
        for h in range(H):
            ref[b, h] = orc.decode_output(wl.to_f64(q_new[b, h], "bf16"), wl.to_f64(kr[h], "bf16"),
                                          wl.to_f64(vr[h], "bf16"), wl.to_f64(ko[h], "bf16"),
                                          wl.to_f64(vo[h], "bf16"), first, L, n, T, w.scale)
    ma, rel = check_close(got, ref, "bf16", "ragged")
    print(f"ragged: max|d|={ma:.3e} rel={rel:.3e}")
    # the new token sits in its ring slot, bit for bit
    kb_all = bits(cache.k)
    for b in range(w.batch):
        L, T = int(r.ref_len[b]), int(r.t_now[b])
        blk = kb_all[bases[b]:bases[b] + H * (L + n) * d].reshape(H, L + n, d)
        assert np.array_equal(blk[:, orc.ring_slot(L, n, T)], storage_bits(k_new[b]))
    assert rs.rswa_check_device_error(cache.desc) == 0


def _small_fp32(L_m=13, n=5, B=3, H=2, d=64, steps=23, seed=5):
    return wl.DecodeWorkload("small-fp32", batch=B, heads=H, head_dim=d, ref_len=L_m, window=n,
                             steps=steps, dtype="fp32", sigma_q=1.0, sigma_kv=1.0, base_seed=seed)


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7, 16, 64])
def test_split_count_invariance(splits):
    w = wl.DecodeWorkload("split-fp32", batch=2, heads=3, head_dim=128, ref_len=700, window=16,
                          steps=40, dtype="fp32", sigma_q=1.0, sigma_kv=1.0, base_seed=77)
    banner(f"split invariance splits={splits}")
    run = DecodeRun(w, num_splits=splits)
    got = run.run(w.steps, keep=[1, 16, 17, 40])
    for T, o in got.items():
        check_close(o.reshape(-1, 128), run.oracle(T), "fp32", f"splits={splits} T={T}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_one_launch_equals_split_and_merge(dtype, d):
    """With one split, the single launch (arrival counters given) and the split + merge
    launches (no counters) give the same bits, step counts and cache images, through
    the wrap; the counters are back at zero after every call."""
    B, H, L, n, steps = 3, 4, 150, 16, 40
    w = wl.DecodeWorkload("one-launch", batch=B, heads=H, head_dim=d, ref_len=L, window=n, steps=steps,
                          dtype=dtype, sigma_q=1.0, sigma_kv=1.0, base_seed=78)
    banner(f"one launch vs split + merge {dtype} d={d}")
    one, two = DecodeRun(w, num_splits=1), DecodeRun(w, num_splits=1)
    two.cache.desc.arrive = None
    for T in range(1, steps + 1):
        q, k, v = (to_dev(x[0], dtype) for x in wl.steps_qkv(w, T, T))
        for r in (one, two):
            rs.rswa_decode_attn(r.cache.desc, q, r.out, k, v, 0.0, 1, r.ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(one.out), bits(two.out)), f"step {T}"
        assert one.cache.arrive.cpu().tolist() == [0] * B
    assert one.cache.step.cpu().tolist() == two.cache.step.cpu().tolist() == [steps] * B
    assert np.array_equal(bits(one.cache.k), bits(two.cache.k))
    assert np.array_equal(bits(one.cache.v), bits(two.cache.v))
    assert rs.rswa_check_device_error(one.cache.desc) == 0


@pytest.mark.parametrize("L_m,n,d", [(0, 4, 64), (1, 1, 128), (3, 2, 64), (130, 128, 128), (64, 300, 64)])
def test_decode_shapes_fp32(L_m, n, d):
    w = _small_fp32(L_m=L_m, n=n, d=d, steps=2 * n + 5 if n < 100 else 140)
    banner(f"fp32 decode L_m={L_m} n={n} d={d}")
    run = DecodeRun(w)
    keep = list(range(1, w.steps + 1))
    got = run.run(w.steps, keep=keep)
    steps = wl.steps_qkv(w, 1, w.steps)
    for T in keep:
        check_close(got[T].reshape(-1, d), run.oracle(T, steps=steps), "fp32", f"L_m={L_m} n={n} T={T}")
    run.check_cache_image()


def test_bf16_head_dim_64():
    w = wl.DecodeWorkload("bf16-d64", batch=2, heads=4, head_dim=64, ref_len=200, window=32, steps=80,
                          dtype="bf16", sigma_q=1.0, sigma_kv=1.0, base_seed=91)
    banner("bf16 d=64 decode")
    run = DecodeRun(w)
    got = run.run(w.steps, keep=[1, 31, 32, 33, 80])
    for T, o in got.items():
        check_close(o.reshape(-1, 64), run.oracle(T), "bf16", f"d64 T={T}")
    run.check_cache_image()


def test_decode_is_deterministic():
    w = wl.ONE_PAGE
    banner("determinism: two identical runs are bit-identical")
    a = DecodeRun(w)
    ga = a.run(300, keep=[129, 300])
    b = DecodeRun(w, ref=(a.kref, a.vref))
    gb = b.run(300, keep=[129, 300])
    for T in ga:
        np.testing.assert_array_equal(ga[T], gb[T])
    assert np.array_equal(bits(a.cache.k), bits(b.cache.k))


def test_checkpoint_and_restore():
    w = wl.ONE_PAGE
    banner("checkpoint / restore of the decode state")
    run = DecodeRun(w)
    run.run(150)
    snap = (run.cache.k.clone(), run.cache.v.clone(), run.cache.step.clone())
    first = run.run(190, keep=range(151, 191))
    run.cache.k.copy_(snap[0])
    run.cache.v.copy_(snap[1])
    run.cache.step.copy_(snap[2])
    run.T = 150
    second = run.run(190, keep=range(151, 191))
    for T in first:
        np.testing.assert_array_equal(first[T], second[T])


# ----------------------------------------------------------- structured probes
def _probe_cache(L_m, n, H, d):
    cache = rs.KVCache.allocate([L_m], H, d, n, dtype=rs.RSWA_FP32)
    return cache


def test_uniform_query_probe():
    """q = 0: the output is the mean of the visible values; V_ref = 0 and output T' has value T'."""
    L_m, n, H, d, S = 64, 8, 2, 64, 40
    banner("uniform-query probe")
    cache = _probe_cache(L_m, n, H, d)
    kref = torch.randn(H * L_m * d, device="cuda")
    vref = torch.zeros(H * L_m * d, device="cuda")
    rs.rswa_cache_init(cache.desc, kref, vref, torch.zeros(1, dtype=torch.int64, device="cuda"))
    ws = cache.workspace()
    out = torch.empty((1, H, d), device="cuda")
    q = torch.zeros((1, H, d), device="cuda")
    for T in range(1, S + 1):
        k = torch.randn((1, H, d), device="cuda")
        v = torch.full((1, H, d), float(T), device="cuda")
        rs.rswa_decode_attn(cache.desc, q, out, k, v, 0.0, 0, ws)
        lo = max(1, T - n + 1)
        expect = sum(range(lo, T + 1)) / (L_m + min(n, T))
        got = out.cpu().numpy()
        np.testing.assert_allclose(got, expect, rtol=2e-6, atol=0, err_msg=f"T={T}")


@pytest.mark.parametrize("offset,visible", [(0, False), (1, True)])
def test_needle_probe_window_edge(offset, visible):
    """A key aligned with q placed at output T-n (evicted) gets no weight; at T-n+1 it dominates."""
    L_m, n, H, d, T = 64, 8, 1, 64, 20
    banner(f"needle probe at output T-n+{offset}")
    cache = _probe_cache(L_m, n, H, d)
    z = torch.zeros(H * L_m * d, device="cuda")
    rs.rswa_cache_init(cache.desc, z, z, torch.zeros(1, dtype=torch.int64, device="cuda"))
    ws = cache.workspace()
    out = torch.empty((1, H, d), device="cuda")
    q = torch.zeros((1, H, d), device="cuda")
    q[..., 0] = 1.0
    needle = T - n + offset
    for t_out in range(1, T + 1):
        k = torch.zeros((1, H, d), device="cuda")
        v = torch.zeros((1, H, d), device="cuda")
        if t_out == needle:
            k[..., 0] = 800.0
            v[..., 1] = 1.0
        rs.rswa_decode_attn(cache.desc, q, out, k, v, 0.0, 0, ws)
    o1 = float(out[0, 0, 1].item())
    if visible:
        assert o1 > 0.999
    else:
        assert o1 == 0.0


# ------------------------------------------------------- device-side checks
def test_device_error_flags():
    banner("device error flags")
    H, d, n = 2, 64, 4
    cache = rs.KVCache.allocate([8, 0], H, d, n, dtype=rs.RSWA_FP32)
    ws = cache.workspace()
    q = torch.randn((2, H, d), device="cuda")
    out = torch.empty_like(q)
    # sequence 1 has L_m = 0 and T = 0: nothing visible without a fused append
    rs.rswa_decode_attn(cache.desc, q, out, None, None, 0.0, 0, ws)
    assert rs.rswa_check_device_error(cache.desc) == rs.RSWA_DEVERR_EMPTY
    assert rs.rswa_check_device_error(cache.desc) == 0          # cleared by the read
    cache.step[0] = -3
    rs.rswa_append_kv(cache.desc, q, q)
    assert rs.rswa_check_device_error(cache.desc) & rs.RSWA_DEVERR_STEP
    assert int(cache.step[0].item()) == -3                       # skipped, untouched
    cache.step[0] = 0
    cache.ref_len[0] = 9                                         # > max_ref_len = 8
    rs.rswa_decode_attn(cache.desc, q, out, q, q, 0.0, 0, ws)
    flags = rs.rswa_check_device_error(cache.desc)
    assert flags & rs.RSWA_DEVERR_REF_LEN
    assert int(cache.step[0].item()) == 0
    assert int(cache.step[1].item()) == 2                        # the valid sequence advanced


def test_one_launch_device_errors_leave_counters_at_zero():
    """A full batch decoded in one launch: sequences with invalid device state are
    flagged, keep their step, get zero outputs, and never count themselves in; the
    other sequences advance and every arrival counter is back at zero."""
    B, H, d, n, L = 32, 16, 128, 8, 40
    banner("one-launch decode with flagged sequences")
    cache = rs.KVCache.allocate([L] * B, H, d, n, dtype=rs.RSWA_BF16)
    cache.k.normal_()
    cache.v.normal_()
    ws = cache.workspace()
    assert ws.numel() == rs.rswa_decode_workspace_size(cache.desc, 1)  # one chunk per (sequence, head)
    q, k, v = (torch.randn((B, H, d), device="cuda").to(torch.bfloat16) for _ in range(3))
    out = torch.empty_like(q)
    cache.ref_len[3] = L + 1   # above max_ref_len
    cache.step[7] = -2
    for _ in range(3):
        rs.rswa_decode_attn(cache.desc, q, out, k, v, 0.0, 0, ws)
    torch.cuda.synchronize()
    flags = rs.rswa_check_device_error(cache.desc)
    assert flags & rs.RSWA_DEVERR_REF_LEN and flags & rs.RSWA_DEVERR_STEP
    steps = cache.step.cpu().tolist()
    assert steps[3] == 0 and steps[7] == -2
    assert all(t == 3 for b, t in enumerate(steps) if b not in (3, 7))
    assert cache.arrive.cpu().tolist() == [0] * B
    o = out.float()
    assert torch.all(o[3] == 0) and torch.all(o[7] == 0)
    assert torch.isfinite(o).all()


def test_active_mask_and_guard_regions():
    """Sequences with active[b] = 0 are untouched; nothing is written outside the blocks."""
    banner("active mask and canary guards")
    H, d, n = 2, 128, 4
    L = [5, 9, 3]
    cache = rs.KVCache.allocate(L, H, d, n, dtype=rs.RSWA_BF16)
    canary = torch.full((4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    big_k = torch.cat([canary, cache.k, canary])
    big_v = torch.cat([canary, cache.v, canary])
    cache.k, cache.v = big_k[4096:-4096], big_v[4096:-4096]
    cache.desc.k, cache.desc.v = cache.k.data_ptr(), cache.v.data_ptr()
    kref = torch.randn(H * max(L) * d * 3, device="cuda").to(torch.bfloat16)
    base = torch.tensor([0, H * max(L) * d, 2 * H * max(L) * d], dtype=torch.int64, device="cuda")
    rs.rswa_cache_init(cache.desc, kref, kref, base)
    active = torch.tensor([1, 0, 1], dtype=torch.uint8, device="cuda")
    for _ in range(7):
        kv = torch.randn((3, H, d), device="cuda").to(torch.bfloat16)
        rs.rswa_append_kv(cache.desc, kv, kv, active)
    assert cache.step.cpu().tolist() == [7, 0, 7]
    for g in (big_k[:4096], big_k[-4096:], big_v[:4096], big_v[-4096:]):
        assert torch.isnan(g.float()).all()
    assert rs.rswa_check_device_error(cache.desc) == 0


# ------------------------------------------------------------ packed form
def _masked_case(N, L_m, n, H, mode, seed):
    mw = wl.MaskedWorkload("masked-small", seq_len=N, heads=H, head_dim=128, ref_len=L_m, window=n,
                           dtype="bf16", sigma=1.0, base_seed=seed)
    Q, K, V = wl.packed_qkv(mw)
    out = torch.empty((N, H, 128), dtype=torch.bfloat16, device="cuda")
    rs.rswa_masked_attn(to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16"), out, N, L_m, n, H, 128,
                        rs.RSWA_BF16, mode, 0.0)
    torch.cuda.synchronize()
    return mw, (Q, K, V), to_f64(out)


@pytest.mark.parametrize("N,L_m,n,mode", [
    (300, 40, 8, rs.RSWA_PREFIX_CAUSAL),
    (300, 40, 8, rs.RSWA_PREFIX_FULL),
    (1, 1, 128, rs.RSWA_PREFIX_CAUSAL),
    (257, 0, 16, rs.RSWA_PREFIX_CAUSAL),
    (200, 200, 4, rs.RSWA_PREFIX_FULL),
    (513, 130, 128, rs.RSWA_PREFIX_CAUSAL),
    (640, 97, 1, rs.RSWA_PREFIX_CAUSAL),
    (700, 300, 200, rs.RSWA_PREFIX_FULL),
    (1, 0, 1, rs.RSWA_PREFIX_CAUSAL),
    (161, 33, 1000, rs.RSWA_PREFIX_CAUSAL),
    (200, 200, 4, rs.RSWA_PREFIX_CAUSAL),
])
def test_masked_small_every_row(N, L_m, n, mode):
    H = 2
    banner(f"packed N={N} L_m={L_m} n={n} mode={mode}")
    mw, (Q, K, V), got = _masked_case(N, L_m, n, H, mode, seed=1000 + N + L_m + n + mode)
    f = lambda a: wl.to_f64(a, "bf16")
    ref = orc.masked_attention_rows(f(Q), f(K), f(V), range(N), L_m, n, mw.scale, mode)
    check_close(got, ref, "bf16", f"packed N={N} L_m={L_m} n={n} mode={mode}")


@pytest.mark.parametrize("mode", [rs.RSWA_PREFIX_CAUSAL, rs.RSWA_PREFIX_FULL])
def test_masked_score_ranges(mode):
    """Scores far from the unit range (score_range_qkv: growing along the sequence, so
    later blocks keep exceeding the running max many times over; strongly negative;
    strongly positive; ordinary). The kernel forms a block's
    probabilities against the running max before looking at the block, so these rows
    exercise its raise-and-retake path; every row against the oracle (Eqs. (3)-(4) of
    the pages' attention do not depend on the max used)."""
    N, L_m, n, H = 700, 200, 64, 4
    banner(f"packed score ranges mode={mode}")
    Qb, Kb, Vb = score_range_qkv(N, H)
    Qf, Kf, Vf = (wl.to_f64(x, "bf16") for x in (Qb, Kb, Vb))
    scale = 1.0 / math.sqrt(128)
    s1 = np.einsum("id,id->i", Qf[:, 1], Kf[:, 1]) * scale
    s2 = np.einsum("id,id->i", Qf[:, 2], Kf[:, 2]) * scale
    assert s1.max() < -30 and s2.min() > 30        # the ranges the heads are built for
    out = torch.empty((N, H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
    rs.rswa_masked_attn(to_dev(Qb, "bf16"), to_dev(Kb, "bf16"), to_dev(Vb, "bf16"), out, N, L_m, n, H, 128,
                        rs.RSWA_BF16, mode, 0.0, lse=lse)
    torch.cuda.synchronize()
    ref = orc.masked_attention_rows(Qf, Kf, Vf, range(N), L_m, n, scale, mode)
    check_close(to_f64(out), ref, "bf16", f"score ranges mode={mode}")
    assert np.isfinite(lse.cpu().numpy()).all()


def test_masked_rows_agree_with_decode_kernel():
    """Teacher-forced rows (packed kernel) equal the decode kernel's outputs at the same step."""
    N, L_m, n, H = 400, 150, 32, 2
    banner("packed rows vs decode kernel")
    mw, (Q, K, V), got = _masked_case(N, L_m, n, H, rs.RSWA_PREFIX_CAUSAL, seed=4242)
    cache = rs.KVCache.allocate([L_m], H, 128, n, dtype=rs.RSWA_BF16)
    kref = to_dev(np.ascontiguousarray(K[:L_m].transpose(1, 0, 2)).reshape(-1), "bf16")
    vref = to_dev(np.ascontiguousarray(V[:L_m].transpose(1, 0, 2)).reshape(-1), "bf16")
    rs.rswa_cache_init(cache.desc, kref, vref, torch.zeros(1, dtype=torch.int64, device="cuda"))
    ws = cache.workspace()
    out = torch.empty((1, H, 128), dtype=torch.bfloat16, device="cuda")
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    for i in range(L_m, N):
        rs.rswa_decode_attn(cache.desc, Qd[i:i + 1], out, Kd[i:i + 1], Vd[i:i + 1], 0.0, 0, ws)
        check_close(to_f64(out)[0], got[i], "bf16", f"row {i}")


@pytest.mark.slow
@pytest.mark.parametrize("mode", [rs.RSWA_PREFIX_CAUSAL, rs.RSWA_PREFIX_FULL])
def test_packed_32k_sampled_rows(mode):
    """All heads of: the rows at the segment and window edges, both edge rows of
    every 128-row tile, and 2048 seeded random rows (oracle on all host cores)."""
    mw = wl.PACKED_32K
    N, L_m, n, H = mw.seq_len, mw.ref_len, mw.window, mw.heads
    banner(f"packed 32K masked forward, N={N} L_m={L_m} n={n} H={H} mode={mode}")
    Q, K, V = wl.packed_qkv(mw)
    out = torch.empty((N, H, 128), dtype=torch.bfloat16, device="cuda")
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    rs.rswa_masked_attn(Qd, Kd, Vd, out, N, L_m, n, H, 128, rs.RSWA_BF16, mode, 0.0)
    torch.cuda.synchronize()
    got = to_f64(out)
    del Qd, Kd, Vd, out
    rng = np.random.default_rng(11)
    special = [0, 1, L_m - 2, L_m - 1, L_m, L_m + 1, L_m + n - 2, L_m + n - 1, L_m + n, L_m + n + 1,
               4095, 4096, 4223, 4224, N - 1]
    edges = [e for t in range(N // 128) for e in (128 * t, 128 * t + 127)]
    rows = sorted(set(special + edges + rng.choice(N, 2048, replace=False).tolist()))
    print(f"oracle: {len(rows)} rows x {H} heads on {opool.workers()} processes", flush=True)
    with opool.SharedArrays() as arrays:
        for name, a in (("Q", Q), ("K", K), ("V", V)):
            arrays.put(name, wl.bf16_bits_to_f32(a))   # exact values of the bf16 inputs
        chunks = [rows[i::64] for i in range(64)]
        parts = opool.pool_map(opool.masked_rows_job,
                               [(c, L_m, n, mw.scale, mode) for c in chunks], arrays, progress="packed rows")
    ref = np.empty((len(rows), H, 128))
    pos = {r: i for i, r in enumerate(rows)}
    for c, part in zip(chunks, parts):
        ref[[pos[r] for r in c]] = part
    ma, rel = check_close(got[rows], ref, "bf16", f"packed 32K rows, mode {mode}")
    print(f"packed 32K: {len(rows)} rows x {H} heads max|d|={ma:.3e} worst (row, head) rel={rel:.3e}")
