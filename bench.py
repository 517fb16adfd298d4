#!/usr/bin/env python3
"""Benchmark of the R-SWA decode hot path on one MI355X.

A step is one fused append + attend decode step of the 40-page workload
(B = 32 sequences, H = 16 heads, d = 128, L_m = 10272, n = 128, bf16, one
attention layer): one call of rswa_decode_attn. The first n = 128 steps fill
the window (untimed), W warm-up steps follow, then exactly K steps are timed
back to back with HIP events on the launch stream, so every timed step sees the
full L_m + n slots; K further steps are timed one by one for the median and
p10/p90. All inputs (reference K/V, per-step q/k/v) are resident in HBM before
the timed region.

Printed: one JSON line. `value` is decode tokens/s (B / step time). The
`roofline` object prices the decode kernel's algorithmic bytes (every visible
K/V row once, plus q, out and the new k/v) against the 8 TB/s HBM peak.
`cpu_baseline` times the CPU oracle on the whole last timed step, on the
host's cores, and `parity` compares that step's outputs with the oracle's
(every sequence and head) and every window slot of the cache after the last
step with the ring rule. `device` records the hardware as the runtime reports
it; the read, matrix-core and per-CU probes give the ceilings the fractions
are read against.
Secondary lines of the same JSON: the full-attention contrast (cache L_m + T)
at a few decode lengths, and the packed 32K masked forward (both prefix modes)
and its backward, a multi-document 32K pack, the prefill -> decode hand-off
at the 40-page shape, and a multi-layer decode step replayed as one HIP graph
at the output lengths of the pages' TPS table (R-SWA against full attention).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "R-SWA decode-attn tokens/s and HBM GB/s (%peak) at L_m=10272, n=128, B=32"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COUNTERS = os.path.join(ROOT, "profiles", "decode_40page_counters.txt")
DECODE_SRC = os.path.join(ROOT, "reference_sliding_window_amd", "csrc", "rswa_decode.hip")


def decode_bytes(B, H, d, L, n, T, elt=2):
    """Algorithmic bytes of one decode step: visible K and V rows once, plus q, out, k_new, v_new."""
    return B * H * (L + min(n, T)) * d * elt * 2 + 4 * B * H * d * elt


def masked_tile_flops(N, L_m, n, H, prefix_full=False):
    """FLOP the packed forward's matrix products execute (d = 128): every 64-key block that meets a
    128-row query block's reference range or window range is multiplied whole, 4 waves x 32 products
    of 32768 FLOP (16 for S^T, 16 for O^T); the algorithmic count takes visible pairs only."""
    blocks = 0
    for q0 in range(0, N, 128):
        q_end = min(N, q0 + 128)
        pre_hi = L_m if (prefix_full and q0 < L_m) else min(L_m, q_end)
        win_lo = max(L_m, max(q0, L_m) - n + 1)
        win_hi = q_end if q_end > L_m else win_lo
        blocks += (pre_hi + 63) // 64 + (win_hi - win_lo + 63) // 64
    return blocks * H * 4 * 32 * 32768


def masked_flops(N, L_m, n, H, d, prefix_full=False):
    """4 d FLOP per visible (query, key) pair of the two-segment mask."""
    pre = L_m * L_m if prefix_full else L_m * (L_m + 1) // 2
    outs = N - L_m
    win = sum(min(n, t) for t in range(1, outs + 1)) if outs > 0 else 0
    return 4 * d * H * (pre + L_m * max(outs, 0) + win)


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(per_launch_units):
    """HBM traffic of the decode kernel from the committed rocprofv3 counter summary,
    or None if the summary is missing or was taken on different kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    for ln in open(COUNTERS):
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != source_sha(DECODE_SRC):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def event_time_ms(fn, iters, stream):
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(iters):
        fn(i)
    b.record(stream)
    b.synchronize()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def cpu_baseline(w, kref, vref, T):
    """Time the oracle on every (sequence, head) of decode step T (all B x H pairs, the
    whole step) on the host's cores: one worker process per core, BLAS on one thread
    each, inputs in shared memory before the clock starts. Returns the timing line and
    the oracle's outputs of that step, [B][H][d] float64."""
    import oracle.pool as opool
    import workloads as wl
    with opool.SharedArrays() as arrays:
        arrays.put("kref", kref)
        arrays.put("vref", vref)
        first = max(1, T - w.window + 1)
        for name, a in zip(("q", "k", "v"), wl.steps_qkv(w, first, T)):
            arrays.new(name, (T,) + a.shape[1:], a.dtype)[first - 1:T] = a   # the job reads only these
        tasks = [(w.dtype, w.ref_len, w.window, w.scale, b, list(range(w.heads)), [T])
                 for b in range(w.batch)]
        with opool.OraclePool(arrays) as pool:
            pool.map(opool.ready, range(4 * pool.processes))   # every worker up before timing
            t0 = time.perf_counter()
            res = pool.map(opool.decode_sequence_job, tasks)
            el = time.perf_counter() - t0
            cores = pool.processes
    ref = np.stack([r[T] for r in res])
    return ref, {"value": w.batch / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole 40-page decode step T={T} (steady state, window full): all "
                      f"{w.batch * w.heads} (sequence, head) pairs in {el:.1f} s wall on {cores} worker "
                      f"processes (one per host core, BLAS on one thread each; {cores * el:.0f} core-seconds); "
                      f"host reports {len(os.sched_getaffinity(0))} cores available"}


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def device_facts(torch, rs):
    """The device as torch and the HIP runtime (through the library) report it: the unit counts and
    sizes the roofline figures assume, and the peak clocks."""
    p = torch.cuda.get_device_properties(0)
    f = rs.rswa_device_facts(torch.cuda.current_device())
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "total_memory_GiB": round(p.total_memory / 2 ** 30, 1),
            "l2_cache_MiB_reported": round(getattr(p, "L2_cache_size", 0) / 2 ** 20, 1),
            "lds_KiB_per_cu": f["lds_bytes_per_cu"] / 1024, "wave_size": f["wave_size"],
            "peak_shader_clock_MHz": f["clock_khz"] / 1000, "peak_memory_clock_MHz": f["mem_clock_khz"] / 1000,
            "memory_bus_width_bits": f["mem_bus_bits"]}


def probe_read_GBps(torch, rs, stream, nbytes=4 << 30):
    """Achievable streaming-read rate with the decode kernel's access pattern (buffer > 256 MB MALL)."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1024, dtype=torch.float32, device="cuda")
    run = lambda i: rs.rswa_probe_stream_read(buf, nbytes, sink, 0, stream=stream)
    for _ in range(3):
        run(0)
    ms = event_time_ms(run, 10, stream) / 10
    del buf, sink
    return nbytes / (ms * 1e-3) / 1e9


def mfma_probe_tflops(torch, rs, stream, iters=4096, workgroups=512):
    """bf16 32x32x16 matrix products issued back to back by two waves per SIMD: the rate the chip
    sustains at the clock it holds under matrix load (the packed kernels' practical ceiling)."""
    sink = torch.empty(workgroups, dtype=torch.float32, device="cuda")
    run = lambda i: rs.rswa_probe_mfma(sink, workgroups, iters, stream=stream)
    for _ in range(3):
        run(0)
    ms = event_time_ms(run, 10, stream) / 10
    return workgroups * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12


def cu_probe(torch, rs, stream, workgroups=256):
    """Per-CU rates of the other units the packed kernels lean on, in shader-clock cycles
    (rswa_probe_cu: one workgroup of 8 waves per CU, cycles counted on the device)."""
    out = torch.zeros(2 * workgroups, dtype=torch.int32, device="cuda")
    res = {}
    for kind, name, iters in ((rs.RSWA_PROBE_LDS_B128, "lds_ds_read_b128", 512),
                              (rs.RSWA_PROBE_LDS_TR16, "lds_ds_read_b64_tr_b16", 512),
                              (rs.RSWA_PROBE_EXP, "v_exp_f32", 8192), (rs.RSWA_PROBE_FMA, "v_fma_f32", 8192)):
        run = lambda i: rs.rswa_probe_cu(out, workgroups, iters, kind, stream=stream)
        for _ in range(3):
            run(0)
        ms = event_time_ms(run, 5, stream) / 5
        cycles = float(np.median(out.view(torch.int32).cpu().numpy()[0::2].astype(np.uint32)))
        if kind in (rs.RSWA_PROBE_LDS_B128, rs.RSWA_PROBE_LDS_TR16):
            res[name + "_bytes_per_clk_per_cu"] = 8 * iters * 16384 / cycles
        else:
            res[name + "_cycles_per_wave_instruction_per_simd"] = cycles / (2 * iters * 8)
        res[name + "_shader_clock_GHz"] = cycles / (ms * 1e-3) / 1e9
    res["how"] = ("rswa_probe_cu: 256 workgroups of 8 waves (one per CU, two waves per SIMD); LDS kinds: 16 KB "
                  "per wave per round, "
                  "the forward's K-fragment (ds_read_b128) and V^T (ds_read_b64_tr_b16) patterns on its "
                  "swizzled tiles; exp/fma: 8 independent instructions per wave per round; median cycles "
                  "over workgroups (s_memtime); the clock is those cycles over the kernel's event time")
    return res


def gemm_tflops(torch, stream, m=8192):
    """A large bf16 GEMM through the vendor library: the measured matrix-core reference."""
    a = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    b = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    c = torch.empty((m, m), device="cuda", dtype=torch.bfloat16)
    run = lambda i: torch.matmul(a, b, out=c)
    for _ in range(3):
        run(0)
    ms = event_time_ms(run, 10, stream) / 10
    del a, b, c
    return 2 * m ** 3 / (ms * 1e-3) / 1e12


def cpu_masked_rows(mw, Q, K, V, rows_per_core=48):
    """Time the oracle's packed forward on random output rows (all heads) on the host's
    cores and scale to all rows."""
    import oracle.pool as opool
    import workloads as wl
    with opool.SharedArrays() as arrays:
        for name, a in (("Q", Q), ("K", K), ("V", V)):
            arrays.put(name, wl.bf16_bits_to_f32(a))   # exact values of the bf16 inputs
        with opool.OraclePool(arrays) as pool:
            cores = pool.processes
            rng = np.random.default_rng(1)
            rows = rng.integers(mw.ref_len, mw.seq_len, rows_per_core * cores).tolist()
            tasks = [(rows[i::cores], mw.ref_len, mw.window, mw.scale, 0) for i in range(cores)]
            pool.map(opool.ready, range(4 * cores))
            t0 = time.perf_counter()
            pool.map(opool.masked_rows_job, tasks)
            el = time.perf_counter() - t0
    per_row = el / len(rows)
    return {"seconds_per_output_row_all_heads": per_row,
            "extrapolated_seconds_for_all_rows": per_row * mw.seq_len, "cores": cores, "kind": "oracle",
            "sample": f"{len(rows)} random output rows x {mw.heads} heads in {el:.1f} s wall on {cores} worker "
                      f"processes (BLAS on one thread each); output rows see the most keys, so the "
                      f"extrapolation to all {mw.seq_len} rows is an upper bound"}


def per_step_curve(torch, rs, w, stream, Tmax):
    """Per-step duration of the fused decode step over T = 1 .. Tmax for the R-SWA cache and for a
    full-attention cache (L_m + Tmax slots), each step bracketed by HIP events: the shape of the
    pages' per-call kernel-duration figure."""
    B, H, d, L, n = w.batch, w.heads, w.head_dim, w.ref_len, w.window
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    curves = {}
    for name, window in (("rswa", n), ("full_attention", Tmax)):
        c = rs.KVCache.allocate([L] * B, H, d, window, dtype=rs.RSWA_BF16)
        c.k.normal_(0.0, w.sigma_kv)
        c.v.normal_(0.0, w.sigma_kv)
        c.step.zero_()
        ws = c.workspace()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(Tmax)]
        for c0 in range(0, Tmax, 512):
            c1 = min(Tmax, c0 + 512)
            x = torch.randn((3, c1 - c0, B, H, d), device="cuda").to(torch.bfloat16)
            for t in range(c0, c1):
                ev[t][0].record(stream)
                rs.rswa_decode_attn(c.desc, x[0, t - c0], out, x[1, t - c0], x[2, t - c0], 0.0, 0, ws,
                                    stream=stream)
                ev[t][1].record(stream)
            torch.cuda.synchronize()
            del x
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        bins = []
        for b0 in range(0, Tmax, 256):
            v = ms[b0:b0 + 256]
            bins.append({"T": f"{b0 + 1}..{min(Tmax, b0 + 256)}", "median_ms": float(np.median(v)),
                         "p10_ms": float(np.percentile(v, 10)), "p90_ms": float(np.percentile(v, 90)),
                         "max_ms": float(v.max())})
        curves[name] = {"bins": bins, "total_s": float(ms.sum() / 1e3),
                        "steady_median_ms": float(np.median(ms[n:])),
                        "tokens_per_s_whole_run": B * Tmax / (ms.sum() / 1e3)}
        if rs.rswa_check_device_error(c.desc):
            print("per-step curve reported device errors", file=sys.stderr)
            sys.exit(1)
        del c, ws
    return curves


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=256)
    ap.add_argument("--splits", type=int, default=0, help="decode key splits per (seq, head); 0 = library")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the contrast and masked lines")
    ap.add_argument("--layers", type=int, default=12,
                    help="attention layers in the multi-layer graph line (the pages do not state the count)")
    ap.add_argument("--curve", action="store_true",
                    help="also time every fused decode step T = 1..6144, R-SWA and full attention")
    ap.add_argument("--copy-reference", action="store_true",
                    help="first run a plain 1 GiB device copy 3 times (scale reference for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (requested --gpus {args.gpus}, WORLD_SIZE {world}); "
              "R-SWA decode shards by sequence and head with no exchange, so the per-GPU figure "
              "is the N=1 line.", file=sys.stderr)
        sys.exit(2)

    import torch
    import reference_sliding_window_amd as rs
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rs.library()  # fail loudly if the HIP library is missing
    # secondary lines draw their timing inputs on the device from torch's seeded generator
    torch.manual_seed(wl.FORTY_PAGE.base_seed)

    if args.copy_reference:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = wl.FORTY_PAGE
    B, H, d, L, n = w.batch, w.heads, w.head_dim, w.ref_len, w.window
    K, W = args.steps, args.warmup
    t_setup = time.perf_counter()
    kref, vref = wl.ref_kv_all(w)
    cache = rs.KVCache.allocate([L] * B, H, d, n, dtype=rs.RSWA_BF16)
    ref_base = torch.arange(B, dtype=torch.int64, device="cuda") * (H * L * d)
    kd = torch.from_numpy(kref.reshape(-1).view(np.int16)).view(torch.bfloat16).cuda()
    vd = torch.from_numpy(vref.reshape(-1).view(np.int16)).view(torch.bfloat16).cuda()
    rs.rswa_cache_init(cache.desc, kd, vd, ref_base)
    torch.cuda.synchronize()
    del kd, vd
    # outputs 1..n fill the window (untimed), then W warm-up and K timed steps, then K
    # more steps timed one by one for the per-step distribution: every timed step has
    # the full L_m + n slots visible (the steady state of Eq. (6))
    fill = n
    steps_total = fill + W + 2 * K
    qs = torch.empty((steps_total, B, H, d), dtype=torch.bfloat16, device="cuda")
    ks = torch.empty_like(qs)
    vs = torch.empty_like(qs)
    for c0 in range(0, steps_total, 512):
        c1 = min(steps_total, c0 + 512)
        q, k, v = wl.steps_qkv(w, c0 + 1, c1)
        for dst, src in ((qs, q), (ks, k), (vs, v)):
            dst[c0:c1].copy_(torch.from_numpy(src.view(np.int16)).view(torch.bfloat16))
    ws = cache.workspace(args.splits)
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    setup_s = time.perf_counter() - t_setup

    def step(i):
        rs.rswa_decode_attn(cache.desc, qs[i], out, ks[i], vs[i], 0.0, args.splits, ws, stream=stream)

    for i in range(fill + W):
        step(i)
    torch.cuda.synchronize()
    t_first = fill + W + 1                       # output index T of the first timed step
    progress(f"window filled and {W} warm-up steps run; timing {K} steps")
    ms = event_time_ms(lambda i: step(fill + W + i), K, stream)
    ms_per_step = ms / K
    out_last_timed = out.clone()                 # output of step t_first + K - 1
    # the same number of further steps, each between its own pair of events
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        step(fill + W + K + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) for a, b in ev])
    flags = rs.rswa_check_device_error(cache.desc)
    if flags:
        print(f"device error flags {flags}", file=sys.stderr)
        sys.exit(1)
    if int(cache.step[0].item()) != steps_total:
        print("decode step counter did not advance as expected", file=sys.stderr)
        sys.exit(1)
    alg_bytes = sum(decode_bytes(B, H, d, L, n, T) for T in range(t_first, t_first + K)) / K
    achieved = alg_bytes / (ms_per_step * 1e-3) / 1e9
    traffic = read_traffic(1)
    achievable = probe_read_GBps(torch, rs, stream)
    result = {
        "metric": METRIC,
        "value": B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "head_dim": d, "ref_len": L,
                   "window": n, "layers": 1, "timed_decode_steps": f"T={t_first}..{t_first + K - 1}",
                   "window_fill_steps": f"T=1..{fill} untimed, then warm-up T={fill + 1}..{fill + W}",
                   "splits": args.splits or "library"},
        "hbm_GBps": achieved,
        "hbm_frac_of_peak": achieved / HBM_PEAK_GBS,
        "per_step_ms": {"median": float(np.median(per_step)), "p10": float(np.percentile(per_step, 10)),
                        "p90": float(np.percentile(per_step, 90)), "mean": float(per_step.mean()),
                        "steps": f"T={t_first + K}..{t_first + 2 * K - 1}",
                        "note": "each step between its own pair of HIP events (the event records add "
                                "a little to every step; ms_per_step times the K steps back to back)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "rswa decode step (split-K attention, merged in the same launch when the plan has one chunk per (sequence, head)), one call",
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "traffic_steps": "steady state (all L_m + n slots visible), as the timed steps",
                     "achievable_read_GBps": achievable, "frac_of_achievable": achieved / achievable},
        "device": device_facts(torch, rs),
    }
    # cache image after the last step (bit for bit): the window slots hold outputs
    # T_last - n + 1 .. T_last at slot L_m + ((t - 1) mod n); ks, vs hold every step's k, v
    t_last = steps_total
    ts = torch.arange(t_last - n + 1, t_last + 1, device="cuda")
    per_seq = H * (L + n) * d
    assert torch.equal(cache.seq_base.cpu(), torch.arange(B, dtype=torch.int64) * per_seq)
    mism = 0
    for pool, src in ((cache.k, ks), (cache.v, vs)):
        win = pool[:B * per_seq].view(B, H, L + n, d)[:, :, L:, :][:, :, (ts - 1) % n, :]
        want = src[ts - 1].permute(1, 2, 0, 3)
        mism += int((win.view(torch.int16) != want.view(torch.int16)).any(-1).sum().item())
    result["parity"] = {"cache_window_slot_mismatches": mism, "cache_step": t_last,
                        "cache_rows_checked": 2 * B * H * n}
    del qs, ks, vs

    progress("contract line measured")
    if not args.no_secondary:
        # full-attention contrast: the same kernels over a cache of exactly L_m + T slots (window T,
        # every output kept), attend-only at output T
        q1 = torch.randn((B, H, d), device="cuda").to(torch.bfloat16)
        contrast = {}
        for T in (256, 2048, 4096, 6144):
            con = rs.KVCache.allocate([L] * B, H, d, T, dtype=rs.RSWA_BF16)
            con.k.normal_(0.0, w.sigma_kv)
            con.v.normal_(0.0, w.sigma_kv)
            con.step.fill_(T)
            cws = con.workspace()
            ms_c = event_time_ms(lambda i: rs.rswa_decode_attn(con.desc, q1, out, None, None, 0.0, 0, cws,
                                                             stream=stream), 20, stream) / 20
            contrast[str(T)] = {"ms_per_step": ms_c, "cache_slots": L + T,
                                "GBps": decode_bytes(B, H, d, L, T, T) / (ms_c * 1e-3) / 1e9}
            del con, cws
        # the R-SWA cache at the same attend-only call, for a like-for-like comparison
        ms_r = event_time_ms(lambda i: rs.rswa_decode_attn(cache.desc, q1, out, None, None, 0.0, 0, ws,
                                                         stream=stream), 20, stream) / 20
        result["contrast_full_attention"] = {
            "what": "attend-only decode call; full attention keeps L_m + T slots (a cache of exactly that "
                    "size, window = T), R-SWA keeps L_m + 128",
            "full_attention_per_T": contrast,
            "rswa_attend_only_ms": ms_r,
            "rswa_fused_step_ms": ms_per_step}
        progress("full-attention contrast measured")
        # ragged batch: 64 sequences, each with its own pages and decode position, one fused step
        rw = wl.RAGGED_64
        rdraw = wl.ragged_lengths(rw)
        rrefs = [int(x) for x in rdraw.ref_len]
        rtnow = [int(x) for x in rdraw.t_now]
        rc = rs.KVCache.allocate(rrefs, rw.heads, rw.head_dim, rw.window, dtype=rs.RSWA_BF16)
        rc.k.normal_()
        rc.v.normal_()
        saved = torch.tensor([t - 1 for t in rtnow], dtype=torch.int32, device="cuda")
        rq, rk, rv = (torch.randn((rw.batch, rw.heads, rw.head_dim), device="cuda").to(torch.bfloat16)
                      for _ in range(3))
        rout = torch.empty_like(rq)
        rws = rc.workspace()
        rc.step.copy_(saved)   # every sequence just before its output t_now
        r_steps = 50
        ragged_step = lambda i: rs.rswa_decode_attn(rc.desc, rq, rout, rk, rv, 0.0, 0, rws, stream=stream)
        for _ in range(3):
            ragged_step(0)
        ms_rg = event_time_ms(ragged_step, r_steps, stream) / r_steps
        if rs.rswa_check_device_error(rc.desc):
            print("ragged step reported device errors", file=sys.stderr)
            sys.exit(1)
        # the timed steps append outputs t_now + 3 .. t_now + 52 of every sequence
        rbytes = sum(rw.heads * (Lb + min(rw.window, t + 3 + i)) * rw.head_dim * 2 * 2
                     for i in range(r_steps) for Lb, t in zip(rrefs, rtnow)) / r_steps \
            + 4 * rw.batch * rw.heads * rw.head_dim * 2
        result["ragged_64"] = {
            "workload": rw.name, "batch": rw.batch, "ms_per_step": ms_rg, "tokens_per_s": rw.batch / (ms_rg * 1e-3),
            "algorithmic_bytes": rbytes, "GBps": rbytes / (ms_rg * 1e-3) / 1e9,
            "frac_of_peak": rbytes / (ms_rg * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "note": f"{r_steps} consecutive fused steps after 3 warm-up steps, each sequence from its own "
                    "decode position (pages ~ U{1..50}, T ~ U{1..8192}); no state restored in between"}
        del rc, rq, rk, rv, rout, rws

        progress("ragged batch measured")
        # packed 32K masked forward (matrix cores); each figure is the median of three
        # timed runs, taken before the GEMM and matrix-core probes below so that
        # their heat does not lower the clock the packed kernels are timed at
        med3 = lambda f, iters: sorted(event_time_ms(f, iters, stream) / iters for _ in range(3))[1]
        mw = wl.PACKED_32K
        Q, Kp, Vp = wl.packed_qkv(mw)
        to_d = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        Qd, Kd, Vd = to_d(Q), to_d(Kp), to_d(Vp)
        Od = torch.empty_like(Qd)
        masked = {}
        for mode, name in ((rs.RSWA_PREFIX_CAUSAL, "prefix_causal"), (rs.RSWA_PREFIX_FULL, "prefix_full")):
            run = lambda i: rs.rswa_masked_attn(Qd, Kd, Vd, Od, mw.seq_len, mw.ref_len, mw.window, mw.heads,
                                                mw.head_dim, rs.RSWA_BF16, mode, 0.0, stream=stream)
            for _ in range(5):
                run(0)
            ms_m = med3(run, 20)
            fl = masked_flops(mw.seq_len, mw.ref_len, mw.window, mw.heads, mw.head_dim,
                              mode == rs.RSWA_PREFIX_FULL)
            tile = masked_tile_flops(mw.seq_len, mw.ref_len, mw.window, mw.heads, mode == rs.RSWA_PREFIX_FULL)
            masked[name] = {"ms": ms_m, "algorithmic_flop": fl, "TFLOPs": fl / (ms_m * 1e-3) / 1e12,
                            "frac_of_bf16_peak": fl / (ms_m * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                            "tile_flop": tile, "tile_over_algorithmic": tile / fl}
        # packed 32K backward (dQ, dK, dV) of the causal-prefix forward
        Gd = to_d(wl.packed_dout(mw))
        lse = torch.empty((mw.heads, mw.seq_len), dtype=torch.float32, device="cuda")
        rs.rswa_masked_attn(Qd, Kd, Vd, Od, mw.seq_len, mw.ref_len, mw.window, mw.heads, mw.head_dim,
                            rs.RSWA_BF16, rs.RSWA_PREFIX_CAUSAL, 0.0, stream=stream, lse=lse)
        ws_b = torch.empty(rs.rswa_masked_bwd_workspace_size(mw.seq_len, mw.ref_len, mw.heads),
                           dtype=torch.uint8, device="cuda")
        dq, dk, dv = torch.empty_like(Qd), torch.empty_like(Qd), torch.empty_like(Qd)
        run_b = lambda i: rs.rswa_masked_attn_bwd(Qd, Kd, Vd, Od, Gd, lse, dq, dk, dv, mw.seq_len, mw.ref_len,
                                                  mw.window, mw.heads, mw.head_dim, rs.RSWA_BF16,
                                                  rs.RSWA_PREFIX_CAUSAL, 0.0, ws_b, stream=stream)
        for _ in range(3):
            run_b(0)
        ms_b = med3(run_b, 5)
        fl_b = 2.5 * masked_flops(mw.seq_len, mw.ref_len, mw.window, mw.heads, mw.head_dim, False)
        masked["backward_prefix_causal"] = {
            "ms": ms_b, "algorithmic_flop": fl_b, "TFLOPs": fl_b / (ms_b * 1e-3) / 1e12,
            "frac_of_bf16_peak": fl_b / (ms_b * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "flop_convention": "2.5x the forward: five products of 2 d flop per visible pair (S, dP, dV, dK, "
                               "dQ); the kernels execute seven (S and dP are formed in both the dQ and "
                               "the dK/dV pass)",
            "calls": "lse-producing forward excluded; dQ (with the per-row D and lse terms), dK/dV and reduction kernels included"}
        del ws_b
        result["masked_32k"] = {"workload": mw.name, "seq_len": mw.seq_len, "ref_len": mw.ref_len,
                                "window": mw.window, "heads": mw.heads, **masked}
        if not args.no_cpu_baseline:
            result["cpu_baseline_masked"] = cpu_masked_rows(mw, Q, Kp, Vp)

        progress("packed 32K forward and backward measured")
        # several documents per 32K pack (samples independent), forward on matrix cores
        cu, refs = wl.varlen_pack_layout(mw.seq_len, mw.base_seed)
        lens = np.diff(cu)
        cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
        refs_d = torch.tensor(refs, dtype=torch.int32, device="cuda")
        run_v = lambda i: rs.rswa_masked_attn_varlen(Qd, Kd, Vd, Od, cu_d, refs_d, len(refs), mw.seq_len,
                                                     int(lens.max()), mw.window, mw.heads, mw.head_dim,
                                                     rs.RSWA_BF16, rs.RSWA_PREFIX_CAUSAL, 0.0, stream=stream)
        for _ in range(5):
            run_v(0)
        ms_v = med3(run_v, 20)
        fl_v = sum(masked_flops(int(N_s), int(L_s), mw.window, mw.heads, mw.head_dim, False)
                   for N_s, L_s in zip(lens, refs))
        # backward of the same pack (dO as for the single-sequence backward)
        rs.rswa_masked_attn_varlen(Qd, Kd, Vd, Od, cu_d, refs_d, len(refs), mw.seq_len, int(lens.max()),
                                   mw.window, mw.heads, mw.head_dim, rs.RSWA_BF16, rs.RSWA_PREFIX_CAUSAL, 0.0,
                                   stream=stream, lse=lse)
        ws_v = torch.empty(rs.rswa_masked_bwd_varlen_workspace_size(mw.seq_len, mw.heads), dtype=torch.uint8,
                           device="cuda")
        run_vb = lambda i: rs.rswa_masked_attn_bwd_varlen(Qd, Kd, Vd, Od, Gd, lse, dq, dk, dv, cu_d, refs_d,
                                                          len(refs), mw.seq_len, int(lens.max()), mw.window,
                                                          mw.heads, mw.head_dim, rs.RSWA_BF16,
                                                          rs.RSWA_PREFIX_CAUSAL, 0.0, ws_v, stream=stream)
        for _ in range(3):
            run_vb(0)
        ms_vb = med3(run_vb, 5)
        result["varlen_32k"] = {
            "workload": "packed-32k-varlen-bf16", "samples": len(refs),
            "sample_rows": [int(x) for x in lens], "ref_lens": [int(x) for x in refs],
            "layout": "pages ~ U{2..16} (L = 256 pages + 32), outputs ~ U{256..2048}, filled front to back",
            "ms": ms_v, "algorithmic_flop": fl_v, "TFLOPs": fl_v / (ms_v * 1e-3) / 1e12,
            "frac_of_bf16_peak": fl_v / (ms_v * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "backward": {"ms": ms_vb, "algorithmic_flop": 2.5 * fl_v,
                         "TFLOPs": 2.5 * fl_v / (ms_vb * 1e-3) / 1e12,
                         "frac_of_bf16_peak": 2.5 * fl_v / (ms_vb * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                         "calls": "rswa_masked_attn_bwd_varlen (dQ, dK/dV); flop convention as "
                                  "for the single-sequence backward"}}
        del Qd, Kd, Vd, Od, cu_d, refs_d, Gd, dq, dk, dv, lse, ws_v

        progress("10-document pack measured")
        # prefill -> decode hand-off at the 40-page decode shape: B sequences of L_m reference
        # rows plus T0 = n outputs (the window full at hand-off), one call for the whole batch
        T0 = n
        rows_b = L + T0
        total = B * rows_b
        gen = torch.Generator(device="cuda")
        gen.manual_seed(w.base_seed)
        pq, pk, pv = (torch.randn((total, H, d), device="cuda", generator=gen).to(torch.bfloat16)
                      for _ in range(3))
        pout = torch.empty_like(pq)
        pcu = torch.arange(0, total + 1, rows_b, dtype=torch.int32, device="cuda")
        pcache = rs.KVCache.allocate([L] * B, H, d, n, dtype=rs.RSWA_BF16)
        run_p = lambda i: rs.rswa_prefill(pcache.desc, pq, pk, pv, pout, pcu, total, rows_b,
                                          rs.RSWA_PREFIX_CAUSAL, 0.0, stream=stream)
        prefs = torch.full((B,), L, dtype=torch.int32, device="cuda")
        run_pf = lambda i: rs.rswa_masked_attn_varlen(pq, pk, pv, pout, pcu, prefs, B, total, rows_b, n, H, d,
                                                      rs.RSWA_BF16, rs.RSWA_PREFIX_CAUSAL, 0.0, stream=stream)
        for _ in range(2):
            run_p(0)
        ms_p = event_time_ms(run_p, 5, stream) / 5
        ms_pf = event_time_ms(run_pf, 5, stream) / 5
        if rs.rswa_check_device_error(pcache.desc):
            print("prefill reported device errors", file=sys.stderr)
            sys.exit(1)
        fl_p = B * masked_flops(rows_b, L, n, H, d, False)
        cache_bytes = 2 * B * H * (L + min(n, T0)) * d * 2  # K and V rows written into the cache
        result["prefill_40page"] = {
            "workload": "40-page-prefill-bf16", "batch": B, "ref_len": L, "outputs_T0": T0,
            "rows": total, "ms": ms_p, "forward_only_ms": ms_pf,
            "forward_algorithmic_flop": fl_p, "forward_TFLOPs": fl_p / (ms_pf * 1e-3) / 1e12,
            "TFLOPs": fl_p / (ms_p * 1e-3) / 1e12, "handoff_cache_bytes": cache_bytes,
            "handoff_overhead_ms": ms_p - ms_pf,
            "note": "one launch: the packed forward with the cache write fused into each workgroup's tail; "
                    "forward_only_ms is the same pack through rswa_masked_attn_varlen"}
        del pq, pk, pv, pout, pcache
        # chip reference rates, measured after every packed kernel was timed
        gemm = gemm_tflops(torch, stream)
        mfma_rate = mfma_probe_tflops(torch, rs, stream)
        result["cu_probe"] = cu_probe(torch, rs, stream)
        mk = result["masked_32k"]
        mk.update({"measured_bf16_gemm_TFLOPs": gemm, "gemm": "8192^3 bf16 torch.matmul",
                   "measured_mfma_rate_TFLOPs": mfma_rate,
                   "mfma_rate": "rswa_probe_mfma: 32x32x16 bf16 products back to back, two waves "
                                "per SIMD, nothing else in the loop; both probes run after the packed "
                                "kernels were timed"})
        for name in ("prefix_causal", "prefix_full", "backward_prefix_causal"):
            if name != "backward_prefix_causal":
                mk[name]["frac_of_measured_gemm"] = mk[name]["TFLOPs"] / gemm
            mk[name]["frac_of_measured_mfma_rate"] = mk[name]["TFLOPs"] / mfma_rate

        progress("prefill measured")
        # a decode step through `layers` attention layers (own cache each) as one HIP graph, at the
        # output lengths of the pages' TPS table, R-SWA against full attention (attention share only)
        layers = args.layers
        r_caches = [rs.KVCache.allocate([L] * B, H, d, n, dtype=rs.RSWA_BF16) for _ in range(layers)]
        for c in r_caches:
            c.k.normal_(0.0, w.sigma_kv)
            c.v.normal_(0.0, w.sigma_kv)
        gq = [torch.randn((B, H, d), device="cuda").to(torch.bfloat16) for _ in range(layers)]
        gk = [torch.randn((B, H, d), device="cuda").to(torch.bfloat16) for _ in range(layers)]
        gv = [torch.randn((B, H, d), device="cuda").to(torch.bfloat16) for _ in range(layers)]
        gout = [torch.empty_like(x) for x in gq]
        ws_r = r_caches[0].workspace()
        _, g_r = rs.rswa_decode_graph_create([c.desc for c in r_caches], gq, gout, workspace=ws_r)
        _, g_rf = rs.rswa_decode_graph_create([c.desc for c in r_caches], gq, gout, gk, gv, workspace=ws_r)
        per_T = {}
        try:
            for T in (256, 2048, 4096, 6144):
                # full attention: per layer a cache of exactly L_m + T slots
                f_caches = [rs.KVCache.allocate([L] * B, H, d, T, dtype=rs.RSWA_BF16) for _ in range(layers)]
                for c in f_caches:
                    c.k.normal_(0.0, w.sigma_kv)
                    c.v.normal_(0.0, w.sigma_kv)
                    c.step.fill_(T)
                for c in r_caches:
                    c.step.fill_(T)
                ws_f = f_caches[0].workspace()
                _, g_f = rs.rswa_decode_graph_create([c.desc for c in f_caches], gq, gout, workspace=ws_f)
                try:
                    rs.rswa_decode_graph_launch(g_r, stream=stream)
                    rs.rswa_decode_graph_launch(g_f, stream=stream)
                    ms_gr = event_time_ms(lambda i: rs.rswa_decode_graph_launch(g_r, stream=stream), 10,
                                          stream) / 10
                    ms_gf = event_time_ms(lambda i: rs.rswa_decode_graph_launch(g_f, stream=stream), 10,
                                          stream) / 10
                finally:
                    rs.rswa_decode_graph_destroy(g_f)
                per_T[str(T)] = {"rswa_ms_per_step": ms_gr, "full_ms_per_step": ms_gf,
                                 "rswa_tokens_per_s": B / (ms_gr * 1e-3), "full_tokens_per_s": B / (ms_gf * 1e-3),
                                 "rswa_over_full": ms_gf / ms_gr}
                del f_caches, ws_f
            for c in r_caches:
                c.step.fill_(w.steps)
            rs.rswa_decode_graph_launch(g_rf, stream=stream)
            ms_rf = event_time_ms(lambda i: rs.rswa_decode_graph_launch(g_rf, stream=stream), 10, stream) / 10
            for c in r_caches:
                if rs.rswa_check_device_error(c.desc):
                    print("multi-layer decode reported device errors", file=sys.stderr)
                    sys.exit(1)
        finally:
            for g in (g_r, g_rf):
                rs.rswa_decode_graph_destroy(g)
        result["multi_layer_graph"] = {
            "what": "one decode step through `layers` attention layers replayed as one HIP graph "
                    "(rswa_decode_graph_*); attend-only at fixed T for both cache kinds; the pages' TPS "
                    "table covers the whole model, this is its attention share",
            "layers": layers, "batch": B, "ref_len": L, "window": n, "per_T": per_T,
            "rswa_fused_step_ms": ms_rf, "rswa_fused_tokens_per_s": B / (ms_rf * 1e-3)}
        del r_caches, ws_r, gq, gk, gv, gout

        progress("multi-layer graph measured")
        # one-page decode (B = 1): 3.4 MB per step, a working set the caches hold, so the step is
        # bound by launch and kernel latency; fused append + attend steps eagerly and replayed as a
        # one-layer HIP graph, past the window fill (T > n)
        ow = wl.ONE_PAGE
        oc = rs.KVCache.allocate([ow.ref_len], ow.heads, ow.head_dim, ow.window, dtype=rs.RSWA_BF16)
        oc.k.normal_()
        oc.v.normal_()
        oq, ok_, ov = (torch.randn((1, ow.heads, ow.head_dim), device="cuda").to(torch.bfloat16)
                       for _ in range(3))
        oout = torch.empty_like(oq)
        ows = oc.workspace()
        o_step = lambda i: rs.rswa_decode_attn(oc.desc, oq, oout, ok_, ov, 0.0, 0, ows, stream=stream)
        for _ in range(2 * ow.window):
            o_step(0)
        o_steps = 1024
        ms_oe = event_time_ms(o_step, o_steps, stream) / o_steps
        _, g_o = rs.rswa_decode_graph_create([oc.desc], [oq], [oout], [ok_], [ov], workspace=ows)
        try:
            for _ in range(16):
                rs.rswa_decode_graph_launch(g_o, stream=stream)
            ms_og = event_time_ms(lambda i: rs.rswa_decode_graph_launch(g_o, stream=stream), o_steps,
                                  stream) / o_steps
        finally:
            rs.rswa_decode_graph_destroy(g_o)
        # the same step through `layers` layers (own cache each): eager calls against one graph launch
        lcs = [rs.KVCache.allocate([ow.ref_len], ow.heads, ow.head_dim, ow.window, dtype=rs.RSWA_BF16)
               for _ in range(layers)]
        for c in lcs:
            c.k.normal_()
            c.v.normal_()
        lq = [torch.randn_like(oq) for _ in range(layers)]
        lk = [torch.randn_like(oq) for _ in range(layers)]
        lv = [torch.randn_like(oq) for _ in range(layers)]
        lo = [torch.empty_like(oq) for _ in range(layers)]

        def l_step(i):
            for li in range(layers):
                rs.rswa_decode_attn(lcs[li].desc, lq[li], lo[li], lk[li], lv[li], 0.0, 0, ows, stream=stream)

        for _ in range(2 * ow.window):
            l_step(0)
        l_steps = 256
        ms_le = event_time_ms(l_step, l_steps, stream) / l_steps
        _, g_l = rs.rswa_decode_graph_create([c.desc for c in lcs], lq, lo, lk, lv, workspace=ows)
        try:
            for _ in range(16):
                rs.rswa_decode_graph_launch(g_l, stream=stream)
            ms_lg = event_time_ms(lambda i: rs.rswa_decode_graph_launch(g_l, stream=stream), l_steps,
                                  stream) / l_steps
        finally:
            rs.rswa_decode_graph_destroy(g_l)
        for c in [oc] + lcs:
            if rs.rswa_check_device_error(c.desc):
                print("one-page decode reported device errors", file=sys.stderr)
                sys.exit(1)
        o_bytes = ow.heads * (ow.ref_len + ow.window) * ow.head_dim * 2 * 2 + 4 * ow.heads * ow.head_dim * 2
        result["one_page"] = {
            "workload": ow.name, "batch": 1, "heads": ow.heads, "ref_len": ow.ref_len, "window": ow.window,
            "bound": "latency (working set far below the 4 MB L2 per XCD and the MALL)",
            "eager_us_per_step": ms_oe * 1e3, "graph_us_per_step": ms_og * 1e3,
            "eager_tokens_per_s": 1 / (ms_oe * 1e-3), "graph_tokens_per_s": 1 / (ms_og * 1e-3),
            "algorithmic_bytes_per_step": o_bytes, "steps_timed": o_steps,
            "layers": layers, "layers_eager_us_per_step": ms_le * 1e3, "layers_graph_us_per_step": ms_lg * 1e3,
            "note": f"fused append + attend, split + merge kernels; eager steps T = {2 * ow.window + 1}.."
                    f"{2 * ow.window + o_steps}, graph steps T = {2 * ow.window + o_steps + 17}.."
                    f"{2 * ow.window + 2 * o_steps + 16}"}
        del oc, oq, ok_, ov, oout, ows, lcs, lq, lk, lv, lo

    if args.curve:
        progress("per-step curve")
        result["per_step_curve"] = per_step_curve(torch, rs, w, stream, w.steps)
    if not args.no_cpu_baseline:
        progress("CPU oracle baseline")
        ref, result["cpu_baseline"] = cpu_baseline(w, kref, vref, t_first + K - 1)
        got = out_last_timed.float().cpu().numpy().astype(np.float64)
        dlt = got - ref
        pair_rel = (np.linalg.norm(dlt, axis=-1) / np.linalg.norm(ref, axis=-1)).max()
        result["parity"]["oracle_step"] = t_first + K - 1
        result["parity"]["max_abs"] = float(np.abs(dlt).max())
        result["parity"]["rel_l2"] = float(np.linalg.norm(dlt) / np.linalg.norm(ref))
        result["parity"]["worst_pair_rel_l2"] = float(pair_rel)
        result["parity"]["bound"] = "max_abs <= 2e-2 and relative L2 <= 1e-2, pooled and per (sequence, head)"
    result["setup_s"] = setup_s
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
