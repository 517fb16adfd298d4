"""The packed calls enqueue all their work on the stream they are given.

A caller that overlaps work or captures a training step into a HIP graph needs
every kernel of a call on the caller's stream: capture fails on a launch to any
other stream. Here the packed forward (with its log-sum-exp) and the backward,
single-sequence (backward split into three runs, so the reduction kernel is
captured too) and over a pack, are captured into one graph with torch.cuda.graph;
every replay, with fresh inputs copied into the captured buffers and the
program's own eager work between replays, must give the bits of the same calls
made eagerly. The same calls, and fused decode steps, on a side stream (default
priority) must give the bits of the default stream's run."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import reference_sliding_window_amd as rs
import workloads as wl
from gpu_util import bits, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

D, H, N_WIN = 128, 4, 64
N, L_M = 1000, 300
CU, REFS = [0, 180, 180, 700], [60, 0, 500]          # a pack of three samples (one empty)
TOTAL = 760


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def draw(seed, rows):
    return [to_dev(wl.draw("bf16", 1.0, (rows, H, D), seed, t), "bf16") for t in range(4)]


class TrainingStep:
    """Device buffers for one packed forward + backward, single-sequence and pack."""

    def __init__(self):
        mk = lambda rows: torch.zeros((rows, H, D), dtype=torch.bfloat16, device="cuda")
        self.x = [mk(N) for _ in range(4)]                 # Q, K, V, dO
        self.y = [mk(N) for _ in range(4)]                 # out, dQ, dK, dV
        self.lse = torch.zeros((H, N), dtype=torch.float32, device="cuda")
        self.ws = torch.empty(rs.rswa_masked_bwd_workspace_size(N, L_M, H, 3), dtype=torch.uint8, device="cuda")
        self.px = [mk(TOTAL) for _ in range(4)]
        self.py = [mk(TOTAL) for _ in range(4)]
        self.plse = torch.zeros((H, TOTAL), dtype=torch.float32, device="cuda")
        self.pws = torch.empty(rs.rswa_masked_bwd_varlen_workspace_size(TOTAL, H), dtype=torch.uint8,
                               device="cuda")
        self.cu = torch.tensor(CU, dtype=torch.int32, device="cuda")
        self.refs = torch.tensor(REFS, dtype=torch.int32, device="cuda")

    def load(self, seed):
        for dst, src in zip(self.x, draw(seed, N)):
            dst.copy_(src)
        for dst, src in zip(self.px, draw(seed + 1, TOTAL)):
            dst.copy_(src)

    def run(self, stream=None):
        (q, k, v, g), (o, dq, dk, dv) = self.x, self.y
        rs.rswa_masked_attn(q, k, v, o, N, L_M, N_WIN, H, D, rs.RSWA_BF16, rs.RSWA_PREFIX_CAUSAL, 0.0,
                            lse=self.lse, stream=stream)
        rs.rswa_masked_attn_bwd(q, k, v, o, g, self.lse, dq, dk, dv, N, L_M, N_WIN, H, D, rs.RSWA_BF16,
                                rs.RSWA_PREFIX_CAUSAL, 0.0, self.ws, num_parts=3, stream=stream)
        (q, k, v, g), (o, dq, dk, dv) = self.px, self.py
        mx = max(b - a for a, b in zip(CU, CU[1:]))
        rs.rswa_masked_attn_varlen(q, k, v, o, self.cu, self.refs, len(REFS), TOTAL, mx, N_WIN, H, D,
                                   rs.RSWA_BF16, rs.RSWA_PREFIX_FULL, 0.0, lse=self.plse, stream=stream)
        rs.rswa_masked_attn_bwd_varlen(q, k, v, o, g, self.plse, dq, dk, dv, self.cu, self.refs, len(REFS),
                                       TOTAL, mx, N_WIN, H, D, rs.RSWA_BF16, rs.RSWA_PREFIX_FULL, 0.0, self.pws,
                                       stream=stream)


def _outputs(step):
    return [bits(t) for t in (*step.y, step.lse, *step.py, step.plse)]


def test_packed_training_step_under_graph_capture():
    banner("packed forward + backward (single sequence and pack) captured into one HIP graph")
    eager, graphed = TrainingStep(), TrainingStep()
    # a first eager call of each entry point outside capture
    for s in (eager, graphed):
        s.load(8300)
        s.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run()
    other = torch.randn(1 << 20, device="cuda")
    for rep, seed in enumerate((8310, 8320, 8330)):
        for s in (eager, graphed):
            s.load(seed)
        eager.run()
        g.replay()
        other.mul_(1.0001)                   # the program's own eager work between replays
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outputs(eager), _outputs(graphed))):
            assert np.array_equal(a, b), f"replay {rep}: output {i} differs from the eager call"


def test_side_stream_gives_the_default_streams_bits():
    banner("packed calls and fused decode steps on a side stream")
    main, side = TrainingStep(), TrainingStep()
    for s in (main, side):
        s.load(8400)
    torch.cuda.synchronize()
    main.run()
    stream = torch.cuda.Stream()             # default priority
    with torch.cuda.stream(stream):
        side.run(stream=stream)
    stream.synchronize()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(_outputs(main), _outputs(side))):
        assert np.array_equal(a, b), f"output {i} differs on the side stream"

    w = wl.DecodeWorkload("side-stream", batch=3, heads=H, head_dim=D, ref_len=500, window=16, steps=40,
                          dtype="bf16", sigma_q=1.0, sigma_kv=1.0, base_seed=8401)
    kref, vref = wl.ref_kv_all(w)
    q, k, v = wl.steps_qkv(w, 1, w.steps)
    runs = []
    for on_side in (False, True):
        cache = rs.KVCache.allocate([w.ref_len] * w.batch, w.heads, w.head_dim, w.window)
        bases = torch.tensor([b * w.heads * w.ref_len * D for b in range(w.batch)], dtype=torch.int64,
                             device="cuda")
        rs.rswa_cache_init(cache.desc, to_dev(kref.reshape(-1), "bf16"), to_dev(vref.reshape(-1), "bf16"), bases)
        ws = cache.workspace(3)
        out = torch.empty((w.batch, w.heads, D), dtype=torch.bfloat16, device="cuda")
        dev = [[to_dev(x[T], "bf16") for T in range(w.steps)] for x in (q, k, v)]
        torch.cuda.synchronize()
        s = stream if on_side else torch.cuda.current_stream()
        outs = []
        with torch.cuda.stream(s):
            for T in range(w.steps):
                rs.rswa_decode_attn(cache.desc, dev[0][T], out, dev[1][T], dev[2][T], 0.0, 3, ws, stream=s)
                outs.append(out.clone())
        s.synchronize()
        torch.cuda.synchronize()
        runs.append(([bits(o) for o in outs], bits(cache.k), bits(cache.v), cache.step.cpu().tolist()))
        assert rs.rswa_check_device_error(cache.desc) == 0
    (o0, k0, v0, s0), (o1, k1, v1, s1) = runs
    assert s0 == s1 == [w.steps] * w.batch
    assert all(np.array_equal(a, b) for a, b in zip(o0, o1)), "decode outputs differ on the side stream"
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1), "cache images differ on the side stream"
