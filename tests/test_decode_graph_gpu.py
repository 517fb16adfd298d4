"""Multi-layer decode step under HIP-graph capture (rswa_decode_graph_*): every
replay must give the bits the eager per-layer rswa_decode_attn calls give, with
the program's own eager work and synchronisations between replays, across the
window's wrap-around; attend-only graphs leave the step counters alone. Layer 0
of the eager path is also checked against the oracle's queue model."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.rswa as orc
import reference_sliding_window_amd as rs
import workloads as wl
from gpu_util import bits, check_close, to_dev, to_f64

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def make_layers(refs, H, d, n, L, dtype, seed):
    """L caches with the same reference lengths, each initialised from its own draw."""
    caches, kref = [], []
    tdt = "bf16" if dtype == rs.RSWA_BF16 else "fp32"
    for l in range(L):
        c = rs.KVCache.allocate(refs, H, d, n, dtype=dtype)
        ks = [wl.draw(tdt, 1.0, (H, Lb, d), seed, 10 + l, b) for b, Lb in enumerate(refs)]
        vs = [wl.draw(tdt, 1.0, (H, Lb, d), seed, 50 + l, b) for b, Lb in enumerate(refs)]
        base = np.concatenate([[0], np.cumsum([H * Lb * d for Lb in refs])[:-1]]).astype(np.int64)
        kd = to_dev(np.concatenate([x.reshape(-1) for x in ks]), tdt)
        vd = to_dev(np.concatenate([x.reshape(-1) for x in vs]), tdt)
        rs.rswa_cache_init(c.desc, kd, vd, torch.tensor(base, device="cuda"))
        caches.append(c)
        kref.append((ks, vs))
    torch.cuda.synchronize()
    return caches, kref


FULL_BATCH = [int(x) for x in np.random.default_rng(8099).integers(0, 120, 32)]


@pytest.mark.parametrize("dtype,d,refs,H", [
    (rs.RSWA_BF16, 128, [40, 0, 77], 2),
    (rs.RSWA_FP32, 64, [40, 0, 77], 2),
    # B * H = 512 short sequences: the library decodes in one launch per layer (one chunk per
    # sequence and head, steps published through the arrival counters)
    (rs.RSWA_BF16, 128, FULL_BATCH, 16),
], ids=["bf16-d128", "fp32-d64", "bf16-one-launch"])
def test_graph_replays_equal_eager_steps(dtype, d, refs, H):
    n, L, steps = 8, 3, 20
    B = len(refs)
    tdt = "bf16" if dtype == rs.RSWA_BF16 else "fp32"
    tt = torch.bfloat16 if dtype == rs.RSWA_BF16 else torch.float32
    banner(f"decode graph vs eager dtype={tdt} d={d} layers={L} steps={steps}")
    eager, kref = make_layers(refs, H, d, n, L, dtype, seed=8100)
    graphed, _ = make_layers(refs, H, d, n, L, dtype, seed=8100)
    ws_e = eager[0].workspace()
    ws_g = graphed[0].workspace()
    sq = [torch.zeros((B, H, d), dtype=tt, device="cuda") for _ in range(L)]
    sk = [torch.zeros_like(x) for x in sq]
    sv = [torch.zeros_like(x) for x in sq]
    sout = [torch.zeros_like(x) for x in sq]
    _, g = rs.rswa_decode_graph_create([c.desc for c in graphed], sq, sout, sk, sv, workspace=ws_g)
    out_e = torch.empty((B, H, d), dtype=tt, device="cuda")
    other = torch.randn(1 << 20, device="cuda")
    hist = []
    try:
        for i in range(steps):
            x = [[to_dev(wl.draw(tdt, 1.0, (B, H, d), 8101, t, i, l), tdt) for t in range(3)] for l in range(L)]
            outs_e = []
            for l in range(L):
                rs.rswa_decode_attn(eager[l].desc, x[l][0], out_e, x[l][1], x[l][2], 0.0, 0, ws_e)
                outs_e.append(bits(out_e))
            for l in range(L):
                sq[l].copy_(x[l][0]); sk[l].copy_(x[l][1]); sv[l].copy_(x[l][2])
            rs.rswa_decode_graph_launch(g)
            other.mul_(1.0001)                     # the program's own eager work between replays
            torch.cuda.synchronize()
            for l in range(L):
                assert np.array_equal(bits(sout[l]), outs_e[l]), f"step {i + 1} layer {l}"
            hist.append([to_f64(sout[0]).copy()])
        for l in range(L):
            assert graphed[l].step.cpu().tolist() == [steps] * B
            assert graphed[l].arrive.cpu().tolist() == [0] * B
            assert rs.rswa_check_device_error(graphed[l].desc) == 0
        # layer 0 against the oracle's queue model, every step, every (sequence, head)
        f = lambda a: wl.to_f64(a, tdt)
        qs = np.stack([f(wl.draw(tdt, 1.0, (B, H, d), 8101, 0, i, 0)) for i in range(steps)])
        ks = np.stack([f(wl.draw(tdt, 1.0, (B, H, d), 8101, 1, i, 0)) for i in range(steps)])
        vs = np.stack([f(wl.draw(tdt, 1.0, (B, H, d), 8101, 2, i, 0)) for i in range(steps)])
        got = np.stack([h[0] for h in hist])
        for b, Lb in enumerate(refs):
            for h in range(H):
                ref = orc.simulate_decode(qs[:, b, h], f(kref[0][0][b][h]), f(kref[0][1][b][h]), ks[:, b, h],
                                          vs[:, b, h], Lb, n, 1.0 / np.sqrt(d))
                check_close(got[:, b, h], ref, tdt, f"graph layer 0 seq {b} head {h}")
    finally:
        rs.rswa_decode_graph_destroy(g)


def test_attend_only_graph_keeps_steps_and_repeats():
    refs, H, d, n, L = [64, 33], 2, 128, 16, 2
    B = len(refs)
    banner("attend-only decode graph")
    caches, _ = make_layers(refs, H, d, n, L, rs.RSWA_BF16, seed=8200)
    for c in caches:
        c.step.fill_(5)
    ws = caches[0].workspace()
    sq = [torch.randn((B, H, d), device="cuda").to(torch.bfloat16) for _ in range(L)]
    sout = [torch.empty_like(x) for x in sq]
    _, g = rs.rswa_decode_graph_create([c.desc for c in caches], sq, sout, workspace=ws)
    try:
        first = None
        for rep in range(4):
            rs.rswa_decode_graph_launch(g)
            torch.cuda.synchronize()
            now = [bits(x) for x in sout]
            if first is None:
                first = now
            for a, b in zip(first, now):
                assert np.array_equal(a, b), f"replay {rep}"
        eager = torch.empty_like(sq[0])
        for l in range(L):
            rs.rswa_decode_attn(caches[l].desc, sq[l], eager, None, None, 0.0, 0, ws)
            torch.cuda.synchronize()
            assert np.array_equal(bits(eager), first[l])
            assert caches[l].step.cpu().tolist() == [5, 5]
    finally:
        rs.rswa_decode_graph_destroy(g)


def test_graph_replays_equal_eager_steps_flat_work_list():
    """A ragged batch large enough for the flat work list (flat kernel + merge per layer):
    every replay gives the eager calls' bits, step counters and cache images, through the
    window's wrap. (The flat path's outputs are checked against the oracle elsewhere.)"""
    refs, H, d, n, L, steps = [33000, 0, 100, 5000], 32, 128, 16, 2, 20
    B = len(refs)
    banner(f"decode graph vs eager, flat work list, refs {refs} H={H}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8300)
    pools = []
    for _ in range(2):          # eager, graphed: identical initial caches
        cs = []
        for l in range(L):
            c = rs.KVCache.allocate(refs, H, d, n, dtype=rs.RSWA_BF16)
            cs.append(c)
        pools.append(cs)
    for l in range(L):
        k0 = torch.randn(pools[0][l].k.shape, device="cuda", generator=gen).to(torch.bfloat16)
        v0 = torch.randn(pools[0][l].v.shape, device="cuda", generator=gen).to(torch.bfloat16)
        for cs in pools:
            cs[l].k.copy_(k0)
            cs[l].v.copy_(v0)
            cs[l].step.zero_()
    eager, graphed = pools
    assert rs.rswa_decode_workspace_size(eager[0].desc, 0) == rs.rswa_workspace_size(B, H, d, max(refs) + n)
    ws_e, ws_g = eager[0].workspace(), graphed[0].workspace()
    sq = [torch.zeros((B, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    sk = [torch.zeros_like(x) for x in sq]
    sv = [torch.zeros_like(x) for x in sq]
    sout = [torch.zeros_like(x) for x in sq]
    _, g = rs.rswa_decode_graph_create([c.desc for c in graphed], sq, sout, sk, sv, workspace=ws_g)
    out_e = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    try:
        for i in range(steps):
            x = [[torch.randn((B, H, d), device="cuda", generator=gen).to(torch.bfloat16) for _ in range(3)]
                 for _ in range(L)]
            outs_e = []
            for l in range(L):
                rs.rswa_decode_attn(eager[l].desc, x[l][0], out_e, x[l][1], x[l][2], 0.0, 0, ws_e)
                outs_e.append(bits(out_e))
            for l in range(L):
                sq[l].copy_(x[l][0]); sk[l].copy_(x[l][1]); sv[l].copy_(x[l][2])
            rs.rswa_decode_graph_launch(g)
            torch.cuda.synchronize()
            for l in range(L):
                assert np.array_equal(bits(sout[l]), outs_e[l]), f"step {i + 1} layer {l}"
        for l in range(L):
            assert graphed[l].step.cpu().tolist() == eager[l].step.cpu().tolist() == [steps] * B
            assert np.array_equal(bits(graphed[l].k), bits(eager[l].k))
            assert np.array_equal(bits(graphed[l].v), bits(eager[l].v))
            assert rs.rswa_check_device_error(graphed[l].desc) == 0
    finally:
        rs.rswa_decode_graph_destroy(g)
