"""Seeded random shapes for the packed paths, through the C ABI, against the oracle.

The hand-picked cases elsewhere cover the edges we thought of; these draw
sequence lengths, reference lengths, windows (below, at and above the block
and tile sizes), head counts, prefix modes and pack layouts at random (fixed
seeds, so every run checks the same cases) and compare every row, key and
cache slot. Tolerances are the ones of the dedicated tests: outputs max|diff|
<= 2e-2 and relative L2 <= 1e-2; gradients relative to their own magnitude;
cache images bit for bit.

RSWA_RANDOM_CASES=k (default 1) draws k times as many cases from the same seeds
(the default cases first), for a wider sweep than the suite runs by default."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle.rswa as orc
import reference_sliding_window_amd as rs
import workloads as wl
from gpu_util import bits, check_close, check_grad, to_dev, to_f64

pytestmark = pytest.mark.gpu

CAUSAL, FULL = rs.RSWA_PREFIX_CAUSAL, rs.RSWA_PREFIX_FULL
D = 128
SCALE = 1.0 / np.sqrt(D)
WINDOWS = [1, 2, 7, 31, 32, 63, 64, 65, 127, 128, 129, 300, 1000]
WIDEN = max(1, int(os.environ.get("RSWA_RANDOM_CASES", "1")))


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def dev_i32(a):
    return torch.tensor(np.asarray(a, np.int32), dtype=torch.int32, device="cuda")


def check_lse(got, ref, what):
    err = np.abs(got - ref)
    assert (err <= 2.0 ** -8 + 2e-4 + 1e-5 * np.abs(ref)).all(), f"{what}: lse max|d|={err.max():.3e}"


def tensors(total, H, seed, with_dout=False):
    shape = (total, H, D)
    out = [wl.draw("bf16", 1.0, shape, seed, tid) for tid in (0, 1, 2)]
    if with_dout:
        out.append(wl.draw("bf16", 1.0, shape, seed, wl.TID_DOUT))
    return out


def single_cases(count, seed, max_n):
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        N = int(g.integers(1, max_n + 1))
        L_m = int(g.integers(0, N + 1)) if g.random() < 0.85 else int(g.choice([0, N]))
        cases.append((N, L_m, int(g.choice(WINDOWS)), int(g.choice([CAUSAL, FULL])), int(g.integers(1, 4))))
    return cases


@pytest.mark.parametrize("case", single_cases(20 * WIDEN, 2026, 600), ids=lambda c: "N%d-L%d-n%d-m%d-H%d" % c)
def test_forward_random_every_row(case):
    N, L_m, n, mode, H = case
    banner(f"random forward N={N} L_m={L_m} n={n} mode={mode} H={H}")
    Q, K, V = tensors(N, H, 9100 + N)
    out = torch.full((N, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, N), float("nan"), dtype=torch.float32, device="cuda")
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    rs.rswa_masked_attn(Qd, Kd, Vd, out, N, L_m, n, H, D, rs.RSWA_BF16, mode, 0.0, lse=lse)
    torch.cuda.synchronize()
    f = lambda a: wl.to_f64(a, "bf16")
    ref = orc.masked_attention_rows(f(Q), f(K), f(V), range(N), L_m, n, SCALE, mode)
    check_close(to_f64(out), ref, "bf16", f"forward N={N} L_m={L_m} n={n} mode={mode}")
    ref_lse = orc.masked_logsumexp_rows(f(Q), f(K), range(N), L_m, n, SCALE, mode)
    check_lse(lse.cpu().numpy().astype(np.float64).T, ref_lse, "forward lse")


@pytest.mark.parametrize("case", single_cases(10 * WIDEN, 2027, 320), ids=lambda c: "N%d-L%d-n%d-m%d-H%d" % c)
def test_backward_random_every_row_and_key(case):
    N, L_m, n, mode, H = case
    parts = int(np.random.default_rng(N + 7 * L_m).integers(0, 4))
    banner(f"random backward N={N} L_m={L_m} n={n} mode={mode} H={H} parts={parts}")
    Q, K, V, G = tensors(N, H, 9200 + N, with_dout=True)
    Qd, Kd, Vd, Gd = (to_dev(x, "bf16") for x in (Q, K, V, G))
    shape = (N, H, D)
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    ws = torch.empty(max(16, rs.rswa_masked_bwd_workspace_size(N, L_m, H, parts)), dtype=torch.uint8,
                     device="cuda")
    rs.rswa_masked_attn(Qd, Kd, Vd, out, N, L_m, n, H, D, rs.RSWA_BF16, mode, 0.0, lse=lse)
    rs.rswa_masked_attn_bwd(Qd, Kd, Vd, out, Gd, lse, dq, dk, dv, N, L_m, n, H, D, rs.RSWA_BF16, mode, 0.0, ws,
                            num_parts=parts)
    torch.cuda.synchronize()
    f = lambda a: wl.to_f64(a, "bf16")
    dQ, dK, dV = orc.masked_attention_backward(f(Q), f(K), f(V), f(G), L_m, n, SCALE, mode)
    tag = f"N={N} L_m={L_m} n={n} mode={mode} parts={parts}"
    check_grad(to_f64(dq), dQ, f"dQ {tag}")
    check_grad(to_f64(dk), dK, f"dK {tag}")
    check_grad(to_f64(dv), dV, f"dV {tag}")


def pack_cases(count, seed):
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        S = int(g.integers(1, 8))
        lens = [int(x) for x in g.integers(0, 300, S)]
        refs = [int(g.integers(0, L + 1)) for L in lens]
        cases.append((lens, refs, int(g.choice(WINDOWS)), int(g.choice([CAUSAL, FULL])), int(g.integers(1, 3)),
                      int(g.integers(0, 6))))
    return cases


@pytest.mark.parametrize("case", pack_cases(8 * WIDEN, 2028), ids=lambda c: "S%d-n%d-m%d" % (len(c[0]), c[2], c[3]))
def test_pack_random_forward_and_backward(case):
    lens, refs, n, mode, H, tail = case
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1]) + tail  # rows outside every sample must stay untouched
    max_len = max(1, max(lens))
    banner(f"random pack lens={lens} refs={refs} n={n} mode={mode} H={H} tail={tail}")
    if total == 0:
        pytest.skip("empty pack")
    Q, K, V, G = tensors(total, H, 9300 + total, with_dout=True)
    Qd, Kd, Vd, Gd = (to_dev(x, "bf16") for x in (Q, K, V, G))
    shape = (total, H, D)
    nan = lambda: torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    out, dq, dk, dv = nan(), nan(), nan(), nan()
    lse = torch.full((H, total), float("nan"), dtype=torch.float32, device="cuda")
    cu_d, refs_d = dev_i32(cu), dev_i32(refs)
    ws = torch.empty(rs.rswa_masked_bwd_varlen_workspace_size(total, H), dtype=torch.uint8, device="cuda")
    rs.rswa_masked_attn_varlen(Qd, Kd, Vd, out, cu_d, refs_d, len(refs), total, max_len, n, H, D, rs.RSWA_BF16,
                               mode, 0.0, lse=lse)
    rs.rswa_masked_attn_bwd_varlen(Qd, Kd, Vd, out, Gd, lse, dq, dk, dv, cu_d, refs_d, len(refs), total, max_len,
                                   n, H, D, rs.RSWA_BF16, mode, 0.0, ws)
    torch.cuda.synchronize()
    f = lambda a: wl.to_f64(a, "bf16")
    got, got_lse = to_f64(out), lse.cpu().numpy().astype(np.float64)
    gq, gk, gv = to_f64(dq), to_f64(dk), to_f64(dv)
    for s, (L, r0, r1) in enumerate(zip(refs, cu[:-1], cu[1:])):
        if r1 == r0:
            continue
        sl = slice(r0, r1)
        ref = orc.masked_attention_rows(f(Q[sl]), f(K[sl]), f(V[sl]), range(r1 - r0), L, n, SCALE, mode)
        check_close(got[sl], ref, "bf16", f"sample {s} outputs")
        ref_lse = orc.masked_logsumexp_rows(f(Q[sl]), f(K[sl]), range(r1 - r0), L, n, SCALE, mode)
        check_lse(got_lse[:, sl].T, ref_lse, f"sample {s} lse")
        dQ, dK, dV = orc.masked_attention_backward(f(Q[sl]), f(K[sl]), f(V[sl]), f(G[sl]), L, n, SCALE, mode)
        check_grad(gq[sl], dQ, f"sample {s} dQ")
        check_grad(gk[sl], dK, f"sample {s} dK")
        check_grad(gv[sl], dV, f"sample {s} dV")
    rest = slice(int(cu[-1]), total)
    for t, name in ((out, "out"), (dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert torch.isnan(t[rest].float()).all(), f"rows outside every sample were written ({name})"


def prefill_cases(count, seed):
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        B = int(g.integers(1, 6))
        n = int(g.choice([1, 5, 16, 64, 128]))
        refs = [int(x) for x in g.integers(0, 200, B)]
        t0s = [int(x) for x in g.integers(0, 3 * n + 2, B)]
        cases.append((refs, t0s, n, int(g.choice([CAUSAL, FULL]))))
    return cases


@pytest.mark.parametrize("case", prefill_cases(6 * WIDEN, 2029), ids=lambda c: "B%d-n%d-m%d" % (len(c[0]), c[2], c[3]))
def test_prefill_random_cache_images(case):
    refs, t0s, n, mode = case
    H = 2
    lens = [L + t for L, t in zip(refs, t0s)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    banner(f"random prefill refs={refs} t0s={t0s} n={n} mode={mode}")
    Q, K, V = tensors(max(total, 1), H, 9400 + total)
    cache = rs.KVCache.allocate(refs, H, D, n, dtype=rs.RSWA_BF16)
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    cache.step.fill_(-5)
    out = torch.full((max(total, 1), H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    rs.rswa_prefill(cache.desc, Qd, Kd, Vd, out, dev_i32(cu), total, max(lens), mode, 0.0)
    torch.cuda.synchronize()
    assert rs.rswa_check_device_error(cache.desc) == 0
    assert cache.step.cpu().tolist() == t0s
    got = to_f64(out)
    kbits, vbits = bits(cache.k), bits(cache.v)
    f = lambda a: wl.to_f64(a, "bf16")
    for b, (L, t0) in enumerate(zip(refs, t0s)):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if r1 > r0:
            sl = slice(r0, r1)
            ref = orc.masked_attention_rows(f(Q[sl]), f(K[sl]), f(V[sl]), range(r1 - r0), L, n, SCALE, mode)
            check_close(got[sl], ref, "bf16", f"sequence {b} outputs")
        base = cache._host_bases()[b]
        blk_k = kbits[base:base + H * (L + n) * D].reshape(H, L + n, D)
        blk_v = vbits[base:base + H * (L + n) * D].reshape(H, L + n, D)
        for slot, pos in enumerate(orc.ring_image(L, n, t0)):
            if pos == 0:
                assert np.all(blk_k[:, slot] == 0x7FC0), f"seq {b} slot {slot} written"
                assert np.all(blk_v[:, slot] == 0x7FC0), f"seq {b} slot {slot} written"
                continue
            assert np.array_equal(blk_k[:, slot], K[r0 + pos - 1]), f"seq {b} slot {slot} K"
            assert np.array_equal(blk_v[:, slot], V[r0 + pos - 1]), f"seq {b} slot {slot} V"


def decode_cases(count, seed):
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        B, H = int(g.integers(1, 5)), int(g.integers(1, 4))
        n = int(g.choice([1, 2, 7, 16, 64, 128, 129, 300]))
        cases.append((B, H, int(g.choice([64, 128])), str(g.choice(["bf16", "fp32"])),
                      [int(x) for x in g.integers(0, 300, B)], n, int(g.integers(1, min(80, 2 * n + 4) + 1)),
                      int(g.choice([0, 1, 3, 8]))))
    return cases


@pytest.mark.parametrize("case", decode_cases(12 * WIDEN, 2030),
                         ids=lambda c: "B%d-H%d-d%d-%s-n%d-T%d-s%d" % (c[0], c[1], c[2], c[3], c[5], c[6], c[7]))
def test_decode_random_every_step_and_cache_image(case):
    """Per-sequence reference lengths, fused append + attend from an empty window
    through wrap-around, every step against the oracle; then the cache bit for bit."""
    B, H, d, dt, refs, n, steps, splits = case
    code = rs.RSWA_BF16 if dt == "bf16" else rs.RSWA_FP32
    banner(f"random decode B={B} H={H} d={d} {dt} refs={refs} n={n} steps={steps} splits={splits}")
    seed = 9500 + sum(refs) + steps
    kref = [wl.draw(dt, 1.0, (H, L, d), seed, 0, b) for b, L in enumerate(refs)]
    vref = [wl.draw(dt, 1.0, (H, L, d), seed, 1, b) for b, L in enumerate(refs)]
    bases = np.concatenate([[0], np.cumsum([H * L * d for L in refs])[:-1]]).astype(np.int64)
    flat = lambda xs: np.concatenate([x.reshape(-1) for x in xs] + [np.zeros(8, xs[0].dtype)])
    cache = rs.KVCache.allocate(refs, H, d, n, dtype=code)
    rs.rswa_cache_init(cache.desc, to_dev(flat(kref), dt), to_dev(flat(vref), dt),
                       torch.tensor(bases, dtype=torch.int64, device="cuda"))
    ws = cache.workspace(splits)
    out = torch.empty((B, H, d), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device="cuda")
    new = [[wl.draw(dt, 1.0, (B, H, d), seed, tid, T) for T in range(1, steps + 1)] for tid in (2, 3, 4)]
    f = lambda a: wl.to_f64(a, dt)
    for T in range(1, steps + 1):
        q, k, v = (to_dev(x[T - 1], dt) for x in new)
        rs.rswa_decode_attn(cache.desc, q, out, k, v, 0.0, splits, ws)
        got = to_f64(out)
        ref = np.empty_like(got)
        for b, L in enumerate(refs):
            ok = np.stack([new[1][t][b] for t in range(T)])  # outputs 1..T, [T][H][d]
            ov = np.stack([new[2][t][b] for t in range(T)])
            for h in range(H):
                ref[b, h] = orc.decode_output(f(new[0][T - 1][b, h]), f(kref[b][h]), f(vref[b][h]),
                                              f(ok[:, h]), f(ov[:, h]), 1, L, n, T, 1.0 / np.sqrt(d))
        check_close(got, ref, dt, f"decode step {T}")
    torch.cuda.synchronize()
    assert rs.rswa_check_device_error(cache.desc) == 0
    assert cache.step.cpu().tolist() == [steps] * B
    kbits, vbits = bits(cache.k), bits(cache.v)
    sb = lambda a: a.view(np.uint16) if dt == "bf16" else a.view(np.uint32)
    for b, L in enumerate(refs):
        base = cache._host_bases()[b]
        blk_k = kbits[base:base + H * (L + n) * d].reshape(H, L + n, d)
        blk_v = vbits[base:base + H * (L + n) * d].reshape(H, L + n, d)
        for slot, pos in enumerate(orc.ring_image(L, n, steps)):
            if pos == 0:
                continue  # never written: the pool was not initialised
            if pos <= L:
                want_k, want_v = kref[b][:, pos - 1], vref[b][:, pos - 1]
            else:
                want_k, want_v = new[1][pos - L - 1][b], new[2][pos - L - 1][b]
            assert np.array_equal(blk_k[:, slot], sb(want_k)), f"seq {b} slot {slot} K"
            assert np.array_equal(blk_v[:, slot], sb(want_v)), f"seq {b} slot {slot} V"
