"""GPU parity of the packed forward's log-sum-exp output and of the packed
backward (rswa_masked_attn_bwd) against the oracle, through the C ABI.

Gradient tolerance: the gradients are bf16 outputs whose size grows with the
number of terms summed (a prefix key's dK/dV gathers every row that sees it),
and the kernels round P and dS to bf16 as matrix-core operands, so the error is
relative to the gradient's magnitude: max|diff| <= 2e-2 * max(1, max|ref|) and
||diff||_2 / ||ref||_2 <= 1e-2, over each gradient tensor and over each head
on its own (see gpu_util.check_grad). The log-sum-exp is fp32, but the forward sums
the probabilities it has rounded to bf16 (8 significant bits: each within 2^-8
relative of its fp32 value), so its normaliser is within a factor 1 +- 2^-8 of
the exact one: |diff| <= 2^-8 + 2e-4 + 1e-5 |ref| (the rest covers fp32 scores
and exp2)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.pool as opool
import oracle.rswa as orc
import reference_sliding_window_amd as rs
import workloads as wl
from gpu_util import check_close, check_grad, score_range_qkv, to_dev, to_f64

pytestmark = pytest.mark.gpu

CAUSAL, FULL = rs.RSWA_PREFIX_CAUSAL, rs.RSWA_PREFIX_FULL


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


class PackedRun:
    """Forward (with lse) and backward of one packed sequence on the device."""

    def __init__(self, N, L_m, n, H, mode, seed, sigma=1.0, parts=0):
        self.mw = wl.MaskedWorkload("masked-bwd", seq_len=N, heads=H, head_dim=128, ref_len=L_m,
                                    window=n, dtype="bf16", sigma=sigma, base_seed=seed)
        self.N, self.L_m, self.n, self.H, self.mode = N, L_m, n, H, mode
        self.Q, self.K, self.V = wl.packed_qkv(self.mw)
        self.G = wl.packed_dout(self.mw)
        self.Qd, self.Kd, self.Vd, self.Gd = (to_dev(x, "bf16") for x in (self.Q, self.K, self.V, self.G))
        shape = (N, H, 128)
        self.out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
        self.dq = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        self.dk = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        self.dv = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        self.parts = parts
        nbytes = rs.rswa_masked_bwd_workspace_size(N, L_m, H, parts)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")

    def forward(self):
        rs.rswa_masked_attn(self.Qd, self.Kd, self.Vd, self.out, self.N, self.L_m, self.n, self.H, 128,
                            rs.RSWA_BF16, self.mode, 0.0, lse=self.lse)

    def backward(self):
        rs.rswa_masked_attn_bwd(self.Qd, self.Kd, self.Vd, self.out, self.Gd, self.lse, self.dq, self.dk,
                                self.dv, self.N, self.L_m, self.n, self.H, 128, rs.RSWA_BF16, self.mode,
                                0.0, self.ws, num_parts=self.parts)

    def f64(self):
        f = lambda a: wl.to_f64(a, "bf16")
        return f(self.Q), f(self.K), f(self.V), f(self.G)


SMALL_CASES = [
    (300, 40, 8, CAUSAL),
    (300, 40, 8, FULL),
    (1, 1, 128, CAUSAL),
    (1, 0, 1, CAUSAL),
    (257, 0, 16, CAUSAL),
    (200, 200, 4, FULL),
    (200, 200, 4, CAUSAL),
    (513, 130, 128, CAUSAL),
    (640, 97, 1, CAUSAL),
    (700, 300, 200, FULL),
    (161, 33, 1000, CAUSAL),
]


@pytest.mark.parametrize("N,L_m,n,mode", SMALL_CASES[:4] + SMALL_CASES[7:8])
def test_forward_lse_every_row(N, L_m, n, mode):
    banner(f"packed lse N={N} L_m={L_m} n={n} mode={mode}")
    r = PackedRun(N, L_m, n, 2, mode, seed=5000 + N + L_m + n + mode)
    r.forward()
    torch.cuda.synchronize()
    Q, K, _, _ = r.f64()
    ref = orc.masked_logsumexp_rows(Q, K, range(N), L_m, n, r.mw.scale, mode)  # [N][H]
    got = r.lse.cpu().numpy().astype(np.float64).T
    err = np.abs(got - ref)
    assert np.isfinite(got).all()
    assert (err <= 2.0 ** -8 + 2e-4 + 1e-5 * np.abs(ref)).all(), f"lse max err {err.max():.3e}"


def test_forward_lse_does_not_change_output():
    banner("packed forward with and without lse")
    r = PackedRun(513, 130, 128, 2, CAUSAL, seed=77)
    r.forward()
    a = r.out.clone()
    rs.rswa_masked_attn(r.Qd, r.Kd, r.Vd, r.out, r.N, r.L_m, r.n, r.H, 128, rs.RSWA_BF16, CAUSAL, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), r.out.view(torch.int16))


@pytest.mark.parametrize("N,L_m,n,mode", SMALL_CASES)
def test_backward_small_every_row_and_key(N, L_m, n, mode):
    banner(f"packed bwd N={N} L_m={L_m} n={n} mode={mode}")
    r = PackedRun(N, L_m, n, 2, mode, seed=6000 + N + L_m + n + mode)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    Q, K, V, G = r.f64()
    dQ, dK, dV = orc.masked_attention_backward(Q, K, V, G, L_m, n, r.mw.scale, mode)
    tag = f"N={N} L_m={L_m} n={n} mode={mode}"
    check_grad(to_f64(r.dq), dQ, f"dQ {tag}")
    check_grad(to_f64(r.dk), dK, f"dK {tag}")
    check_grad(to_f64(r.dv), dV, f"dV {tag}")


@pytest.mark.parametrize("N,L_m,n,mode,parts", [
    (300, 40, 8, CAUSAL, 2),
    (700, 300, 200, FULL, 3),
    (513, 130, 128, CAUSAL, 7),
    (200, 200, 4, CAUSAL, 64),   # more parts than query blocks: empty runs
    (1, 1, 128, CAUSAL, 5),
])
def test_backward_split_walks_every_row_and_key(N, L_m, n, mode, parts):
    """Reference-segment keys with their row walks cut into parts (fp32 partials
    summed by the reduction kernel)."""
    banner(f"packed bwd parts={parts} N={N} L_m={L_m} n={n} mode={mode}")
    r = PackedRun(N, L_m, n, 2, mode, seed=7000 + N + L_m + n + mode, parts=parts)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    Q, K, V, G = r.f64()
    dQ, dK, dV = orc.masked_attention_backward(Q, K, V, G, L_m, n, r.mw.scale, mode)
    tag = f"parts={parts} N={N} L_m={L_m} n={n} mode={mode}"
    check_grad(to_f64(r.dq), dQ, f"dQ {tag}")
    check_grad(to_f64(r.dk), dK, f"dK {tag}")
    check_grad(to_f64(r.dv), dV, f"dV {tag}")


def test_backward_parts_change_only_rounding():
    """One walk against several: the same gradients up to fp32 summation order."""
    banner("packed bwd parts invariance")
    runs = []
    for parts in (1, 4):
        r = PackedRun(2048, 700, 128, 2, CAUSAL, seed=99, parts=parts)
        r.forward()
        r.backward()
        torch.cuda.synchronize()
        runs.append([to_f64(t) for t in (r.dq, r.dk, r.dv)])
    for name, a, b in zip(("dQ", "dK", "dV"), *runs):
        check_grad(b, a, f"{name} parts 4 vs 1")
        if name == "dQ":
            assert np.array_equal(a, b)  # dQ does not depend on the split


def test_backward_is_deterministic():
    banner("packed bwd determinism")
    r = PackedRun(700, 300, 200, 2, FULL, seed=9)
    r.forward()
    r.backward()
    first = [t.clone() for t in (r.dq, r.dk, r.dv)]
    r.backward()
    torch.cuda.synchronize()
    for a, b in zip(first, (r.dq, r.dk, r.dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_backward_medium_every_row_and_key():
    """Long query walks for the prefix keys (~3000 rows each), several heads."""
    N, L_m, n, H = 4096, 1000, 128, 2
    banner(f"packed bwd medium N={N} L_m={L_m} n={n} H={H}")
    r = PackedRun(N, L_m, n, H, CAUSAL, seed=31337)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    Q, K, V, G = r.f64()
    dQ, dK, dV = orc.masked_attention_backward(Q, K, V, G, L_m, n, r.mw.scale, CAUSAL)
    for name, got, ref in (("dQ", r.dq, dQ), ("dK", r.dk, dK), ("dV", r.dv, dV)):
        ma, rel = check_grad(to_f64(got), ref, f"{name} medium")
        print(f"{name}: max|d|={ma:.3e} rel={rel:.3e}")


@pytest.mark.slow
@pytest.mark.parametrize("mode", [CAUSAL, FULL])
def test_backward_32k_sampled_and_column_sums(mode):
    """Full packed 32K size: dQ on sampled rows and dK/dV on sampled output-segment
    keys exactly (the rows that see such a key are the n rows from it on), and for
    every key the column sums the softmax fixes: sum_j dV_j = sum_i dO_i (each
    row's weights sum to one) and sum_j dK_j = 0 (each row's dS sums to zero)."""
    mw = wl.PACKED_32K
    N, L_m, n, H = mw.seq_len, mw.ref_len, mw.window, mw.heads
    banner(f"packed 32K bwd N={N} L_m={L_m} n={n} H={H} mode={mode}")
    r = PackedRun(N, L_m, n, H, mode, seed=mw.base_seed, sigma=mw.sigma)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    dq, dk, dv = to_f64(r.dq), to_f64(r.dk), to_f64(r.dv)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    f = lambda a: wl.to_f64(a, "bf16")
    K, V = f(r.K), f(r.V)
    rng = np.random.default_rng(12)
    rows = sorted(set([0, 1, L_m - 1, L_m, L_m + 1, L_m + n - 1, L_m + n, 4095, 4096, N - 1] +
                      rng.integers(0, N, 24).tolist()))
    Qr, Gr = _RowView(f(r.Q[rows]), rows), _RowView(f(r.G[rows]), rows)
    dQ, _, _ = orc.masked_attention_backward(Qr, K, V, Gr, L_m, n, mw.scale, mode, rows=rows)
    ma, rel = check_grad(dq[rows], dQ, "dQ 32K sampled rows")
    print(f"dQ rows: max|d|={ma:.3e} rel={rel:.3e}")
    # output-segment keys in three runs of 8 (near L_m, mid-sequence, the tail);
    # heads 0 and H-1 only (a head's gradients depend on that head alone)
    hs = [0, H - 1]
    Kh, Vh = K[:, hs], V[:, hs]
    mid = (L_m + N) // 2
    for a in (L_m, mid, N - 8):
        see = list(range(a, min(N, a + 8 + n - 1)))
        Qs = _RowView(f(r.Q[see])[:, hs], see)
        Gs = _RowView(f(r.G[see])[:, hs], see)
        _, dK, dV = orc.masked_attention_backward(Qs, Kh, Vh, Gs, L_m, n, mw.scale, mode, rows=see)
        check_grad(dk[a:a + 8][:, hs], dK[a:a + 8], f"dK keys {a}..{a + 7}")
        check_grad(dv[a:a + 8][:, hs], dV[a:a + 8], f"dV keys {a}..{a + 7}")
    # column sums over every key, per head and dimension (fp64 sums of the bf16 results)
    g_sum = f(r.G).sum(axis=0)
    dv_sum = dv.sum(axis=0)
    check_grad(dv_sum, g_sum, "sum_j dV_j vs sum_i dO_i")
    # sum_j dK_j vanishes in exact arithmetic; here each row's dS sums to a
    # rounding residue (the forward rounds P to bf16 for its normaliser and
    # output, the backward rounds dS), each at most bf16's unit roundoff 2^-8
    # of that row's mass. The rows round independently, so over 32K rows their
    # sum grows like the square root of the count while the mass grows
    # linearly: bound it by 2^-9 of the mass that cancels, sum_j |dK_j|, per
    # head and dimension.
    dk_sum = dk.sum(axis=0)
    bound = 2.0 ** -9 * np.abs(dk).sum(axis=0)
    worst = float((np.abs(dk_sum) / bound).max())
    print(f"sum_j dK_j: max |sum| = {np.abs(dk_sum).max():.3e}, worst |sum| / bound = {worst:.3f}")
    assert worst <= 1.0, f"sum_j dK_j exceeds 2^-9 sum_j |dK_j| (ratio {worst:.3f})"


@pytest.mark.slow
def test_backward_32k_reference_keys_elementwise():
    """The library's default plan at 32K cuts each reference key's walk over the
    query rows into 4 runs whose fp32 partials the reduction kernel adds. Here dK
    and dV of reference keys at the segment's edges, its middle and 5 seeded
    positions are compared element by element, heads 0 and H-1, both prefix
    modes, against the oracle's backward over every row that sees them (on all
    host cores). Output rows see the same keys in both modes, so their
    contributions are computed once and the prefix rows' per mode."""
    mw = wl.PACKED_32K
    N, L_m, n, H = mw.seq_len, mw.ref_len, mw.window, mw.heads
    default = rs.rswa_masked_bwd_workspace_size(N, L_m, H, 0)
    assert default == rs.rswa_masked_bwd_workspace_size(N, L_m, H, 4) != \
        rs.rswa_masked_bwd_workspace_size(N, L_m, H, 1), "the default plan at 32K is 4 runs"
    rng = np.random.default_rng(13)
    keys = sorted(set([0, 1, 127, 128, L_m // 2, L_m - 2, L_m - 1] +
                      rng.integers(2, L_m - 2, 5).tolist()))
    hs = [0, H - 1]
    got = {}
    for mode in (CAUSAL, FULL):
        banner(f"packed 32K bwd, default plan, reference keys {keys}, heads {hs}, mode={mode}")
        r = PackedRun(N, L_m, n, H, mode, seed=mw.base_seed, sigma=mw.sigma)
        r.forward()
        r.backward()
        torch.cuda.synchronize()
        got[mode] = (to_f64(r.dk)[keys][:, hs], to_f64(r.dv)[keys][:, hs])
        inputs = (r.Q, r.K, r.V, r.G)
        del r
    print(f"oracle: {N} rows x {len(hs)} heads on {opool.workers()} processes", flush=True)
    out_rows = list(range(L_m, N))
    pre_rows = list(range(L_m))
    with opool.SharedArrays() as arrays:
        for name, a in zip(("Q", "K", "V", "dO"), inputs):
            arrays.put(name, wl.bf16_bits_to_f32(a))   # exact values of the bf16 inputs
        tasks = [(out_rows[i::96], keys, hs, L_m, n, mw.scale, CAUSAL) for i in range(96)]
        for mode in (CAUSAL, FULL):
            tasks += [(pre_rows[i::16], keys, hs, L_m, n, mw.scale, mode) for i in range(16)]
        parts = opool.pool_map(opool.masked_bwd_keys_job, tasks, arrays, progress="backward row runs")
    out_dk = sum(p[0] for p in parts[:96])
    out_dv = sum(p[1] for p in parts[:96])
    for k, mode in enumerate((CAUSAL, FULL)):
        pre = parts[96 + 16 * k:96 + 16 * (k + 1)]
        ref_dk = out_dk + sum(p[0] for p in pre)
        ref_dv = out_dv + sum(p[1] for p in pre)
        ma, rel = check_grad(got[mode][0], ref_dk, f"dK reference keys, mode {mode}")
        print(f"mode {mode} dK: max|d|={ma:.3e} worst head rel={rel:.3e}")
        ma, rel = check_grad(got[mode][1], ref_dv, f"dV reference keys, mode {mode}")
        print(f"mode {mode} dV: max|d|={ma:.3e} worst head rel={rel:.3e}")


class _RowView:
    """Indexes like the full [N][H][d] array for the given rows only."""

    def __init__(self, rows_arr, rows):
        self.a = rows_arr
        self.pos = {r: i for i, r in enumerate(rows)}
        self.shape = (max(rows) + 1,) + rows_arr.shape[1:]

    def __getitem__(self, i):
        if isinstance(i, tuple):
            return self.a[self.pos[int(i[0])]][i[1:]]
        return self.a[self.pos[int(i)]]


@pytest.mark.parametrize("mode", [CAUSAL, FULL])
def test_backward_score_ranges(mode):
    """Gradients where the scores leave the unit range (score_range_qkv: a head whose
    scores grow to about +-100 along the sequence, one strongly negative, one strongly
    positive, one ordinary): dQ, dK, dV of every row and key against the oracle."""
    N, L_m, n, H = 700, 200, 64, 4
    banner(f"backward score ranges mode={mode}")
    r = PackedRun(N, L_m, n, H, mode, seed=77001)
    r.Q, r.K, r.V = score_range_qkv(N, H)
    r.Qd, r.Kd, r.Vd = (to_dev(x, "bf16") for x in (r.Q, r.K, r.V))
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    Qf, Kf, Vf, Gf = r.f64()
    scale = 1.0 / np.sqrt(128)
    ref_o = orc.masked_attention_rows(Qf, Kf, Vf, range(N), L_m, n, scale, mode)
    check_close(to_f64(r.out), ref_o, "bf16", f"forward score ranges mode={mode}")
    dQ, dK, dV = orc.masked_attention_backward(Qf, Kf, Vf, Gf, L_m, n, scale, mode)
    tag = f"score ranges mode={mode}"
    check_grad(to_f64(r.dq), dQ, f"dQ {tag}")
    check_grad(to_f64(r.dk), dK, f"dK {tag}")
    check_grad(to_f64(r.dv), dV, f"dV {tag}")
