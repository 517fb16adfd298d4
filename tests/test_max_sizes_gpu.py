"""The packed forward and backward at the largest tensors the C ABI accepts.

The packed calls take seq_len * heads * head_dim below 2^31 elements, so with
16 heads of 128 the longest sequence is N = 2^20 - 1 rows: 4 GB per tensor,
and the kernels' 32-bit byte offsets reach 2^32 - 4 KB (the other tests stay
below 2^31). Rows and keys on both sides of the 2^31-byte point, at the ends
and at the segment edges are checked against the oracle.

A row's output, log-sum-exp and dQ depend only on the keys it sees, and a key's
dK and dV only on the rows that see it and on those rows' own visible keys
(WeThinkIn "Unlimited OCR Works：一篇读懂 R-SWA…", 方法展开.3, Eqs. (1)-(4)).
Each check therefore runs the oracle on a compact sequence made of just those
rows, in order, with the same reference length and window, after asserting with
the oracle's own visible-set function that the compact sequence gives the
checked row or key exactly the visible sets it has in the full one."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.rswa as orc
import reference_sliding_window_amd as rs
from gpu_util import check_close, check_grad

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

H, D = 16, 128
N = (1 << 31) // (H * D) - 1          # 2^20 - 1 rows: 2^31 - 2048 elements per tensor
SCALE = 1.0 / np.sqrt(D)
N_WIN = 128
EDGE = (1 << 31) // (H * D * 2)       # first row at byte offset 2^31


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def device_normal(seed, shape):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)


def host_rows(t, rows):
    """float64 copy of the listed rows (every head) of a device [N][H][D] tensor."""
    idx = torch.as_tensor(np.asarray(rows, np.int64), device="cuda")
    return t.index_select(0, idx).float().cpu().numpy().astype(np.float64)


def check_lse(got, ref, what):
    err = np.abs(got - ref)
    assert (err <= 2.0 ** -8 + 2e-4 + 1e-5 * np.abs(ref)).all(), f"{what}: lse max|d|={err.max():.3e}"


def compact_for_row(i, L_m, mode):
    """The rows row i sees, in order (row i among them), the compact sequence's
    reference length, and row i's place p in it: there row p sees every row, as
    row i does in the full sequence."""
    rows = orc.masked_visible_columns(i, L_m, N_WIN, mode)
    Lc = min(L_m, len(rows))
    p = rows.index(i)
    assert orc.masked_visible_columns(p, Lc, N_WIN, mode) == list(range(len(rows)))
    return rows, Lc, p


@pytest.fixture(scope="module")
def rng():
    return np.random.default_rng(20261203)


@pytest.mark.parametrize("mode", [rs.RSWA_PREFIX_CAUSAL, rs.RSWA_PREFIX_FULL])
def test_forward_at_the_largest_size(mode, rng):
    L_m = 256
    banner(f"packed forward N={N} H={H} L_m={L_m} n={N_WIN} mode={mode} (4 GB per tensor)")
    Q, K, V = (device_normal(7100 + t, (N, H, D)) for t in range(3))
    out = torch.full((N, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, N), float("nan"), dtype=torch.float32, device="cuda")
    rs.rswa_masked_attn(Q, K, V, out, N, L_m, N_WIN, H, D, rs.RSWA_BF16, mode, 0.0, lse=lse)
    torch.cuda.synchronize()
    rows = [0, 1, L_m - 1, L_m, L_m + 1, L_m + N_WIN - 2, L_m + N_WIN - 1, L_m + N_WIN, EDGE - 1, EDGE,
            N - 2, N - 1] + sorted(rng.integers(L_m + N_WIN, N, 8).tolist())
    got = host_rows(out, rows)
    got_lse = lse[:, torch.as_tensor(rows, device="cuda")].cpu().numpy().astype(np.float64).T
    ref, ref_lse = np.empty_like(got), np.empty_like(got_lse)
    for k, i in enumerate(rows):
        vis, Lc, p = compact_for_row(i, L_m, mode)
        Qc, Kc, Vc = (host_rows(t, vis) for t in (Q, K, V))
        ref[k] = orc.masked_attention_rows(Qc, Kc, Vc, [p], Lc, N_WIN, SCALE, mode)[0]
        ref_lse[k] = orc.masked_logsumexp_rows(Qc, Kc, [p], Lc, N_WIN, SCALE, mode)[0]
    check_close(got, ref, "bf16", f"forward at N={N}, rows {rows}")
    check_lse(got_lse, ref_lse, "forward lse at the largest size")
    del Q, K, V, out, lse
    torch.cuda.empty_cache()


def test_backward_at_the_largest_size(rng):
    L_m, mode = 0, rs.RSWA_PREFIX_CAUSAL
    banner(f"packed backward N={N} H={H} L_m={L_m} n={N_WIN} (4 GB per tensor, 8 tensors)")
    Q, K, V, G = (device_normal(7200 + t, (N, H, D)) for t in range(4))
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.full((N, H, D), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    ws = torch.empty(rs.rswa_masked_bwd_workspace_size(N, L_m, H, 0), dtype=torch.uint8, device="cuda")
    rs.rswa_masked_attn(Q, K, V, out, N, L_m, N_WIN, H, D, rs.RSWA_BF16, mode, 0.0, lse=lse)
    rs.rswa_masked_attn_bwd(Q, K, V, out, G, lse, dq, dk, dv, N, L_m, N_WIN, H, D, rs.RSWA_BF16, mode, 0.0, ws)
    torch.cuda.synchronize()
    picks = [0, 1, N_WIN - 1, N_WIN, EDGE - 1, EDGE, N - N_WIN - 1, N - 2, N - 1] + \
        sorted(rng.integers(N_WIN, N - N_WIN, 4).tolist())

    # dQ of row i: the compact sequence of the keys it sees.
    got_dq = host_rows(dq, picks)
    ref_dq = np.empty_like(got_dq)
    for k, i in enumerate(picks):
        vis, Lc, p = compact_for_row(i, L_m, mode)
        Qc, Kc, Vc, Gc = (host_rows(t, vis) for t in (Q, K, V, G))
        dQc, _, _ = orc.masked_attention_backward(Qc, Kc, Vc, Gc, Lc, N_WIN, SCALE, mode)
        ref_dq[k] = dQc[p]
    check_grad(got_dq, ref_dq, f"dQ at N={N}, rows {picks}")

    # dK, dV of key j: rows [a, b) with a = j - n + 1 (clamped) hold every row that sees j
    # (j .. j + n - 1) and every key those rows see.
    got_dk, got_dv = host_rows(dk, picks), host_rows(dv, picks)
    ref_dk, ref_dv = np.empty_like(got_dk), np.empty_like(got_dv)
    for k, j in enumerate(picks):
        a, b = max(0, j - N_WIN + 1), min(N, j + N_WIN)
        seers = [i for i in range(j, b) if j in orc.masked_visible_columns(i, L_m, N_WIN, mode)]
        assert seers == list(range(j, min(N, j + N_WIN)))
        for i in seers:   # each sees the same keys, shifted by a, in the compact sequence
            assert orc.masked_visible_columns(i - a, L_m, N_WIN, mode) == \
                [c - a for c in orc.masked_visible_columns(i, L_m, N_WIN, mode)]
        Qc, Kc, Vc, Gc = (host_rows(t, range(a, b)) for t in (Q, K, V, G))
        _, dKc, dVc = orc.masked_attention_backward(Qc, Kc, Vc, Gc, L_m, N_WIN, SCALE, mode)
        ref_dk[k], ref_dv[k] = dKc[j - a], dVc[j - a]
    check_grad(got_dk, ref_dk, f"dK at N={N}, keys {picks}")
    check_grad(got_dv, ref_dv, f"dV at N={N}, keys {picks}")
    del Q, K, V, G, out, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
