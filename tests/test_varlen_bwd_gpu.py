"""GPU parity of the multi-sample packed backward (rswa_masked_attn_bwd_varlen)
against the oracle, through the C ABI.

Reading under test (as for the multi-sample forward): samples are independent,
so each sample's dQ, dK, dV must equal the single-sequence oracle backward on
that sample's rows alone. Gradient tolerance as for the single-sequence
backward: max|diff| <= 2e-2 * max(1, max|ref|) and ||diff||_2 / ||ref||_2 <=
1e-2 (bf16 outputs; P and dS rounded to bf16 as matrix-core operands)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.rswa as orc
import reference_sliding_window_amd as rs
import workloads as wl
from gpu_util import bits, check_grad, to_dev, to_f64

pytestmark = pytest.mark.gpu

CAUSAL, FULL = rs.RSWA_PREFIX_CAUSAL, rs.RSWA_PREFIX_FULL
D = 128
SCALE = 1.0 / np.sqrt(D)


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def dev_i32(a):
    return torch.tensor(np.asarray(a, np.int32), dtype=torch.int32, device="cuda")


class PackRun:
    """Forward (with lse) and backward of a pack of samples on the device. Gradient
    buffers start as NaN so rows the kernels must not write stay visible."""

    def __init__(self, cu, refs, n, H, mode, seed, total=None, max_len=None):
        self.cu = np.asarray(cu, np.int32)
        self.refs = np.asarray(refs, np.int32)
        self.total = int(total if total is not None else self.cu[-1])
        lens = np.diff(self.cu)
        self.max_len = int(max_len if max_len is not None else lens.max(initial=0))
        self.n, self.H, self.mode = n, H, mode
        shape = (self.total, H, D)
        self.Q, self.K, self.V = (wl.draw("bf16", 1.0, shape, seed, tid) for tid in (0, 1, 2))
        self.G = wl.draw("bf16", 1.0, shape, seed, wl.TID_DOUT)
        self.Qd, self.Kd, self.Vd, self.Gd = (to_dev(x, "bf16") for x in (self.Q, self.K, self.V, self.G))
        self.cu_d, self.refs_d = dev_i32(self.cu), dev_i32(self.refs)
        nan = lambda: torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        self.out, self.dq, self.dk, self.dv = nan(), nan(), nan(), nan()
        self.lse = torch.full((H, self.total), float("nan"), dtype=torch.float32, device="cuda")
        nbytes = rs.rswa_masked_bwd_varlen_workspace_size(self.total, H)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def forward(self):
        rs.rswa_masked_attn_varlen(self.Qd, self.Kd, self.Vd, self.out, self.cu_d, self.refs_d,
                                   len(self.refs), self.total, self.max_len, self.n, self.H, D,
                                   rs.RSWA_BF16, self.mode, 0.0, lse=self.lse)

    def backward(self):
        rs.rswa_masked_attn_bwd_varlen(self.Qd, self.Kd, self.Vd, self.out, self.Gd, self.lse, self.dq,
                                       self.dk, self.dv, self.cu_d, self.refs_d, len(self.refs),
                                       self.total, self.max_len, self.n, self.H, D, rs.RSWA_BF16,
                                       self.mode, 0.0, self.ws)

    def sample_ref(self, r0, r1, L, heads=None):
        hs = slice(None) if heads is None else heads
        f = lambda a: wl.to_f64(a[r0:r1][:, hs], "bf16")
        return orc.masked_attention_backward(f(self.Q), f(self.K), f(self.V), f(self.G), L, self.n, SCALE,
                                             self.mode)


@pytest.mark.parametrize("mode", [CAUSAL, FULL])
def test_varlen_bwd_every_row_and_key(mode):
    # samples: ordinary, no reference, all reference, one row, empty, window wider than sample
    lens = [300, 150, 97, 1, 0, 260]
    refs = [40, 0, 97, 1, 0, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1]) + 5  # five trailing rows outside every sample
    banner(f"varlen bwd mode={mode} lens={lens} refs={refs}")
    r = PackRun(cu, refs, 16, 2, mode, seed=8100 + mode, total=total)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    dq, dk, dv = to_f64(r.dq), to_f64(r.dk), to_f64(r.dv)
    for s, (L, r0, r1) in enumerate(zip(refs, cu[:-1], cu[1:])):
        if r1 == r0:
            continue
        dQ, dK, dV = r.sample_ref(r0, r1, L)
        tag = f"sample {s} (rows {r0}..{r1}, L={L})"
        check_grad(dq[r0:r1], dQ, f"dQ {tag}")
        check_grad(dk[r0:r1], dK, f"dK {tag}")
        check_grad(dv[r0:r1], dV, f"dV {tag}")
    for t in (r.dq, r.dk, r.dv):
        assert torch.isnan(t[int(cu[-1]):].float()).all(), "rows outside every sample were written"


def test_varlen_bwd_one_sample_equals_single_sequence_kernel():
    """A pack of one sample gives the single-sequence call's bits (one part there)."""
    N, L, n, H = 777, 200, 128, 3
    banner("varlen bwd one sample vs rswa_masked_attn_bwd")
    r = PackRun([0, N], [L], n, H, CAUSAL, seed=8200)
    r.forward()
    r.backward()
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
    rs.rswa_masked_attn(r.Qd, r.Kd, r.Vd, out, N, L, n, H, D, rs.RSWA_BF16, CAUSAL, 0.0, lse=lse)
    g = [torch.empty_like(out) for _ in range(3)]
    ws = torch.empty(rs.rswa_masked_bwd_workspace_size(N, L, H), dtype=torch.uint8, device="cuda")
    rs.rswa_masked_attn_bwd(r.Qd, r.Kd, r.Vd, out, r.Gd, lse, g[0], g[1], g[2], N, L, n, H, D, rs.RSWA_BF16,
                            CAUSAL, 0.0, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(r.out), bits(out))
    for name, a, b in zip(("dQ", "dK", "dV"), (r.dq, r.dk, r.dv), g):
        assert np.array_equal(bits(a), bits(b)), f"{name} differs from the single-sequence kernel"


def test_varlen_bwd_sample_offset_does_not_change_results():
    """A sample gives the same gradient bits wherever it sits in the pack."""
    n, H = 32, 2
    lens, refs = [333, 190], [70, 64]
    banner("varlen bwd offset invariance")
    a = PackRun(np.concatenate([[0], np.cumsum(lens)]), refs, n, H, CAUSAL, seed=8300)
    a.forward()
    a.backward()
    # the second sample alone, at row 0, from the same input rows
    b = PackRun([0, lens[1]], [refs[1]], n, H, CAUSAL, seed=8300, total=lens[1])
    sl = slice(lens[0], lens[0] + lens[1])
    for dst, src in ((b.Qd, a.Qd), (b.Kd, a.Kd), (b.Vd, a.Vd), (b.Gd, a.Gd)):
        dst.copy_(src[sl])
    b.forward()
    b.backward()
    torch.cuda.synchronize()
    for name, x, y in (("dQ", a.dq, b.dq), ("dK", a.dk, b.dk), ("dV", a.dv, b.dv)):
        assert np.array_equal(bits(x[sl]), bits(y)), f"{name} depends on the sample's offset"


def test_varlen_bwd_malformed_samples_are_skipped():
    """Device-side metadata the kernels cannot trust: a sample whose end lies before
    its start, or that is longer than max_seq_len, is skipped; the others are exact."""
    banner("varlen bwd malformed samples")
    cu, refs = [0, 200, 100, 420], [50, 10, 20]
    r = PackRun(cu, refs, 64, 2, CAUSAL, seed=8400, total=420, max_len=200)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    dQ, dK, dV = r.sample_ref(0, 200, 50)
    check_grad(to_f64(r.dq)[:200], dQ, "dQ valid sample")
    check_grad(to_f64(r.dk)[:200], dK, "dK valid sample")
    check_grad(to_f64(r.dv)[:200], dV, "dV valid sample")
    for t in (r.dq, r.dk, r.dv):
        assert torch.isnan(t[200:].float()).all(), "a skipped sample's rows were written"


def test_varlen_bwd_is_deterministic():
    banner("varlen bwd determinism")
    r = PackRun([0, 300, 700], [100, 40], 128, 2, FULL, seed=8500)
    r.forward()
    r.backward()
    first = [t.clone() for t in (r.dq, r.dk, r.dv)]
    r.backward()
    torch.cuda.synchronize()
    for a, b in zip(first, (r.dq, r.dk, r.dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.slow
def test_varlen_bwd_32k_pack():
    """The 32K ten-document pack (pages ~ U{2..16}, outputs ~ U{256..2048}): the two
    shortest samples exactly on two heads, and for every sample the column sums the
    softmax fixes: sum_j dV_j = sum_i dO_i and |sum_j dK_j| <= 2^-9 sum_j |dK_j| (the
    rounding residues of thousands of rows, each at most 2^-8 of its row's mass,
    largely cancel; see test_masked_bwd_gpu)."""
    mw = wl.PACKED_32K
    H, n = mw.heads, mw.window
    cu, refs = wl.varlen_pack_layout(mw.seq_len, 20260004)
    banner(f"varlen bwd 32K pack: {len(refs)} samples, rows {np.diff(cu).tolist()}")
    r = PackRun(cu, refs, n, H, CAUSAL, seed=20260004, total=mw.seq_len)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    dq, dk, dv = to_f64(r.dq), to_f64(r.dk), to_f64(r.dv)
    lens = np.diff(cu)
    hs = [0, H - 1]
    for s in np.argsort(lens)[:2]:
        r0, r1, L = int(cu[s]), int(cu[s + 1]), int(refs[s])
        dQ, dK, dV = r.sample_ref(r0, r1, L, heads=hs)
        for name, got, ref in (("dQ", dq, dQ), ("dK", dk, dK), ("dV", dv, dV)):
            ma, rel = check_grad(got[r0:r1][:, hs], ref, f"{name} sample {s} ({r1 - r0} rows)")
            print(f"{name} sample {s}: max|d|={ma:.3e} rel={rel:.3e}")
    G = wl.to_f64(r.G, "bf16")
    for s in range(len(refs)):
        r0, r1 = int(cu[s]), int(cu[s + 1])
        check_grad(dv[r0:r1].sum(axis=0), G[r0:r1].sum(axis=0), f"sum dV vs sum dO, sample {s}")
        dk_sum = dk[r0:r1].sum(axis=0)
        bound = 2.0 ** -9 * np.abs(dk[r0:r1]).sum(axis=0)
        worst = float((np.abs(dk_sum) / bound).max())
        assert worst <= 1.0, f"sample {s}: sum_j dK_j exceeds 2^-9 sum_j |dK_j| (ratio {worst:.3f})"
    tail = int(cu[-1])
    for t in (r.dq, r.dk, r.dv):
        assert torch.isnan(t[tail:].float()).all(), "rows outside every sample were written"
