"""GPU parity of the multi-sample packed forward (rswa_masked_attn_varlen) and
of the prefill -> decode hand-off (rswa_prefill) against the oracle, through
the C ABI.

Reading under test (the pages pack several documents per 32K sequence without
stating a cross-sample mask): samples are independent, so each sample of a pack
must equal the single-sequence oracle on that sample alone. The hand-off must
leave the cache exactly as the oracle's ring image after T0 outputs (bit-exact
K/V in every slot, untouched slots keep their old contents) and decoding must
continue from output T0 + 1 as the oracle's queue model does."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.rswa as orc
import reference_sliding_window_amd as rs
import workloads as wl
from gpu_util import bits, check_close, to_dev, to_f64

pytestmark = pytest.mark.gpu

CAUSAL, FULL = rs.RSWA_PREFIX_CAUSAL, rs.RSWA_PREFIX_FULL
D = 128
SCALE = 1.0 / np.sqrt(D)


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def pack_tensors(total, H, seed):
    """q, k, v of a pack in storage form (bf16 bits), [total][H][D]."""
    return tuple(wl.draw("bf16", 1.0, (total, H, D), seed, tid) for tid in (0, 1, 2))


def dev_i32(a):
    return torch.tensor(np.asarray(a, np.int32), dtype=torch.int32, device="cuda")


def sample_oracle(Q, K, V, r0, r1, L, n, mode):
    f = lambda a: wl.to_f64(a[r0:r1], "bf16")
    out = orc.masked_attention_rows(f(Q), f(K), f(V), range(r1 - r0), L, n, SCALE, mode)
    lse = orc.masked_logsumexp_rows(f(Q), f(K), range(r1 - r0), L, n, SCALE, mode)
    return out, lse


def run_varlen(Q, K, V, cu, refs, n, H, mode, max_len=None, total=None):
    total = total if total is not None else Q.shape[0]
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    out = torch.full((total, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, total), float("nan"), dtype=torch.float32, device="cuda")
    lens = np.diff(cu)
    max_len = max_len if max_len is not None else int(lens.max(initial=0))
    rs.rswa_masked_attn_varlen(Qd, Kd, Vd, out, dev_i32(cu), dev_i32(refs), len(refs), total, max_len, n, H, D,
                               rs.RSWA_BF16, mode, 0.0, lse=lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("mode", [CAUSAL, FULL])
def test_varlen_every_row_of_every_sample(mode):
    # samples: ordinary, no reference, all reference, one row, empty, window wider than sample
    lens = [300, 150, 97, 1, 0, 260]
    refs = [40, 0, 97, 1, 0, 33]
    n, H = 16, 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1]) + 5  # five trailing rows outside every sample
    Q, K, V = pack_tensors(total, H, 7100 + mode)
    banner(f"varlen mode={mode} lens={lens} refs={refs}")
    out, lse = run_varlen(Q, K, V, cu, refs, n, H, mode, total=total)
    got, got_lse = to_f64(out), lse.cpu().numpy().astype(np.float64)
    for s, (L, r0, r1) in enumerate(zip(refs, cu[:-1], cu[1:])):
        if r1 == r0:
            continue
        ref, ref_lse = sample_oracle(Q, K, V, r0, r1, L, n, mode)
        check_close(got[r0:r1], ref, "bf16", f"sample {s} (rows {r0}..{r1}, L={L})")
        err = np.abs(got_lse[:, r0:r1].T - ref_lse)
        assert (err <= 2.0 ** -8 + 2e-4 + 1e-5 * np.abs(ref_lse)).all(), f"sample {s} lse {err.max():.3e}"
    assert torch.isnan(out[int(cu[-1]):].float()).all(), "rows outside every sample were written"


def test_varlen_one_sample_equals_single_sequence_kernel():
    N, L, n, H = 777, 200, 128, 3
    Q, K, V = pack_tensors(N, H, 7200)
    banner("varlen one sample vs rswa_masked_attn")
    out_v, lse_v = run_varlen(Q, K, V, np.array([0, N], np.int32), [L], n, H, CAUSAL)
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
    rs.rswa_masked_attn(Qd, Kd, Vd, out, N, L, n, H, D, rs.RSWA_BF16, CAUSAL, 0.0, lse=lse)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_v), bits(out))
    assert torch.equal(lse_v, lse)


def test_varlen_sample_offset_does_not_change_results():
    """A sample gives the same bits wherever it sits in the pack."""
    n, H = 32, 2
    A = pack_tensors(400, H, 7300)
    lead = pack_tensors(123, H, 7301)
    banner("varlen sample at offset 0 and 123")
    out0, _ = run_varlen(*A, np.array([0, 400], np.int32), [90], n, H, CAUSAL)
    Q, K, V = (np.concatenate([x, y]) for x, y in zip(lead, A))
    out1, _ = run_varlen(Q, K, V, np.array([0, 123, 523], np.int32), [10, 90], n, H, CAUSAL)
    assert np.array_equal(bits(out0), bits(out1)[123:])


def test_varlen_malformed_samples_are_skipped():
    n, H = 8, 2
    cu = np.array([0, 200, 300, 420], np.int32)
    Q, K, V = pack_tensors(420, H, 7400)
    banner("varlen malformed metadata")
    # sample 1: ref_len larger than the sample; sample 2 longer than max_seq_len
    out, _ = run_varlen(Q, K, V, cu, [30, 101, 20], n, H, CAUSAL, max_len=110)
    ref, _ = sample_oracle(Q, K, V, 0, 200, 30, n, CAUSAL)
    # sample 0 is longer than max_seq_len too: skipped as well
    assert torch.isnan(out.float()).all()
    out, _ = run_varlen(Q, K, V, cu, [30, 101, 20], n, H, CAUSAL, max_len=200)
    got = to_f64(out)
    check_close(got[0:200], ref, "bf16", "sample 0")
    assert torch.isnan(out[200:300].float()).all()
    ref2, _ = sample_oracle(Q, K, V, 300, 420, 20, n, CAUSAL)
    check_close(got[300:420], ref2, "bf16", "sample 2")
    # decreasing boundaries (sample 1), and a sample longer than max_seq_len (sample 2)
    out, _ = run_varlen(Q, K, V, np.array([0, 200, 100, 420], np.int32), [30, 10, 20], n, H, CAUSAL,
                        max_len=200)
    check_close(to_f64(out)[0:200], ref, "bf16", "sample 0 beside malformed ones")
    assert torch.isnan(out[200:].float()).all()


# ----------------------------------------------------------------- hand-off
class Prefilled:
    """A cache of B sequences prefilled from one pack, then decoded further."""

    def __init__(self, refs, t0s, n, H, seed, mode=CAUSAL):
        self.refs, self.t0s, self.n, self.H = list(refs), list(t0s), n, H
        lens = [L + t for L, t in zip(refs, t0s)]
        self.cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        self.total = int(self.cu[-1])
        self.Q, self.K, self.V = pack_tensors(self.total, H, seed)
        self.seed = seed
        self.cache = rs.KVCache.allocate(refs, H, D, n, dtype=rs.RSWA_BF16)
        self.cache.k.fill_(float("nan"))
        self.cache.v.fill_(float("nan"))
        self.cache.step.fill_(-5)
        self.out = torch.full((self.total, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((H, self.total), dtype=torch.float32, device="cuda")
        Qd, Kd, Vd = (to_dev(x, "bf16") for x in (self.Q, self.K, self.V))
        rs.rswa_prefill(self.cache.desc, Qd, Kd, Vd, self.out, dev_i32(self.cu), self.total,
                        int(np.diff(self.cu).max()), mode, 0.0, lse=self.lse)
        torch.cuda.synchronize()

    def rows(self, a, b):
        return a[self.cu[b]:self.cu[b + 1]]


def test_prefill_outputs_cache_images_and_steps():
    refs = [40, 0, 64, 100, 7]
    t0s = [5, 30, 16, 0, 50]  # T0 < n, T0 > n (wrap), T0 = n, T0 = 0, several wraps
    n, H = 16, 2
    banner(f"prefill refs={refs} t0s={t0s}")
    pf = Prefilled(refs, t0s, n, H, seed=7500)
    assert pf.cache.step.cpu().tolist() == t0s
    assert rs.rswa_check_device_error(pf.cache.desc) == 0
    got = to_f64(pf.out)
    kbits, vbits = bits(pf.cache.k), bits(pf.cache.v)
    for b, (L, t0) in enumerate(zip(refs, t0s)):
        r0, r1 = pf.cu[b], pf.cu[b + 1]
        ref, _ = sample_oracle(pf.Q, pf.K, pf.V, r0, r1, L, n, CAUSAL)
        check_close(got[r0:r1], ref, "bf16", f"prefill sequence {b}")
        img = orc.ring_image(L, n, t0)  # 1-based position per slot, 0 = never written
        base = pf.cache._host_bases()[b]
        blk_k = kbits[base:base + H * (L + n) * D].reshape(H, L + n, D)
        blk_v = vbits[base:base + H * (L + n) * D].reshape(H, L + n, D)
        for slot, pos in enumerate(img):
            if pos == 0:
                assert np.all(blk_k[:, slot] == 0x7FC0), f"seq {b} slot {slot} written"
                continue
            row = r0 + pos - 1
            assert np.array_equal(blk_k[:, slot], pf.K[row]), f"seq {b} slot {slot} K"
            assert np.array_equal(blk_v[:, slot], pf.V[row]), f"seq {b} slot {slot} V"


def test_prefill_then_decode_continues():
    """After the hand-off, fused decode steps T0+1 .. T0+12 equal the oracle's
    queue model run over the whole sequence (pack outputs, then new tokens)."""
    refs = [48, 96, 20]
    t0s = [3, 40, 16]
    n, H, steps = 16, 2, 12
    banner("prefill then decode")
    pf = Prefilled(refs, t0s, n, H, seed=7600)
    B = len(refs)
    ws = pf.cache.workspace()
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    new = [wl.draw("bf16", 1.0, (steps, B, H, D), 7601, tid) for tid in (0, 1, 2)]
    got = []
    for i in range(steps):
        q, k, v = (to_dev(x[i], "bf16") for x in new)
        rs.rswa_decode_attn(pf.cache.desc, q, out, k, v, 0.0, 0, ws)
        got.append(to_f64(out))
    torch.cuda.synchronize()
    assert rs.rswa_check_device_error(pf.cache.desc) == 0
    assert pf.cache.step.cpu().tolist() == [t + steps for t in t0s]
    got = np.stack(got)  # [steps][B][H][D]
    f = lambda a: wl.to_f64(a, "bf16")
    for b, (L, t0) in enumerate(zip(refs, t0s)):
        Qs, Ks, Vs = (f(pf.rows(x, b)) for x in (pf.Q, pf.K, pf.V))
        for h in range(H):
            q_steps = np.concatenate([Qs[L:, h], f(new[0][:, b, h])])
            out_k = np.concatenate([Ks[L:, h], f(new[1][:, b, h])])
            out_v = np.concatenate([Vs[L:, h], f(new[2][:, b, h])])
            ref = orc.simulate_decode(q_steps, Ks[:L, h], Vs[:L, h], out_k, out_v, L, n, SCALE)
            check_close(got[:, b, h], ref[t0:], "bf16", f"decode after prefill, seq {b} head {h}")
            if t0:
                check_close(to_f64(pf.out)[pf.cu[b] + L:pf.cu[b + 1], h], ref[:t0], "bf16",
                            f"prefill rows = decode steps 1..T0, seq {b} head {h}")


def test_prefill_flags_bad_sequences_and_keeps_the_rest():
    refs = [30, 50]
    n, H = 8, 2
    banner("prefill error flags")
    pf_cu = np.array([0, 20, 80], np.int32)  # sequence 0 has 20 rows < ref_len 30
    Q, K, V = pack_tensors(80, H, 7700)
    cache = rs.KVCache.allocate(refs, H, D, n, dtype=rs.RSWA_BF16)
    cache.k.fill_(float("nan"))
    cache.step.fill_(-5)
    out = torch.full((80, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    rs.rswa_prefill(cache.desc, Qd, Kd, Vd, out, dev_i32(pf_cu), 80, 60, CAUSAL, 0.0)
    torch.cuda.synchronize()
    assert rs.rswa_check_device_error(cache.desc) == rs.RSWA_DEVERR_PACK
    assert cache.step.cpu().tolist() == [-5, 10]
    assert torch.isnan(out[:20].float()).all()
    ref, _ = sample_oracle(Q, K, V, 20, 80, 50, n, CAUSAL)
    check_close(to_f64(out)[20:80], ref, "bf16", "good sequence of a pack with a bad one")



def test_prefill_empty_pack_publishes_steps():
    """No rows at all: sequences without a reference start at step 0; a sequence
    whose reference does not fit its (empty) sample is flagged and keeps its state."""
    n, H = 8, 2
    banner("prefill of an empty pack")
    cache = rs.KVCache.allocate([0, 0, 5], H, D, n, dtype=rs.RSWA_BF16)
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    cache.step.fill_(-5)
    A = torch.zeros((16, H, D), dtype=torch.bfloat16, device="cuda")
    rs.rswa_prefill(cache.desc, A, A, A, A, dev_i32([0, 0, 0, 0]), 0, 0, CAUSAL, 0.0)
    torch.cuda.synchronize()
    assert rs.rswa_check_device_error(cache.desc) == rs.RSWA_DEVERR_PACK
    assert cache.step.cpu().tolist() == [0, 0, -5]
    assert torch.isnan(cache.k.float()).all() and torch.isnan(cache.v.float()).all()


def test_prefill_misaligned_sequence_is_flagged_and_skipped():
    """A sequence whose cache block is not 16-byte aligned is flagged and left
    untouched; its outputs are still computed, and the other sequences are handed
    off as usual (prefix rows seeing the whole reference here)."""
    refs, t0s, n, H = [16, 24, 8], [5, 20, 3], 8, 2
    lens = [L + t for L, t in zip(refs, t0s)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    banner(f"prefill with a misaligned sequence, refs={refs} t0s={t0s}")
    Q, K, V = pack_tensors(total, H, 7800)
    cache = rs.KVCache.allocate(refs, H, D, n, dtype=rs.RSWA_BF16)
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    cache.step.fill_(-5)
    bases = list(cache._host_bases())
    cache.seq_base[1] += 4  # 8 bytes off: not 16-byte aligned
    out = torch.full((total, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    Qd, Kd, Vd = (to_dev(x, "bf16") for x in (Q, K, V))
    rs.rswa_prefill(cache.desc, Qd, Kd, Vd, out, dev_i32(cu), total, max(lens), FULL, 0.0)
    torch.cuda.synchronize()
    assert rs.rswa_check_device_error(cache.desc) == rs.RSWA_DEVERR_ALIGN
    assert cache.step.cpu().tolist() == [t0s[0], -5, t0s[2]]
    got = to_f64(out)
    for b, L in enumerate(refs):
        ref, _ = sample_oracle(Q, K, V, cu[b], cu[b + 1], L, n, FULL)
        check_close(got[cu[b]:cu[b + 1]], ref, "bf16", f"sequence {b} outputs")
    kbits, vbits = bits(cache.k), bits(cache.v)
    size1 = H * (refs[1] + n) * D
    assert np.all(kbits[bases[1]:bases[1] + size1] == 0x7FC0), "misaligned sequence written"
    assert np.all(vbits[bases[1]:bases[1] + size1] == 0x7FC0), "misaligned sequence written"
    for b in (0, 2):
        L, t0 = refs[b], t0s[b]
        blk_k = kbits[bases[b]:bases[b] + H * (L + n) * D].reshape(H, L + n, D)
        blk_v = vbits[bases[b]:bases[b] + H * (L + n) * D].reshape(H, L + n, D)
        for slot, pos in enumerate(orc.ring_image(L, n, t0)):
            if pos == 0:
                assert np.all(blk_k[:, slot] == 0x7FC0), f"seq {b} slot {slot} written"
                continue
            row = cu[b] + pos - 1
            assert np.array_equal(blk_k[:, slot], K[row]), f"seq {b} slot {slot} K"
            assert np.array_equal(blk_v[:, slot], V[row]), f"seq {b} slot {slot} V"

@pytest.mark.slow
@pytest.mark.parametrize("t0", [128, 200])
def test_prefill_40page_full_size(t0):
    """The hand-off at the 40-page decode shape (32 sequences of L_m = 10272 reference rows plus
    T0 outputs, one call): every sequence's K/V block equals the oracle's ring image built from
    the packed rows, bit for bit; every step counter is T0; the output equals the plain packed
    forward of the same pack bit for bit and matches the oracle on sampled rows of two sequences.
    T0 = n is the configuration the benchmark times; T0 = 200 has wrapped the ring."""
    w = wl.FORTY_PAGE
    B, H, L, n = w.batch, w.heads, w.ref_len, w.window
    rows_b = L + t0
    total = B * rows_b
    banner(f"40-page prefill B={B} L_m={L} n={n} T0={t0} rows={total}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.base_seed + t0)
    q, k, v = (torch.randn((total, H, D), device="cuda", generator=gen).to(torch.bfloat16) for _ in range(3))
    cu = torch.arange(0, total + 1, rows_b, dtype=torch.int32, device="cuda")
    cache = rs.KVCache.allocate([L] * B, H, D, n, dtype=rs.RSWA_BF16)
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    cache.step.fill_(-5)
    out = torch.full_like(q, float("nan"))
    rs.rswa_prefill(cache.desc, q, k, v, out, cu, total, rows_b, CAUSAL, 0.0)
    torch.cuda.synchronize()
    assert rs.rswa_check_device_error(cache.desc) == 0
    assert cache.step.cpu().tolist() == [t0] * B

    # cache images, compared on the device: slot s of sequence b holds packed row b*rows_b + pos - 1
    img = orc.ring_image(L, n, t0)
    assert (img > 0).all()  # T0 >= n: every slot written
    src = torch.as_tensor(img - 1, dtype=torch.int64, device="cuda")
    kb, vb = k.view(torch.int16), v.view(torch.int16)
    ck, cv = cache.k.view(torch.int16), cache.v.view(torch.int16)
    for b in range(B):
        rows = src + b * rows_b
        assert torch.equal(cache.block(ck, b), kb[rows].permute(1, 0, 2)), f"sequence {b} K block"
        assert torch.equal(cache.block(cv, b), vb[rows].permute(1, 0, 2)), f"sequence {b} V block"

    # the output is the packed forward's: same bits as the forward call alone
    fwd = torch.full_like(q, float("nan"))
    refs = torch.full((B,), L, dtype=torch.int32, device="cuda")
    rs.rswa_masked_attn_varlen(q, k, v, fwd, cu, refs, B, total, rows_b, n, H, D, rs.RSWA_BF16, CAUSAL, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), fwd.view(torch.int16))
    del fwd

    rng = np.random.default_rng(t0)
    special = [0, 1, L - 1, L, L + 1, L + n - 2, L + n - 1, rows_b - 1]
    local = sorted(set(special + rng.integers(0, rows_b, 8).tolist()))
    for b in (0, B - 1):
        r0 = b * rows_b
        f = lambda a: a[r0:r0 + rows_b].float().cpu().numpy().astype(np.float64)
        Qs, Ks, Vs = f(q), f(k), f(v)
        ref = orc.masked_attention_rows(Qs, Ks, Vs, local, L, n, SCALE, CAUSAL)
        got = to_f64(out[r0:r0 + rows_b])[local]
        ma, rel = check_close(got, ref, "bf16", f"40-page prefill sequence {b} sampled rows")
        print(f"sequence {b}: {len(local)} rows x {H} heads max|d|={ma:.3e} rel={rel:.3e}", flush=True)
