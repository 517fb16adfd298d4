"""Helpers for the GPU parity tests: host<->device transfer of the generator's
storage arrays, the tolerance rule, and a decode driver over the C ABI."""
from __future__ import annotations

import numpy as np
import torch

import oracle.pool as opool
import oracle.rswa as orc
import reference_sliding_window_amd as rs
import workloads as wl

# bf16: max|diff| <= 2e-2 and ||diff||_2 / ||ref||_2 <= 1e-2; fp32: both 1e-5. The
# relative bound holds over the whole array AND for every output vector on its
# own (the last axis: one (sequence, head) of a decode step, one (row, head) of
# the packed form), so one wrong head cannot hide among hundreds of good ones.
TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-5, 1e-5)}
DTYPE_CODE = {"bf16": rs.RSWA_BF16, "fp32": rs.RSWA_FP32}


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a device tensor (uint16 for bf16, uint32 for fp32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def storage_bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def _vector_rel(d: np.ndarray, ref: np.ndarray, floor: float = 0.0):
    """Per-vector ||d|| / max(||ref||, floor) over the last axis; (worst, its index).
    A vector whose reference and floor are both zero (e.g. the exact zero gradient of
    a row that sees one key) has no relative error and is left to the max-abs bound."""
    dn = np.linalg.norm(d.reshape(-1, d.shape[-1]), axis=1)
    rn = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    den = np.maximum(rn, floor)
    rel = np.where(den > 0, dn / np.where(den > 0, den, 1.0), 0.0)
    i = int(np.argmax(rel))
    return float(rel[i]), np.unravel_index(i, ref.shape[:-1]) if ref.ndim > 1 else ()


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    """Returns (max|diff|, worst per-vector relative L2); asserts the rule above."""
    atol, rtol = TOL[dtype]
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if got.size == 0:
        return 0.0, 0.0
    d = got - ref
    maxabs = float(np.abs(d).max())
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    vrel, where = _vector_rel(d, ref)
    elem_out = int((np.abs(d) > atol + rtol * np.abs(ref)).sum())   # reported only
    msg = (f"{what}: max|d|={maxabs:.3e} (<= {atol}) rel={rel:.3e} (<= {rtol}) "
           f"worst vector rel={vrel:.3e} at {tuple(int(x) for x in where)} (<= {rtol}); "
           f"{elem_out} of {d.size} elements outside |d| <= atol + rtol|ref|")
    assert maxabs <= atol and rel <= rtol and vrel <= rtol, msg
    return maxabs, vrel


def check_grad(got: np.ndarray, ref: np.ndarray, what: str):
    """Gradient rule: max|diff| <= 2e-2 max(1, max|ref|) and relative L2 <= 1e-2, over
    the whole tensor and over each head (axis -2 of [rows][H][d]) on its own, so one
    wrong head cannot hide among the others. Not per row: the backward forms
    D_i = dO_i . O_i from the forward's bf16 output (up to 2^-8 relative), and for a row
    that sees a few keys dS = P (dP - D) turns that into a few per cent of the
    row's own dQ where dP is close to D. Returns (max|diff|, worst per-head
    relative L2)."""
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if ref.size == 0:
        return 0.0, 0.0
    d = got - ref
    scale = max(1.0, float(np.abs(ref).max()))
    maxabs = float(np.abs(d).max())
    rn = np.linalg.norm(ref)
    rel = 0.0 if rn == 0.0 else float(np.linalg.norm(d) / rn)   # e.g. one visible key: dS = 0
    hrel, worst_h = rel, None
    if ref.ndim >= 2:
        dh = np.linalg.norm(np.moveaxis(d, -2, 0).reshape(d.shape[-2], -1), axis=1)
        rh = np.linalg.norm(np.moveaxis(ref, -2, 0).reshape(ref.shape[-2], -1), axis=1)
        per = np.where(rh > 0, dh / np.where(rh > 0, rh, 1.0), 0.0)   # zero heads: max-abs only
        worst_h = int(np.argmax(per))
        hrel = float(per[worst_h])
    assert maxabs <= 2e-2 * scale and rel <= 1e-2 and hrel <= 1e-2, (
        f"{what}: max|d|={maxabs:.3e} (<= {2e-2 * scale:.3e}) rel={rel:.3e} (<= 1e-2) "
        f"worst head rel={hrel:.3e} (head {worst_h}) (<= 1e-2)")
    return maxabs, hrel


def score_range_qkv(N: int, H: int = 4, d: int = 128, seed: int = 20261204):
    """Packed Q, K, V ([N][H][d], bf16 storage bits) whose scores leave the unit range,
    per head: head 0 grows along the sequence (key j scaled by 1 + j/60, queries by 2:
    about -105 .. 107 at N = 700, d = 128, so later blocks keep exceeding the running
    max), head 1 is strongly negative (q = -5u, k = u, plus unit noise: about -84 .. -46),
    head 2 strongly positive (q = 8u: about 68 .. 131), head 3 ordinary N(0, 1). The
    construction only scales and mixes seeded Gaussian draws."""
    g = lambda i, shape: wl.to_f64(wl.draw("bf16", 1.0, shape, seed, i), "bf16")
    Q, K, V = g(0, (N, H, d)), g(1, (N, H, d)), g(2, (N, H, d))
    u = g(3, (d,))
    j = np.arange(N, dtype=np.float64)[:, None]
    K[:, 0] *= 1.0 + j / 60.0
    Q[:, 0] *= 2.0
    K[:, 1] = u + K[:, 1]
    Q[:, 1] = -5.0 * u + Q[:, 1]
    K[:, 2] = u + K[:, 2]
    Q[:, 2] = 8.0 * u + Q[:, 2]
    return tuple(wl.f32_to_bf16_bits(x.astype(np.float32)) for x in (Q, K, V))


class DecodeRun:
    """Drives a batch-synchronous decode workload through the C ABI."""

    def __init__(self, w: wl.DecodeWorkload, window: int | None = None, num_splits: int = 0,
                 ref=None):
        self.w = w
        self.n = window or w.window
        self.dtype = w.dtype
        self.num_splits = num_splits
        self.cache = rs.KVCache.allocate([w.ref_len] * w.batch, w.heads, w.head_dim, self.n,
                                         dtype=DTYPE_CODE[w.dtype])
        self.kref, self.vref = ref if ref is not None else wl.ref_kv_all(w)
        kd = to_dev(self.kref.reshape(-1), w.dtype)
        vd = to_dev(self.vref.reshape(-1), w.dtype)
        per = w.heads * w.ref_len * w.head_dim
        ref_base = torch.arange(w.batch, dtype=torch.int64, device="cuda") * per
        rs.rswa_cache_init(self.cache.desc, kd, vd, ref_base)
        torch.cuda.synchronize()
        del kd, vd
        self.ws = self.cache.workspace(num_splits)
        self.out = torch.empty((w.batch, w.heads, w.head_dim), dtype=self.cache.k.dtype, device="cuda")
        self.T = 0

    def run(self, T_end: int, keep=(), chunk: int = 256, fused: bool = True, steps=None) -> dict:
        """Advance to step T_end; returns {T: output (float64 numpy)} for T in keep.
        steps: optional pre-drawn (q, k, v), each [S][B][H][d] for outputs 1..S >= T_end."""
        outs = {}
        keep = set(keep)
        while self.T < T_end:
            first = self.T + 1
            last = min(T_end, first + chunk - 1)
            if steps is not None:
                q, k, v = (x[first - 1:last] for x in steps)
            else:
                q, k, v = wl.steps_qkv(self.w, first, last)
            qd, kd, vd = (to_dev(x, self.dtype) for x in (q, k, v))
            for i in range(last - first + 1):
                if fused:
                    rs.rswa_decode_attn(self.cache.desc, qd[i], self.out, kd[i], vd[i], 0.0,
                                        self.num_splits, self.ws)
                else:
                    rs.rswa_append_kv(self.cache.desc, kd[i], vd[i])
                    rs.rswa_decode_attn(self.cache.desc, qd[i], self.out, None, None, 0.0,
                                        self.num_splits, self.ws)
                self.T += 1
                if self.T in keep:
                    outs[self.T] = self.out.clone()
        torch.cuda.synchronize()
        return {T: to_f64(o) for T, o in outs.items()}

    def oracle(self, T: int, bh=None, steps=None) -> np.ndarray:
        """Oracle outputs of step T for the listed (b, h) pairs (default all): [len][d].
        steps: optional pre-drawn step inputs for outputs 1..>=T (as from steps_qkv)."""
        w, n = self.w, self.n
        first = max(1, T - n + 1)
        if steps is not None:
            q, k, v = (x[first - 1:T] for x in steps)
        else:
            q, k, v = wl.steps_qkv(w, first, T)
        if bh is None:
            bh = [(b, h) for b in range(w.batch) for h in range(w.heads)]
        res = []
        for b, h in bh:
            res.append(orc.decode_output(
                wl.to_f64(q[-1, b, h], w.dtype),
                wl.to_f64(self.kref[b, h], w.dtype), wl.to_f64(self.vref[b, h], w.dtype),
                wl.to_f64(k[:, b, h], w.dtype), wl.to_f64(v[:, b, h], w.dtype),
                first, w.ref_len, n, T, w.scale))
        return np.asarray(res)

    def check_cache_image(self, bs=None, heads=None, ref_rows=None):
        """Bit-exact check of the cache against the ring rule after self.T outputs."""
        w, n, T = self.w, self.n, self.T
        first = max(1, T - n + 1)
        _, k, v = wl.steps_qkv(self.w, first, T) if T >= 1 else (None, None, None)
        bs = range(w.batch) if bs is None else bs
        heads = range(w.heads) if heads is None else heads
        L = w.ref_len
        for b in bs:
            kb = bits(self.cache.block(self.cache.k, b))
            vb = bits(self.cache.block(self.cache.v, b))
            for h in heads:
                rows = range(L) if ref_rows is None else ref_rows
                rows = np.asarray(list(rows), dtype=np.int64)
                assert np.array_equal(kb[h, rows], storage_bits(self.kref[b, h][rows])), (b, h, "ref K")
                assert np.array_equal(vb[h, rows], storage_bits(self.vref[b, h][rows])), (b, h, "ref V")
                for t_out in range(first, T + 1):
                    slot = orc.ring_slot(L, n, t_out)
                    assert np.array_equal(kb[h, slot], storage_bits(k[t_out - first, b, h])), (b, h, t_out)
                    assert np.array_equal(vb[h, slot], storage_bits(v[t_out - first, b, h])), (b, h, t_out)


def shared_decode_inputs(w: wl.DecodeWorkload, arrays: "opool.SharedArrays", S: int, ref=None):
    """Draws the workload's reference K/V and the inputs of outputs 1..S into shared
    memory ("kref", "vref" [B][H][L_m][d]; "q", "k", "v" [S][B][H][d], storage form)
    for the oracle's worker pool; returns (kref, vref, (q, k, v)) as views."""
    kref, vref = ref if ref is not None else wl.ref_kv_all(w)
    kref, vref = arrays.put("kref", kref), arrays.put("vref", vref)
    dt = kref.dtype
    shape = (S, w.batch, w.heads, w.head_dim)
    q, k, v = (arrays.new(name, shape, dt) for name in ("q", "k", "v"))
    for c0 in range(0, S, 512):
        c1 = min(S, c0 + 512)
        for dst, src in zip((q, k, v), wl.steps_qkv(w, c0 + 1, c1)):
            dst[c0:c1] = src
    return kref, vref, (q, k, v)


def oracle_decode_all_pairs(w: wl.DecodeWorkload, n: int, arrays: "opool.SharedArrays", checks):
    """Oracle outputs of every (sequence, head) at each step in checks, computed on
    all host cores from the shared inputs: {T: [B][H][d]}."""
    tasks = [(w.dtype, w.ref_len, n, w.scale, b, list(range(w.heads)), list(checks))
             for b in range(w.batch)]
    per_seq = opool.pool_map(opool.decode_sequence_job, tasks, arrays, progress="decode (sequence) tasks")
    return {T: np.stack([r[T] for r in per_seq]) for T in checks}
