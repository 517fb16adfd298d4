"""Helpers for the GPU parity tests: host<->device transfer of the generator's
storage arrays, the tolerance rule, and a decode driver over the C ABI."""
from __future__ import annotations

import numpy as np
import torch

import oracle.rswa as orc
import reference_sliding_window_amd as rs
import workloads as wl

# bf16: max|diff| <= 2e-2 and ||diff||_2 / ||ref||_2 <= 1e-2; fp32: both 1e-5.
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


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    atol, rtol = TOL[dtype]
    d = got - ref
    maxabs = float(np.abs(d).max()) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert maxabs <= atol and rel <= rtol, f"{what}: max|d|={maxabs:.3e} (<= {atol}) rel={rel:.3e} (<= {rtol})"
    return maxabs, rel


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

    def run(self, T_end: int, keep=(), chunk: int = 256, fused: bool = True) -> dict:
        """Advance to step T_end; returns {T: output (float64 numpy)} for T in keep."""
        outs = {}
        keep = set(keep)
        while self.T < T_end:
            first = self.T + 1
            last = min(T_end, first + chunk - 1)
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
