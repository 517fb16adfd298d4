"""Python binding of librswa, the HIP/gfx950 R-SWA library (include/rswa.h).

Argument marshalling only: every step of the attention path runs in the
library's HIP kernels. torch supplies device memory and streams. The functions
carry the C names; each takes torch tensors (or a CacheDesc) and returns the
library's status, raising RswaError for a non-zero status.

There is no CPU fallback: if librswa.so is missing this module raises at
first use.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librswa.so")

RSWA_OK = 0
RSWA_ERR_NULL = -1
RSWA_ERR_SHAPE = -2
RSWA_ERR_UNSUPPORTED = -3
RSWA_ERR_ALIGN = -4
RSWA_ERR_CAPACITY = -5
RSWA_ERR_WORKSPACE = -6
RSWA_ERR_STATE = -7
RSWA_ERR_HIP = -8

RSWA_BF16 = 0
RSWA_FP32 = 1
RSWA_PREFIX_CAUSAL = 0
RSWA_PREFIX_FULL = 1

RSWA_DEVERR_REF_LEN = 1
RSWA_DEVERR_STEP = 2
RSWA_DEVERR_EMPTY = 4
RSWA_DEVERR_ALIGN = 8
RSWA_DEVERR_PACK = 16

EXPORTED = ("rswa_abi_version", "rswa_status_str", "rswa_cache_init", "rswa_append_kv",
            "rswa_workspace_size", "rswa_decode_workspace_size", "rswa_decode_attn",
            "rswa_decode_attn_noalloc", "rswa_masked_attn",
            "rswa_masked_attn_varlen", "rswa_prefill", "rswa_masked_bwd_workspace_size",
            "rswa_masked_attn_bwd", "rswa_masked_bwd_varlen_workspace_size",
            "rswa_masked_attn_bwd_varlen", "rswa_decode_graph_create", "rswa_decode_graph_launch",
            "rswa_decode_graph_destroy", "rswa_probe_stream_read", "rswa_probe_mfma",
            "rswa_probe_cu", "rswa_device_facts", "rswa_check_device_error")


class RswaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status} ({_lib().rswa_status_str(status).decode()})")
        self.status = status


class CacheDesc(ctypes.Structure):
    """Mirror of rswa_cache_t."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("max_ref_len", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("seq_base", ctypes.c_void_p),
        ("ref_len", ctypes.c_void_p),
        ("step", ctypes.c_void_p),
        ("error", ctypes.c_void_p),
        ("arrive", ctypes.c_void_p),
    ]


_LIB = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (run reference_sliding_window_amd/build.py)")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        D = ctypes.POINTER(CacheDesc)
        sig = {
            "rswa_abi_version": (I32, []),
            "rswa_status_str": (ctypes.c_char_p, [I32]),
            "rswa_cache_init": (I32, [D, P, P, P, P]),
            "rswa_append_kv": (I32, [D, P, P, P, P]),
            "rswa_workspace_size": (SZ, [I32, I32, I32, I32]),
            "rswa_decode_workspace_size": (SZ, [D, I32]),
            "rswa_decode_attn": (I32, [D, P, P, P, P, F, I32, P, SZ, P]),
            "rswa_decode_attn_noalloc": (I32, [D, P, P, P, P, F, I32, P]),
            "rswa_masked_attn": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F, P]),
            "rswa_masked_attn_varlen": (I32, [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                              I32, F, P]),
            "rswa_prefill": (I32, [D, P, P, P, P, P, P, I32, I32, I32, F, P]),
            "rswa_masked_bwd_workspace_size": (SZ, [I32, I32, I32, I32]),
            "rswa_masked_attn_bwd": (I32, [P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                           I32, F, I32, P, SZ, P]),
            "rswa_masked_bwd_varlen_workspace_size": (SZ, [I32, I32]),
            "rswa_masked_attn_bwd_varlen": (I32, [P, P, P, P, P, P, P, P, P, P, P, I32, I32, I32, I32,
                                                  I32, I32, I32, I32, F, P, SZ, P]),
            "rswa_decode_graph_create": (I32, [D, I32, P, P, P, P, F, I32, P, SZ, ctypes.POINTER(P)]),
            "rswa_decode_graph_launch": (I32, [P, P]),
            "rswa_decode_graph_destroy": (I32, [P]),
            "rswa_probe_stream_read": (I32, [P, SZ, P, I32, P]),
            "rswa_probe_mfma": (I32, [P, I32, I32, P]),
            "rswa_probe_cu": (I32, [P, I32, I32, I32, P]),
            "rswa_device_facts": (I32, [I32, ctypes.POINTER(ctypes.c_int64), I32]),
            "rswa_check_device_error": (I32, [D, ctypes.POINTER(I32), P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _LIB = lib
    return _LIB


def library() -> ctypes.CDLL:
    """The loaded librswa (raises ImportError if it is not built)."""
    return _lib()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to librswa must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> int:
    if status != RSWA_OK:
        raise RswaError(status, where)
    return status


# ------------------------------------------------------------- C entry points
def rswa_abi_version() -> int:
    return _lib().rswa_abi_version()


def rswa_status_str(status: int) -> str:
    return _lib().rswa_status_str(status).decode()


def rswa_cache_init(desc: CacheDesc, k_ref, v_ref, ref_base, stream=None, check=True) -> int:
    st = _lib().rswa_cache_init(ctypes.byref(desc), _ptr(k_ref), _ptr(v_ref), _ptr(ref_base),
                                _stream(stream))
    return _check(st, "rswa_cache_init") if check else st


def rswa_append_kv(desc: CacheDesc, k_new, v_new, active=None, stream=None, check=True) -> int:
    st = _lib().rswa_append_kv(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(active),
                               _stream(stream))
    return _check(st, "rswa_append_kv") if check else st


def rswa_workspace_size(batch: int, num_heads: int, head_dim: int, max_len: int) -> int:
    return _lib().rswa_workspace_size(batch, num_heads, head_dim, max_len)


def rswa_decode_workspace_size(desc: CacheDesc, num_splits: int = 0) -> int:
    return _lib().rswa_decode_workspace_size(ctypes.byref(desc), num_splits)


def rswa_decode_attn(desc: CacheDesc, q, out, k_new=None, v_new=None, scale: float = 0.0,
                     num_splits: int = 0, workspace=None, workspace_bytes: int | None = None,
                     stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    st = _lib().rswa_decode_attn(ctypes.byref(desc), _ptr(q), _ptr(out), _ptr(k_new), _ptr(v_new),
                                 float(scale), int(num_splits), _ptr(workspace), int(workspace_bytes),
                                 _stream(stream))
    return _check(st, "rswa_decode_attn") if check else st


def rswa_decode_attn_noalloc(desc: CacheDesc, q, out, k_new=None, v_new=None, scale: float = 0.0,
                             num_splits: int = 0, stream=None, check=True) -> int:
    st = _lib().rswa_decode_attn_noalloc(ctypes.byref(desc), _ptr(q), _ptr(out), _ptr(k_new), _ptr(v_new),
                                         float(scale), int(num_splits), _stream(stream))
    return _check(st, "rswa_decode_attn_noalloc") if check else st


def rswa_masked_attn(q, k, v, out, seq_len: int, ref_len: int, window: int, num_heads: int,
                     head_dim: int, dtype: int = RSWA_BF16, prefix_mode: int = RSWA_PREFIX_CAUSAL,
                     scale: float = 0.0, stream=None, check=True, lse=None) -> int:
    st = _lib().rswa_masked_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), seq_len, ref_len,
                                 window, num_heads, head_dim, dtype, prefix_mode, float(scale),
                                 _stream(stream))
    return _check(st, "rswa_masked_attn") if check else st


def rswa_masked_attn_varlen(q, k, v, out, cu_seqlens, ref_lens, num_seqs: int, total_tokens: int,
                            max_seq_len: int, window: int, num_heads: int, head_dim: int,
                            dtype: int = RSWA_BF16, prefix_mode: int = RSWA_PREFIX_CAUSAL,
                            scale: float = 0.0, stream=None, check=True, lse=None) -> int:
    st = _lib().rswa_masked_attn_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
                                        _ptr(ref_lens), num_seqs, total_tokens, max_seq_len, window,
                                        num_heads, head_dim, dtype, prefix_mode, float(scale),
                                        _stream(stream))
    return _check(st, "rswa_masked_attn_varlen") if check else st


def rswa_prefill(desc: CacheDesc, q, k, v, out, cu_seqlens, total_tokens: int, max_seq_len: int,
                 prefix_mode: int = RSWA_PREFIX_CAUSAL, scale: float = 0.0, stream=None, check=True,
                 lse=None) -> int:
    st = _lib().rswa_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                             _ptr(cu_seqlens), total_tokens, max_seq_len, prefix_mode, float(scale),
                             _stream(stream))
    return _check(st, "rswa_prefill") if check else st


def rswa_masked_bwd_workspace_size(seq_len: int, ref_len: int, num_heads: int,
                                   num_parts: int = 0) -> int:
    return _lib().rswa_masked_bwd_workspace_size(seq_len, ref_len, num_heads, num_parts)


def rswa_masked_attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, seq_len: int, ref_len: int,
                         window: int, num_heads: int, head_dim: int, dtype: int = RSWA_BF16,
                         prefix_mode: int = RSWA_PREFIX_CAUSAL, scale: float = 0.0,
                         workspace=None, workspace_bytes: int | None = None, num_parts: int = 0,
                         stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    st = _lib().rswa_masked_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                     _ptr(dq), _ptr(dk), _ptr(dv), seq_len, ref_len, window,
                                     num_heads, head_dim, dtype, prefix_mode, float(scale),
                                     int(num_parts), _ptr(workspace), int(workspace_bytes),
                                     _stream(stream))
    return _check(st, "rswa_masked_attn_bwd") if check else st


def rswa_masked_bwd_varlen_workspace_size(total_tokens: int, num_heads: int) -> int:
    return _lib().rswa_masked_bwd_varlen_workspace_size(total_tokens, num_heads)


def rswa_masked_attn_bwd_varlen(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens, ref_lens,
                                num_seqs: int, total_tokens: int, max_seq_len: int, window: int,
                                num_heads: int, head_dim: int, dtype: int = RSWA_BF16,
                                prefix_mode: int = RSWA_PREFIX_CAUSAL, scale: float = 0.0,
                                workspace=None, workspace_bytes: int | None = None, stream=None,
                                check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    st = _lib().rswa_masked_attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens),
                                            _ptr(ref_lens), num_seqs, total_tokens, max_seq_len,
                                            window, num_heads, head_dim, dtype, prefix_mode,
                                            float(scale), _ptr(workspace), int(workspace_bytes),
                                            _stream(stream))
    return _check(st, "rswa_masked_attn_bwd_varlen") if check else st


def _ptr_array(items):
    if items is None:
        return None
    arr = (ctypes.c_void_p * len(items))(*[_ptr(t) for t in items])
    return ctypes.cast(arr, ctypes.c_void_p), arr


def rswa_decode_graph_create(descs, q, out, k_new=None, v_new=None, scale: float = 0.0,
                             num_splits: int = 0, workspace=None, workspace_bytes: int | None = None,
                             check=True):
    """Returns (status, handle). descs: sequence of CacheDesc, one per layer; q, out,
    k_new, v_new: sequences of per-layer device tensors (k_new/v_new may be None)."""
    L = len(descs)
    arr = (CacheDesc * L)(*descs)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    keep = []
    ptrs = []
    for items in (q, out, k_new, v_new):
        if items is None:
            ptrs.append(None)
        else:
            p, a = _ptr_array(items)
            keep.append(a)
            ptrs.append(p)
    handle = ctypes.c_void_p(None)
    st = _lib().rswa_decode_graph_create(arr, L, *ptrs, float(scale), int(num_splits), _ptr(workspace),
                                         int(workspace_bytes), ctypes.byref(handle))
    if check:
        _check(st, "rswa_decode_graph_create")
    return st, handle.value


def rswa_decode_graph_launch(handle, stream=None, check=True) -> int:
    st = _lib().rswa_decode_graph_launch(handle, _stream(stream))
    return _check(st, "rswa_decode_graph_launch") if check else st


def rswa_decode_graph_destroy(handle, check=True) -> int:
    st = _lib().rswa_decode_graph_destroy(handle)
    return _check(st, "rswa_decode_graph_destroy") if check else st


def rswa_probe_stream_read(buf, nbytes: int, sink, workgroups: int = 0, stream=None, check=True) -> int:
    st = _lib().rswa_probe_stream_read(_ptr(buf), int(nbytes), _ptr(sink), int(workgroups), _stream(stream))
    return _check(st, "rswa_probe_stream_read") if check else st


def rswa_probe_mfma(sink, workgroups: int = 0, iters: int = 4096, stream=None, check=True) -> int:
    st = _lib().rswa_probe_mfma(_ptr(sink), int(workgroups), int(iters), _stream(stream))
    return _check(st, "rswa_probe_mfma") if check else st


RSWA_PROBE_LDS_B128, RSWA_PROBE_LDS_TR16, RSWA_PROBE_EXP, RSWA_PROBE_FMA = 0, 1, 2, 3


def rswa_probe_cu(out, workgroups: int = 0, iters: int = 1024, kind: int = RSWA_PROBE_LDS_B128, stream=None,
                  check=True) -> int:
    st = _lib().rswa_probe_cu(_ptr(out), int(workgroups), int(iters), int(kind), _stream(stream))
    return _check(st, "rswa_probe_cu") if check else st


DEVICE_FACTS = ("compute_units", "lds_bytes_per_cu", "l2_bytes", "clock_khz", "mem_clock_khz",
                "mem_bus_bits", "global_mem_bytes", "wave_size")


def rswa_device_facts(device: int = 0) -> dict:
    """The HIP runtime's facts of one device, keyed by DEVICE_FACTS."""
    out = (ctypes.c_int64 * len(DEVICE_FACTS))()
    _check(_lib().rswa_device_facts(int(device), out, len(DEVICE_FACTS)), "rswa_device_facts")
    return dict(zip(DEVICE_FACTS, (int(x) for x in out)))


def rswa_check_device_error(desc: CacheDesc, stream=None) -> int:
    """Returns the device error bits (0 = none) and clears them."""
    flags = ctypes.c_int32(0)
    st = _lib().rswa_check_device_error(ctypes.byref(desc), ctypes.byref(flags), _stream(stream))
    if st not in (RSWA_OK, RSWA_ERR_STATE):
        raise RswaError(st, "rswa_check_device_error")
    return flags.value


# ------------------------------------------------------- caller-side plumbing
_TORCH_DTYPE = {RSWA_BF16: torch.bfloat16, RSWA_FP32: torch.float32}


@dataclass
class KVCache:
    """Device memory for an R-SWA cache, allocated with torch, plus its descriptor.

    Pools are flat; sequence b's block starts at seq_base[b] and is laid out
    [H][ref_len[b] + window][head_dim] (the ABI's layout).
    """
    desc: CacheDesc
    k: torch.Tensor
    v: torch.Tensor
    seq_base: torch.Tensor
    ref_len: torch.Tensor
    step: torch.Tensor
    error: torch.Tensor
    arrive: torch.Tensor
    ref_lens: list
    window: int
    heads: int
    head_dim: int

    @staticmethod
    def allocate(ref_lens, heads: int, head_dim: int, window: int, dtype: int = RSWA_BF16,
                 device="cuda") -> "KVCache":
        ref_lens = [int(x) for x in ref_lens]
        align = 16 // (2 if dtype == RSWA_BF16 else 4)
        bases, off = [], 0
        for L in ref_lens:
            bases.append(off)
            off += heads * (L + window) * head_dim
            off = (off + align - 1) // align * align
        tdt = _TORCH_DTYPE[dtype]
        # zero-filled: slots no call has written yet (a window not yet full,
        # alignment gaps) hold zeros, not whatever the allocator handed back, so
        # two caches driven alike compare equal bit for bit and checkpoints of
        # the pools are reproducible
        k = torch.zeros(max(off, align), dtype=tdt, device=device)
        v = torch.zeros(max(off, align), dtype=tdt, device=device)
        seq_base = torch.tensor(bases, dtype=torch.int64, device=device)
        ref_len = torch.tensor(ref_lens, dtype=torch.int32, device=device)
        step = torch.zeros(len(ref_lens), dtype=torch.int32, device=device)
        error = torch.zeros(4, dtype=torch.int32, device=device)
        arrive = torch.zeros(len(ref_lens), dtype=torch.int32, device=device)  # zero before first use
        desc = CacheDesc(len(ref_lens), heads, head_dim, window, max(ref_lens), dtype,
                         k.data_ptr(), v.data_ptr(), seq_base.data_ptr(), ref_len.data_ptr(),
                         step.data_ptr(), error.data_ptr(), arrive.data_ptr())
        return KVCache(desc, k, v, seq_base, ref_len, step, error, arrive, ref_lens, window, heads, head_dim)

    def block(self, pool: torch.Tensor, b: int) -> torch.Tensor:
        """View of sequence b's [H][L_m + n][d] block of a pool."""
        L = self.ref_lens[b]
        start = int(self.seq_base[b].item()) if self.seq_base.device.type == "cpu" else None
        if start is None:
            start = self._host_bases()[b]
        size = self.heads * (L + self.window) * self.head_dim
        return pool[start:start + size].view(self.heads, L + self.window, self.head_dim)

    def _host_bases(self):
        if not hasattr(self, "_hb"):
            self._hb = self.seq_base.cpu().tolist()
        return self._hb

    def workspace(self, num_splits: int = 0) -> torch.Tensor:
        nbytes = rswa_decode_workspace_size(self.desc, num_splits)
        if nbytes == 0:
            raise RswaError(RSWA_ERR_SHAPE, "rswa_decode_workspace_size")
        return torch.zeros(nbytes, dtype=torch.uint8, device=self.k.device)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
