"""Seeded synthetic inputs for R-SWA decode and masked attention.

This module holds the workload shapes and the random-number recipe that both
the GPU path's callers (tests, bench) and the CPU oracle draw their inputs
from. It contains no attention arithmetic: no softmax, no visibility rule, no
slot or eviction rule. It only draws Gaussian numbers from counter-style seeds
and rounds them to the storage dtype.

Workload shapes follow the pages' workloads:
  * one 1024x1024 page is 256 vision tokens (WeThinkIn "Unlimited OCR Works：
    一篇读懂 R-SWA…", section 方法展开.2, DeepEncoder paragraph);
  * the reference segment is vision tokens + prompt (same page, section
    方法展开.3, Eq. (1)); the prompt length is not stated there and is taken as
    32 tokens;
  * the output window defaults to n = 128 (same page, 核心导读);
  * up to 6144 output tokens (same page, 实验与证据.5, Table 4 prose);
  * training packs samples of 2..50 pages into 32K tokens (same page,
    实验与证据.1).

Seeding: every tensor is drawn from numpy's PCG64 seeded with
SeedSequence([base, tensor_id, *index]), so any one step, sequence or tensor
can be regenerated on its own without replaying the others.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# tensor ids used in seed words
TID_Q, TID_K, TID_V, TID_KREF, TID_VREF, TID_RAGGED, TID_DOUT, TID_PACK = 0, 1, 2, 3, 4, 5, 6, 7

PAGE_TOKENS = 256   # vision tokens per 1024x1024 page
PROMPT_TOKENS = 32  # prompt length (not stated on the pages; fixed here)


@dataclass(frozen=True)
class DecodeWorkload:
    """A batch-synchronous decode run: B sequences, same L_m, T steps."""
    name: str
    batch: int
    heads: int
    head_dim: int
    ref_len: int
    window: int
    steps: int
    dtype: str            # "fp32" or "bf16"
    sigma_q: float
    sigma_kv: float
    base_seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass(frozen=True)
class MaskedWorkload:
    """One packed sequence of N tokens with a reference prefix of L_m."""
    name: str
    seq_len: int
    heads: int
    head_dim: int
    ref_len: int
    window: int
    dtype: str
    sigma: float
    base_seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass(frozen=True)
class RaggedWorkload:
    """Many sequences, each with its own page count and decode position."""
    name: str
    batch: int
    heads: int
    head_dim: int
    window: int
    max_pages: int
    max_steps: int
    dtype: str
    sigma: float
    base_seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


TINY_FP32 = DecodeWorkload("tiny-decode-fp32", batch=1, heads=2, head_dim=64, ref_len=64,
                           window=8, steps=40, dtype="fp32", sigma_q=1.0, sigma_kv=1.0,
                           base_seed=20260001)
ONE_PAGE = DecodeWorkload("one-page-decode-bf16", batch=1, heads=16, head_dim=128,
                          ref_len=1 * PAGE_TOKENS + PROMPT_TOKENS, window=128, steps=2048,
                          dtype="bf16", sigma_q=1.0, sigma_kv=1.0, base_seed=20260002)
FORTY_PAGE = DecodeWorkload("40-page-decode-bf16", batch=32, heads=16, head_dim=128,
                            ref_len=40 * PAGE_TOKENS + PROMPT_TOKENS, window=128, steps=6144,
                            dtype="bf16", sigma_q=1.0, sigma_kv=0.5, base_seed=20260003)
PACKED_32K = MaskedWorkload("packed-32k-masked-bf16", seq_len=32768, heads=16, head_dim=128,
                            ref_len=16 * PAGE_TOKENS + PROMPT_TOKENS, window=128, dtype="bf16",
                            sigma=1.0, base_seed=20260004)
RAGGED_64 = RaggedWorkload("ragged-64-decode-bf16", batch=64, heads=16, head_dim=128, window=128,
                           max_pages=50, max_steps=8192, dtype="bf16", sigma=1.0,
                           base_seed=20260005)

WORKLOADS = {1: TINY_FP32, 2: ONE_PAGE, 3: FORTY_PAGE, 4: PACKED_32K, 5: RAGGED_64}


# ---------------------------------------------------------------- dtype helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Inputs here are finite Gaussian draws; NaN/Inf are not produced.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(w) for w in words])))


def draw(dtype: str, sigma: float, shape, *words: int) -> np.ndarray:
    """One seeded Gaussian tensor in storage form.

    dtype "fp32" -> float32 array; "bf16" -> uint16 array of bf16 bit patterns.
    """
    x = _rng(*words).standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype == "fp32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form -> exact float64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ------------------------------------------------------- decode (batch-synchronous)
def ref_kv(w: DecodeWorkload, b: int):
    """Reference K and V of sequence b, each [H][L_m][d] in storage form."""
    shape = (w.heads, w.ref_len, w.head_dim)
    k = draw(w.dtype, w.sigma_kv, shape, w.base_seed, TID_KREF, b)
    v = draw(w.dtype, w.sigma_kv, shape, w.base_seed, TID_VREF, b)
    return k, v


def ref_kv_all(w: DecodeWorkload, threads: int = 16):
    """Reference K and V for all sequences, each [B][H][L_m][d]."""
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda b: ref_kv(w, b), range(w.batch)))
    return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


def step_qkv(w: DecodeWorkload, t_out: int):
    """q, k_new, v_new of decode step t_out (1-based output index), each [B][H][d].

    k_new/v_new are the K/V of output token t_out; q is the query formed at
    that token's position.
    """
    shape = (w.batch, w.heads, w.head_dim)
    q = draw(w.dtype, w.sigma_q, shape, w.base_seed, TID_Q, t_out)
    k = draw(w.dtype, w.sigma_kv, shape, w.base_seed, TID_K, t_out)
    v = draw(w.dtype, w.sigma_kv, shape, w.base_seed, TID_V, t_out)
    return q, k, v


def steps_qkv(w: DecodeWorkload, first: int, last: int, threads: int = 16):
    """Stacked step inputs for outputs first..last inclusive: each [S][B][H][d]."""
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda t: step_qkv(w, t), range(first, last + 1)))
    return tuple(np.stack([p[i] for p in parts]) for i in range(3))


# ------------------------------------------------------------------ masked / packed
def packed_qkv(w: MaskedWorkload, threads: int = 3):
    """Q, K, V of the packed sequence, each [N][H][d] in storage form."""
    shape = (w.seq_len, w.heads, w.head_dim)
    with ThreadPoolExecutor(threads) as ex:
        return tuple(ex.map(lambda tid: draw(w.dtype, w.sigma, shape, w.base_seed, tid),
                            (TID_Q, TID_K, TID_V)))


def packed_dout(w: MaskedWorkload, sigma: float = 1.0):
    """Upstream gradient dO of the packed forward's output, [N][H][d] in storage
    form, N(0, sigma^2) (the loss is sum(dO * O))."""
    return draw(w.dtype, sigma, (w.seq_len, w.heads, w.head_dim), w.base_seed, TID_DOUT)


def varlen_pack_layout(total_tokens: int, base_seed: int, pages=(2, 16), outputs=(256, 2048),
                       page_tokens: int = 256, prompt_tokens: int = 32):
    """Sample boundaries of a pack of several documents, filled front to back.

    Each sample is a reference segment of L = page_tokens * pages + prompt_tokens
    (pages ~ U{pages}) followed by T ~ U{outputs} output tokens. When the next
    sample does not fit, it is shrunk to the rows left (fewer pages, then fewer
    outputs, at least one output); rows too few for a two-page sample stay
    outside every sample. Returns (cu_seqlens [S+1], ref_lens [S]) as int32.
    """
    g = _rng(base_seed, TID_PACK)
    cu, refs, used = [0], [], 0
    min_len = page_tokens * pages[0] + prompt_tokens + 1
    while total_tokens - used >= min_len:
        left = total_tokens - used
        p = int(g.integers(pages[0], pages[1] + 1))
        t = int(g.integers(outputs[0], outputs[1] + 1))
        p = min(p, (left - prompt_tokens - 1) // page_tokens)
        L = page_tokens * p + prompt_tokens
        t = min(t, left - L)
        used += L + t
        cu.append(used)
        refs.append(L)
    return np.asarray(cu, np.int32), np.asarray(refs, np.int32)


# --------------------------------------------------------------------------- ragged
@dataclass
class RaggedDraw:
    pages: np.ndarray        # [B] int
    ref_len: np.ndarray      # [B] int  (pages*256 + 32)
    t_now: np.ndarray        # [B] int  output index of the fused step (1-based)
    extra: dict = field(default_factory=dict)


def ragged_lengths(w: RaggedWorkload) -> RaggedDraw:
    g = _rng(w.base_seed, TID_RAGGED)
    pages = g.integers(1, w.max_pages + 1, size=w.batch)
    t_now = g.integers(1, w.max_steps + 1, size=w.batch)
    return RaggedDraw(pages=pages, ref_len=pages * PAGE_TOKENS + PROMPT_TOKENS, t_now=t_now)


def ragged_ref_kv(w: RaggedWorkload, b: int, ref_len: int):
    shape = (w.heads, int(ref_len), w.head_dim)
    return (draw(w.dtype, w.sigma, shape, w.base_seed, TID_KREF, b),
            draw(w.dtype, w.sigma, shape, w.base_seed, TID_VREF, b))


def ragged_token_kv(w: RaggedWorkload, b: int, t_out: int):
    """K and V of output token t_out (1-based) of sequence b, each [H][d]."""
    shape = (w.heads, w.head_dim)
    return (draw(w.dtype, w.sigma, shape, w.base_seed, TID_K, b, t_out),
            draw(w.dtype, w.sigma, shape, w.base_seed, TID_V, b, t_out))


def ragged_query(w: RaggedWorkload, b: int, t_out: int):
    return draw(w.dtype, w.sigma, (w.heads, w.head_dim), w.base_seed, TID_Q, b, t_out)
