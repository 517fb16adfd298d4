"""R-SWA oracle: the visible set, attention and KV-cache rules in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
HIP path.

Sources, cited by page title and section:
  [WeThinkIn] "Unlimited OCR Works：一篇读懂 R-SWA 如何把长文档 OCR 从 for-loop
              推向 one-shot" -- section 方法展开.3 (Eqs. (1)-(4)), section
              方法展开.4 (Eqs. (5)-(9)).
  [yhxrc]     news article on Unlimited OCR, section "R-SWA 如何穩住長程解碼？"
              (fixed-capacity output KV buffer of width n on top of the
              reference KV cache).
  [夜雨聆风]  "多模态文档解析开源新进展:Unlimited OCR技术方案" -- section
              "为什么它能”无限”读下去？关键在 KV cache 恒定" (queue of capacity
              m+n; each new token evicts the KV at position m+1).

Notation (the pages'): positions are 1-based; the reference segment P holds
positions 1..L_m (vision tokens + prompt); output token number T (1-based)
sits at position L_m + T. The query q_t predicts output t; it is formed at
position L_m + t - 1, i.e. from output t-1 (or, for t = 1, from the last
reference token). "Decode step T" below means: output T has been appended to
the cache, and the query formed at its position, q_{T+1}, attends.

Readings taken where the pages leave a step open (all listed in the design
notes of the repository):
  * Eq. (2)'s upper bound L_m+t-1 is the query's own position, so the window
    holds the min(n, T) most recent outputs including the query's own token;
    this is the only reading that matches Eq. (6)'s occupancy L_m + min(n, T).
  * Queue eviction is realised as a ring: output T lives in physical slot
    L_m + ((T-1) mod n) (0-based). Attention is order-free, so the visible set
    is unchanged; the slot rule is a layout convention.
  * Rows of the reference prefix in the packed (teacher-forced) form are not
    covered by Eq. (1); PREFIX_CAUSAL (default) lets row i see j <= i,
    PREFIX_FULL lets it see the whole prefix. Prefix rows: parity unpinned by
    the pages (pinned only by this convention).
"""
from __future__ import annotations

import numpy as np

PREFIX_CAUSAL = 0
PREFIX_FULL = 1


# ----------------------------------------------------------------- visible set
def reference_segment(L_m: int) -> list[int]:
    """P = {1, ..., L_m}  ([WeThinkIn] 方法展开.3, Eq. (1))."""
    return list(range(1, L_m + 1))


def decode_window(L_m: int, n: int, t: int) -> list[int]:
    """D_n(t) = { j : max(L_m+1, L_m+t-n) <= j <= L_m+t-1 }  ([WeThinkIn] Eq. (2))."""
    lo = max(L_m + 1, L_m + t - n)
    hi = L_m + t - 1
    return list(range(lo, hi + 1))


def visible_positions(L_m: int, n: int, t: int) -> list[int]:
    """N(t) = P ∪ D_n(t)  ([WeThinkIn] Eq. (1)); 1-based positions, sorted."""
    return sorted(set(reference_segment(L_m)) | set(decode_window(L_m, n, t)))


# ------------------------------------------------------------------- attention
def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query over the given keys.

    alpha_j = exp(q.k_j * scale) / sum_i exp(q.k_i * scale)   ([WeThinkIn] Eq. (3))
    o = sum_j alpha_j v_j                                      ([WeThinkIn] Eq. (4))
    The max score is subtracted before exp (exact in real arithmetic).
    q: [d], K, V: [m][d]; all float64.
    """
    if K.shape[0] == 0:
        raise ValueError("attention over an empty visible set is undefined")
    s = (K @ q) * scale
    w = np.exp(s - s.max())
    alpha = w / w.sum()
    return alpha @ V


def decode_output(q, ref_k, ref_v, out_k, out_v, out_first: int, L_m: int, n: int,
                  T: int, scale: float) -> np.ndarray:
    """Output of decode step T for one (sequence, head).

    After T outputs are in the cache, the query q_{T+1} (formed at output T's
    position) attends over N(T+1). ref_k/ref_v: [L_m][d] (positions 1..L_m);
    out_k/out_v: rows for outputs out_first, out_first+1, ... (at least up to
    T). Raises if a visible output is not supplied.
    """
    t = T + 1
    ks, vs = [], []
    for p in visible_positions(L_m, n, t):
        if p <= L_m:
            ks.append(ref_k[p - 1])
            vs.append(ref_v[p - 1])
        else:
            row = (p - L_m) - out_first
            if row < 0:
                raise ValueError(f"output {p - L_m} is visible but not supplied")
            ks.append(out_k[row])
            vs.append(out_v[row])
    d = np.shape(q)[-1]
    K = np.asarray(ks, dtype=np.float64).reshape(-1, d)
    V = np.asarray(vs, dtype=np.float64).reshape(-1, d)
    return attend(np.asarray(q, dtype=np.float64), K, V, scale)


# -------------------------------------------------------------- KV-cache rules
def cache_size_mha(L_m: int, T: int) -> int:
    """C_MHA(T) = L_m + T  ([WeThinkIn] 方法展开.4, Eq. (5))."""
    return L_m + T


def cache_size_rswa(L_m: int, n: int, T: int) -> int:
    """C_R-SWA(T) = L_m + min(n, T) <= L_m + n  ([WeThinkIn] Eq. (6))."""
    return L_m + min(n, T)


def cache_ratio(L_m: int, n: int, T: int) -> float:
    """rho(T) = C_R-SWA(T) / C_MHA(T)  ([WeThinkIn] Eq. (7))."""
    return cache_size_rswa(L_m, n, T) / cache_size_mha(L_m, T)


class FifoCache:
    """The queue model of the cache, taken literally from [夜雨聆风]: a queue of
    capacity m + n (m = L_m) that starts with the reference positions; each new
    token is appended at the back, and when the queue is full the entry at
    (1-based) queue index m+1 -- the oldest output -- is evicted first.
    Holds 1-based positions."""

    def __init__(self, L_m: int, n: int):
        self.m, self.n = L_m, n
        self.items = list(range(1, L_m + 1))

    def append(self, position: int) -> int | None:
        evicted = None
        if len(self.items) == self.m + self.n:
            evicted = self.items.pop(self.m)  # 1-based index m+1
        self.items.append(position)
        return evicted


def ring_slot(L_m: int, n: int, T: int) -> int:
    """Physical 0-based slot of output T (T >= 1) in a cache of L_m + n slots:
    L_m + ((T - 1) mod n). Layout convention realising the queue of [夜雨聆风]."""
    if T < 1:
        raise ValueError("outputs are numbered from 1")
    return L_m + (T - 1) % n


def ring_image(L_m: int, n: int, T: int) -> np.ndarray:
    """Which 1-based position each of the L_m + n physical slots holds after T
    outputs were appended under the ring rule (0 = never written). Built by
    replaying the appends one by one."""
    img = np.zeros(L_m + n, dtype=np.int64)
    img[:L_m] = np.arange(1, L_m + 1)
    for t_out in range(1, T + 1):
        img[ring_slot(L_m, n, t_out)] = L_m + t_out
    return img


def simulate_decode(q_steps, ref_k, ref_v, out_k, out_v, L_m: int, n: int, scale: float):
    """Run decode steps 1..S through the queue model of [夜雨聆风] and attend over
    the queue's contents (order-free), independently of Eq. (2)'s index
    arithmetic. q_steps/out_k/out_v: [S][d] for outputs 1..S. Returns [S][d]."""
    cache = FifoCache(L_m, n)
    K_all = np.concatenate([ref_k, out_k]).astype(np.float64)
    V_all = np.concatenate([ref_v, out_v]).astype(np.float64)
    outs = []
    for i in range(len(q_steps)):
        cache.append(L_m + i + 1)
        idx = np.asarray(cache.items) - 1
        outs.append(attend(np.asarray(q_steps[i], np.float64), K_all[idx], V_all[idx], scale))
    return np.asarray(outs)


# ------------------------------------------------- packed (teacher-forced) form
def masked_visible_columns(i: int, L_m: int, n: int, prefix_mode: int = PREFIX_CAUSAL) -> list[int]:
    """0-based key columns visible to 0-based row i of a packed sequence.

    Row i >= L_m is output T = i - L_m + 1; its query is q_{T+1} and sees N(T+1)
    ([WeThinkIn] Eqs. (1)-(2)). Rows i < L_m belong to the reference prefix,
    which Eq. (1) does not cover: PREFIX_CAUSAL sees columns 0..i, PREFIX_FULL
    sees 0..L_m-1 (parity unpinned by the pages for these rows).
    """
    if i >= L_m:
        return [p - 1 for p in visible_positions(L_m, n, i - L_m + 2)]
    if prefix_mode == PREFIX_CAUSAL:
        return list(range(i + 1))
    if prefix_mode == PREFIX_FULL:
        return list(range(L_m))
    raise ValueError(prefix_mode)


def masked_attention_rows(Q, K, V, rows, L_m: int, n: int, scale: float,
                          prefix_mode: int = PREFIX_CAUSAL) -> np.ndarray:
    """Packed-sequence attention for the selected rows, all heads.

    Q, K, V: [N][H][d] (any real dtype, promoted to float64). Returns
    [len(rows)][H][d] float64. Each row gathers its own visible columns and
    applies Eqs. (3)-(4) per head.
    """
    H = Q.shape[1]
    out = np.empty((len(rows), H, Q.shape[2]), dtype=np.float64)
    for r, i in enumerate(rows):
        cols = np.asarray(masked_visible_columns(int(i), L_m, n, prefix_mode))
        Kc = np.asarray(K[cols], dtype=np.float64)
        Vc = np.asarray(V[cols], dtype=np.float64)
        qi = np.asarray(Q[i], dtype=np.float64)
        for h in range(H):
            out[r, h] = attend(qi[h], Kc[:, h], Vc[:, h], scale)
    return out


# ------------------------------------------- packed form: log-sum-exp and backward
def masked_logsumexp_rows(Q, K, rows, L_m: int, n: int, scale: float,
                          prefix_mode: int = PREFIX_CAUSAL) -> np.ndarray:
    """Natural-log normaliser of each selected row's softmax (Eq. (3)'s denominator):
    lse_i = log sum_{j visible} exp(scale q_i.k_j). Returns [len(rows)][H] float64."""
    H = Q.shape[1]
    out = np.empty((len(rows), H), dtype=np.float64)
    for r, i in enumerate(rows):
        cols = np.asarray(masked_visible_columns(int(i), L_m, n, prefix_mode))
        Kc = np.asarray(K[cols], dtype=np.float64)
        qi = np.asarray(Q[i], dtype=np.float64)
        for h in range(H):
            s = (Kc[:, h] @ qi[h]) * scale
            mx = s.max()
            out[r, h] = mx + np.log(np.exp(s - mx).sum())
    return out


def masked_attention_backward(Q, K, V, dO, L_m: int, n: int, scale: float,
                              prefix_mode: int = PREFIX_CAUSAL, rows=None):
    """Gradients of the packed forward (Eqs. (3)-(4)) for the loss sum(dO * O).

    For each row i with visible set J(i), p = softmax(scale K_J q_i), o_i = p V_J:
      dV_j += p_j dO_i;   dP_j = dO_i . v_j;   D_i = dO_i . o_i = sum_j p_j dP_j;
      dS_j = p_j (dP_j - D_i);   dQ_i = scale sum_j dS_j k_j;   dK_j += scale dS_j q_i.
    rows: the query rows whose contributions are included (default all). Returns
    (dQ [len(rows)][H][d] for those rows, dK [N][H][d], dV [N][H][d]) in float64;
    dK and dV are exact only when rows covers every row that sees the key.
    """
    N, H, d = Q.shape
    rows = range(N) if rows is None else rows
    dQ = np.zeros((len(rows), H, d))
    dK = np.zeros((N, H, d))
    dV = np.zeros((N, H, d))
    for r, i in enumerate(rows):
        cols = np.asarray(masked_visible_columns(int(i), L_m, n, prefix_mode))
        for h in range(H):
            q = np.asarray(Q[i, h], np.float64)
            Kc = np.asarray(K[cols, h], np.float64)
            Vc = np.asarray(V[cols, h], np.float64)
            g = np.asarray(dO[i, h], np.float64)
            s = (Kc @ q) * scale
            p = np.exp(s - s.max())
            p /= p.sum()
            o = p @ Vc
            dP = Vc @ g
            D = g @ o
            dS = p * (dP - D)
            dQ[r, h] = scale * (dS @ Kc)
            dK[cols, h] += scale * np.outer(dS, q)
            dV[cols, h] += np.outer(p, g)
    return dQ, dK, dV
