"""Pins for the CPU oracle (no GPU).

Each check ties the oracle to something other than itself: visible sets,
queue states and probe outputs worked by hand from the pages (tests/golden/),
torch's scaled_dot_product_attention in float64 for the special cases that
reduce to ordinary causal or banded attention, brute force with a dense mask,
and the literal queue model. The mutation tests at the end plant plausible
mistakes in the oracle (on the CPU) and confirm the pins catch each one.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.rswa as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def _sdpa(Q, K, V, mask, scale):
    """torch's library attention in float64; Q,K,V: [N][d], mask [N][N] bool."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x, np.float64))[None, None] for x in (Q, K, V))
    m = torch.from_numpy(mask)[None, None]
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0, 0].numpy()


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------------ pin suite
# Each pin returns True when the oracle passes it. The suite is run as-is on
# the oracle, and again on planted mistakes (see the mutation tests).

def pin_golden_visible():
    for ln in _rows("visible_sets_Lm3_n2.txt"):
        t, *pos = map(int, ln.split())
        if orc.visible_positions(3, 2, t) != pos:
            return False
    return True


def pin_golden_queue():
    c = orc.FifoCache(3, 2)
    for ln in _rows("fifo_queue_Lm3_n2.txt"):
        T, queue, ev = (s.strip() for s in ln.split("|"))
        evicted = c.append(3 + int(T))
        if c.items != list(map(int, queue.split())):
            return False
        if (evicted is None) != (ev == "-") or (evicted is not None and evicted != int(ev)):
            return False
    return True


def pin_golden_ring():
    for ln in _rows("ring_image_Lm3_n2.txt"):
        T, img = (s.strip() for s in ln.split("|"))
        if list(orc.ring_image(3, 2, int(T))) != list(map(int, img.split())):
            return False
    return True


def pin_visible_equals_queue(cases=((0, 1), (0, 3), (1, 1), (3, 2), (5, 4), (7, 8))):
    """N(T+1) must equal the queue contents after T appends, for every T."""
    for L_m, n in cases:
        c = orc.FifoCache(L_m, n)
        for T in range(0, 3 * n + 3):
            if T:
                c.append(L_m + T)
            if L_m + T == 0:
                continue
            if orc.visible_positions(L_m, n, T + 1) != sorted(c.items):
                return False
            img = orc.ring_image(L_m, n, T)
            if sorted(img[img > 0].tolist()) != sorted(c.items):
                return False
            if len(c.items) != orc.cache_size_rswa(L_m, n, T):
                return False
    return True


def pin_short_decode_is_full_causal():
    """T <= n: R-SWA equals full causal attention over L_m + T (library routine)."""
    L_m, n, d, S = 5, 6, 8, 6
    Kall, Vall, Qall = _rand((L_m + S, d), 1), _rand((L_m + S, d), 2), _rand((L_m + S, d), 3)
    scale = 1 / math.sqrt(d)
    N = L_m + S
    ref = _sdpa(Qall, Kall, Vall, np.tril(np.ones((N, N), bool)), scale)
    for T in range(1, S + 1):
        pos = L_m + T - 1            # 0-based row of output T; its query is q_{T+1}
        o = orc.decode_output(Qall[pos], Kall[:L_m], Vall[:L_m], Kall[L_m:], Vall[L_m:], 1,
                              L_m, n, T, scale)
        if not np.allclose(o, ref[pos], rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_lm0_is_banded_causal():
    """L_m = 0: textbook causal sliding-window attention of width n (library routine + band mask)."""
    n, d, S = 3, 4, 9
    K, V, Q = _rand((S, d), 4), _rand((S, d), 5), _rand((S, d), 6)
    ones = np.ones((S, S), bool)
    band = np.tril(ones) & np.triu(ones, -(n - 1))
    ref = _sdpa(Q, K, V, band, 0.5)
    for T in range(1, S + 1):
        o = orc.decode_output(Q[T - 1], K[:0], V[:0], K, V, 1, 0, n, T, 0.5)
        if not np.allclose(o, ref[T - 1], rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_uniform_probe():
    """q = 0 probe against the hand-worked values in tests/golden/."""
    d = 3
    L_m, n = 3, 2
    S = 5
    ref_v = np.zeros((L_m, d))
    out_v = np.repeat(np.arange(1, S + 1, dtype=float)[:, None], d, axis=1)
    ref_k, out_k = _rand((L_m, d), 7), _rand((S, d), 8)
    for ln in _rows("uniform_probe_Lm3_n2.txt"):
        T, _, _, expect = ln.split()
        o = orc.decode_output(np.zeros(d), ref_k, ref_v, out_k, out_v, 1, L_m, n, int(T), 0.125)
        if not np.allclose(o, float(expect), rtol=0, atol=1e-14):
            return False
    return True


def pin_masked_brute_force():
    """Packed form vs a dense boolean mask built from band operations (library routine)."""
    N, L_m, n, H, d = 23, 7, 4, 2, 5
    Q, K, V = _rand((N, H, d), 9), _rand((N, H, d), 10), _rand((N, H, d), 11)
    ones = np.ones((N, N), bool)
    col_is_ref = np.zeros((N, N), bool)
    col_is_ref[:, :L_m] = True
    row_is_ref = np.zeros((N, N), bool)
    row_is_ref[:L_m, :] = True
    for mode in (orc.PREFIX_CAUSAL, orc.PREFIX_FULL):
        causal = np.tril(ones)
        mask = causal & (col_is_ref | np.triu(ones, -(n - 1)))
        if mode == orc.PREFIX_FULL:
            mask = np.where(row_is_ref, col_is_ref, mask)
        got = orc.masked_attention_rows(Q, K, V, range(N), L_m, n, 0.3, mode)
        for h in range(H):
            ref = _sdpa(Q[:, h], K[:, h], V[:, h], mask, 0.3)
            if not np.allclose(got[:, h], ref, rtol=1e-12, atol=1e-12):
                return False
    return True


def pin_queue_simulation_equals_eq2():
    """Decode through the literal queue model == Eq. (2) gather, every step (incl. wrap)."""
    L_m, n, d, S = 4, 3, 6, 11
    rk, rv = _rand((L_m, d), 12), _rand((L_m, d), 13)
    ok, ov, q = _rand((S, d), 14), _rand((S, d), 15), _rand((S, d), 16)
    sim = orc.simulate_decode(q, rk, rv, ok, ov, L_m, n, 0.4)
    for T in range(1, S + 1):
        o = orc.decode_output(q[T - 1], rk, rv, ok, ov, 1, L_m, n, T, 0.4)
        if not np.allclose(o, sim[T - 1], rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_masked_rows_equal_decode():
    """Teacher-forced rows at positions >= L_m equal the decode output of the same step."""
    N, L_m, n, H, d = 20, 6, 3, 2, 4
    Q, K, V = _rand((N, H, d), 17), _rand((N, H, d), 18), _rand((N, H, d), 19)
    rows = list(range(L_m, N))
    got = orc.masked_attention_rows(Q, K, V, rows, L_m, n, 0.5)
    for r, i in enumerate(rows):
        T = i - L_m + 1
        for h in range(H):
            o = orc.decode_output(Q[i, h], K[:L_m, h], V[:L_m, h], K[L_m:, h], V[L_m:, h], 1,
                                  L_m, n, T, 0.5)
            if not np.allclose(o, got[r, h], rtol=1e-12, atol=1e-12):
                return False
    return True


PINS = [pin_golden_visible, pin_golden_queue, pin_golden_ring, pin_visible_equals_queue,
        pin_short_decode_is_full_causal, pin_lm0_is_banded_causal, pin_uniform_probe,
        pin_masked_brute_force, pin_queue_simulation_equals_eq2, pin_masked_rows_equal_decode]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_passes_pin(pin):
    assert pin()


# ----------------------------------------------------------- closed forms, special cases
def test_occupancy_eq6_and_eq5():
    """Queue length is L_m + min(n, T) (Eq. 6); a queue that never evicts grows as L_m + T (Eq. 5)."""
    for L_m, n in [(64, 8), (288, 128), (0, 5)]:
        c = orc.FifoCache(L_m, n)
        big = orc.FifoCache(L_m, 10 ** 9)
        for T in range(1, 3 * n):
            c.append(L_m + T)
            big.append(L_m + T)
            assert len(c.items) == orc.cache_size_rswa(L_m, n, T) <= L_m + n
            assert len(big.items) == orc.cache_size_mha(L_m, T)


def test_cache_ratio_eq7_to_eq9():
    L_m, n = 40 * 256 + 32, 128
    assert orc.cache_ratio(L_m, n, 6144) == pytest.approx(10400 / 16416, rel=1e-15)
    for T in (1, 50, 128):           # T <= n: nothing is evicted, ratio 1
        assert orc.cache_ratio(L_m, n, T) == 1.0
    for T in (129, 1000, 10 ** 6):   # Eq. (8) once T >= n
        assert orc.cache_ratio(L_m, n, T) == pytest.approx((L_m + n) / (L_m + T), rel=1e-15)
    # Eq. (9): rho * T / (L_m + n) -> 1 as T grows
    assert orc.cache_ratio(L_m, n, 10 ** 9) * 10 ** 9 / (L_m + n) == pytest.approx(1.0, rel=1e-4)


def test_large_window_is_full_attention_every_step():
    """n >= total outputs: every step equals full causal attention (Eq. 5 cache)."""
    L_m, n, d, S = 3, 50, 4, 12
    K, V, Q = _rand((L_m + S, d), 20), _rand((L_m + S, d), 21), _rand((L_m + S, d), 22)
    N = L_m + S
    ref = _sdpa(Q, K, V, np.tril(np.ones((N, N), bool)), 0.7)
    for T in range(1, S + 1):
        o = orc.decode_output(Q[L_m + T - 1], K[:L_m], V[:L_m], K[L_m:], V[L_m:], 1, L_m, n, T, 0.7)
        np.testing.assert_allclose(o, ref[L_m + T - 1], rtol=1e-12, atol=1e-12)


def test_single_key_and_constant_values():
    d = 5
    v = _rand((1, d), 23)
    o = orc.decode_output(_rand(d, 24), _rand((1, d), 25), v, np.zeros((0, d)), np.zeros((0, d)), 1,
                          1, 4, 0, 0.3)
    np.testing.assert_array_equal(o, v[0])       # one visible key: o = v exactly
    L_m, n, S = 6, 3, 8
    const = np.full(d, 1.25)
    o = orc.decode_output(_rand(d, 26), _rand((L_m, d), 27), np.tile(const, (L_m, 1)),
                          _rand((S, d), 28), np.tile(const, (S, 1)), 1, L_m, n, S, 0.3)
    np.testing.assert_allclose(o, const, rtol=0, atol=1e-15)


def test_scale_folds_into_query():
    d = 6
    q, K, V = _rand(d, 29), _rand((9, d), 30), _rand((9, d), 31)
    np.testing.assert_allclose(orc.attend(q * 3.0, K, V, 0.1), orc.attend(q, K, V, 0.3), rtol=1e-13)


def test_needle_probe_marks_window_edge():
    """A key aligned with q at the evicted output T-n gets no weight; at T-n+1 it dominates."""
    L_m, n, d = 4, 3, 8
    T = 9
    q = np.zeros(d)
    q[0] = 1.0
    ref_k = np.zeros((L_m, d))
    ref_v = np.zeros((L_m, d))
    out_k = np.zeros((T, d))
    out_v = np.zeros((T, d))
    for needle, expect_big in ((T - n, False), (T - n + 1, True)):
        ok = out_k.copy()
        ov = out_v.copy()
        ok[needle - 1, 0] = 60.0
        ov[needle - 1, 1] = 1.0
        o = orc.decode_output(q, ref_k, ref_v, ok, ov, 1, L_m, n, T, 1.0)
        assert (o[1] > 0.99) == expect_big
        if not expect_big:
            assert o[1] == 0.0


def test_empty_visible_set_raises():
    with pytest.raises(ValueError):
        orc.decode_output(np.zeros(4), np.zeros((0, 4)), np.zeros((0, 4)), np.zeros((0, 4)),
                          np.zeros((0, 4)), 1, 0, 4, 0, 1.0)


def test_ring_slot_rule():
    assert [orc.ring_slot(10, 4, T) for T in range(1, 10)] == [10, 11, 12, 13, 10, 11, 12, 13, 10]
    with pytest.raises(ValueError):
        orc.ring_slot(10, 4, 0)


# ------------------------------------------------------------ planted mistakes
def _window_too_narrow(L_m, n, t):
    return list(range(max(L_m + 1, L_m + t - n + 1), L_m + t))


def _window_too_wide(L_m, n, t):
    return list(range(max(L_m + 1, L_m + t - n - 1), L_m + t))


def _window_without_own_token(L_m, n, t):
    return list(range(max(L_m + 1, L_m + t - n - 1), L_m + t - 1))


def _window_shifted(L_m, n, t):
    return list(range(max(L_m + 1, L_m + t - n + 1), L_m + t + 1))


def _attend_no_scale(q, K, V, scale):
    s = K @ q
    w = np.exp(s - s.max())
    return (w / w.sum()) @ V


def _attend_k_v_swapped(q, K, V, scale):
    s = (V @ q) * scale
    w = np.exp(s - s.max())
    return (w / w.sum()) @ K


def _attend_unnormalised(q, K, V, scale):
    s = (K @ q) * scale
    return np.exp(s - s.max()) @ V


def _evict_newest(self, position):
    if len(self.items) == self.m + self.n:
        self.items.pop(-1)
    self.items.append(position)


def _ring_slot_off_by_one(L_m, n, T):
    return L_m + T % n


_true_columns = orc.masked_visible_columns


def _columns_without_diagonal(i, L_m, n, prefix_mode=orc.PREFIX_CAUSAL):
    return [j for j in _true_columns(i, L_m, n, prefix_mode) if j != i]


def _causal_prefix_sees_whole_prefix(i, L_m, n, prefix_mode=orc.PREFIX_CAUSAL):
    return list(range(L_m)) if i < L_m else _true_columns(i, L_m, n, prefix_mode)


def _output_rows_one_step_early(i, L_m, n, prefix_mode=orc.PREFIX_CAUSAL):
    if i < L_m:
        return _true_columns(i, L_m, n, prefix_mode)
    return [p - 1 for p in orc.visible_positions(L_m, n, i - L_m + 1)]


MUTANTS = [
    ("decode_window", _window_too_narrow),
    ("decode_window", _window_too_wide),
    ("decode_window", _window_without_own_token),
    ("decode_window", _window_shifted),
    ("attend", _attend_no_scale),
    ("attend", _attend_k_v_swapped),
    ("attend", _attend_unnormalised),
    ("ring_slot", _ring_slot_off_by_one),
    ("masked_visible_columns", _columns_without_diagonal),
    ("masked_visible_columns", _causal_prefix_sees_whole_prefix),
    ("masked_visible_columns", _output_rows_one_step_early),
]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f.__name__ for _, f in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, fn):
    monkeypatch.setattr(orc, name, fn)
    failed = []
    for pin in PINS:
        try:
            ok = pin()
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {fn.__name__}"


def test_pins_catch_wrong_eviction(monkeypatch):
    monkeypatch.setattr(orc.FifoCache, "append", _evict_newest)
    assert not pin_golden_queue()
    assert not pin_queue_simulation_equals_eq2()


def test_oracle_package_exports():
    for name in ("visible_positions", "decode_output", "masked_attention_rows", "FifoCache",
                 "ring_image", "cache_ratio"):
        assert hasattr(oracle, name)


# ------------------------------------------------------ packed backward and normaliser
def _torch_masked_grads(Q, K, V, dO, L_m, n, scale, mode):
    """torch autograd through its own float64 attention with a band-built mask."""
    N, H, d = Q.shape
    ones = np.ones((N, N), bool)
    col_is_ref = np.zeros((N, N), bool)
    col_is_ref[:, :L_m] = True
    mask = np.tril(ones) & (col_is_ref | np.triu(ones, -(n - 1)))
    if mode == orc.PREFIX_FULL:
        row_is_ref = np.zeros((N, N), bool)
        row_is_ref[:L_m, :] = True
        mask = np.where(row_is_ref, col_is_ref, mask)
    t = [torch.tensor(x.transpose(1, 0, 2), dtype=torch.float64, requires_grad=True) for x in (Q, K, V)]
    out = F.scaled_dot_product_attention(t[0][None], t[1][None], t[2][None],
                                         attn_mask=torch.from_numpy(mask)[None, None], scale=scale)[0]
    out.backward(torch.tensor(dO.transpose(1, 0, 2)))
    lse = torch.logsumexp((t[0] @ t[1].transpose(1, 2)) * scale
                          + torch.where(torch.from_numpy(mask), 0.0, -torch.inf), dim=-1)
    return [x.grad.numpy().transpose(1, 0, 2) for x in t], lse.detach().numpy().T


@pytest.mark.parametrize("mode", [orc.PREFIX_CAUSAL, orc.PREFIX_FULL])
def test_backward_matches_torch_autograd(mode):
    N, L_m, n, H, d = 19, 6, 4, 2, 5
    Q, K, V, dO = (_rand((N, H, d), s) for s in (40, 41, 42, 43))
    dQ, dK, dV = orc.masked_attention_backward(Q, K, V, dO, L_m, n, 0.6, mode)
    (tq, tk, tv), lse = _torch_masked_grads(Q, K, V, dO, L_m, n, 0.6, mode)
    np.testing.assert_allclose(dQ, tq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, tk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, tv, rtol=1e-10, atol=1e-12)
    got = orc.masked_logsumexp_rows(Q, K, range(N), L_m, n, 0.6, mode)
    np.testing.assert_allclose(got, lse, rtol=1e-12, atol=1e-12)


def test_backward_column_sums():
    """sum_j dV_j = sum_i dO_i (rows of the softmax sum to 1); sum_j dK_j = 0."""
    N, L_m, n, H, d = 23, 7, 3, 2, 4
    Q, K, V, dO = (_rand((N, H, d), s) for s in (44, 45, 46, 47))
    _, dK, dV = orc.masked_attention_backward(Q, K, V, dO, L_m, n, 0.5)
    np.testing.assert_allclose(dV.sum(0), dO.sum(0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dK.sum(0), 0.0, atol=1e-12)


def test_backward_row_subset_dq():
    N, L_m, n, H, d = 17, 5, 3, 1, 4
    Q, K, V, dO = (_rand((N, H, d), s) for s in (48, 49, 50, 51))
    full, _, _ = orc.masked_attention_backward(Q, K, V, dO, L_m, n, 0.7)
    part, _, _ = orc.masked_attention_backward(Q, K, V, dO, L_m, n, 0.7, rows=[3, 11, 16])
    np.testing.assert_allclose(part, full[[3, 11, 16]], rtol=1e-14)
