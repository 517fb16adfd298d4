"""bench.py's host-side figures, checked without a GPU.

The roofline and matrix-rate fractions divide measured times into algorithmic
byte and FLOP counts that bench.py computes in closed form. These tests count
the same quantities by brute force from the oracle's visible sets (WeThinkIn
"Unlimited OCR Works：一篇读懂 R-SWA…", 方法展开.3 Eqs. (1)-(2) for the sets,
方法展开.4 Eq. (6) for the decode occupancy), and check that more than one GPU
is refused before anything is imported or touched."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench
import oracle.rswa as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("L_m,n,T", [(10272, 128, 1), (10272, 128, 127), (10272, 128, 128),
                                     (10272, 128, 153), (64, 8, 3), (0, 8, 20), (5, 1, 9)])
def test_decode_bytes_count_every_visible_slot_once(L_m, n, T):
    B, H, d = 3, 2, 128
    # the query of fused step T sees N(T + 1): L_m + min(n, T) slots
    slots = len(orc.visible_positions(L_m, n, T + 1))
    assert slots == orc.cache_size_rswa(L_m, n, T)
    expect = B * H * (slots * 2 * d * 2 + 4 * d * 2)   # K and V rows, then q, out, k_new, v_new
    assert bench.decode_bytes(B, H, d, L_m, n, T) == expect


def test_decode_bytes_of_the_headline_step():
    # 32 sequences x 16 heads x 10400 slots x 512 B + 32 x 16 x 1 KB
    assert bench.decode_bytes(32, 16, 128, 10272, 128, 153) == 2_726_821_888


CASES = [(300, 100, 16), (50, 0, 8), (64, 64, 8), (257, 130, 64), (200, 7, 300), (129, 1, 1)]


@pytest.mark.parametrize("N,L_m,n", CASES)
@pytest.mark.parametrize("mode", [orc.PREFIX_CAUSAL, orc.PREFIX_FULL])
def test_masked_flops_count_the_visible_pairs(N, L_m, n, mode):
    H, d = 3, 128
    pairs = sum(len(orc.masked_visible_columns(i, L_m, n, mode)) for i in range(N))
    assert bench.masked_flops(N, L_m, n, H, d, prefix_full=mode == orc.PREFIX_FULL) == 4 * d * H * pairs


@pytest.mark.parametrize("N,L_m,n", CASES)
@pytest.mark.parametrize("mode", [orc.PREFIX_CAUSAL, orc.PREFIX_FULL])
def test_masked_tile_flops_cover_tight_key_ranges(N, L_m, n, mode):
    """The forward visits, per 128-row query block, whole 64-key blocks over the
    reference keys up to the last one any row of the block sees, and over the
    output keys from the first to the last one any row sees. Count those blocks
    from the visible sets and compare with bench's figure, which is at least the
    algorithmic count."""
    H = 2
    blocks = 0
    for q0 in range(0, N, 128):
        cols = set()
        for i in range(q0, min(N, q0 + 128)):
            cols.update(orc.masked_visible_columns(i, L_m, n, mode))
        pre = [c for c in cols if c < L_m]
        win = [c for c in cols if c >= L_m]
        if pre:
            blocks += -(-(max(pre) + 1) // 64)
        if win:
            blocks += -(-(max(win) + 1 - min(win)) // 64)
    full = mode == orc.PREFIX_FULL
    tile = bench.masked_tile_flops(N, L_m, n, H, prefix_full=full)
    assert tile == blocks * H * 4 * 32 * 32768
    assert tile >= bench.masked_flops(N, L_m, n, H, 128, prefix_full=full)


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
