"""C ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments on the host with the
documented status before anything is enqueued (no HIP call is reached)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import reference_sliding_window_amd as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rswa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(rs.LIB_PATH), reason="librswa.so not built")

A = 0x7f0000000000  # a fake, 16-byte aligned device address; never dereferenced here


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"RSWA_API\s+[\w\s\*]*?\b(rswa_\w+)\s*\(", text)))


def test_header_declares_the_four_calls_and_helpers():
    names = header_functions()
    for n in ("rswa_cache_init", "rswa_append_kv", "rswa_decode_attn", "rswa_masked_attn"):
        assert n in names
    assert set(names) == set(rs.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = rs.library()
    for name in header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", rs.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (rswa_\w+)", out))
    assert set(header_functions()) <= exported


def test_abi_version_and_status_strings():
    ver = int(re.search(r"#define RSWA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert rs.rswa_abi_version() == ver
    for code in range(0, -9, -1):
        assert rs.rswa_status_str(code) not in ("", "unknown status")
    assert rs.rswa_status_str(-99) == "unknown status"


def good_desc(**kw):
    d = dict(batch=2, num_heads=4, head_dim=128, window=8, max_ref_len=100, dtype=rs.RSWA_BF16,
             k=A, v=A + 0x100000, seq_base=A + 0x200000, ref_len=A + 0x300000, step=A + 0x400000,
             error=A + 0x500000)
    d.update(kw)
    return rs.CacheDesc(**d)


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, rs.RSWA_ERR_UNSUPPORTED),
    ("head_dim", 0, rs.RSWA_ERR_UNSUPPORTED),
    ("dtype", 7, rs.RSWA_ERR_UNSUPPORTED),
    ("batch", 0, rs.RSWA_ERR_SHAPE),
    ("num_heads", -1, rs.RSWA_ERR_SHAPE),
    ("window", 0, rs.RSWA_ERR_SHAPE),
    ("max_ref_len", -5, rs.RSWA_ERR_SHAPE),
    ("max_ref_len", 2 ** 31 - 4, rs.RSWA_ERR_CAPACITY),
    ("k", None, rs.RSWA_ERR_NULL),
    ("step", None, rs.RSWA_ERR_NULL),
    ("error", None, rs.RSWA_ERR_NULL),
    ("v", A + 8, rs.RSWA_ERR_ALIGN),
    ("arrive", A + 2, rs.RSWA_ERR_ALIGN),
])
def test_bad_descriptor_rejected_by_every_cache_call(field, value, status):
    desc = good_desc(**{field: value})
    assert rs.rswa_append_kv(desc, A, A, check=False) == status
    assert rs.rswa_cache_init(desc, A, A, A, check=False) == status
    assert rs.rswa_decode_attn(desc, A, A, workspace=A, workspace_bytes=1 << 30, check=False) == status
    assert rs.rswa_decode_workspace_size(desc, 0) == 0


def test_decode_argument_checks():
    desc = good_desc()
    ws = rs.rswa_decode_workspace_size(desc, 0)
    assert ws > 0
    call = lambda **kw: rs.rswa_decode_attn(desc, **{**dict(q=A, out=A, workspace=A, workspace_bytes=ws), **kw},
                                             check=False)
    assert call(q=None) == rs.RSWA_ERR_NULL
    assert call(out=None) == rs.RSWA_ERR_NULL
    assert call(k_new=A) == rs.RSWA_ERR_NULL          # k_new without v_new
    assert call(v_new=A) == rs.RSWA_ERR_NULL
    assert call(q=A + 4) == rs.RSWA_ERR_ALIGN
    assert call(k_new=A + 2, v_new=A) == rs.RSWA_ERR_ALIGN
    assert call(scale=math.nan) == rs.RSWA_ERR_SHAPE
    assert call(scale=math.inf) == rs.RSWA_ERR_SHAPE
    assert call(num_splits=-1) == rs.RSWA_ERR_SHAPE
    assert call(workspace=None, workspace_bytes=0) == rs.RSWA_ERR_WORKSPACE
    assert call(workspace_bytes=ws - 1) == rs.RSWA_ERR_WORKSPACE
    assert call(workspace=A + 4) == rs.RSWA_ERR_ALIGN


def test_workspace_grows_with_splits():
    desc = good_desc(max_ref_len=10272, window=128, batch=32, num_heads=16)
    s1 = rs.rswa_decode_workspace_size(desc, 1)
    s16 = rs.rswa_decode_workspace_size(desc, 16)
    assert 0 < s1 < s16
    # 16 splits: 32*16*16 partial states of 128 floats plus (max, sum) pairs
    assert s16 >= 32 * 16 * 16 * (128 + 2) * 4


def test_library_split_choice():
    """One chunk per (sequence, head) -- one launch -- for a batch that fills the GPU with
    sequences of at most 12288 slots; otherwise a flat work list for large steps and
    short per-(sequence, head) chunks for small ones."""
    ws = lambda s, **kw: rs.rswa_decode_workspace_size(good_desc(**kw), s)
    forty = dict(batch=32, num_heads=16, max_ref_len=10272, window=128)
    assert ws(0, **forty) == ws(1, **forty)
    one_page = dict(batch=1, num_heads=16, max_ref_len=288, window=128)
    assert ws(0, **one_page) > ws(1, **one_page)
    # a large step (>= 4M slots of capacity) not decoded in one launch: the flat work
    # list over 512 workgroups, partial states for 512 + B*H (sequence, head) pieces
    r256 = lambda x: (x + 255) // 256 * 256
    flat = lambda B, H: r256((512 + B * H) * 128 * 4) + r256((512 + B * H) * 8) + r256(B * 4) + r256((B + 1) * 8)
    ragged = dict(batch=64, num_heads=16, max_ref_len=12832, window=128)
    assert ws(0, **ragged) == flat(64, 16) < ws(7, **ragged)
    contrast = dict(batch=32, num_heads=16, max_ref_len=10272, window=6144)
    assert ws(0, **contrast) == flat(32, 16)
    few = dict(batch=2, num_heads=16, max_ref_len=10272, window=128)   # 333K slots: chunks
    assert ws(0, **few) > ws(8, **few) and ws(0, **few) != flat(2, 16)
    # small steps keep per-(sequence, head) chunks: one page, 16 heads -> 7 chunks of 64 slots
    assert ws(0, **one_page) == ws(7, **one_page)


def test_append_and_init_argument_checks():
    desc = good_desc()
    assert rs.rswa_append_kv(desc, None, A, check=False) == rs.RSWA_ERR_NULL
    assert rs.rswa_append_kv(desc, A, A + 8, check=False) == rs.RSWA_ERR_ALIGN
    assert rs.rswa_cache_init(desc, A, A, None, check=False) == rs.RSWA_ERR_NULL
    assert rs.rswa_cache_init(desc, A + 2, A, A, check=False) == rs.RSWA_ERR_ALIGN


def test_masked_argument_checks():
    m = lambda **kw: rs.rswa_masked_attn(**{**dict(q=A, k=A, v=A, out=A, seq_len=300, ref_len=40, window=8,
                                                    num_heads=2, head_dim=128), **kw}, check=False)
    assert m(q=None) == rs.RSWA_ERR_NULL
    assert m(ref_len=301) == rs.RSWA_ERR_SHAPE
    assert m(seq_len=-1) == rs.RSWA_ERR_SHAPE
    assert m(window=0) == rs.RSWA_ERR_SHAPE
    assert m(num_heads=0) == rs.RSWA_ERR_SHAPE
    assert m(head_dim=64) == rs.RSWA_ERR_UNSUPPORTED
    assert m(dtype=rs.RSWA_FP32) == rs.RSWA_ERR_UNSUPPORTED
    assert m(prefix_mode=3) == rs.RSWA_ERR_UNSUPPORTED
    assert m(k=A + 2) == rs.RSWA_ERR_ALIGN
    assert m(scale=math.nan) == rs.RSWA_ERR_SHAPE
    assert m(lse=A + 2) == rs.RSWA_ERR_ALIGN
    assert m(seq_len=2 ** 20, ref_len=0, num_heads=16) == rs.RSWA_ERR_CAPACITY
    assert m(seq_len=2, ref_len=0, num_heads=2 ** 16) == rs.RSWA_ERR_CAPACITY   # 24-bit row products
    assert m(seq_len=0, ref_len=0) == rs.RSWA_OK   # nothing to do, nothing enqueued


def test_varlen_argument_checks():
    base = dict(q=A, k=A, v=A, out=A, cu_seqlens=A, ref_lens=A + 64, num_seqs=3, total_tokens=900,
                max_seq_len=400, window=8, num_heads=2, head_dim=128)
    m = lambda **kw: rs.rswa_masked_attn_varlen(**{**base, **kw}, check=False)
    for name in ("q", "k", "v", "out", "cu_seqlens", "ref_lens"):
        assert m(**{name: None}) == rs.RSWA_ERR_NULL, name
    assert m(num_seqs=-1) == rs.RSWA_ERR_SHAPE
    assert m(total_tokens=-1) == rs.RSWA_ERR_SHAPE
    assert m(max_seq_len=-1) == rs.RSWA_ERR_SHAPE
    assert m(window=0) == rs.RSWA_ERR_SHAPE
    assert m(num_heads=0) == rs.RSWA_ERR_SHAPE
    assert m(head_dim=64) == rs.RSWA_ERR_UNSUPPORTED
    assert m(dtype=rs.RSWA_FP32) == rs.RSWA_ERR_UNSUPPORTED
    assert m(prefix_mode=9) == rs.RSWA_ERR_UNSUPPORTED
    assert m(total_tokens=2 ** 20, num_heads=16) == rs.RSWA_ERR_CAPACITY
    assert m(total_tokens=2, max_seq_len=2, num_heads=2 ** 16) == rs.RSWA_ERR_CAPACITY
    assert m(q=A + 8) == rs.RSWA_ERR_ALIGN
    assert m(cu_seqlens=A + 2) == rs.RSWA_ERR_ALIGN
    assert m(lse=A + 1) == rs.RSWA_ERR_ALIGN
    assert m(scale=math.nan) == rs.RSWA_ERR_SHAPE
    assert m(num_seqs=0) == rs.RSWA_OK            # nothing to do, nothing enqueued
    assert m(total_tokens=0) == rs.RSWA_OK
    assert m(max_seq_len=0) == rs.RSWA_OK


def test_prefill_argument_checks():
    desc = good_desc()
    p = lambda **kw: rs.rswa_prefill(**{**dict(desc=desc, q=A, k=A, v=A, out=A, cu_seqlens=A, total_tokens=500,
                                              max_seq_len=300), **kw}, check=False)
    for name in ("q", "k", "v", "out", "cu_seqlens"):
        assert p(**{name: None}) == rs.RSWA_ERR_NULL, name
    assert p(desc=good_desc(head_dim=64)) == rs.RSWA_ERR_UNSUPPORTED
    assert p(desc=good_desc(dtype=rs.RSWA_FP32)) == rs.RSWA_ERR_UNSUPPORTED
    assert p(desc=good_desc(k=None)) == rs.RSWA_ERR_NULL
    assert p(desc=good_desc(batch=0)) == rs.RSWA_ERR_SHAPE
    assert p(total_tokens=-1) == rs.RSWA_ERR_SHAPE
    assert p(max_seq_len=-3) == rs.RSWA_ERR_SHAPE
    assert p(prefix_mode=5) == rs.RSWA_ERR_UNSUPPORTED
    assert p(total_tokens=2 ** 22) == rs.RSWA_ERR_CAPACITY
    assert p(desc=good_desc(batch=1, num_heads=2 ** 16), total_tokens=2, max_seq_len=2) == rs.RSWA_ERR_CAPACITY
    assert p(out=A + 4) == rs.RSWA_ERR_ALIGN
    assert p(cu_seqlens=A + 1) == rs.RSWA_ERR_ALIGN
    assert p(scale=math.inf) == rs.RSWA_ERR_SHAPE


def test_decode_graph_argument_checks():
    """Validation happens before any stream or capture is created."""
    desc = good_desc()
    ws = rs.rswa_decode_workspace_size(desc, 0)
    g = lambda **kw: rs.rswa_decode_graph_create(**{**dict(descs=[desc, desc], q=[A, A], out=[A, A],
                                                           workspace=A, workspace_bytes=ws), **kw},
                                                 check=False)[0]
    assert g(q=[A, None]) == rs.RSWA_ERR_NULL
    assert g(out=[None, A]) == rs.RSWA_ERR_NULL
    assert g(k_new=[A, A]) == rs.RSWA_ERR_NULL            # k_new without v_new
    assert g(k_new=[A, None], v_new=[A, A]) == rs.RSWA_ERR_NULL
    assert g(q=[A, A + 8]) == rs.RSWA_ERR_ALIGN
    assert g(descs=[desc, good_desc(head_dim=96)]) == rs.RSWA_ERR_UNSUPPORTED
    assert g(workspace_bytes=ws - 1) == rs.RSWA_ERR_WORKSPACE
    assert g(workspace=None, workspace_bytes=0) == rs.RSWA_ERR_WORKSPACE
    assert g(scale=math.nan) == rs.RSWA_ERR_SHAPE
    assert g(num_splits=-2) == rs.RSWA_ERR_SHAPE
    assert g(descs=[], q=[], out=[]) == rs.RSWA_ERR_SHAPE
    assert rs.rswa_decode_graph_destroy(None) == rs.RSWA_OK
    assert rs.rswa_decode_graph_launch(None, check=False) == rs.RSWA_ERR_NULL


def test_probe_argument_checks():
    pr = lambda **kw: rs.rswa_probe_stream_read(**{**dict(buf=A, nbytes=1 << 20, sink=A + 64), **kw}, check=False)
    assert pr(buf=None) == rs.RSWA_ERR_NULL
    assert pr(sink=None) == rs.RSWA_ERR_NULL
    assert pr(nbytes=1000) == rs.RSWA_ERR_SHAPE
    assert pr(workgroups=-1) == rs.RSWA_ERR_SHAPE
    assert pr(buf=A + 8) == rs.RSWA_ERR_ALIGN
    assert pr(sink=A + 2) == rs.RSWA_ERR_ALIGN
    assert pr(nbytes=0) == rs.RSWA_OK


def test_probe_mfma_argument_checks():
    pm = lambda **kw: rs.rswa_probe_mfma(**{**dict(sink=A, workgroups=0, iters=16), **kw}, check=False)
    assert pm(sink=None) == rs.RSWA_ERR_NULL
    assert pm(workgroups=-1) == rs.RSWA_ERR_SHAPE
    assert pm(iters=0) == rs.RSWA_ERR_SHAPE
    assert pm(sink=A + 2) == rs.RSWA_ERR_ALIGN


def test_device_facts_argument_checks():
    lib = rs._lib()
    buf = (ctypes.c_int64 * 8)()
    assert lib.rswa_device_facts(0, None, 8) == rs.RSWA_ERR_NULL
    assert lib.rswa_device_facts(-1, buf, 8) == rs.RSWA_ERR_SHAPE
    assert lib.rswa_device_facts(0, buf, 0) == rs.RSWA_ERR_SHAPE
    assert len(rs.DEVICE_FACTS) == int(re.search(r"RSWA_FACT_COUNT = (\d+)", open(HEADER).read()).group(1))


def test_probe_cu_argument_checks():
    pc = lambda **kw: rs.rswa_probe_cu(**{**dict(out=A, workgroups=0, iters=16, kind=0), **kw}, check=False)
    assert pc(out=None) == rs.RSWA_ERR_NULL
    assert pc(workgroups=-1) == rs.RSWA_ERR_SHAPE
    assert pc(iters=0) == rs.RSWA_ERR_SHAPE
    assert pc(kind=-1) == rs.RSWA_ERR_SHAPE
    assert pc(kind=4) == rs.RSWA_ERR_SHAPE
    assert pc(out=A + 2) == rs.RSWA_ERR_ALIGN


def test_masked_bwd_workspace_size():
    ws = rs.rswa_masked_bwd_workspace_size
    assert ws(-1, 0, 2) == 0
    assert ws(10, 0, 0) == 0
    assert ws(10, 11, 2) == 0          # ref_len > seq_len
    assert ws(10, 5, 2, -1) == 0
    assert ws(10, 5, 2, 65) == 0
    assert ws(0, 0, 2) == 0
    assert ws(2 ** 31 - 1, 0, 1) == 0   # sizes the call rejects with RSWA_ERR_CAPACITY
    assert ws(2, 0, 2 ** 16) == 0
    # one part: two float arrays [H][roundup(N, 32)]
    assert ws(1, 1, 2, 1) == 2 * 2 * 32 * 4
    assert ws(300, 40, 3, 1) == 2 * 3 * 320 * 4
    # parts > 1 add fp32 partial dK and dV for the 128-key blocks below ref_len
    assert ws(300, 40, 3, 4) == 2 * 3 * 320 * 4 + 2 * 4 * 3 * 128 * 128 * 4
    assert ws(300, 0, 3, 4) == 2 * 3 * 320 * 4    # no reference segment: nothing to split
    # the library's choice at the packed 32K shape: runs of about 256 query blocks
    assert ws(32768, 4128, 16) == 2 * 16 * 32768 * 4 + 2 * 4 * 16 * 4224 * 128 * 4


def test_masked_bwd_argument_checks():
    ws = rs.rswa_masked_bwd_workspace_size(300, 40, 2)
    base = dict(q=A, k=A, v=A, out=A, dout=A, lse=A, dq=A, dk=A, dv=A, seq_len=300, ref_len=40,
                window=8, num_heads=2, head_dim=128, workspace=A, workspace_bytes=ws)
    b = lambda **kw: rs.rswa_masked_attn_bwd(**{**base, **kw}, check=False)
    for name in ("q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv"):
        assert b(**{name: None}) == rs.RSWA_ERR_NULL, name
    for name in ("q", "k", "v", "out", "dout", "dq", "dk", "dv"):
        assert b(**{name: A + 8}) == rs.RSWA_ERR_ALIGN, name
    assert b(lse=A + 2) == rs.RSWA_ERR_ALIGN
    assert b(ref_len=301) == rs.RSWA_ERR_SHAPE
    assert b(seq_len=-1) == rs.RSWA_ERR_SHAPE
    assert b(window=0) == rs.RSWA_ERR_SHAPE
    assert b(num_heads=0) == rs.RSWA_ERR_SHAPE
    assert b(head_dim=64) == rs.RSWA_ERR_UNSUPPORTED
    assert b(dtype=rs.RSWA_FP32) == rs.RSWA_ERR_UNSUPPORTED
    assert b(prefix_mode=2) == rs.RSWA_ERR_UNSUPPORTED
    assert b(scale=math.inf) == rs.RSWA_ERR_SHAPE
    assert b(seq_len=2 ** 20, ref_len=0, num_heads=16) == rs.RSWA_ERR_CAPACITY
    assert b(seq_len=2, ref_len=0, num_heads=2 ** 16) == rs.RSWA_ERR_CAPACITY
    assert b(workspace=None, workspace_bytes=0) == rs.RSWA_ERR_NULL
    assert b(workspace_bytes=ws - 1) == rs.RSWA_ERR_WORKSPACE
    assert b(workspace=A + 4) == rs.RSWA_ERR_ALIGN
    assert b(num_parts=-1) == rs.RSWA_ERR_SHAPE
    assert b(num_parts=65) == rs.RSWA_ERR_SHAPE
    assert b(num_parts=3) == rs.RSWA_ERR_WORKSPACE   # more parts need more workspace
    assert b(seq_len=0, ref_len=0, workspace=None, workspace_bytes=0) == rs.RSWA_OK


def test_masked_bwd_varlen_workspace_size():
    # two float rows per head and row of the pack, rows padded to 32
    assert rs.rswa_masked_bwd_varlen_workspace_size(300, 2) == 2 * 2 * 320 * 4
    assert rs.rswa_masked_bwd_varlen_workspace_size(0, 3) == 0
    assert rs.rswa_masked_bwd_varlen_workspace_size(-1, 2) == 0
    assert rs.rswa_masked_bwd_varlen_workspace_size(64, 0) == 0
    assert rs.rswa_masked_bwd_varlen_workspace_size(2 ** 20, 16) == 0   # rejected by the call
    assert rs.rswa_masked_bwd_varlen_workspace_size(2, 2 ** 16) == 0


def test_varlen_bwd_argument_checks():
    ws = rs.rswa_masked_bwd_varlen_workspace_size(300, 2)
    base = dict(q=A, k=A, v=A, out=A, dout=A, lse=A, dq=A, dk=A, dv=A, cu_seqlens=A, ref_lens=A,
                num_seqs=2, total_tokens=300, max_seq_len=200, window=8, num_heads=2, head_dim=128,
                workspace=A, workspace_bytes=ws)
    b = lambda **kw: rs.rswa_masked_attn_bwd_varlen(**{**base, **kw}, check=False)
    for name in ("q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv", "cu_seqlens", "ref_lens"):
        assert b(**{name: None}) == rs.RSWA_ERR_NULL, name
    for name in ("q", "k", "v", "out", "dout", "dq", "dk", "dv"):
        assert b(**{name: A + 8}) == rs.RSWA_ERR_ALIGN, name
    for name in ("lse", "cu_seqlens", "ref_lens"):
        assert b(**{name: A + 2}) == rs.RSWA_ERR_ALIGN, name
    assert b(num_seqs=-1) == rs.RSWA_ERR_SHAPE
    assert b(total_tokens=-1) == rs.RSWA_ERR_SHAPE
    assert b(max_seq_len=-1) == rs.RSWA_ERR_SHAPE
    assert b(window=0) == rs.RSWA_ERR_SHAPE
    assert b(num_heads=0) == rs.RSWA_ERR_SHAPE
    assert b(head_dim=64) == rs.RSWA_ERR_UNSUPPORTED
    assert b(dtype=rs.RSWA_FP32) == rs.RSWA_ERR_UNSUPPORTED
    assert b(prefix_mode=2) == rs.RSWA_ERR_UNSUPPORTED
    assert b(scale=math.nan) == rs.RSWA_ERR_SHAPE
    assert b(total_tokens=2 ** 20, num_heads=16) == rs.RSWA_ERR_CAPACITY
    assert b(total_tokens=2, max_seq_len=2, num_heads=2 ** 16) == rs.RSWA_ERR_CAPACITY
    assert b(num_seqs=2 ** 20, max_seq_len=2 ** 20, num_heads=16, total_tokens=1) == rs.RSWA_ERR_CAPACITY
    assert b(workspace=None, workspace_bytes=0) == rs.RSWA_ERR_NULL
    assert b(workspace_bytes=ws - 1) == rs.RSWA_ERR_WORKSPACE
    assert b(workspace=A + 4) == rs.RSWA_ERR_ALIGN
    # nothing to do: no sample, no row or no row per sample
    for kw in (dict(num_seqs=0), dict(total_tokens=0), dict(max_seq_len=0)):
        assert b(workspace=None, workspace_bytes=0, **kw) == rs.RSWA_OK, kw


def test_check_device_error_null_arguments():
    lib = rs.library()
    flags = ctypes.c_int32(0)
    assert lib.rswa_check_device_error(None, ctypes.byref(flags), None) == rs.RSWA_ERR_NULL
    desc = good_desc()
    assert lib.rswa_check_device_error(ctypes.byref(desc), None, None) == rs.RSWA_ERR_NULL


def test_workspace_size_by_sizes_matches_descriptor_form():
    """rswa_workspace_size(batch, heads, head_dim, max_len) is the library's split
    choice for a cache whose longest sequence holds max_len = max_ref_len + window slots."""
    for B, H, d, L, n in ((32, 16, 128, 10272, 128), (1, 16, 128, 288, 128), (64, 16, 128, 12832, 128),
                          (2, 16, 128, 10272, 128), (1, 2, 64, 64, 8), (3, 4, 64, 0, 5)):
        desc = good_desc(batch=B, num_heads=H, head_dim=d, max_ref_len=L, window=n)
        assert rs.rswa_workspace_size(B, H, d, L + n) == rs.rswa_decode_workspace_size(desc, 0) > 0
    ws = rs.rswa_workspace_size
    assert ws(0, 16, 128, 100) == 0
    assert ws(1, 0, 128, 100) == 0
    assert ws(1, 16, 96, 100) == 0
    assert ws(1, 16, 128, 0) == 0
    assert ws(2 ** 30, 16, 128, 100) == 0


def test_packed_calls_reject_a_negative_scale():
    """The packed kernels need scale > 0 (or 0 for the default); decode accepts any finite scale."""
    neg = -0.125
    assert rs.rswa_masked_attn(A, A, A, A, 300, 40, 8, 2, 128, scale=neg, check=False) == rs.RSWA_ERR_SHAPE
    assert rs.rswa_masked_attn_varlen(A, A, A, A, A, A + 64, 3, 900, 400, 8, 2, 128, scale=neg,
                                      check=False) == rs.RSWA_ERR_SHAPE
    assert rs.rswa_prefill(good_desc(), A, A, A, A, A, 500, 300, scale=neg, check=False) == rs.RSWA_ERR_SHAPE
    ws = rs.rswa_masked_bwd_workspace_size(300, 40, 2)
    assert rs.rswa_masked_attn_bwd(A, A, A, A, A, A, A, A, A, 300, 40, 8, 2, 128, scale=neg, workspace=A,
                                   workspace_bytes=ws, check=False) == rs.RSWA_ERR_SHAPE
    wsv = rs.rswa_masked_bwd_varlen_workspace_size(300, 2)
    assert rs.rswa_masked_attn_bwd_varlen(A, A, A, A, A, A, A, A, A, A, A, 2, 300, 200, 8, 2, 128, scale=neg,
                                          workspace=A, workspace_bytes=wsv, check=False) == rs.RSWA_ERR_SHAPE


def test_noalloc_decode_checks_before_touching_the_device():
    """Argument checks and the buffer-size limit come first (nothing enqueued)."""
    desc = good_desc(batch=32, num_heads=16, max_ref_len=10272, window=128)
    call = lambda **kw: rs.rswa_decode_attn_noalloc(desc, **{**dict(q=A, out=A), **kw}, check=False)
    assert rs.rswa_decode_workspace_size(desc, 64) > 8 << 20
    assert call(num_splits=64) == rs.RSWA_ERR_WORKSPACE
    assert call(q=None) == rs.RSWA_ERR_NULL
    assert call(k_new=A) == rs.RSWA_ERR_NULL
    assert call(out=A + 4) == rs.RSWA_ERR_ALIGN
    assert call(scale=math.nan) == rs.RSWA_ERR_SHAPE
    assert call(num_splits=-1) == rs.RSWA_ERR_SHAPE
    assert rs.rswa_decode_attn_noalloc(good_desc(head_dim=96), A, A, check=False) == rs.RSWA_ERR_UNSUPPORTED
