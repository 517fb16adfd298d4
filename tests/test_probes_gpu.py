"""The measurement helpers the bench reports beside the kernels (not on the
attention path) run through the C ABI and give sane figures: the streaming-read
probe touches every workgroup's sink entry, the matrix-core probe's folds are
finite, the per-CU probe records positive cycle counts for every kind, with
LDS rates and instruction costs inside what any CDNA part can do, and the
device facts agree with what torch reports of the same device."""
import numpy as np
import pytest
import torch

import reference_sliding_window_amd as rs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_stream_read_and_mfma_probes():
    print("\n[case] stream-read and matrix-core probes", flush=True)
    buf = torch.ones(1 << 22, dtype=torch.int32, device="cuda")       # 16 MiB
    sink = torch.full((64,), -1.0, device="cuda")
    rs.rswa_probe_stream_read(buf, buf.numel() * 4, sink, 64)
    torch.cuda.synchronize()
    assert (sink.cpu().numpy() >= 0).all()
    sink = torch.full((32,), float("nan"), device="cuda")
    rs.rswa_probe_mfma(sink, 32, 8)
    torch.cuda.synchronize()
    assert np.isfinite(sink.cpu().numpy()).all()


@pytest.mark.parametrize("kind", [rs.RSWA_PROBE_LDS_B128, rs.RSWA_PROBE_LDS_TR16, rs.RSWA_PROBE_EXP,
                                  rs.RSWA_PROBE_FMA])
def test_cu_probe(kind):
    print(f"\n[case] per-CU probe kind {kind}", flush=True)
    wg, iters = 256, 64
    out = torch.zeros(2 * wg, dtype=torch.int32, device="cuda")
    rs.rswa_probe_cu(out, wg, iters, kind)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.uint32)
    cycles = o[0::2].astype(np.float64)
    assert (cycles > 0).all()
    med = float(np.median(cycles))
    if kind in (rs.RSWA_PROBE_LDS_B128, rs.RSWA_PROBE_LDS_TR16):
        bpc = 8 * iters * 16384 / med
        print(f"LDS bytes per clock per CU: {bpc:.1f}", flush=True)
        assert 16 <= bpc <= 1024
    else:
        cpi = med / (2 * iters * 8)
        print(f"cycles per wave instruction per SIMD: {cpi:.2f}", flush=True)
        assert 1 <= cpi <= 64
        assert (o[1::2] != 0).any()          # the fold of the arithmetic results was written


def test_device_facts():
    print("\n[case] device facts", flush=True)
    f = rs.rswa_device_facts(0)
    p = torch.cuda.get_device_properties(0)
    print(f, flush=True)
    assert f["compute_units"] == p.multi_processor_count
    assert f["global_mem_bytes"] == p.total_memory
    assert f["wave_size"] == 64
    assert f["lds_bytes_per_cu"] >= 64 * 1024
    assert f["clock_khz"] > 0 and f["mem_clock_khz"] > 0 and f["mem_bus_bits"] > 0
