"""The streaming-read measurement kernel (la_stream_read) on the GPU: it
reads the largest whole number of 64 KiB units per workgroup, leaves the
source untouched, rejects bad grids and too-small buffers, and its rate is
a plausible fraction of the 8 TB/s peak on a large buffer."""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def la():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_phase_attention_amd as la
    la.lib()
    return la


def test_bytes_read_and_source_untouched(la):
    src = torch.randint(0, 255, ((64 << 20) + 12345,), dtype=torch.uint8, device="cuda")
    before = src.clone()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for grid in (0, 1, 7, 256, 1000):
        g = grid or torch.cuda.get_device_properties(0).multi_processor_count
        n = la.la_stream_read(src, sink, grid=grid)
        unit = 16 * 256 * 16
        assert n == src.numel() // g // unit * unit * g
    la.la_sync_check()
    assert torch.equal(src, before)


def test_rejects_bad_arguments(la):
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    small = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(la.LaError):
        la.la_stream_read(small, sink, grid=2)   # less than 64 KiB per workgroup
    with pytest.raises(la.LaError):
        la.la_stream_read(small, sink, grid=70000)
    assert la.la_stream_read(small, sink, grid=1) == 1 << 16


def test_rate_is_plausible(la):
    buf = torch.zeros(2 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    la.la_stream_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    n = la.la_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    print(f"streaming read: {gbs:.0f} GB/s", flush=True)
    assert 1000 < gbs < 8000
    del buf
    torch.cuda.empty_cache()
