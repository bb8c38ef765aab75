"""The streaming-read ceiling kernel (tern_stream_read) that the bench rates
the layer kernels against: it must read every byte of the buffer, whatever
the size, depth and spread, or the ceiling it gives is too optimistic.

A buffer of zeros gets one 16-byte chunk whose first word is the constant
that makes the kernel write its sink; every other lane folds to zero. The
sink is written only if the load that covers that chunk happened."""
from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu

MARK = 0x9E3779B9


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def tl(torch):
    import ternary_weight_linear_amd as tl
    tl.lib()
    return tl


# sizes with runs that do not split evenly over the waves (KiB: 1, 3, 1000,
# 46,387 = the gemv's bytes on the 5120 -> 34816 layer rounded up)
@pytest.mark.parametrize("kib", [1, 3, 1000, 46387])
@pytest.mark.parametrize("depth,waves", [(4, 4), (8, 8), (16, 16), (16, 1)])
def test_stream_read_reads_every_chunk(torch, tl, kib, depth, waves):
    dev = torch.device("cuda:0")
    nbytes = kib * 1024
    buf = torch.zeros((nbytes // 4,), dtype=torch.int32, device=dev)
    sink = torch.zeros((1,), dtype=torch.int32, device=dev)
    mark = MARK - 2**32 if MARK >= 2**31 else MARK
    chunks = nbytes // 16
    for c in sorted({0, chunks // 2 + 1, chunks - 1}):
        buf.zero_()
        sink.zero_()
        buf[4 * c] = mark
        tl.stream_read(buf, depth=depth, waves_per_cu=waves, sink=sink)
        torch.cuda.synchronize()
        assert sink.item() == mark, (kib, depth, waves, c)
    # nothing marked: the sink stays untouched
    buf.zero_()
    sink.zero_()
    tl.stream_read(buf, depth=depth, waves_per_cu=waves, sink=sink)
    torch.cuda.synchronize()
    assert sink.item() == 0


def test_stream_read_rejects_bad_arguments(torch, tl):
    dev = torch.device("cuda:0")
    buf = torch.zeros((4096,), dtype=torch.uint8, device=dev)
    with pytest.raises(tl.TernError):
        tl.stream_read(buf, nbytes=1000)
    with pytest.raises(tl.TernError):
        tl.stream_read(buf, depth=3)
    with pytest.raises(ValueError):
        tl.stream_read(buf, nbytes=8192)
