"""The streaming-read measurement kernel reads every byte of its range once:
in its checking mode the wrapping 32-bit sums its workgroups write add up to
the sum of the range's words, for ragged sizes, several grids and both load
depths (a piece read twice or skipped would change the sum)."""

import numpy as np
import pytest
import torch

import quantized_gemm_decode_amd as ql
from tests.gpu_util import requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("nbytes", [0, 16, 1040, 16 * ((1 << 20) + 3), 50 << 20])
@pytest.mark.parametrize("workgroups", [1, 3, 256, 1024, 4096])
@pytest.mark.parametrize("lif", [4, 8])
def test_stream_read_reads_every_byte_once(nbytes, workgroups, lif):
    g = torch.Generator().manual_seed(nbytes % 9973 + workgroups)
    host = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, generator=g)
    src = host.cuda()
    sink = torch.full((workgroups,), 0xDEAD, dtype=torch.int32, device="cuda")
    ql.qlinear_stream_read(src, nbytes, workgroups, sink, loads_in_flight=lif, check=True)
    torch.cuda.synchronize()
    got = int(sink.cpu().numpy().view(np.uint32).astype(np.uint64).sum()) & 0xFFFFFFFF
    words = host[:nbytes].numpy().view(np.uint32).astype(np.uint64)
    assert got == int(words.sum()) & 0xFFFFFFFF


def test_stream_read_timing_mode_writes_nothing_in_practice():
    src = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((512,), 7, dtype=torch.int32, device="cuda")
    ql.qlinear_stream_read(src, 1 << 20, 512, sink)
    torch.cuda.synchronize()
    assert bool(torch.all(sink == 7))


def test_stream_read_arguments_are_checked():
    src = torch.empty(64, dtype=torch.uint8, device="cuda")
    sink = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(ql.QLinearError):
        ql.qlinear_stream_read(src, 24, 4, sink)          # not a multiple of 16
    with pytest.raises(ValueError):
        ql.qlinear_stream_read(src, 128, 4, sink)         # beyond the source
    with pytest.raises(ValueError):
        ql.qlinear_stream_read(src, 64, 32, sink)         # sink too small for the grid
    with pytest.raises(ql.QLinearError):
        ql.qlinear_stream_read(src, 64, 4, sink, loads_in_flight=3)


@pytest.mark.parametrize("nbytes,bbytes", [(0, 0), (16, 0), (0, 4096), (1040, 48), (16 * ((1 << 20) + 3), 131072),
                                           (50 << 20, 393216)])
@pytest.mark.parametrize("workgroups", [1, 3, 256])
@pytest.mark.parametrize("threads,lif", [(256, 2), (512, 4), (1024, 2), (1024, 4)])
def test_stream_read_bcast_reads_its_slice_and_the_whole_block(nbytes, bbytes, workgroups, threads, lif):
    """Workgroup w's checking sum is that of its slice of src (the slices of
    qlinear_stream_read) plus that of every word of the broadcast block."""
    g = torch.Generator().manual_seed(nbytes % 9973 + bbytes + workgroups)
    host = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, generator=g)
    bhost = torch.randint(0, 256, (bbytes + 64,), dtype=torch.uint8, generator=g)
    src, bc = host.cuda(), bhost.cuda()
    sink = torch.full((workgroups,), 0xDEAD, dtype=torch.int32, device="cuda")
    ql.qlinear_stream_read_bcast(src, nbytes, bc, bbytes, sink, workgroups=workgroups, threads=threads,
                                 loads_in_flight=lif, check=True)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32).astype(np.uint64)
    words = host[:nbytes].numpy().view(np.uint32).astype(np.uint64)
    bsum = int(bhost[:bbytes].numpy().view(np.uint32).astype(np.uint64).sum())
    n16 = nbytes // 16
    per = -(-n16 // workgroups)
    for w in range(workgroups):
        lo, hi = min(n16, w * per) * 4, min(n16, (w + 1) * per) * 4
        assert int(got[w]) == (int(words[lo:hi].sum()) + bsum) & 0xFFFFFFFF, w


def test_stream_read_bcast_arguments_are_checked():
    src = torch.empty(64, dtype=torch.uint8, device="cuda")
    sink = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(ql.QLinearError):
        ql.qlinear_stream_read_bcast(src, 64, src, 24, sink, workgroups=4)      # broadcast not a multiple of 16
    with pytest.raises(ql.QLinearError):
        ql.qlinear_stream_read_bcast(src, 64, src, 32, sink, workgroups=4, threads=128)
    with pytest.raises(ql.QLinearError):
        ql.qlinear_stream_read_bcast(src, 64, src, 32, sink, workgroups=4, loads_in_flight=8)
    with pytest.raises(ValueError):
        ql.qlinear_stream_read_bcast(src, 64, src, 128, sink, workgroups=4)     # beyond the broadcast source
