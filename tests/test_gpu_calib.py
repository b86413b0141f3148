"""The read-ceiling calibration kernels run through the C ABI on the
benchmark's page layouts (windowed NHD, padded batch, head size 512) and
leave the sink untouched."""

import pytest
import torch

import paged_kv_decode_block_amd as pad
import workloads as wl
from gpu_check import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,ctx,M", [(2, 4096, 4), (3, 16384, 4), (4, 1500, 8), (5, 3000, 4)])
def test_gather_read_runs(cfg, ctx, M):
    say(f"calibration gather: config {cfg} context {ctx} M={M}")
    c = wl.config_case(cfg, ctx, M, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    D = c.q.shape[3]
    for waves in (4, 8):
        for tif in ((1,) if D == 512 else (1, 2)):
            for segs in (1, 7, 256):
                pad.pad_calib_gather_read(c.kv_cache, c.block_tables[0], c.seq_lens, M, c.q.shape[2], c.window,
                                          sink, layout=c.layout, waves=waves, tiles_in_flight=tif, segments=segs)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_stream_read_runs():
    say("calibration stream read: 3 MiB + 48 B")
    src = torch.randn((3 << 20) // 2 + 24, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for blocks in (1, 13, 4096):
        for threads in (256, 512, 1024):
            for loads in (4, 8, 16):
                pad.pad_calib_stream_read(src, sink, blocks=blocks, threads=threads, loads_in_flight=loads)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
