"""pad_decode_attn_noalloc (workspace in the library's fixed device array)
against pad_decode_attn (caller-supplied workspace), through the C ABI.

Both entry points plan the same launch and run the same kernels, so their
outputs must be the same bits; each is also held to the oracle's gates.
Calls follow one another with shrinking inputs, so the array holds the
previous call's partials and control words when the next one starts.
"""

import pytest
import torch

import paged_kv_decode_block_amd as pad
import workloads as wl
from gpu_check import check, oracle_out, run_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc(c, out=None, **kw):
    if out is None:
        out = torch.full_like(c.q, float("nan"))
    pad.pad_decode_attn_noalloc(c.q, c.kv_cache, c.block_tables[0], c.seq_lens, c.scale, c.window, out,
                                layout=c.layout, **kw)
    return out


# (config, context, M): the persistent batch (about 27 MB of partials), the
# wide-head split with merge helpers, the window, then smaller calls.
SEQUENCE = [(5, 16384, 4), (4, 32768, 8), (3, 16384, 4), (2, 4096, 4), (2, 1000, 1), (1, 256, 1)]


def test_noalloc_matches_the_workspace_entry_point():
    for cfg, ctx, M in SEQUENCE:
        say(f"noalloc: config {cfg} context {ctx} M={M}")
        c = wl.config_case(cfg, ctx, M, device=DEV)
        shape = pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout)
        need = pad.pad_decode_attn_workspace_size(shape)
        assert need <= pad.PAD_NOALLOC_SCRATCH_BYTES
        ref = run_gpu(c)
        got = _noalloc(c)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"config {cfg}: the two entry points must give the same bits"
        check(got, oracle_out(c), c.q.dtype, f"noalloc config {cfg} L={ctx} M={M} (workspace {need} B)")
        del c


def test_noalloc_two_calls_second_smaller():
    big = wl.config_case(4, 16384, 8, device=DEV)
    small = wl.make_case(wl.CONFIGS[4], [700], 3, seed=1234, device=DEV)
    for c in (big, small):
        say(f"noalloc back to back: lens {c.seq_lens.tolist()[:4]} M={c.query_len}")
        ref = run_gpu(c)
        got = _noalloc(c)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        check(got, oracle_out(c), c.q.dtype, "noalloc back to back")


def test_noalloc_forced_schedules_and_segments():
    c = wl.config_case(5, 3000, 4, device=DEV)
    ref_o = oracle_out(c)
    for sched, nseg in ((pad.PAD_SCHED_GRID, 4), (pad.PAD_SCHED_PERSISTENT, 0), (pad.PAD_SCHED_GRID, 0)):
        say(f"noalloc schedule {sched} segments {nseg}")
        ref = run_gpu(c, schedule=sched, num_segments=nseg)
        got = _noalloc(c, schedule=sched, num_segments=nseg)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        check(got, ref_o, c.q.dtype, f"noalloc schedule {sched} segments {nseg}")


def test_noalloc_graph_replay():
    c = wl.config_case(2, 4096, 4, device=DEV, instances=2)
    eager = [run_gpu(c, i) for i in range(2)]
    torch.cuda.synchronize()
    static_out = torch.zeros_like(c.q)
    g = torch.cuda.CUDAGraph()
    say("noalloc captured in a graph")
    with torch.cuda.graph(g):
        pad.pad_decode_attn_noalloc(c.q, c.kv_cache, c.block_tables[0], c.seq_lens, c.scale, c.window, static_out,
                                    layout=c.layout)
    for it in range(5):
        static_out.fill_(float("nan"))
        g.replay()
        other = torch.full_like(c.q, float("nan"))
        pad.pad_decode_attn_noalloc(c.q, c.kv_cache, c.block_tables[1], c.seq_lens, c.scale, c.window, other,
                                    layout=c.layout)
        torch.cuda.synchronize()
        assert torch.equal(static_out, eager[0]), f"replay {it}"
        assert torch.equal(other, eager[1]), f"eager call after replay {it}"


def test_noalloc_rejects_calls_beyond_its_array():
    spec = wl.Spec("bf16", 512, 64, 8, 16, wl.HND)
    q = torch.zeros((64, 8, 64, 512), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((2, 8, 16, 2, 512), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((64, 2048), dtype=torch.int32, device=DEV)
    lens = torch.zeros(64, dtype=torch.int32, device=DEV)
    kw = dict(num_segments=64, schedule=pad.PAD_SCHED_GRID)
    shape = pad.make_shape(q, kv, bt, wl.HND, **kw)
    assert pad.pad_decode_attn_workspace_size(shape) > pad.PAD_NOALLOC_SCRATCH_BYTES
    with pytest.raises(pad.PadError) as e:
        pad.pad_decode_attn_noalloc(q, kv, bt, lens, 0.1, 0, torch.empty_like(q), layout=spec.layout, **kw)
    assert e.value.status == pad.PAD_ESCRATCH
