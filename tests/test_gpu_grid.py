"""HIP path vs the fp64 oracle over every point of the five benchmark
configurations, each at the planner's automatic launch (the launch
``bench.py`` times), plus the bitwise pins that the mathematics fixes.

Grid: configuration 1 (256 keys, M=1); configuration 2 at 128..32768 keys
and M in {1, 2, 4}; configuration 3 (512-key window over 16384 keys, NHD)
at M in {1, 4}; configuration 4 at 1024..32768 keys and M = 1..8;
configuration 5 (64 live sequences of 512..16384 keys plus one padded) with
every sequence compared.  Each point is compared element by element with
the oracle at both gates (the absolute gate of the task and the
scale-aware bound), and prints its case before it runs.

Bitwise pins:
* one key (L = 1, M = 1): the softmax weight is exactly 1, so every output
  row is V_0 of its kv head, bit for bit;
* window 1: every query token sees only its own key, so its output is
  V_qpos bit for bit;
* a padded sequence (length 0) changes nothing for the others: the batch
  with it gives the same bits as the batch without it, and its own rows
  are exactly zero.
(The decode and speculative-verify rules: ROCm/vllm pull request 1330,
"Summary"; the K length of query i, seq_len - q_len + i + 1, and the zero
rows of padding: RocmOctaveMetadataBuilder._fill_query_maps on the
rocm_octave_attn page.)
"""

import numpy as np
import pytest
import torch

import paged_kv_decode_block_amd as pad
import workloads as wl
from gpu_check import check, oracle_out, run_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

GRID = [(cfg, ctx, M) for cfg, pts in sorted(wl.CONFIG_POINTS.items())
        for ctx in pts["contexts"] for M in pts["queries"]]


@pytest.mark.parametrize("cfg,ctx,M", GRID, ids=[f"c{c}-L{l}-M{m}" for c, l, m in GRID])
def test_config_point(cfg, ctx, M):
    say(f"grid point: config {cfg} context {ctx} M={M} (automatic plan)")
    c = wl.config_case(cfg, ctx, M, device=DEV)
    shape = pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout)
    plan = pad.pad_decode_attn_plan(shape, c.window)
    say(f"  plan: segments {plan['num_segments']} row groups {plan['row_groups']} "
        f"persistent {plan['persistent']} slices {plan['merge_slices']}")
    out = run_gpu(c)
    torch.cuda.synchronize()
    if cfg == 5:
        assert torch.all(out[-1] == 0), "the padded sequence's rows must be zero"
    check(out, oracle_out(c), c.q.dtype, f"config {cfg} L={ctx} M={M}")
    del c


def _v_rows(case, seq, keys, kv_head):
    """V rows (device dtype) of logical ``keys`` of one sequence."""
    bt = case.block_tables[0][seq].cpu()
    P = case.spec.page_size
    rows = []
    for t in keys:
        blk = int(bt[t // P])
        slot = case.kv_cache[blk, kv_head, t % P] if case.layout == wl.HND else case.kv_cache[blk, t % P, kv_head]
        rows.append(slot[1])
    return torch.stack(rows)


ONE_KEY = [
    # D, Hq, Hkv, P, dtype, layout
    (64, 4, 1, 16, "fp16", wl.HND),
    (128, 32, 8, 16, "bf16", wl.HND),
    (256, 8, 2, 32, "fp16", wl.NHD),
    (512, 16, 2, 32, "bf16", wl.HND),
    (256, 16, 2, 1056, "bf16", wl.HND),
]


@pytest.mark.parametrize("shape", ONE_KEY, ids=[f"k{i}" for i in range(len(ONE_KEY))])
def test_one_key_gives_v0_bitwise(shape):
    D, Hq, Hkv, P, dt, layout = shape
    spec = wl.Spec(dt, D, Hq, Hkv, P, layout)
    say(f"one key: D={D} {Hq}/{Hkv} P={P} {dt} layout={layout}")
    c = wl.make_case(spec, [1, 1, 1], 1, seed=611 + D, device=DEV)
    for path in (pad.PAD_PATH_AUTO, pad.PAD_PATH_DOT):
        if path == pad.PAD_PATH_DOT and (Hq // Hkv > 4 or D > 128):
            continue
        out = run_gpu(c, path=path)
        torch.cuda.synchronize()
        G = Hq // Hkv
        for s in range(3):
            for h in range(Hq):
                v0 = _v_rows(c, s, [0], h // G)[0]
                assert torch.equal(out[s, 0, h], v0), f"seq {s} head {h} (path {path}): output is not V_0"


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("layout", [wl.HND, wl.NHD])
def test_window_one_gives_v_qpos_bitwise(M, layout):
    spec = wl.Spec("bf16", 128, 16, 2, 32, layout, window=1, window_table_only=True)
    lens = [1000, 37, M + 3]
    say(f"window 1: M={M} layout={layout} lens={lens}")
    c = wl.make_case(spec, lens, M, seed=733 + M, device=DEV)
    out = run_gpu(c)
    torch.cuda.synchronize()
    G = spec.num_q_heads // spec.num_kv_heads
    for s, L in enumerate(lens):
        for kvh in range(spec.num_kv_heads):
            v = _v_rows(c, s, [L - M + m for m in range(M)], kvh)
            for m in range(M):
                for g in range(G):
                    assert torch.equal(out[s, m, kvh * G + g], v[m]), f"seq {s} token {m} head {kvh * G + g}"


def test_padded_sequence_changes_no_bits():
    say("config 5 full: 64 live + 1 padded against the 64 live alone")
    c = wl.config_case(5, 16384, 4, device=DEV)
    with_pad = run_gpu(c)
    live = wl.Case(c.spec, c.q[:64].contiguous(), c.kv_cache, [c.block_tables[0][:64].contiguous()],
                   c.seq_lens[:64].contiguous(), c.scale, c.window, c.poison_block, c.seed)
    without = run_gpu(live)
    torch.cuda.synchronize()
    assert torch.all(with_pad[64] == 0), "the padded sequence's rows must be exactly zero"
    assert torch.equal(with_pad[:64], without), "a padded sequence must not change the other sequences' bits"
    # A padded sequence in the middle of the batch, on both schedules (the
    # segment count is forced: the grid schedule's automatic count depends
    # on the number of sequences).
    order = list(range(32)) + [64] + list(range(32, 64))
    mid = wl.Case(c.spec, c.q[order].contiguous(), c.kv_cache, [c.block_tables[0][order].contiguous()],
                  c.seq_lens[order].contiguous(), c.scale, c.window, c.poison_block, c.seed)
    for sched in (pad.PAD_SCHED_GRID, pad.PAD_SCHED_PERSISTENT):
        got = run_gpu(mid, schedule=sched, num_segments=4)
        ref = run_gpu(live, schedule=sched, num_segments=4)
        torch.cuda.synchronize()
        assert torch.all(got[32] == 0)
        assert torch.equal(got[:32], ref[:32]) and torch.equal(got[33:], ref[32:]), f"schedule {sched}"
    np.testing.assert_array_equal(c.seq_lens[64].item(), 0)
