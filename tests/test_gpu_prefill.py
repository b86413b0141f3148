"""Prefill chunks (M > 8 query tokens per sequence) on the HIP path against
the fp64 oracle: each row group reads only the keys its own tokens reach
(the row-tile work list of plan_prefill on the rdna_hip page), on both
schedules."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_block_amd as pad
import workloads as wl
from gpu_check import check, oracle_out, run_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (spec, lens, M, window, nseg)
CHUNKS = [
    (wl.CONFIGS[2], [2000], 64, 0, 0),          # a chunk over a 1936-key context, 256 rows
    (wl.CONFIGS[2], [200], 200, 0, 0),          # a whole prompt: no context, 800 rows
    (wl.CONFIGS[2], [3000], 96, 128, 0),        # window shorter than the chunk
    (wl.CONFIGS[4], [1500], 32, 0, 5),          # head size 512, 256 rows in 16 row groups
    (wl.CONFIGS[3], [16384], 40, 512, 0),       # NHD fp16, window table
    (wl.CONFIGS[1], [256], 48, 0, 3),           # fp16 head size 64
]


@pytest.mark.parametrize("case", CHUNKS, ids=[f"p{i}" for i in range(len(CHUNKS))])
def test_prefill_chunk(case):
    spec, lens, M, window, nseg = case
    say(f"prefill: D={spec.head_size} Hq={spec.num_q_heads} Hkv={spec.num_kv_heads} lens={lens} M={M} "
        f"window={window} nseg={nseg}")
    c = wl.make_case(spec, lens, M, seed=8000 + M, device=DEV, window=window)
    out = run_gpu(c, num_segments=nseg)
    check(out, oracle_out(c), c.q.dtype, "prefill chunk")


def test_prefill_batch_schedules():
    """A batch of chunks of different lengths: both schedules match the
    oracle, and the balanced grid gives the same bits on every call."""
    spec = wl.CONFIGS[2]
    c = wl.make_case(spec, [1500, 300, 0, 2600], 48, seed=8101, device=DEV)
    say("prefill batch: config 2 shapes, lens [1500, 300, 0, 2600], M=48")
    ref = oracle_out(c)
    grid = run_gpu(c, num_segments=4, schedule=pad.PAD_SCHED_GRID)
    per = run_gpu(c, schedule=pad.PAD_SCHED_PERSISTENT)
    again = run_gpu(c, schedule=pad.PAD_SCHED_PERSISTENT)
    check(grid, ref, c.q.dtype, "prefill batch, grid")
    check(per, ref, c.q.dtype, "prefill batch, balanced grid")
    assert torch.equal(per, again), "deterministic"


def test_mixed_decode_and_prefill_counts():
    """One packed call with decode (1), verify (4) and prefill (100, 33)
    counts."""
    spec = wl.CONFIGS[2]
    counts = [1, 100, 4, 33]
    lens = [4000, 900, 1200, 33]
    mmax = max(counts)
    c = wl.make_case(spec, lens, mmax, seed=8202, device=DEV)
    say(f"mixed counts: lens {lens} counts {counts}")
    q = torch.cat([c.q[s, :n] for s, n in enumerate(counts)], dim=0).contiguous()
    starts = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    out = torch.full_like(q, float("nan"))
    pad.pad_decode_attn_varlen(q, torch.from_numpy(starts).to(DEV), c.kv_cache, c.block_tables[0], c.seq_lens,
                               c.scale, c.window, out, max_query_len=mmax, layout=c.layout)
    kv64, table, lens64 = wl.compact(c)
    ref = oracle.decode_attention_varlen(wl.as_f64(q), starts, kv64, table, lens64, c.scale, c.window, c.layout)
    check(out, ref, c.q.dtype, "mixed counts")
