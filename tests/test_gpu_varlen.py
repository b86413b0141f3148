"""Per-sequence query counts (packed queries) on the HIP path, through the C
ABI, against the fp64 oracle of the query-map rule."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_block_amd as pad
import workloads as wl
from gpu_check import check, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _packed(spec, lens, counts, seed, window=0, lead=0):
    """A case with M = max(counts) and its packed queries: sequence s keeps
    its first counts[s] query rows; `lead` unowned rows come first."""
    mmax = max(1, max(counts))
    say(f"varlen case: D={spec.head_size} Hq={spec.num_q_heads} Hkv={spec.num_kv_heads} P={spec.page_size} "
        f"{spec.dtype} layout={spec.layout} lens={list(lens)} counts={list(counts)} window={window} lead={lead}")
    c = wl.make_case(spec, lens, mmax, seed=seed, device=DEV, window=window)
    Hq, D = c.q.shape[2], c.q.shape[3]
    filler = torch.zeros((lead, Hq, D), dtype=c.q.dtype, device=DEV)
    q = torch.cat([filler] + [c.q[s, :n] for s, n in enumerate(counts)], dim=0).contiguous()
    q_start = np.concatenate([[lead], lead + np.cumsum(counts)]).astype(np.int32)
    return c, q, torch.from_numpy(q_start).to(DEV), q_start, mmax


def _oracle(c, q, q_start_np):
    kv64, table, lens = wl.compact(c)
    return oracle.decode_attention_varlen(wl.as_f64(q), q_start_np, kv64, table, lens, c.scale, c.window, c.layout)


def _run(c, q, q_start, mmax, out=None, **kw):
    if out is None:
        out = torch.full_like(q, float("nan"))
    pad.pad_decode_attn_varlen(q, q_start, c.kv_cache, c.block_tables[0], c.seq_lens, c.scale, c.window, out,
                               max_query_len=mmax, layout=c.layout, **kw)
    return out


# (spec, lens, counts, window)
MIXED = [
    (wl.CONFIGS[2], [4096, 700, 1, 0, 2500], [4, 1, 3, 2, 2], 0),   # decode + verify, L < M, padding
    (wl.CONFIGS[4], [1500, 90, 2200], [8, 1, 5], 0),                 # wide heads, 8..64 rows
    (wl.CONFIGS[3], [16384, 600], [4, 1], 512),                      # window, NHD, fp16
    (wl.CONFIGS[5], [3000, 512, 0, 9000, 1057], [4, 2, 4, 1, 3], 0),  # batch layout, page 1056
]


@pytest.mark.parametrize("case", MIXED, ids=[f"v{i}" for i in range(len(MIXED))])
def test_mixed_counts(case):
    spec, lens, counts, window = case
    c, q, q_start, q_start_np, mmax = _packed(spec, lens, counts, 900 + len(lens), window=window)
    ref = _oracle(c, q, q_start_np)
    out = _run(c, q, q_start, mmax)
    check(out, ref, c.q.dtype, "varlen")
    again = _run(c, q, q_start, mmax)
    assert torch.equal(out, again), "bitwise deterministic"


def test_sequence_without_queries_and_unowned_rows():
    """Rows before q_start[0] belong to no sequence and a sequence with no
    query owns none: the call leaves such rows untouched."""
    spec = wl.CONFIGS[2]
    c, q, q_start, q_start_np, mmax = _packed(spec, [800, 300, 1200], [2, 0, 3], 31, lead=3)
    out = torch.full_like(q, 7.0)
    _run(c, q, q_start, mmax, out=out)
    assert torch.all(out[:3] == 7.0), "unowned rows written"
    ref = _oracle(c, q, q_start_np)
    check(out[3:], ref[3:], c.q.dtype, "owned rows")


def test_uniform_counts_match_uniform_call():
    """Equal counts give the bits of the uniform [S, M, Hq, D] entry point."""
    c = wl.make_case(wl.CONFIGS[4], [2500, 700], 4, seed=41, device=DEV)
    S, M, Hq, D = c.q.shape
    say("varlen vs uniform: config 4 shapes, lens [2500, 700], M=4")
    uni = torch.full_like(c.q, float("nan"))
    pad.pad_decode_attn(c.q, c.kv_cache, c.block_tables[0], c.seq_lens, c.scale, c.window, uni, layout=c.layout)
    q_start = torch.arange(S + 1, dtype=torch.int32, device=DEV) * M
    q = c.q.reshape(S * M, Hq, D)
    var = _run(c, q, q_start, M)
    assert torch.equal(var.reshape(S, M, Hq, D), uni)


def test_schedules_and_dot_family():
    spec = wl.CONFIGS[5]
    c, q, q_start, q_start_np, mmax = _packed(spec, [3000, 600, 0, 5000, 40], [4, 1, 2, 3, 4], 57)
    ref = _oracle(c, q, q_start_np)
    shape = pad.make_shape(torch.empty((c.num_seqs, mmax) + tuple(c.q.shape[2:]), device="meta",
                                       dtype=c.q.dtype), c.kv_cache, c.block_tables[0], c.layout, num_segments=6)
    n = pad.pad_decode_attn_plan(shape, c.window)["num_segments"]
    grid = _run(c, q, q_start, mmax, num_segments=n, schedule=pad.PAD_SCHED_GRID)
    per = _run(c, q, q_start, mmax, schedule=pad.PAD_SCHED_PERSISTENT)
    again = _run(c, q, q_start, mmax, schedule=pad.PAD_SCHED_PERSISTENT)
    check(grid, ref, c.q.dtype, "varlen grid")
    check(per, ref, c.q.dtype, "varlen balanced grid")
    assert torch.equal(per, again), "deterministic"
    # the dot family: G = 4 query heads per kv head and at most one query each
    d = _packed(wl.CONFIGS[2], [3000, 17, 900], [1, 1, 0], 61)
    cd, qd, qsd, qsd_np, md = d
    out = _run(cd, qd, qsd, md, path=pad.PAD_PATH_DOT)
    check(out, _oracle(cd, qd, qsd_np), cd.q.dtype, "varlen dot")


def test_graph_replay_follows_device_counts():
    """The counts are read on the device: a captured call follows new
    q_start contents written between replays, with no host sync."""
    spec = wl.CONFIGS[2]
    c, q, q_start, a_np, mmax = _packed(spec, [2000, 1000, 3000], [4, 4, 4], 71)
    out = torch.zeros_like(q)
    ws = pad.Workspace(q.device)
    shape = pad.make_shape(torch.empty((c.num_seqs, mmax) + tuple(c.q.shape[2:]), device="meta",
                                       dtype=c.q.dtype), c.kv_cache, c.block_tables[0], c.layout)
    buf = ws.get(shape)
    _run(c, q, q_start, mmax, out=out, workspace=buf)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run(c, q, q_start, mmax, out=out, workspace=buf)
    b_np = np.array([0, 1, 5, 8], dtype=np.int32)  # counts 1, 4, 3 over the same packed rows
    for it, starts in enumerate([a_np, b_np, a_np, b_np]):
        q_start.copy_(torch.from_numpy(starts).to(DEV))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        used = int(starts[-1])
        ref = _oracle(c, q[:used], starts)
        check(out[:used], ref, c.q.dtype, f"replay {it}")
