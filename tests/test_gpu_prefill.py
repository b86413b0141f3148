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


# ------------------------------------------------- the prefill family

PREFILL = pad.PAD_PATH_PREFILL
FAMILY_SHAPES = [
    # D, Hq, Hkv, P, dtype, layout
    (128, 32, 8, 16, "bf16", wl.HND),
    (64, 8, 2, 32, "fp16", wl.NHD),
    (128, 12, 4, 48, "fp16", wl.HND),
]
FAMILY_CASES = [
    # lens, M, window, nseg
    ([1], 1, 0, 0),                  # one key, one row of 128
    ([40, 1, 0, 77], 33, 0, 0),      # ragged, a padded sequence, L < M rows with no key
    ([1000], 100, 0, 3),             # forced segments
    ([700], 64, 50, 0),              # window shorter than the chunk
    ([300, 513], 130, 1, 7),         # window 1: each row sees its own key only
    ([5, 3], 8, 0, 0),               # every row past the keys for some tokens
]


@pytest.mark.parametrize("shape", FAMILY_SHAPES, ids=[f"d{s[0]}g{s[1] // s[2]}" for s in FAMILY_SHAPES])
@pytest.mark.parametrize("case", FAMILY_CASES, ids=[f"c{i}" for i in range(len(FAMILY_CASES))])
def test_prefill_family(shape, case):
    """The prefill family forced on small, ragged and degenerate chunks
    (NaN-poisoned page tails, empty rows of a 128-row block, windows,
    forced segments) against the oracle."""
    D, Hq, Hkv, P, dt, layout = shape
    lens, M, window, nseg = case
    spec = wl.Spec(dt, D, Hq, Hkv, P, layout, window=window)
    say(f"prefill family: D={D} Hq={Hq} Hkv={Hkv} P={P} {dt} layout={layout} lens={lens} M={M} W={window} "
        f"nseg={nseg}")
    c = wl.make_case(spec, lens, M, seed=8300 + D + M + sum(lens), device=DEV, window=window)
    out = run_gpu(c, path=PREFILL, num_segments=nseg, schedule=pad.PAD_SCHED_GRID)
    for s, L in enumerate(lens):
        if L == 0:
            assert torch.all(out[s] == 0), "padded sequence must be zero"
    check(out, oracle_out(c), c.q.dtype, "prefill family")


def test_prefill_bench_chunk_full():
    """The benchmark's chunk at full size (256 tokens over a 4096-key
    context, 32/8 heads of 128, bf16) through the automatic plan, which is
    the prefill family, against the oracle on every row."""
    spec = wl.CONFIGS[2]
    c = wl.make_case(spec, [4096 + 256], 256, seed=20261202 + 7, device=DEV)
    sh = pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout)
    assert pad.pad_decode_attn_plan(sh)["path"] == PREFILL
    say("prefill bench chunk: 256 tokens over 4096 keys, config 2 shapes")
    check(run_gpu(c), oracle_out(c), c.q.dtype, "prefill bench chunk")


def _sampled_prompt_check(c, spec, M, window, what):
    """Sampled tokens of a whole prompt (the first, the last and 62 spread
    between) of every head against the oracle's own gather-and-softmax
    steps: the full oracle is too slow at these sizes."""
    out = run_gpu(c)
    assert torch.isfinite(out).all()
    kv64, table, lens = wl.compact(c)
    q64 = wl.as_f64(c.q)
    G = spec.num_q_heads // spec.num_kv_heads
    toks = sorted(set([0, M - 1] + list(np.linspace(1, M - 2, 62).astype(int))))
    ref = np.zeros((len(toks), spec.num_q_heads, spec.head_size))
    for kvh in range(spec.num_kv_heads):
        K_all, V_all = oracle.gather_kv(kv64, c.layout, table[0], kvh, range(M))
        for i, m in enumerate(toks):
            lo, hi = oracle.key_bounds(M, M, m, window)
            for g in range(G):
                h = kvh * G + g
                ref[i, h] = oracle.attention._softmax_attend(q64[0, m, h], K_all[lo:hi + 1], V_all[lo:hi + 1], c.scale)
    check(out[0, toks], ref, c.q.dtype, what)


def test_prefill_2048_token_prompt():
    """A 2048-token prompt (no earlier context) in one call: 8192 GQA-packed
    rows per kv head, 64 row blocks, on sampled tokens."""
    spec = wl.CONFIGS[2]
    M = 2048
    c = wl.make_case(spec, [M], M, seed=8400, device=DEV)
    say("prefill prompt: 2048 tokens, config 2 shapes")
    _sampled_prompt_check(c, spec, M, 0, "2048-token prompt, sampled tokens")


@pytest.mark.parametrize(
    "spec,window",
    [
        (wl.Spec("bf16", 128, 32, 4, 16, wl.HND), 0),
        (wl.Spec("fp16", 64, 16, 2, 32, wl.NHD, window=777), 777),
    ],
    ids=["bf16_d128_hnd", "fp16_d64_nhd_window"],
)
def test_prefill_largest_prompt(spec, window):
    """The largest call the planner takes: a 4096-token prompt with eight
    query heads per kv head, 32768 GQA-packed rows per kv head (256 row
    blocks), through the automatic plan (the prefill family), on sampled
    tokens; once with a sliding window over a token-major cache."""
    M = 4096
    c = wl.make_case(spec, [M], M, seed=8500 + spec.head_size, device=DEV, window=window)
    sh = pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout)
    p = pad.pad_decode_attn_plan(sh, window)
    assert p["path"] == PREFILL and p["rows"] == 32768 and p["row_groups"] == 256, p
    say(f"prefill prompt: 4096 tokens, {spec.dtype} D={spec.head_size} "
        f"{spec.num_q_heads}/{spec.num_kv_heads} heads, window {window}")
    _sampled_prompt_check(c, spec, M, window, f"4096-token prompt, window {window}, sampled tokens")


def test_prefill_graph_replay():
    """A prefill-family call (96 tokens over a 1904-key context, forced
    segments, so its split-KV merge runs) captured in a HIP graph and
    replayed 20 times, with eager decode calls through the same workspace
    between replays: every replay gives the eager call's bits, and the
    control words end zero."""
    spec = wl.CONFIGS[2]
    c = wl.make_case(spec, [2000], 96, seed=8600, device=DEV, instances=2)
    d = wl.make_case(spec, [3000], 4, seed=8601, device=DEV)
    need = max(pad.pad_decode_attn_workspace_size(pad.make_shape(x.q, x.kv_cache, x.block_tables[0], x.layout,
                                                                 num_segments=n, path=p))
               for x, n, p in ((c, 3, PREFILL), (d, 0, 0)))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    pad.pad_decode_attn_workspace_init(ws)
    say("prefill graph replay: 96 tokens over 1904 keys, config 2 shapes, 3 segments")
    eager = run_gpu(c, 0, workspace=ws, path=PREFILL, num_segments=3)
    dref = run_gpu(d, workspace=ws)
    torch.cuda.synchronize()
    static_out = torch.zeros_like(c.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_gpu(c, 0, workspace=ws, out=static_out, path=PREFILL, num_segments=3)
    for it in range(20):
        static_out.fill_(float("nan"))
        g.replay()
        if it % 5 == 0:
            other = run_gpu(d, workspace=ws)  # eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(other, dref), f"eager decode call {it} changed"
        torch.cuda.synchronize()
        assert torch.equal(static_out, eager), f"replay {it} differs from the eager result"
    assert int(ws[: 1 << 20].view(torch.int32).abs().sum()) == 0, "control words must be left zero"
    check(static_out, oracle_out(c), c.q.dtype, "prefill graph replay")
