"""HIP path vs the fp64 oracle, through the C ABI, on seeded inputs.

Small cases span several 16-key tiles and a ragged tail; full-size cases
run the benchmark's sizes and launch configuration and compare whole
sequences (or sampled sequences of the batch)."""

import math

import numpy as np
import pytest
import torch

import paged_kv_decode_block_amd as pad
import workloads as wl
from gpu_check import ABS_TOL, check, errors, oracle_out, passes, run_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(spec, lens, M, seed, **kw):
    say(f"case: D={spec.head_size} Hq={spec.num_q_heads} Hkv={spec.num_kv_heads} P={spec.page_size} "
        f"{spec.dtype} layout={spec.layout} lens={list(lens)[:6]} M={M} seed={seed} {kw}")
    return wl.make_case(spec, lens, M, seed=seed, device=DEV, **kw)


# ---------------------------------------------------------------- configs


@pytest.mark.parametrize("M", [1])
def test_config1_exact(M):
    c = wl.config_case(1, 256, M, device=DEV)
    say("config 1: fp16 D64 4/1 M1 P16 L256 HND")
    check(run_gpu(c), oracle_out(c), c.q.dtype, "config1")


@pytest.mark.parametrize("ctx", [128, 1000, 4096, 5003])
@pytest.mark.parametrize("M", [1, 2, 4])
def test_config2_small(ctx, M):
    spec = wl.CONFIGS[2]
    c = _case(spec, [ctx], M, wl.seed_for(2, ctx, M))
    check(run_gpu(c), oracle_out(c), c.q.dtype, f"config2 L={ctx} M={M}")


@pytest.mark.parametrize("M", [1, 4])
def test_config3_window_nhd(M):
    c = wl.config_case(3, 16384, M, device=DEV)
    say(f"config 3: fp16 D256 8/2 W512 P32 L16384 NHD M={M}")
    check(run_gpu(c), oracle_out(c), c.q.dtype, f"config3 M={M}")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_config4_small(M):
    spec = wl.CONFIGS[4]
    c = _case(spec, [1500], M, wl.seed_for(4, 1500, M))
    check(run_gpu(c), oracle_out(c), c.q.dtype, f"config4 L=1500 M={M}")


def test_config5_small_batch():
    c = wl.config_case(5, 3000, 4, device=DEV)
    say("config 5 (length mix up to 3000): 64 seqs + 1 padded, P1056")
    out = run_gpu(c)
    assert torch.all(out[-1] == 0), "padded sequence must be zero"
    check(out, oracle_out(c), c.q.dtype, "config5 small")


def test_length_past_table_capacity():
    """A device length above the block table's capacity is treated as that
    capacity: no key past the table is read."""
    c = _case(wl.CONFIGS[2], [1024, 700], 4, 91, max_blocks=64)
    ref = oracle_out(c)
    lens = c.seq_lens.clone()
    lens[0] = 1 << 30
    for nseg in (0, 1, 7):
        out = torch.full_like(c.q, float("nan"))
        pad.pad_decode_attn(c.q, c.kv_cache, c.block_tables[0], lens, c.scale, 0, out, layout=c.layout,
                            num_segments=nseg)
        check(out, ref, c.q.dtype, f"length clamped to the table, nseg={nseg}")


@pytest.mark.parametrize("window", [0, 700])
@pytest.mark.parametrize("schedule", [pad.PAD_SCHED_GRID, pad.PAD_SCHED_PERSISTENT])
def test_lengths_past_planning_bound(window, schedule):
    """Device lengths above the host's max_seq_len bound (up to the table's
    capacity) stretch the planned segments: the block ids a segment stages
    before its length is known are then replaced, and the result matches
    the oracle; shorter sequences in the same batch keep the plan."""
    c = _case(wl.CONFIGS[2], [3000, 200, 1000], 4, 93, max_blocks=192)
    out = run_gpu(c, max_seq_len=1000, window=window, schedule=schedule)
    check(out, oracle_out(c, window=window), c.q.dtype, f"lengths past the bound, window={window}")


# ------------------------------------------------------- random shapes


RANDOM_SHAPES = [
    # D, Hq, Hkv, P, dtype, layout, lens, M, window
    (64, 8, 8, 16, "fp16", wl.HND, [77, 1, 16], 1, 0),
    (64, 16, 1, 32, "bf16", wl.NHD, [300, 45], 3, 0),
    (128, 8, 2, 48, "fp16", wl.HND, [999], 8, 0),
    (128, 12, 3, 16, "bf16", wl.NHD, [513, 0, 64], 2, 100),
    (256, 4, 4, 528, "bf16", wl.HND, [1100, 17], 5, 0),
    (256, 32, 2, 32, "fp16", wl.HND, [400], 4, 0),   # 64 rows: two row groups at D=256
    (512, 8, 1, 16, "fp16", wl.HND, [333], 2, 0),
    (512, 16, 1, 32, "bf16", wl.NHD, [200], 8, 0),   # 128 rows: 8 row groups at D=512
    (128, 4, 1, 16, "bf16", wl.HND, [5, 3, 2, 1], 4, 0),  # L < M: rows with no key
    (64, 4, 2, 16, "fp16", wl.HND, [40, 41], 3, 1),   # window 1
    (128, 8, 4, 544, "fp16", wl.NHD, [2000], 7, 3000),  # window wider than the context
    (256, 16, 2, 784, "bf16", wl.HND, [1600, 784, 785], 4, 0),
]


@pytest.mark.parametrize("shape", RANDOM_SHAPES, ids=[f"s{i}" for i in range(len(RANDOM_SHAPES))])
def test_random_shapes(shape):
    D, Hq, Hkv, P, dt, layout, lens, M, W = shape
    spec = wl.Spec(dt, D, Hq, Hkv, P, layout, window=W)
    c = _case(spec, lens, M, 4242 + D + Hq + P + M)
    out = run_gpu(c)
    check(out, oracle_out(c), c.q.dtype, f"random {shape}")


# ------------------------------------------------ split-KV and the merge


@pytest.mark.parametrize("nseg", [1, 2, 3, 17, 256])
def test_forced_segments(nseg):
    spec = wl.CONFIGS[2]
    c = _case(spec, [2000], 4, 77)
    ref = oracle_out(c)
    out = run_gpu(c, num_segments=nseg)
    check(out, ref, c.q.dtype, f"nseg={nseg}")
    base = run_gpu(c, num_segments=1)
    assert float((out.float() - base.float()).abs().max()) < 1e-2


@pytest.mark.parametrize("nseg", [8, 9, 16, 17, 32, 36, 63, 84, 125, 250])
def test_merge_lane_counts(nseg):
    """Every lanes-per-item count of the merge (one lane for up to 8 slots,
    then 2, 4, 8, 16 and 32 lanes up to 256 slots), near both edges of each
    range, matches the oracle (4000 keys are 250 tiles: these counts split
    them evenly enough that the planner keeps them)."""
    c = _case(wl.CONFIGS[2], [4000], 4, 91)
    shape = pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout, num_segments=nseg)
    assert pad.pad_decode_attn_plan(shape, c.window)["num_segments"] == nseg
    out = run_gpu(c, num_segments=nseg)
    check(out, oracle_out(c), c.q.dtype, f"merge of {nseg} slots")


def test_counters_left_zero_and_nan_scratch():
    spec = wl.CONFIGS[4]
    c = _case(spec, [3000], 8, 11)
    shape = pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout)
    need = pad.pad_decode_attn_workspace_size(shape)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    pad.pad_decode_attn_workspace_init(ws)
    plan = pad.pad_decode_attn_plan(shape, 0)
    assert plan["num_segments"] > 1
    ref = oracle_out(c)
    # counters occupy a fixed 1 MiB prefix of the workspace
    cnt_bytes = 1 << 20
    for it in range(3):
        # poison the partial area: a stale read would surface as NaN
        ws[cnt_bytes:].fill_(0xFF)
        out = run_gpu(c, workspace=ws)
        torch.cuda.synchronize()
        check(out, ref, c.q.dtype, f"poisoned scratch run {it}")
        assert int(ws[:cnt_bytes].view(torch.int32).abs().sum()) == 0, "arrival counters must be left zero"


def test_workspace_shared_across_shapes():
    """One workspace serves calls of different shapes one after another
    (counters stay in their own region and are left zero by every call)."""
    cases = [
        _case(wl.CONFIGS[2], [2000], 4, 41),
        _case(wl.CONFIGS[4], [3000], 8, 42),
        _case(wl.CONFIGS[2], [5000], 1, 43),
        _case(wl.Spec("bf16", 256, 16, 2, 1056, wl.HND), [9000, 3000, 0], 4, 44),
    ]
    need = max(
        pad.pad_decode_attn_workspace_size(pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout,
                                                          num_segments=n))
        for c in cases for n in (0, 256, 3))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    pad.pad_decode_attn_workspace_init(ws)
    refs = [oracle_out(c) for c in cases]
    for rnd in range(2):
        for i, c in enumerate(cases):
            for nseg in (0, 256, 3):
                out = run_gpu(c, workspace=ws, num_segments=nseg)
                check(out, refs[i], c.q.dtype, f"shared workspace round {rnd} case {i} nseg={nseg}")
    torch.cuda.synchronize()
    assert int(ws[: 1 << 20].view(torch.int32).abs().sum()) == 0


def test_deterministic():
    c = _case(wl.CONFIGS[2], [5000], 4, 5)
    a = run_gpu(c)
    b = run_gpu(c)
    assert torch.equal(a, b)


# (config, lengths, M, forced segments): merges of 4 to 32 slices, with
# row groups, wide heads and a ragged batch.
# Helpers take part only when the grid is resident at once (at most one
# workgroup per CU), so every case keeps its grid within 256 workgroups.
MERGE_CASES = [
    (2, [4096], 4, 0),
    (2, [4096], 4, 32),
    (4, [3000], 8, 0),
    (4, [2048], 1, 128),
    (5, [9000, 700, 0, 13000], 4, 32),
]


@pytest.mark.parametrize("cfg,lens,M,nseg", MERGE_CASES, ids=[f"m{i}" for i in range(len(MERGE_CASES))])
def test_merge_handover(cfg, lens, M, nseg):
    """Merge helpers that stop waiting at once leave their slices to the
    last segment: the output keeps the same bits and every merge control
    word is left zero."""
    c = _case(wl.CONFIGS[cfg], lens, M, 300 + cfg)
    shape = pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout, num_segments=nseg)
    plan = pad.pad_decode_attn_plan(shape, c.window)
    assert plan["num_segments"] > 1 and plan["merge_slices"] > 1, plan
    ws = torch.empty(pad.pad_decode_attn_workspace_size(shape), dtype=torch.uint8, device=DEV)
    pad.pad_decode_attn_workspace_init(ws)
    ref = oracle_out(c)
    a = run_gpu(c, workspace=ws, num_segments=nseg)
    try:
        pad.pad_set_merge_wait(0)
        b = run_gpu(c, workspace=ws, num_segments=nseg)
        torch.cuda.synchronize()
    finally:
        pad.pad_set_merge_wait(200)
    check(a, ref, c.q.dtype, f"merge slices {plan['merge_slices']}")
    assert torch.equal(a, b), "the fallback merge must give the same bits"
    assert int(ws[: 1 << 20].view(torch.int32).abs().sum()) == 0


# (config, lengths, M, window, segments): batches with ragged, empty and
# windowed sequences.
SCHEDULE_CASES = [
    (5, None, 4, 0, 8),
    (2, [3000, 17, 0, 900, 1], 4, 0, 16),
    (3, [2000, 700, 40], 4, 512, 4),
]


@pytest.mark.parametrize("cfg,lens,M,window,nseg", SCHEDULE_CASES, ids=[f"sch{i}" for i in range(len(SCHEDULE_CASES))])
def test_both_schedules(cfg, lens, M, window, nseg):
    """One workgroup per item and the balanced persistent grid both match
    the oracle, each gives the same bits on every call, and each leaves the
    workspace's control prefix zero."""
    if lens is None:
        c = wl.config_case(cfg, 3000, M, device=DEV)
    else:
        c = _case(wl.CONFIGS[cfg], lens, M, 500 + cfg, window=window)
    ref = oracle_out(c)
    for sched in (pad.PAD_SCHED_GRID, pad.PAD_SCHED_PERSISTENT):
        shape = pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout, num_segments=nseg, schedule=sched)
        plan = pad.pad_decode_attn_plan(shape, c.window)
        assert plan["persistent"] == (sched == pad.PAD_SCHED_PERSISTENT)
        ws = torch.empty(pad.pad_decode_attn_workspace_size(shape), dtype=torch.uint8, device=DEV)
        pad.pad_decode_attn_workspace_init(ws)
        outs = [run_gpu(c, workspace=ws, num_segments=nseg, schedule=sched) for _ in range(3)]
        torch.cuda.synchronize()
        check(outs[0], ref, c.q.dtype, f"schedule {sched}")
        assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2]), "deterministic"
        assert int(ws[: 1 << 20].view(torch.int32).abs().sum()) == 0


# Batches for the balanced persistent grid: a unit split over every share,
# fewer tiles than workgroups, row groups, windows and zero-length
# sequences.
BALANCED_CASES = [
    # spec, lens, M, window
    (wl.CONFIGS[2], [32768], 4, 0),                      # 8 units over 256 shares
    (wl.Spec("bf16", 128, 4, 1, 16, wl.HND), [20000], 1, 0),  # one unit in every share: 256 partials
    (wl.CONFIGS[2], [40, 1, 0, 17], 2, 0),               # 7 tiles per kv head: fewer tiles than workgroups
    (wl.Spec("bf16", 128, 8, 8, 16, wl.HND), [70000, 65000, 90], 1, 0),  # 264-tile shares over 24 units
    (wl.CONFIGS[4], [3000, 900, 0, 2500], 8, 0),         # 4 row groups per kv head
    (wl.CONFIGS[3], [5000, 700, 16384], 4, 512),         # windows, NHD
]


@pytest.mark.parametrize("case", BALANCED_CASES, ids=[f"bal{i}" for i in range(len(BALANCED_CASES))])
def test_balanced_grid(case):
    spec, lens, M, window = case
    c = _case(spec, lens, M, 650 + len(lens) + M, window=window)
    ref = oracle_out(c)
    shape = pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout, schedule=pad.PAD_SCHED_PERSISTENT)
    plan = pad.pad_decode_attn_plan(shape, c.window)
    assert plan["persistent"] == 1
    ws = torch.empty(pad.pad_decode_attn_workspace_size(shape), dtype=torch.uint8, device=DEV)
    pad.pad_decode_attn_workspace_init(ws)
    for it in range(2):
        ws[1 << 20:].fill_(0xFF)  # NaN partials: every slot the merge reads must be written first
        out = run_gpu(c, workspace=ws, schedule=pad.PAD_SCHED_PERSISTENT)
        torch.cuda.synchronize()
        check(out, ref, c.q.dtype, f"balanced grid {lens} M={M} call {it}")
        assert int(ws[: 1 << 20].view(torch.int32).abs().sum()) == 0, "control words left zero"


def test_balanced_grid_long_shares_periodic_cache():
    """Shares longer than the LDS block-id area (4096 tiles) are walked in
    chunks.  Closed form: a sequence of 20M keys whose block table maps
    every page to the same physical block holds 1.25M copies of that
    block's 16 keys, so its softmax gives each copy the same weight and the
    output equals attention over the single 16-key page (oracle).  One unit
    spans all shares: its 256 partials take the 32-lane merge."""
    spec = wl.Spec("bf16", 128, 4, 1, 16, wl.HND)
    base = _case(spec, [16, 16], 1, 4711)
    L = 20 * (1 << 20)
    nb = L // 16
    blk = int(base.block_tables[0][0, 0])
    table = torch.full((2, nb), blk, dtype=torch.int32, device=DEV)
    table[1, 1:] = base.poison_block  # a 16-key sequence beside it
    table[1, 0] = int(base.block_tables[0][1, 0])
    lens = torch.tensor([L, 16], dtype=torch.int32, device=DEV)
    big = wl.Case(spec, base.q, base.kv_cache, [table], lens, base.scale, 0, base.poison_block, base.seed)
    shape = pad.make_shape(big.q, big.kv_cache, table, big.layout, schedule=pad.PAD_SCHED_PERSISTENT)
    plan = pad.pad_decode_attn_plan(shape, 0)
    assert plan["persistent"] == 1 and (nb + 1) // 256 > 4096
    say(f"periodic cache: {L} keys in one block, shares of {(nb + 1) // 256} tiles")
    out = run_gpu(big, schedule=pad.PAD_SCHED_PERSISTENT)
    torch.cuda.synchronize()
    check(out, oracle_out(base), big.q.dtype, "20M keys of one repeated page")


def test_graph_replay():
    c = _case(wl.CONFIGS[4], [2500], 4, 6, instances=2)
    ref = [oracle_out(c, i) for i in range(2)]
    ws = pad.Workspace(c.q.device)
    shape = pad.make_shape(c.q, c.kv_cache, c.block_tables[0], c.layout)
    buf = ws.get(shape)
    eager = run_gpu(c, 0, workspace=buf)
    torch.cuda.synchronize()
    static_out = torch.zeros_like(c.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_gpu(c, 0, workspace=buf, out=static_out)
    for it in range(100):
        static_out.fill_(float("nan"))
        g.replay()
        if it % 10 == 0:
            other = run_gpu(c, 1, workspace=buf)  # eager work between replays
            torch.cuda.synchronize()
            check(other, ref[1], c.q.dtype, f"eager between replays {it}")
        torch.cuda.synchronize()
        assert torch.equal(static_out, eager), f"replay {it} differs from the eager result"
    check(static_out, ref[0], c.q.dtype, "graph replay")


# ------------------------------------------------------ layouts, GQA


def test_hnd_equals_nhd():
    spec = wl.Spec("bf16", 128, 16, 4, 32, wl.HND)
    c = _case(spec, [700, 33], 3, 9)
    out_h = run_gpu(c)
    kv_n = c.kv_cache.permute(0, 2, 1, 3, 4).contiguous()
    out_n = torch.empty_like(out_h)
    pad.pad_decode_attn(c.q, kv_n, c.block_tables[0], c.seq_lens, c.scale, 0, out_n, layout=pad.PAD_NHD)
    assert torch.equal(out_h, out_n)


def test_planted_keys_unit_scale():
    """A dominant key gives unit-scale outputs, so the absolute gate bites:
    planted inside the window it must win; one past the token (causal) or
    one before the window it must be ignored."""
    spec = wl.Spec("bf16", 512, 16, 2, 32, wl.HND, window=64, kv_std=0.5)
    L, M = 1200, 4
    c = _case(spec, [L], M, 21)
    bt = c.block_tables[0].cpu()

    def key(t, kvh):
        return c.kv_cache[int(bt[0, t // 32]), kvh, t % 32]

    for t_star, expect_win in [(L - M - 10, True), (L - M + 1, False), (L - M - 64, False)]:
        q = c.q.clone()
        for kvh in range(2):
            k = key(t_star, kvh)[0].float()
            beta = 60.0 / (k.dot(k).item() * c.scale)
            for g in range(8):
                q[0, 0, kvh * 8 + g] = (beta * k).to(q.dtype)
        c2 = wl.Case(spec, q, c.kv_cache, c.block_tables, c.seq_lens, c.scale, 64, c.poison_block, c.seed)
        out = run_gpu(c2)
        ref = oracle_out(c2)
        check(out, ref, q.dtype, f"planted at {t_star}")
        v = wl.as_f64(key(t_star, 0)[1])
        won = np.abs(ref[0, 0, 0] - v).max() < 1e-2
        assert won == expect_win


# ------------------------------------------------ negative controls


def test_negative_controls_fail_the_checker():
    spec = wl.CONFIGS[2]
    c = _case(spec, [20000], 4, 31)
    ref = oracle_out(c)
    out = run_gpu(c)
    check(out, ref, c.q.dtype, "control baseline")
    assert not passes(torch.zeros_like(out), ref, c.q.dtype), "zero output must fail"
    # wrong GQA map: q heads grouped modulo instead of contiguously
    Hq, Hkv = spec.num_q_heads, spec.num_kv_heads
    G = Hq // Hkv
    perm = [(h % Hkv) * G + h // Hkv for h in range(Hq)]
    wrong = run_gpu(wl.Case(spec, c.q[:, :, perm].contiguous(), c.kv_cache, c.block_tables, c.seq_lens,
                            c.scale, 0, c.poison_block, c.seed))
    inv = np.argsort(perm)
    assert not passes(wrong[:, :, inv], ref, c.q.dtype), "wrong GQA map must fail"
    # off-by-one causal mask (every row one position early), on a short
    # context where one key carries visible weight
    s2 = _case(spec, [60, 45], 4, 32)
    ref2 = oracle_out(s2)
    early = wl.Case(spec, s2.q, s2.kv_cache, s2.block_tables, s2.seq_lens - 1, s2.scale, 0, s2.poison_block,
                    s2.seed)
    assert not passes(run_gpu(early), ref2, s2.q.dtype), "off-by-one mask must fail"


# ---------------------------------------------- full benchmark sizes


POOL = 512 << 20


@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("ctx", [4096, 32768])
def test_config2_full(ctx, M):
    say(f"config 2 full: L={ctx} M={M} pool=512MiB")
    inst = max(1, (POOL // wl.CONFIGS[2].block_bytes) // (ctx // 16))
    c = wl.config_case(2, ctx, M, device=DEV, instances=inst, pool_bytes=POOL)
    for i in sorted({0, inst - 1}):
        check(run_gpu(c, i), oracle_out(c, i), c.q.dtype, f"config2 L={ctx} M={M} inst={i}")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_config4_full(M):
    ctx = 32768
    say(f"config 4 full: L={ctx} M={M}")
    c = wl.config_case(4, ctx, M, device=DEV, instances=1, pool_bytes=POOL)
    check(run_gpu(c), oracle_out(c), c.q.dtype, f"config4 L={ctx} M={M}")


def test_config5_full_sampled():
    say("config 5 full: 64 seqs L~U[512,16384] + padded, P1056")
    c = wl.config_case(5, 16384, 4, device=DEV)
    out = run_gpu(c)
    assert torch.all(out[-1] == 0)
    lens = c.seq_lens.tolist()
    order = np.argsort(lens[:-1])
    pick = [int(order[0]), int(order[len(order) // 2]), int(order[-1]), 3, 64]
    ref = oracle_out(c, 0, seqs=pick)
    check(out[pick], ref, c.q.dtype, f"config5 seqs {pick}")


# ------------------------------------------- dot-product family (G*M <= 4)


DOT_SHAPES = [
    # D, Hq, Hkv, P, dtype, layout, lens, M, window
    (64, 4, 1, 16, "fp16", wl.HND, [256], 1, 0),          # config 1
    (128, 32, 8, 16, "bf16", wl.HND, [4096], 1, 0),       # config 2, M = 1
    (128, 8, 4, 32, "fp16", wl.NHD, [777, 0, 5], 2, 0),   # padded and short sequences
    (64, 2, 2, 16, "bf16", wl.HND, [300, 41], 3, 17),     # 3 rows, window
    (128, 4, 4, 48, "bf16", wl.HND, [2, 1000], 4, 0),     # L < M rows
    (64, 8, 2, 528, "fp16", wl.HND, [1100], 1, 0),
]


@pytest.mark.parametrize("shape", DOT_SHAPES, ids=[f"d{i}" for i in range(len(DOT_SHAPES))])
@pytest.mark.parametrize("nseg", [0, 1, 5])
def test_dot_path(shape, nseg):
    D, Hq, Hkv, P, dt, layout, lens, M, W = shape
    spec = wl.Spec(dt, D, Hq, Hkv, P, layout, window=W)
    c = _case(spec, lens, M, 777 + D + Hq + M)
    ref = oracle_out(c)
    out_dot = run_gpu(c, path=pad.PAD_PATH_DOT, num_segments=nseg)
    check(out_dot, ref, c.q.dtype, f"dot path {shape} nseg={nseg}")
    out_mfma = run_gpu(c, path=pad.PAD_PATH_MFMA, num_segments=nseg)
    check(out_mfma, ref, c.q.dtype, f"mfma path {shape} nseg={nseg}")
    assert float((out_dot.float() - out_mfma.float()).abs().max()) <= 2 * ABS_TOL[c.q.dtype]


def test_dot_path_full_config2():
    say("config 2 full, M=1, dot family")
    c = wl.config_case(2, 32768, 1, device=DEV, instances=2, pool_bytes=POOL)
    check(run_gpu(c, 1, path=pad.PAD_PATH_DOT), oracle_out(c, 1), c.q.dtype, "dot config2 L=32768 M=1")
