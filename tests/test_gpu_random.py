"""Seeded random shapes on the HIP path against the fp64 oracle: head sizes,
GQA ratios, query counts, page sizes, layouts, dtypes, windows, lengths
(including 0 and L < M), forced segment counts, both schedules, both
kernel families and packed per-sequence queries.  Sizes stay small enough
for the oracle to finish in seconds."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_block_amd as pad
import workloads as wl
from gpu_check import check, oracle_out, run_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 40


def _draw(i):
    r = np.random.default_rng(5000 + i)
    D = int(r.choice([64, 128, 256, 512]))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8, 16]))
    M = int(r.integers(1, 9))
    P = int(r.choice([16, 32, 48, 64, 1056]))
    layout = int(r.choice([wl.HND, wl.NHD]))
    dtype = str(r.choice(["fp16", "bf16"]))
    S = int(r.integers(1, 5))
    lens = [int(x) for x in r.integers(0, 2500, size=S)]
    if r.random() < 0.3:
        lens[int(r.integers(0, S))] = int(r.integers(0, M + 1))  # empty or shorter than M
    window = int(r.choice([0, 0, 1, 7, 100, 700]))
    nseg = int(r.choice([0, 0, 1, 3, 16]))
    schedule = int(r.choice([pad.PAD_SCHED_AUTO, pad.PAD_SCHED_GRID, pad.PAD_SCHED_PERSISTENT]))
    path = pad.PAD_PATH_DOT if (G * M <= 4 and D <= 128 and r.random() < 0.5) else pad.PAD_PATH_AUTO
    varlen = bool(r.random() < 0.3)
    counts = [int(x) for x in r.integers(0, M + 1, size=S)] if varlen else None
    return D, Hkv, G, M, P, layout, dtype, S, lens, window, nseg, schedule, path, counts


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    D, Hkv, G, M, P, layout, dtype, S, lens, window, nseg, schedule, path, counts = _draw(i)
    if counts is not None and path == pad.PAD_PATH_DOT:
        path = pad.PAD_PATH_AUTO
    if path == pad.PAD_PATH_DOT and schedule == pad.PAD_SCHED_PERSISTENT:
        schedule = pad.PAD_SCHED_GRID  # the dot family runs on the grid schedule only
    say(f"random {i}: D={D} Hkv={Hkv} G={G} M={M} P={P} layout={layout} {dtype} lens={lens} window={window} "
        f"nseg={nseg} schedule={schedule} path={path} counts={counts}")
    spec = wl.Spec(dtype, D, G * Hkv, Hkv, P, layout)
    c = wl.make_case(spec, lens, M, seed=7000 + i, device=DEV, window=window)
    if counts is None:
        out = run_gpu(c, num_segments=nseg, path=path, schedule=schedule)
        check(out, oracle_out(c), c.q.dtype, f"random {i}")
        return
    q = torch.cat([c.q[s, :n] for s, n in enumerate(counts)], dim=0).contiguous()
    starts = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    if q.shape[0] == 0:
        return  # no query token in the whole batch
    out = torch.full_like(q, float("nan"))
    pad.pad_decode_attn_varlen(q, torch.from_numpy(starts).to(DEV), c.kv_cache, c.block_tables[0], c.seq_lens,
                               c.scale, c.window, out, max_query_len=M, layout=c.layout, num_segments=nseg,
                               path=path, schedule=schedule)
    kv64, table, lens64 = wl.compact(c)
    ref = oracle.decode_attention_varlen(wl.as_f64(q), starts, kv64, table, lens64, c.scale, c.window, c.layout)
    check(out, ref, c.q.dtype, f"random varlen {i}")
