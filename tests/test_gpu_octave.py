"""The quantized ("octave") packed cache on the HIP path, through the C ABI,
against the fp64 oracle (oracle/octave.py) on seeded inputs.

* Decode over a packed cache the oracle encoded: every format, both
  dtypes of q/out, both layouts, both schedules, forced segment counts,
  row groups, padded and short sequences (rows with no key).  Slots past a
  sequence's end and the never-read block hold NaN steps: they must not
  reach the output.
* The store kernel against the oracle's encoder: steps and codes equal,
  except where the value sits within rounding of a decision boundary
  (either neighbour is correct there); skipped and other slots untouched.
* Store then decode on the GPU against encode then decode in the oracle.
"""

import numpy as np
import pytest
import torch

import paged_kv_decode_block_amd as pad
import workloads as wl
from gpu_check import check, say
from oracle import octave as oc

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = {pad.PAD_KV_OCTAVE_K3V4: "octave_k3v4", pad.PAD_KV_OCTAVE_K3V3: "octave_k3v3",
         pad.PAD_KV_OCTAVE_K3V3_COMPACT: "octave_k3v3_compact"}


def _signs(seed):
    w = wl.sign_words(seed)
    return w, oc.signs_from_bits(w.numpy().view(np.uint32), 256)


def _packed_case(fmt, dtype, layout, lens, M, Hq, Hkv, P, seed, **kw):
    """Host case, its cache encoded by the oracle, slots of NaN rows set to
    all-ones bytes (NaN steps)."""
    spec = wl.Spec(dtype, 256, Hq, Hkv, P, layout)
    c = wl.make_case(spec, lens, M, seed=seed, device="cpu", **kw)
    kw_, sk = _signs(seed + 1)
    vw_, sv = _signs(seed + 2)
    kv = c.kv_cache.to(torch.float64).numpy()
    bad = np.isnan(kv).any(axis=(-1, -2))
    with np.errstate(invalid="ignore"):
        packed = oc.encode_rows(np.nan_to_num(kv[..., 0, :]), np.nan_to_num(kv[..., 1, :]), sk, sv, NAMES[fmt])
    packed[bad] = 0xFF
    return c, packed, kw_, vw_, sk, sv


def _oracle(c, packed, fmt, sk, sv, seqs=None):
    bt = c.block_tables[0].numpy()
    idx = list(range(c.num_seqs)) if seqs is None else list(seqs)
    sub = bt[idx]
    used = np.unique(sub)
    remap = {int(b): i for i, b in enumerate(used)}
    table = np.vectorize(lambda b: remap[int(b)], otypes=[np.int64])(sub)
    lens = c.seq_lens.numpy()[idx]
    q64 = c.q[idx].to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):
        return oc.decode_attention_quant(q64, packed[used], table, lens, c.scale, c.layout, NAMES[fmt], sk, sv)


def _run(c, packed, fmt, kw_, vw_, **kw):
    q = c.q.to(DEV)
    out = torch.full_like(q, float("nan"))
    pad.pad_decode_attn_octave(q, torch.from_numpy(packed).to(DEV), c.block_tables[0].to(DEV), c.seq_lens.to(DEV),
                               kw_.to(DEV), vw_.to(DEV), c.scale, out, fmt, layout=c.layout, **kw)
    torch.cuda.synchronize()
    return out


CASES = [
    # fmt, dtype, layout, lens, M, Hq, Hkv, P, run kwargs
    (1, "bf16", wl.HND, [3000, 17, 0, 1200], 4, 16, 2, 32, {}),
    (2, "fp16", wl.NHD, [2100], 1, 8, 2, 16, {}),
    (3, "bf16", wl.HND, [1500, 800], 8, 16, 2, 1056, {}),           # 64 rows: two row groups
    (1, "fp16", wl.HND, [5, 3, 40], 4, 8, 2, 16, {}),               # L < M: rows with no key
    (1, "bf16", wl.NHD, [2500], 2, 16, 2, 32, {"num_segments": 1}),
    (2, "bf16", wl.HND, [2500], 2, 16, 2, 32, {"num_segments": 17}),
    (3, "fp16", wl.HND, [4000, 900, 0, 2000], 4, 16, 2, 544, {"schedule": pad.PAD_SCHED_PERSISTENT}),
    (1, "bf16", wl.HND, [4000, 900, 0, 2000], 4, 16, 2, 544, {"schedule": pad.PAD_SCHED_GRID, "num_segments": 5}),
    (1, "bf16", wl.HND, [1200, 30], 40, 16, 2, 32, {}),                # a 40-token chunk: 320 rows, 20 row groups
    (3, "fp16", wl.NHD, [2500], 24, 8, 2, 16, {"schedule": pad.PAD_SCHED_PERSISTENT}),
]


@pytest.mark.parametrize("case", CASES, ids=[f"o{i}" for i in range(len(CASES))])
def test_decode_matches_oracle(case):
    fmt, dt, layout, lens, M, Hq, Hkv, P, kw = case
    say(f"octave decode: {NAMES[fmt]} {dt} layout={layout} lens={lens} M={M} {Hq}/{Hkv} P={P} {kw}")
    c, packed, kw_, vw_, sk, sv = _packed_case(fmt, dt, layout, lens, M, Hq, Hkv, P, 900 + fmt + M + len(lens))
    out = _run(c, packed, fmt, kw_, vw_, **kw)
    check(out, _oracle(c, packed, fmt, sk, sv), c.q.dtype, f"octave {NAMES[fmt]} {dt}")
    if 0 in lens:
        assert torch.all(out[lens.index(0)] == 0)


def test_decode_batch_workload_shapes():
    """64 sequences of 512..4000 keys plus a padded one, the batch
    workload's heads and page size (16/2 heads of 256, page 1056, M=4),
    k3v4 bf16: the balanced persistent grid."""
    g = torch.Generator().manual_seed(77)
    lens = torch.randint(512, 4001, (64,), generator=g).tolist() + [0]
    c, packed, kw_, vw_, sk, sv = _packed_case(1, "bf16", wl.HND, lens, 4, 16, 2, 1056, 4242)
    say("octave decode: batch of 64 + 1 padded, k3v4 bf16, page 1056")
    out = _run(c, packed, 1, kw_, vw_)
    assert torch.all(out[64] == 0)
    pick = [0, 13, 31, 47, 63]
    check(out[pick], _oracle(c, packed, 1, sk, sv, seqs=pick), c.q.dtype, "octave batch (5 sequences)")


@pytest.mark.parametrize("fmt", [1, 3])
def test_decode_batch_poisoned_workspace(fmt):
    """The balanced persistent grid at two workgroups per CU on a 64-sequence
    batch (lengths 512..3000, 16/2 heads of 256, page 1056, M=4) with an
    explicit workspace whose partial area is NaN-filled before every call:
    three calls give the same bits, the control words are left zero, and
    eight sequences (the longest among them) match the oracle."""
    g = torch.Generator().manual_seed(78 + fmt)
    lens = torch.randint(512, 3001, (64,), generator=g).tolist() + [0]
    c, packed, kw_, vw_, sk, sv = _packed_case(fmt, "bf16", wl.HND, lens, 4, 16, 2, 1056, 4300 + fmt)
    q = c.q.to(DEV)
    cache = torch.from_numpy(packed).to(DEV)
    bt, sl = c.block_tables[0].to(DEV), c.seq_lens.to(DEV)
    shape = pad._octave_shape(q, cache, bt, c.layout, fmt)
    need = pad.pad_decode_attn_octave_workspace_size(shape, fmt)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    pad.pad_decode_attn_workspace_init(ws)
    say(f"octave batch, {NAMES[fmt]}: 64 + 1 padded, workspace {need} B poisoned before each call")
    outs = []
    for _ in range(3):
        ws[1 << 20:].fill_(0xFF)
        out = torch.full_like(q, float("nan"))
        pad.pad_decode_attn_octave(q, cache, bt, sl, kw_.to(DEV), vw_.to(DEV), c.scale, out, fmt, layout=c.layout,
                                   workspace=ws)
        torch.cuda.synchronize()
        outs.append(out)
        assert int(ws[: 1 << 20].view(torch.int32).abs().sum()) == 0, "control words must be left zero"
    assert all(torch.equal(outs[0], o) for o in outs[1:]), "repeated calls must give the same bits"
    assert torch.all(outs[0][64] == 0)
    longest = int(np.argmax(lens[:64]))
    pick = sorted({0, 9, 21, 33, 42, 55, 63, longest})
    check(outs[0][pick], _oracle(c, packed, fmt, sk, sv, seqs=pick), c.q.dtype, f"octave batch {NAMES[fmt]}")


def test_graph_replay_packed():
    """A packed-cache (k3v4) call on the balanced grid (two workgroups per
    CU) captured in a HIP graph and replayed 20 times, with eager calls on
    the grid schedule through the same workspace between replays: every
    replay gives the eager call's bits, and the control words end zero."""
    g = torch.Generator().manual_seed(91)
    lens = torch.randint(512, 2001, (16,), generator=g).tolist() + [0]
    c, packed, kw_, vw_, sk, sv = _packed_case(1, "bf16", wl.HND, lens, 4, 16, 2, 544, 4400)
    q = c.q.to(DEV)
    cache = torch.from_numpy(packed).to(DEV)
    bt, sl, ks, vs = c.block_tables[0].to(DEV), c.seq_lens.to(DEV), kw_.to(DEV), vw_.to(DEV)
    need = max(pad.pad_decode_attn_octave_workspace_size(pad._octave_shape(q, cache, bt, c.layout, 1, schedule=sch), 1)
               for sch in (pad.PAD_SCHED_PERSISTENT, pad.PAD_SCHED_GRID))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    pad.pad_decode_attn_workspace_init(ws)

    def call(out, sch):
        pad.pad_decode_attn_octave(q, cache, bt, sl, ks, vs, c.scale, out, 1, layout=c.layout, workspace=ws,
                                   schedule=sch)
        return out

    say("octave graph replay: 16 + 1 padded sequences, k3v4 bf16, persistent schedule captured")
    eager = call(torch.empty_like(q), pad.PAD_SCHED_PERSISTENT)
    grid_ref = call(torch.empty_like(q), pad.PAD_SCHED_GRID)
    torch.cuda.synchronize()
    static_out = torch.zeros_like(q)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static_out, pad.PAD_SCHED_PERSISTENT)
    for it in range(20):
        static_out.fill_(float("nan"))
        graph.replay()
        if it % 5 == 0:
            other = call(torch.empty_like(q), pad.PAD_SCHED_GRID)  # eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(other, grid_ref), f"eager grid call {it} changed"
        torch.cuda.synchronize()
        assert torch.equal(static_out, eager), f"replay {it} differs from the eager result"
    assert int(ws[: 1 << 20].view(torch.int32).abs().sum()) == 0, "control words must be left zero"
    pick = [0, 5, 11, 15]
    check(static_out[pick], _oracle(c, packed, 1, sk, sv, seqs=pick), c.q.dtype, "octave graph replay")
    assert torch.all(static_out[16] == 0)


VARLEN_CASES = [
    # fmt, dtype, layout, lens, counts, schedule
    (1, "bf16", wl.HND, [1500, 40, 0, 900, 2600, 3], [1, 4, 2, 0, 3, 4], pad.PAD_SCHED_AUTO),
    (3, "fp16", wl.NHD, [700, 1200, 64], [2, 1, 4], pad.PAD_SCHED_PERSISTENT),
    (2, "bf16", wl.HND, [2000, 33, 900], [4, 2, 1], pad.PAD_SCHED_GRID),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[f"v{i}" for i in range(len(VARLEN_CASES))])
def test_decode_varlen_matches_oracle(case):
    """A query count per sequence over a packed cache
    (pad_decode_attn_octave_varlen): sequence s owns its packed rows and its
    M_s tokens sit at the last M_s positions; each sequence against the
    oracle's own call with M_s tokens.  A count of 0 skips the sequence, a
    padded sequence gets zero rows, L < M rows see no key, and the three
    leading rows no sequence owns are left untouched."""
    fmt, dt, layout, lens, counts, sched = case
    mmax = max(counts)
    say(f"octave varlen: {NAMES[fmt]} {dt} layout={layout} lens={lens} counts={counts} schedule={sched}")
    c, packed, kw_, vw_, sk, sv = _packed_case(fmt, dt, layout, lens, mmax, 16, 2, 32, 9500 + fmt + len(lens))
    lead = 3
    rows = [c.q[s, :m] for s, m in enumerate(counts)]
    q_packed = torch.cat([torch.zeros((lead,) + tuple(c.q.shape[2:]), dtype=c.q.dtype)] + rows).to(DEV)
    starts = np.concatenate([[lead], lead + np.cumsum(counts)]).astype(np.int32)
    out = torch.full_like(q_packed, float("nan"))
    pad.pad_decode_attn_octave_varlen(q_packed, torch.from_numpy(starts).to(DEV), torch.from_numpy(packed).to(DEV),
                                      c.block_tables[0].to(DEV), c.seq_lens.to(DEV), kw_.to(DEV), vw_.to(DEV),
                                      c.scale, out, fmt, max_query_len=mmax, layout=layout, schedule=sched)
    torch.cuda.synchronize()
    assert torch.isnan(out[:lead]).all(), "rows no sequence owns are left untouched"
    bt = c.block_tables[0].numpy()
    for s, (L, m) in enumerate(zip(lens, counts)):
        if m == 0:
            continue
        got = out[starts[s]:starts[s + 1]]
        if L == 0:
            assert torch.all(got == 0), "padded sequence must be zero"
            continue
        used = np.unique(bt[s])
        table = np.searchsorted(used, bt[s])[None, :]
        q64 = c.q[s:s + 1, :m].to(torch.float64).numpy()
        with np.errstate(invalid="ignore"):
            ref = oc.decode_attention_quant(q64, packed[used], table, [L], c.scale, layout, NAMES[fmt], sk, sv)
        check(got[None], ref, c.q.dtype, f"octave varlen seq {s} (L={L}, M={m})")


def _ambiguous(x, step):
    r = x / np.where(step > 0, step, 1.0)
    return np.abs(r - np.round(r)) < 1e-4


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("dtype,layout", [("bf16", wl.HND), ("fp16", wl.NHD)])
def test_cache_write_matches_encoder(fmt, dtype, layout):
    T, Hkv, P, nb = 300, 2, 16, 40
    say(f"octave store: {NAMES[fmt]} {dtype} layout={layout} T={T}")
    g = torch.Generator().manual_seed(31 + fmt)
    tdt = wl._DTYPES[dtype]
    key = torch.randn((T, Hkv, 256), generator=g).to(tdt)
    value = (torch.randn((T, Hkv, 256), generator=g) * 0.5).to(tdt)
    slots = torch.randperm(nb * P, generator=g)[:T].to(torch.int64)
    slots[5] = -1                 # padding token: skipped
    slots[7] = nb * P             # past the cache: skipped
    kw_, sk = _signs(500 + fmt)
    vw_, sv = _signs(600 + fmt)
    sb = pad.pad_octave_slot_bytes(fmt)
    shape = (nb, Hkv, P, sb) if layout == wl.HND else (nb, P, Hkv, sb)
    cache = torch.full(shape, 0xAB, dtype=torch.uint8, device=DEV)
    pad.pad_octave_cache_write(key.to(DEV), value.to(DEV), cache, slots.to(DEV), kw_.to(DEV), vw_.to(DEV), fmt,
                               layout=layout)
    torch.cuda.synchronize()
    got_all = cache.cpu().numpy()
    name = NAMES[fmt]
    kb, vb, compact = oc.FORMATS[name]
    gk = 256 if compact else 64
    k64, v64 = key.to(torch.float64).numpy(), value.to(torch.float64).numpy()
    want = oc.encode_rows(k64, v64, sk, sv, name)
    kr = oc.rotate(k64, sk, gk)
    vr = oc.rotate(v64, sv, 256)
    written = np.zeros(got_all.shape[:-1], dtype=bool)
    n_codes = n_equal = 0
    for t in range(T):
        s = int(slots[t])
        if s < 0 or s >= nb * P:
            continue
        blk, off = divmod(s, P)
        for h in range(Hkv):
            got = got_all[blk, h, off] if layout == wl.HND else got_all[blk, off, h]
            written[(blk, h, off) if layout == wl.HND else (blk, off, h)] = True
            w = want[t, h]
            nk, nv = kb * 32, vb * 32
            ng = 256 // gk
            st_got = got[nk + nv: nk + nv + 2 * (ng + 1)].view(np.float16).astype(np.float64)
            st_want = w[nk + nv: nk + nv + 2 * (ng + 1)].view(np.float16).astype(np.float64)
            assert np.all(got[nk + nv + 2 * (ng + 1):] == 0), "padding bytes are zero"
            kc_got, kc_want = oc.unpack_codes(got[:nk], kb, 256), oc.unpack_codes(w[:nk], kb, 256)
            vc_got, vc_want = oc.unpack_codes(got[nk:nk + nv], vb, 256), oc.unpack_codes(w[nk:nk + nv], vb, 256)
            # a step may differ only where absmax / 2^(b-1) is within rounding of an fp16 midpoint
            for i in range(ng + 1):
                if st_got[i] != st_want[i]:
                    a = np.abs(kr[t, h, i * gk:(i + 1) * gk]).max() / 4 if i < ng else np.abs(vr[t, h]).max() / (1 << (vb - 1))
                    assert abs(st_got[i] - st_want[i]) <= 2 ** -10 * a and abs(a - (st_got[i] + st_want[i]) / 2) < 1e-6 * a
            for codes_g, codes_w, x, steps, groups in ((kc_got, kc_want, kr[t, h], st_got[:ng], ng),
                                                        (vc_got, vc_want, vr[t, h], st_got[ng:], 1)):
                step = np.repeat(steps, 256 // groups)
                diff = codes_g != codes_w
                n_codes += codes_g.size
                n_equal += int((~diff).sum())
                assert np.all(~diff | _ambiguous(x, step) | (np.repeat(st_got[:ng] if groups == ng else st_got[ng:], 256 // groups) != np.repeat(st_want[:ng] if groups == ng else st_want[ng:], 256 // groups)))
                assert np.all(np.abs(codes_g - codes_w) <= 1)
    assert np.all(got_all[~written] == 0xAB), "slots of skipped tokens and unused slots are untouched"
    assert n_equal >= 0.999 * n_codes
    say(f"  codes equal: {n_equal}/{n_codes}")


@pytest.mark.parametrize("fmt,dtype", [(1, "bf16"), (3, "fp16")])
def test_store_then_decode(fmt, dtype):
    """New tokens stored by the GPU, then decoded by the GPU, against the
    oracle's encode-then-decode of the same rows (a code taken on the
    other side of a decision boundary moves an output by far less than
    the tolerance at these lengths)."""
    spec = wl.Spec(dtype, 256, 16, 2, 32, wl.HND)
    lens, M = [900, 600], 4
    c = wl.make_case(spec, lens, M, seed=71 + fmt, device="cpu", poison_tail=False)
    kw_, sk = _signs(81 + fmt)
    vw_, sv = _signs(91 + fmt)
    nb = c.kv_cache.shape[0]
    # token rows in the order of their slots: slot = block * P + offset
    kv = c.kv_cache.permute(0, 2, 1, 3, 4).reshape(nb * 32, 2, 2, 256)  # [slot, Hkv, 2, D]
    slots = torch.arange(nb * 32, dtype=torch.int64)
    sb = pad.pad_octave_slot_bytes(fmt)
    cache = torch.zeros((nb, 2, 32, sb), dtype=torch.uint8, device=DEV)
    say(f"octave store then decode: {NAMES[fmt]} {dtype}")
    pad.pad_octave_cache_write(kv[:, :, 0].contiguous().to(DEV), kv[:, :, 1].contiguous().to(DEV), cache,
                               slots.to(DEV), kw_.to(DEV), vw_.to(DEV), fmt)
    q = c.q.to(DEV)
    out = torch.empty_like(q)
    pad.pad_decode_attn_octave(q, cache, c.block_tables[0].to(DEV), c.seq_lens.to(DEV), kw_.to(DEV), vw_.to(DEV),
                               c.scale, out, fmt)
    torch.cuda.synchronize()
    kv64 = c.kv_cache.to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):
        packed = oc.encode_rows(np.nan_to_num(kv64[..., 0, :]), np.nan_to_num(kv64[..., 1, :]), sk, sv, NAMES[fmt])
    check(out, _oracle(c, packed, fmt, sk, sv), c.q.dtype, f"store then decode {NAMES[fmt]}")
