"""The KV-cache write with its rotation on the HIP path, through the C ABI,
against the fp64 oracle (oracle/rope.py): stored K within one rounding of
the dtype, V and unrotated elements bit-exact, skipped and foreign slots
untouched, query rows rotated in place; and a decode call over keys
written this way."""

import numpy as np
import pytest
import torch

import oracle
from oracle import rope as orope
import paged_kv_decode_block_amd as pad
import workloads as wl
from gpu_check import check, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
EPS = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}  # unit roundoff


def _table(max_pos, rope_dim):
    half = rope_dim // 2
    inv = 10000.0 ** (-np.arange(half) * 2.0 / rope_dim)
    ang = np.arange(max_pos)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def _close(got, want, dtype, what):
    """Each element within one rounding to the dtype (two units of
    roundoff, relative) of the fp64 value, plus the fp32 arithmetic's own
    error where the two products of a rotation cancel (2^-20 absolute for
    unit-scale inputs)."""
    g = got.detach().cpu().to(torch.float64).numpy()
    err = np.abs(g - want)
    bound = 2 * EPS[dtype] * np.abs(want) + 2.0 ** -20
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off, worst {float((err - bound).max())}"


CASES = [  # (dtype, layout, D, Hkv, G, P, rope_dim, T)
    (torch.bfloat16, wl.HND, 128, 8, 4, 16, 128, 300),
    (torch.bfloat16, wl.NHD, 256, 2, 8, 32, 64, 97),
    (torch.float16, wl.HND, 64, 1, 4, 16, 32, 50),
    (torch.float16, wl.NHD, 512, 2, 8, 32, 0, 33),
    (torch.bfloat16, wl.HND, 256, 2, 8, 1056, 16, 1500),
]


@pytest.mark.parametrize("case", CASES, ids=[f"w{i}" for i in range(len(CASES))])
def test_cache_write_against_oracle(case):
    dtype, layout, D, Hkv, G, P, rd, T = case
    say(f"cache write: {dtype} layout={layout} D={D} Hkv={Hkv} G={G} P={P} rope_dim={rd} T={T}")
    g = torch.Generator().manual_seed(1000 + D + rd + T)
    nb = -(-2 * T // P) + 2
    cap = nb * P
    key = torch.randn((T, Hkv, D), generator=g).to(dtype)
    val = torch.randn((T, Hkv, D), generator=g).to(dtype)
    q = torch.randn((T, Hkv * G, D), generator=g).to(dtype)
    slots = torch.randperm(cap, generator=g)[:T].to(torch.int64)
    slots[torch.rand(T, generator=g) < 0.1] = -1  # padding tokens
    max_pos = 4096
    pos = torch.randint(0, max_pos, (T,), generator=g, dtype=torch.int64)
    tab = _table(max_pos, rd) if rd else None
    shape = (nb, Hkv, P, 2, D) if layout == wl.HND else (nb, P, Hkv, 2, D)
    cache0 = torch.randn(shape, generator=g).to(dtype)  # every slot starts with distinct values

    kv = cache0.to(DEV)
    qd = q.to(DEV)
    pad.pad_rope_cache_write(key.to(DEV), val.to(DEV), kv, slots.to(DEV), layout=layout, q=qd,
                             positions=pos.to(DEV) if rd else None,
                             cos_sin_cache=torch.from_numpy(tab).to(DEV) if rd else None)
    torch.cuda.synchronize()

    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    want, q_want = orope.cache_write(f64(cache0), layout, f64(key), f64(val), slots.numpy(), pos.numpy(), tab, rd,
                                     f64(q))
    got = kv.cpu()
    # slots no token was written to keep their contents, bit for bit
    written = slots >= 0
    keep = np.ones(cap, dtype=bool)
    keep[slots[written].numpy()] = False
    if layout == wl.HND:
        at = lambda s: (s // P, slice(None), s % P)  # noqa: E731
    else:
        at = lambda s: (s // P, s % P, slice(None))  # noqa: E731
    for s in np.nonzero(keep)[0][:200]:
        assert torch.equal(got[at(int(s))], cache0[at(int(s))]), f"slot {s} changed"
    # V halves bit-exact; K rotated part within one rounding, the rest bit-exact
    kk, vv = got[:, :, :, 0], got[:, :, :, 1]
    kw, vw = want[:, :, :, 0], want[:, :, :, 1]
    assert np.array_equal(f64(vv), vw), "V halves"
    _close(kk[..., :rd], kw[..., :rd], dtype, "rotated K")
    assert np.array_equal(f64(kk[..., rd:]), kw[..., rd:]), "unrotated K"
    qg = qd.cpu()
    _close(qg[..., :rd], q_want[..., :rd], dtype, "rotated q")
    assert torch.equal(qg[..., rd:], q[..., rd:]), "unrotated q"


def test_empty_mapping_writes_nothing():
    kv = torch.zeros((2, 1, 16, 2, 64), dtype=torch.bfloat16, device=DEV)
    key = torch.ones((0, 1, 64), dtype=torch.bfloat16, device=DEV)
    pad.pad_rope_cache_write(key, key.clone(), kv, torch.zeros(0, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert not kv.any()


def test_decode_reads_what_the_write_stored():
    """Tokens stored through the cache write, then decoded: matches the
    oracle run on the oracle's own stored cache."""
    spec = wl.CONFIGS[2]
    c = wl.make_case(spec, [700], 4, seed=77, device=DEV)
    say("write-then-decode: config 2 shapes, 700 keys, M=4")
    L, Hkv, D, P = 700, spec.num_kv_heads, spec.head_size, spec.page_size
    g = torch.Generator().manual_seed(78)
    key = torch.randn((L, Hkv, D), generator=g).to(torch.bfloat16)
    val = torch.randn((L, Hkv, D), generator=g).to(torch.bfloat16)
    table = c.block_tables[0][0].cpu().to(torch.int64)
    t = torch.arange(L, dtype=torch.int64)
    slots = table[t // P] * P + t % P
    rd, max_pos = 64, 1024
    tab = _table(max_pos, rd)
    cache_before = c.kv_cache.cpu()
    pad.pad_rope_cache_write(key.to(DEV), val.to(DEV), c.kv_cache, slots.to(DEV), layout=c.layout,
                             positions=t.to(DEV), cos_sin_cache=torch.from_numpy(tab).to(DEV))
    out = torch.full_like(c.q, float("nan"))
    pad.pad_decode_attn(c.q, c.kv_cache, c.block_tables[0], c.seq_lens, c.scale, 0, out, layout=c.layout)
    torch.cuda.synchronize()
    # the oracle: its own cache write (rounded to the dtype like any stored key), then its attention
    f64 = lambda x: x.to(torch.float64).numpy()  # noqa: E731
    want_cache, _ = orope.cache_write(f64(cache_before), c.layout, f64(key), f64(val), slots.numpy(), t.numpy(), tab,
                                      rd)
    stored = torch.from_numpy(want_cache).to(torch.bfloat16).to(torch.float64).numpy()
    ref = oracle.decode_attention(wl.as_f64(c.q), stored, c.block_tables[0].cpu().numpy(), [L], c.scale, 0, c.layout)
    check(out, ref, torch.bfloat16, "decode after write")
