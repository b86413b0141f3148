"""Pins for the fp64 oracle: properties fixed by the pages and by mathematics.

Each ``pin_*`` takes the oracle functions it checks as arguments, so the
same pins run against the real oracle (tests/test_oracle.py) and against
oracle copies with a planted mistake (tests/test_oracle_mutants.py), which
must fail at least one pin.  Every pin raises ``AssertionError`` on failure.
"""

from __future__ import annotations

import math

import numpy as np
import torch

HND, NHD = 1, 0


def tiny_case(rng, S=2, M=3, Hq=4, Hkv=2, D=8, P=16, lens=(37, 20), layout=HND, spare=3):
    """Random fp64 inputs with a shuffled block table over a small pool."""
    need = [-(-L // P) for L in lens]
    maxb = max(1, max(need))
    nb = sum(need) + spare
    perm = rng.permutation(nb)
    table = np.full((S, maxb), nb - 1, dtype=np.int64)
    c = 0
    for s in range(S):
        table[s, : need[s]] = perm[c : c + need[s]]
        c += need[s]
    shape = (nb, Hkv, P, 2, D) if layout == HND else (nb, P, Hkv, 2, D)
    kv = rng.standard_normal(shape)
    q = rng.standard_normal((S, M, Hq, D))
    return q, kv, table, np.asarray(lens, dtype=np.int64)


def to_nhd(kv_hnd):
    return np.ascontiguousarray(np.transpose(kv_hnd, (0, 2, 1, 3, 4)))


def brute_force(q, kv, table, lens, scale, window, layout):
    """Pure-Python loop over every (sequence, token, head, key) with the
    visibility predicate written directly: key t is visible to the token at
    position p iff t <= p and (window == 0 or p - t < window)."""
    S, M, Hq, D = q.shape
    P = kv.shape[2] if layout == HND else kv.shape[1]
    Hkv = kv.shape[1] if layout == HND else kv.shape[2]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for s in range(S):
        L = int(lens[s])
        for m in range(M):
            p = L - M + m
            for h in range(Hq):
                kvh = h // G
                zs, vs = [], []
                for t in range(L):
                    if not (t <= p and (window == 0 or p - t < window)):
                        continue
                    b, o = int(table[s, t // P]), t % P
                    sl = kv[b, kvh, o] if layout == HND else kv[b, o, kvh]
                    zs.append(scale * sum(float(q[s, m, h, d]) * float(sl[0, d]) for d in range(D)))
                    vs.append(sl[1])
                if not zs:
                    continue
                mx = max(zs)
                ws = [math.exp(z - mx) for z in zs]
                tot = sum(ws)
                out[s, m, h] = sum(w * v for w, v in zip(ws, vs)) / tot
    return out


def pin_context_one(attn, rng):
    """Seq length 1, one query: out = V_0 of kv head h // G, exactly."""
    for layout in (HND, NHD):
        q, kv, table, _ = tiny_case(rng, S=1, M=1, Hq=6, Hkv=2, lens=(1,), layout=layout)
        out = attn(q, kv, table, [1], 0.37, 0, layout)
        for h in range(6):
            b = table[0, 0]
            v = kv[b, h // 3, 0, 1] if layout == HND else kv[b, 0, h // 3, 1]
            assert np.array_equal(out[0, 0, h], v), "context 1 must return V_0"


def pin_constant_keys(attn, rng):
    """Equal keys (or scale 0): every visible key has the same weight, so
    out is the mean of the visible V rows."""
    q, kv, table, lens = tiny_case(rng, S=2, M=4, lens=(45, 9))
    kv[:, :, :, 0, :] = kv[0, 0, 0, 0, :]  # every K row identical
    for window in (0, 5):
        for scale in (0.3, 0.0):
            out = attn(q, kv, table, lens, scale, window, HND)
            for s in range(2):
                L = int(lens[s])
                for m in range(4):
                    p = L - 4 + m
                    lo = max(0, p - window + 1) if window else 0
                    keys = range(lo, p + 1)
                    for h in range(4):
                        vs = [kv[table[s, t // 16], h // 2, t % 16, 1] for t in keys]
                        np.testing.assert_allclose(out[s, m, h], np.mean(vs, axis=0), rtol=0, atol=1e-12)
    # scale 0 with arbitrary keys is the same closed form
    q, kv, table, lens = tiny_case(rng, S=1, M=2, lens=(30,))
    out = attn(q, kv, table, lens, 0.0, 0, HND)
    for m in range(2):
        p = 30 - 2 + m
        vs = [kv[table[0, t // 16], 0, t % 16, 1] for t in range(p + 1)]
        np.testing.assert_allclose(out[0, m, 0], np.mean(vs, axis=0), rtol=0, atol=1e-12)


def pin_window_one(attn, rng):
    """Window 1: each token sees only itself, out[m] = V at position qpos."""
    for layout in (HND, NHD):
        q, kv, table, lens = tiny_case(rng, S=2, M=3, lens=(33, 3), layout=layout)
        out = attn(q, kv, table, lens, 0.5, 1, layout)
        for s in range(2):
            L = int(lens[s])
            for m in range(3):
                p = L - 3 + m
                b, o = table[s, p // 16], p % 16
                for h in range(4):
                    v = kv[b, h // 2, o, 1] if layout == HND else kv[b, o, h // 2, 1]
                    assert np.array_equal(out[s, m, h], v), "window 1 must return V_qpos"


def pin_brute_force(attn, rng):
    """Range-based oracle equals the predicate brute force on tiny inputs."""
    for P in (16, 32):
        for window in (0, 1, 3, 17):
            for layout in (HND, NHD):
                lens = (40, 17, 2)
                q, kv, table, lens = tiny_case(rng, S=3, M=3, Hq=4, Hkv=2, D=4, P=P, lens=lens, layout=layout)
                got = attn(q, kv, table, lens, 0.7, window, layout)
                ref = brute_force(q, kv, table, lens, 0.7, window, layout)
                np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def pin_split_merge(attn, split, rng):
    """Segment partials + LSE merge equal the one-pass result for any split,
    including empty segments and segments wholly outside a window."""
    q, kv, table, lens = tiny_case(rng, S=2, M=4, lens=(70, 23), D=8)
    # scale 150 puts logits near +-1000: softmax is shift invariant, so the
    # split result must still be exact (no overflow of exp).
    for scale in (0.6, 150.0):
        for window in (0, 6):
            ref = attn(q, kv, table, lens, scale, window, HND)
            assert np.all(np.isfinite(ref))
            for cuts in ([], [16], [1, 2, 3], [5, 5, 60], list(range(0, 70, 7)), [64, 65, 66, 67, 68, 69]):
                got = split(q, kv, table, lens, scale, window, HND, cuts)
                np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def pin_merge_formula(merge, rng):
    """Direct check of the merge identity against a softmax over the union."""
    D = 5
    z = rng.standard_normal(23) * 3
    V = rng.standard_normal((23, D))
    w = np.exp(z - z.max())
    ref = (w @ V) / w.sum()
    for cuts in ([0, 23], [0, 1, 23], [0, 10, 10, 23], [0, 5, 9, 17, 23]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            if b == a:
                parts.append((np.zeros(D), -math.inf, 0.0))
                continue
            m = z[a:b].max()
            e = np.exp(z[a:b] - m)
            parts.append((e @ V[a:b], float(m), float(e.sum())))
        np.testing.assert_allclose(merge(parts), ref, rtol=0, atol=1e-12)
    assert np.array_equal(merge([(np.zeros(D), -math.inf, 0.0)] * 3), np.zeros(D))


def pin_causal_consistency(attn, rng):
    """Row m of an M-token call equals a one-token call with seq length
    L - M + m + 1 on the same cache (speculative-verify rows)."""
    q, kv, table, lens = tiny_case(rng, S=2, M=5, lens=(41, 7))
    for window in (0, 4):
        full = attn(q, kv, table, lens, 0.45, window, HND)
        for s in range(2):
            for m in range(5):
                L1 = int(lens[s]) - 5 + m + 1
                one = attn(q[s : s + 1, m : m + 1], kv, table[s : s + 1], [L1], 0.45, window, HND)
                np.testing.assert_allclose(full[s, m], one[0, 0], rtol=0, atol=1e-13)


def pin_block_permutation(attn, rng):
    """Renumbering physical blocks (and the table with them) and switching
    HND to NHD leave the output unchanged."""
    q, kv, table, lens = tiny_case(rng, S=2, M=2, lens=(50, 31))
    ref = attn(q, kv, table, lens, 0.8, 0, HND)
    perm = rng.permutation(kv.shape[0])
    inv = np.argsort(perm)
    kv2 = kv[perm]  # new block i holds old block perm[i]
    table2 = inv[table]
    np.testing.assert_allclose(attn(q, kv2, table2, lens, 0.8, 0, HND), ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(attn(q, to_nhd(kv), table, lens, 0.8, 0, NHD), ref, rtol=0, atol=1e-13)


def pin_planted_keys(attn, rng):
    """A key planted with a logit gap > 30 dominates when visible and is
    ignored when it lies one past the token (causal) or one before the
    window."""
    D = 16
    q, kv, table, lens = tiny_case(rng, S=1, M=3, Hq=2, Hkv=1, D=D, lens=(60,))
    L, M = 60, 3

    def kslot(t):
        return kv[table[0, t // 16], 0, t % 16]

    # Visible: plant at key 20 for every token.
    t_star = 20
    k = kslot(t_star)[0]
    qq = q.copy()
    beta = 400.0 / (np.dot(k, k) * 0.25)
    qq[0, :, :, :] = beta * k
    out = attn(qq, kv, table, [L], 0.25, 0, HND)
    for m in range(M):
        np.testing.assert_allclose(out[0, m, 0], kslot(t_star)[1], rtol=0, atol=1e-9)
    # Causal: plant at position qpos+1 of token 0 (visible to tokens 1 and 2 only).
    t_star = L - M + 1
    k = kslot(t_star)[0]
    beta = 400.0 / (np.dot(k, k) * 0.25)
    qq[0, :, :, :] = beta * k
    out = attn(qq, kv, table, [L], 0.25, 0, HND)
    assert np.abs(out[0, 0, 0] - kslot(t_star)[1]).max() > 1e-3, "future key must be ignored"
    np.testing.assert_allclose(out[0, 1, 0], kslot(t_star)[1], rtol=0, atol=1e-9)
    # Window: plant one key before the window of token 0 (window 10).
    W = 10
    t_star = (L - M) - W
    k = kslot(t_star)[0]
    beta = 400.0 / (np.dot(k, k) * 0.25)
    qq[0, :, :, :] = beta * k
    out = attn(qq, kv, table, [L], 0.25, W, HND)
    assert np.abs(out[0, 0, 0] - kslot(t_star)[1]).max() > 1e-3, "pre-window key must be ignored"
    outw = attn(qq, kv, table, [L], 0.25, W + 1, HND)
    np.testing.assert_allclose(outw[0, 0, 0], kslot(t_star)[1], rtol=0, atol=1e-9)


def pin_gqa(attn, rng):
    """Hq = Hkv * G equals a call with Hkv' = Hq where kv head j is copied G
    times (q head h keeps kv head h // G)."""
    G = 3
    q, kv, table, lens = tiny_case(rng, S=2, M=2, Hq=6, Hkv=2, lens=(29, 18))
    ref = attn(q, kv, table, lens, 0.5, 0, HND)
    kv_dup = np.repeat(kv, G, axis=1)  # kv head j -> heads j*G .. j*G+G-1
    np.testing.assert_allclose(attn(q, kv_dup, table, lens, 0.5, 0, HND), ref, rtol=0, atol=1e-13)


def pin_sdpa(attn, rng):
    """fp64 torch scaled_dot_product_attention with an explicit boolean mask
    on the dense gathered K/V (a library routine independent of the oracle)."""
    for window in (0, 7):
        for layout in (HND, NHD):
            q, kv, table, lens = tiny_case(rng, S=2, M=4, Hq=8, Hkv=2, D=16, lens=(53, 5), layout=layout)
            got = attn(q, kv, table, lens, 0.3, window, layout)
            P = 16
            for s in range(2):
                L = int(lens[s])
                keys = np.arange(L)
                blocks, offs = table[s, keys // P], keys % P
                for kvh in range(2):
                    slots = kv[blocks, kvh, offs] if layout == HND else kv[blocks, offs, kvh]
                    K = torch.from_numpy(np.ascontiguousarray(slots[:, 0]))
                    V = torch.from_numpy(np.ascontiguousarray(slots[:, 1]))
                    pos = torch.arange(4, dtype=torch.int64) + (L - 4)
                    t = torch.arange(L, dtype=torch.int64)
                    mask = t[None, :] <= pos[:, None]
                    if window:
                        mask &= t[None, :] > pos[:, None] - window
                    for g in range(4):
                        h = kvh * 4 + g
                        qs = torch.from_numpy(np.ascontiguousarray(q[s, :, h]))  # [M, D]
                        ref = torch.nn.functional.scaled_dot_product_attention(
                            qs[None, None], K[None, None], V[None, None], attn_mask=mask[None, None], scale=0.3
                        )[0, 0]
                        live = mask.any(dim=1)
                        np.testing.assert_allclose(got[s, live.numpy(), h], ref[live].numpy(), rtol=0, atol=1e-12)
                        assert np.all(got[s, ~live.numpy(), h] == 0)


def pin_padding(attn, rng):
    """A padded sequence (length 0) outputs exact zeros and leaves the other
    sequences bit-identical to a call without it."""
    q, kv, table, lens = tiny_case(rng, S=3, M=2, lens=(26, 0, 40))
    out = attn(q, kv, table, lens, 0.5, 0, HND)
    assert np.all(out[1] == 0)
    sub = attn(q[[0, 2]], kv, table[[0, 2]], lens[[0, 2]], 0.5, 0, HND)
    assert np.array_equal(out[[0, 2]], sub)


# ---- per-request query counts (packed queries) ----

def pin_varlen_maps(maps):
    """Query maps of a hand-worked batch: q_start [0, 1, 4, 4, 6] over
    lengths [10, 3, 5, 0].  Request 0 has one query at position 9 (K length
    10); request 1 has three queries at positions 0, 1, 2 (K lengths 1, 2,
    3); request 2 has none; request 3 is padding (K length 0)."""
    req, klen = maps([0, 1, 4, 4, 6], [10, 3, 5, 0])
    assert list(req) == [0, 1, 1, 1, 3, 3], req
    assert list(klen) == [10, 1, 2, 3, 0, 0], klen


def varlen_brute_force(q, q_start, kv, table, lens, scale, window, layout):
    """Pure-Python loop over packed tokens: token i of request s (with
    M_s = q_start[s + 1] - q_start[s] tokens) sits at position
    p = L_s - M_s + i and sees key t iff t <= p and (window == 0 or
    p - t < window)."""
    T, Hq, D = q.shape
    P = kv.shape[2] if layout == HND else kv.shape[1]
    Hkv = kv.shape[1] if layout == HND else kv.shape[2]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for s in range(len(q_start) - 1):
        a, b = int(q_start[s]), int(q_start[s + 1])
        L, Ms = int(lens[s]), b - a
        for i in range(Ms):
            p = L - Ms + i
            for h in range(Hq):
                kvh = h // G
                zs, vs = [], []
                for t in range(L):
                    if not (t <= p and (window == 0 or p - t < window)):
                        continue
                    blk, o = int(table[s, t // P]), t % P
                    sl = kv[blk, kvh, o] if layout == HND else kv[blk, o, kvh]
                    zs.append(scale * sum(float(q[a + i, h, d]) * float(sl[0, d]) for d in range(D)))
                    vs.append(sl[1])
                if not zs:
                    continue
                mx = max(zs)
                ws = [math.exp(z - mx) for z in zs]
                out[a + i, h] = sum(w * v for w, v in zip(ws, vs)) / sum(ws)
    return out


def pin_varlen_brute_force(varlen, rng):
    """Mixed counts (including a request with no query, one with more
    queries than keys, and padding) against the brute-force loop, with and
    without a window, in both layouts."""
    lens = (37, 3, 20, 0, 16)
    counts = (3, 5, 0, 2, 1)
    q_start = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    _, kv, table, lens = tiny_case(rng, S=5, M=1, lens=lens)
    q = rng.standard_normal((int(q_start[-1]), 4, 8))
    for layout, kvl in ((HND, kv), (NHD, to_nhd(kv))):
        for window in (0, 4):
            got = varlen(q, q_start, kvl, table, lens, 0.3, window, layout)
            want = varlen_brute_force(q, q_start, kvl, table, lens, 0.3, window, layout)
            assert np.max(np.abs(got - want)) < 1e-12


def pin_varlen_uniform(varlen, attn, rng):
    """Equal counts reproduce the uniform [S, M, Hq, D] call row for row."""
    q, kv, table, lens = tiny_case(rng, S=2, M=3, lens=(37, 2))
    S, M, Hq, D = q.shape
    q_start = np.arange(S + 1) * M
    for window in (0, 5):
        got = varlen(q.reshape(S * M, Hq, D), q_start, kv, table, lens, 0.7, window, HND)
        want = attn(q, kv, table, lens, 0.7, window, HND).reshape(S * M, Hq, D)
        assert np.max(np.abs(got - want)) < 1e-12
