"""Host check of the balanced persistent grid's work split (no GPU).

The device code (balanced_loop in csrc/decode_common.h) lays every unit
with tiles end to end as `lead` positions (the item's fixed cost) followed
by one position per 16-key tile, and gives workgroup b of Gs = min(G, T)
the share [b T / Gs, (b + 1) T / Gs) of the T positions.  This test
restates that arithmetic and checks, over seeded batches and lead counts,
the properties the kernel relies on:
* every tile of every unit is computed by exactly one item;
* every share holds at least one position, and a share meets a unit only
  where it holds one of its tiles (so every counted item arrives);
* a unit cut by share boundaries has one item per share it meets, and the
  count the items carry (n_parts) is that number;
* the slots the items publish to are exactly the slots the merge reads, in
  share order (first .. first + n - 2, then last), each slot is written at
  most once per launch, and every slot lies in [0, 2 G);
* a unit inside one share is a single item that writes the output.
"""

import numpy as np
import pytest


def split(unit_tiles, G, lead=0):
    """Items of the balanced split: (unit, t0, t1, n_parts, slot, first, last, share)."""
    span = [lead + int(t) if t > 0 else 0 for t in unit_tiles]
    T = int(sum(span))
    Gs = min(G, T)
    items = []
    if T == 0:
        return items, Gs
    owner = lambda t: ((t + 1) * Gs - 1) // T  # noqa: E731
    share_end = lambda bb: (bb + 1) * T // Gs  # noqa: E731
    pref = np.concatenate([[0], np.cumsum(span)]).astype(np.int64)
    for b in range(Gs):
        start, end = b * T // Gs, (b + 1) * T // Gs
        assert end > start, "every share holds a position"
        pos = start
        for u in range(len(unit_tiles)):
            ub, ue = int(pref[u]), int(pref[u + 1])
            if ue <= pos or ue == ub:
                continue
            if pos >= end:
                break
            rb = ub + lead  # first tile position
            f0, f1 = max(rb, pos), min(ue, end)
            if f0 >= f1:  # the share ends among the lead positions
                break
            b0, b1 = owner(rb), owner(ue - 1)
            n = b1 - b0 + 1
            slot = b if f1 == end else G + b
            last = b1 if ue == share_end(b1) else G + b1
            items.append((u, f0 - rb, f1 - rb, n, slot, b0, last, b))
            pos = f1
    return items, Gs


@pytest.mark.parametrize("lead", [0, 1, 6, 12, 40, 64])
@pytest.mark.parametrize("seed", range(40))
def test_balanced_split_invariants(seed, lead):
    r = np.random.default_rng(seed)
    G = int(r.choice([1, 3, 8, 256, 512]))
    U = int(r.integers(1, 300))
    kind = seed % 4
    if kind == 0:
        tiles = r.integers(0, 40, U)
    elif kind == 1:
        tiles = r.integers(0, 3, U)  # fewer tiles than workgroups
    elif kind == 2:
        tiles = np.zeros(U, dtype=np.int64)
        tiles[r.integers(0, U)] = int(r.integers(1, 5000))  # one long unit
    else:
        tiles = r.integers(30, 1100, U)
    items, Gs = split(tiles, G, lead)
    T = int(sum(lead + int(t) for t in tiles if t > 0))
    # every tile of every unit exactly once
    cover = [np.zeros(int(t), dtype=np.int64) for t in tiles]
    for u, t0, t1, *_ in items:
        cover[u][t0:t1] += 1
    assert all(np.all(c == 1) for c in cover)
    # slots written at most once, inside [0, 2G)
    written = [it[4] for it in items if it[3] > 1]
    assert len(written) == len(set(written))
    assert all(0 <= s < 2 * G for s in written)
    # per unit: item count, merge layout and share order
    by_unit = {}
    for it in items:
        by_unit.setdefault(it[0], []).append(it)
    for u, its in by_unit.items():
        its.sort(key=lambda it: it[7])  # share order
        n = its[0][3]
        assert all(it[3] == n for it in its) and len(its) == n
        if n == 1:
            assert its[0][1] == 0 and its[0][2] == tiles[u]
            continue
        first, last = its[0][5], its[0][6]
        want = [first + j for j in range(n - 1)] + [last]
        assert [it[4] for it in its] == want
        # the shares are consecutive
        assert [it[7] for it in its] == list(range(first, first + n))
    # each workgroup publishes at most two partials
    per_wg = {}
    for it in items:
        if it[3] > 1:
            per_wg[it[7]] = per_wg.get(it[7], 0) + 1
    assert all(v <= 2 for v in per_wg.values())
    # shares are equal to within one position
    if T:
        sizes = [(b + 1) * T // Gs - b * T // Gs for b in range(Gs)]
        assert max(sizes) - min(sizes) <= 1 and min(sizes) >= 1
