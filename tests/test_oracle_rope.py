"""The fp64 oracle of the KV-cache write and its rotation against pins:
hand-worked fixtures, closed forms (identity, norm, inverse), the relative
position property, and planted mistakes that must fail.  CPU only."""

import inspect
import json
import os
import types

import numpy as np
import pytest

from oracle import rope as orope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HND, NHD = 1, 0


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def freq_table(max_pos, rope_dim, base=10000.0):
    """A standard frequency table: angle p * base^(-2i / rope_dim)."""
    half = rope_dim // 2
    inv = base ** (-np.arange(half) * 2.0 / rope_dim)
    ang = np.arange(max_pos)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def pin_golden_pairs(mod):
    g = _load("rope_pairs.json")
    got = mod.rope(np.asarray(g["x"]), np.asarray(g["cos"]), np.asarray(g["sin"]))
    np.testing.assert_array_equal(got, np.asarray(g["expected"]))


def pin_identity_norm_inverse(mod, rng):
    x = rng.standard_normal((5, 64))
    half = 16
    assert np.array_equal(mod.rope(x, np.ones(half), np.zeros(half)), x)
    ang = rng.uniform(-3, 3, half)
    y = mod.rope(x, np.cos(ang), np.sin(ang))
    pair = lambda a: a[:, :half] ** 2 + a[:, half : 2 * half] ** 2  # noqa: E731
    assert np.max(np.abs(pair(y) - pair(x))) < 1e-12
    assert np.array_equal(y[:, 2 * half :], x[:, 2 * half :])
    back = mod.rope(y, np.cos(ang), -np.sin(ang))
    assert np.max(np.abs(back - x)) < 1e-12


def pin_relative_position(mod, rng):
    """With a frequency table, q.k after rotation depends only on the
    distance between the two positions."""
    rd = 32
    tab = freq_table(64, rd)
    q, k = rng.standard_normal(48), rng.standard_normal(48)

    def r(x, p):
        return mod.rope(x, tab[p, : rd // 2], tab[p, rd // 2 : rd])

    for p1, p2, d in ((5, 2, 7), (30, 30, 11), (0, 9, 40)):
        a = r(q, p1) @ r(k, p2)
        b = r(q, p1 + d) @ r(k, p2 + d)
        assert abs(a - b) < 1e-9, (p1, p2, d, a, b)


def pin_golden_slots(mod):
    g = _load("cache_slots.json")
    P, nb = g["page_size"], g["num_blocks"]
    for layout in (HND, NHD):
        kv = np.zeros((nb, 1, P, 2, 1)) if layout == HND else np.zeros((nb, P, 1, 2, 1))
        key = np.asarray(g["k"]).reshape(-1, 1, 1)
        val = np.asarray(g["v"]).reshape(-1, 1, 1)
        out, _ = mod.cache_write(kv, layout, key, val, g["slots"])
        kk = out[:, 0, :, 0, 0] if layout == HND else out[:, :, 0, 0, 0]
        vv = out[:, 0, :, 1, 0] if layout == HND else out[:, :, 0, 1, 0]
        np.testing.assert_array_equal(kk, np.asarray(g["expected_k"]))
        np.testing.assert_array_equal(vv, np.asarray(g["expected_v"]))


def pin_cache_rotation(mod, rng):
    """The stored K is the rotated key at its token's position; V and the
    query rows follow the same rule."""
    rd, D, P = 16, 32, 4
    tab = freq_table(20, rd)
    key, val = rng.standard_normal((3, 2, D)), rng.standard_normal((3, 2, D))
    q = rng.standard_normal((3, 4, D))
    pos = [3, 0, 17]
    kv = np.zeros((4, 2, P, 2, D))
    out, qo = mod.cache_write(kv, HND, key, val, [1, 6, 13], pos, tab, rd, q)
    for t, s in enumerate([1, 6, 13]):
        want = mod.rope(key[t], tab[pos[t], : rd // 2], tab[pos[t], rd // 2 : rd])
        np.testing.assert_array_equal(out[s // P, :, s % P, 0], want)
        np.testing.assert_array_equal(out[s // P, :, s % P, 1], val[t])
        np.testing.assert_array_equal(qo[t], mod.rope(q[t], tab[pos[t], : rd // 2], tab[pos[t], rd // 2 : rd]))
    # position 0 leaves the key unrotated
    np.testing.assert_array_equal(out[6 // P, :, 6 % P, 0], key[1])


def _all(mod, rng):
    yield lambda: pin_golden_pairs(mod)
    yield lambda: pin_identity_norm_inverse(mod, rng)
    yield lambda: pin_relative_position(mod, rng)
    yield lambda: pin_golden_slots(mod)
    yield lambda: pin_cache_rotation(mod, rng)


def test_pins():
    rng = np.random.default_rng(3)
    for pin in _all(orope, rng):
        pin()


MUTATIONS = [
    ("adjacent_pairs", "x1, x2 = x[..., :half], x[..., half : 2 * half]", "x1, x2 = x[..., 0 : 2 * half : 2], x[..., 1 : 2 * half : 2]"),
    ("sign_flipped", "y[..., :half] = x1 * cos - x2 * sin", "y[..., :half] = x1 * cos + x2 * sin"),
    ("sin_from_cos_half", "return rope(x, row[:half], row[half:rope_dim])", "return rope(x, row[:half], row[:half])"),
    ("slot_offset_swapped", "b, o = s // P, s % P", "b, o = s % P, s // P"),
    ("negative_slot_written", "        if s < 0:\n            continue\n", ""),
    ("k_v_swapped", "kv_out[b, h, o, 0] = k\n                kv_out[b, h, o, 1] = value[t, h]",
     "kv_out[b, h, o, 1] = k\n                kv_out[b, h, o, 0] = value[t, h]"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(name, old, new):
    src = inspect.getsource(orope)
    assert src.count(old) >= 1, f"anchor not found: {old!r}"
    mod = types.ModuleType("rope_mutant")
    exec(compile(src.replace(old, new, 1), "rope_mutant", "exec"), mod.__dict__)
    rng = np.random.default_rng(5)
    for pin in _all(mod, rng):
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return
    pytest.fail(f"planted mistake {name!r} passed every pin")
