"""Pins of the quantized-cache oracle (oracle/octave.py): checks against
closed forms, brute force and hand-derived fixtures.  Each takes the oracle
module, so tests/test_oracle_octave.py can also run them on copies with a
planted mistake, each of which must fail at least one."""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "octave_codec.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _signs(rng, n):
    return np.where(rng.random(n) < 0.5, -1.0, 1.0)


def pin_hadamard_closed_form(oc, rng):
    """H_n[i, j] = (-1)^popcount(i & j) (a closed form independent of the
    recursive construction); H_n H_n = n I."""
    for n in (1, 2, 4, 64, 256):
        h = oc.hadamard(n)
        want = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(n)] for i in range(n)])
        assert np.array_equal(h, want)
        assert np.array_equal(h @ h, n * np.eye(n))


def pin_rotation(oc, rng):
    """Orthogonal (norm kept per block, inverse undoes it), blocks
    independent, and the hand-derived rotation of e_1."""
    g = golden()["hadamard_rotation"]
    x = np.array(g["x"], dtype=float)
    assert np.allclose(oc.rotate(x, np.ones(4), 4), g["plus"], atol=1e-15)
    assert np.allclose(oc.rotate(x, np.array([1.0, -1.0, 1.0, 1.0]), 4), g["sign1_negated"], atol=1e-15)
    for block in (64, 256):
        s = _signs(rng, 256)
        v = rng.standard_normal((3, 256))
        r = oc.rotate(v, s, block)
        for b0 in range(0, 256, block):
            assert np.allclose(np.linalg.norm(r[:, b0:b0 + block], axis=1), np.linalg.norm(v[:, b0:b0 + block], axis=1))
        assert np.allclose(oc.rotate(r, s, block, inverse=True), v, atol=1e-12)
        # the rotation of each basis vector is the matching Hadamard column
        j = int(rng.integers(0, 256))
        e = np.zeros(256)
        e[j] = 1.0
        col = np.zeros(256)
        b0 = j - j % block
        col[b0:b0 + block] = [s[j] * (-1.0) ** bin(i & (j - b0)).count("1") / math.sqrt(block) for i in range(block)]
        assert np.allclose(oc.rotate(e, s, block), col, atol=1e-14)
    # a block's rotation ignores the other blocks' signs and values
    s1, s2 = _signs(rng, 256), _signs(rng, 256)
    s2[:64] = s1[:64]
    v = rng.standard_normal(256)
    w = v.copy()
    w[64:] = rng.standard_normal(192)
    assert np.allclose(oc.rotate(v, s1, 64)[:64], oc.rotate(w, s2, 64)[:64])


def pin_sign_bits(oc, rng):
    g = golden()["sign_bits"]
    s = oc.signs_from_bits(np.array(g["words"], dtype=np.uint32), g["n"])
    assert set(np.flatnonzero(s < 0).tolist()) == set(g["negative"]) and np.all(np.abs(s) == 1)


def pin_quantizer(oc, rng):
    """Hand-derived example; every code is the nearest level (brute force
    over all levels), the error is at most half a step (plus the fp16
    rounding of the step); zero groups are exact."""
    g = golden()["quantize_3bit"]
    c, d = oc.quantize(np.array([g["x"]]), 3)
    assert c[0].tolist() == g["codes"] and float(d[0]) == g["step"]
    assert np.allclose(oc.dequantize(c, d, 3)[0], g["values"])
    g2 = golden()["quantize_fp16_step"]  # the step is rounded to fp16 before the codes are taken
    c, d = oc.quantize(np.array([g2["x"]]), 3)
    assert c[0].tolist() == g2["codes"] and float(d[0]) == g2["step"]
    assert np.array_equal(oc.dequantize(c, d, 3)[0], np.array(g2["values"]))
    for bits in (3, 4):
        half = 1 << (bits - 1)
        x = rng.standard_normal((40, 64)) * rng.uniform(0.01, 10, (40, 1))
        c, d = oc.quantize(x, bits)
        q = oc.dequantize(c, d, bits)
        levels = (np.arange(2 * half) - half + 0.5)[None, None, :] * d[:, None, None]
        nearest = np.abs(x[..., None] - levels).argmin(axis=-1)
        tie = np.isclose(np.sort(np.abs(x[..., None] - levels), axis=-1)[..., 0],
                         np.sort(np.abs(x[..., None] - levels), axis=-1)[..., 1])
        assert np.all((c == nearest) | tie)
        amax = np.abs(x).max(axis=1, keepdims=True)
        assert np.all(np.abs(q - x) <= 0.5 * d[:, None] + amax * 2.0 ** -10)
        z, dz = oc.quantize(np.zeros((2, 64)), bits)
        assert np.all(dz == 0) and np.all(oc.dequantize(z, dz, bits) == 0)


def pin_packing(oc, rng):
    g = golden()
    assert {f: oc.slot_bytes(f) for f in oc.FORMATS} == {k: v for k, v in g["slot_bytes"].items() if k.startswith("octave")}
    p = g["pack_3bit"]
    codes = np.zeros(256, dtype=np.int64)
    for d, v in p["codes_at"].items():
        codes[int(d)] = v
    raw = oc.pack_codes(codes, 3)
    want = np.zeros(p["nbytes"], dtype=np.uint8)
    for i, v in p["bytes"].items():
        want[int(i)] = v
    assert np.array_equal(raw, want)
    for bits in (3, 4):
        c = rng.integers(0, 1 << bits, (5, 256))
        assert np.array_equal(oc.unpack_codes(oc.pack_codes(c, bits), bits, 256), c)


def pin_encode_unit_key(oc, rng):
    """K = e_0, V = 0, all signs +: the hand-derived slot of each layout."""
    g = golden()["encode_unit_key"]
    k = np.zeros(256)
    k[0] = 1.0
    v = np.zeros(256)
    ones = np.ones(256)
    for fmt, key in (("octave_k3v4", "k3v4"), ("octave_k3v3_compact", "compact")):
        raw = oc.encode_rows(k, v, ones, ones, fmt)
        kb, vb, compact = oc.FORMATS[fmt]
        ng = 1 if compact else 4
        off = kb * 32 + vb * 32
        scales = raw[off:off + 2 * (ng + 1)].view(np.float16).astype(float)
        assert scales[:ng].tolist() == g[key]["k_scales"] and scales[ng] == g[key]["v_scale"]
        kq, vq = oc.decode_rows(raw, fmt)
        codes = oc.unpack_codes(raw[:kb * 32], kb, 256)
        if compact:
            assert np.all(kq == g[key]["k_value"]) and np.all(codes == g[key]["k_code"])
        else:
            assert np.all(kq[:64] == g[key]["k_value_block0"]) and np.all(kq[64:] == 0)
            assert np.all(codes[:64] == g[key]["k_code_block0"]) and np.all(codes[64:] == g[key]["k_code_rest"])
        assert np.all(vq == 0)


def pin_encode_error_bound(oc, rng):
    """Decoding and undoing the rotation returns K and V within the
    quantizer's bound: per element at most half a step in the rotated space,
    so at most sqrt(group) * step / 2 in L2 per group after the inverse
    rotation (orthogonal) -- with the signs each rotation was made with."""
    ks, vs = _signs(rng, 256), _signs(rng, 256)
    k, v = rng.standard_normal((6, 256)), rng.standard_normal((6, 256))
    for fmt in oc.FORMATS:
        kb, vb, compact = oc.FORMATS[fmt]
        gk = 256 if compact else 64
        raw = oc.encode_rows(k, v, ks, vs, fmt)
        kq, vq = oc.decode_rows(raw, fmt)
        k_back = oc.rotate(kq, ks, gk, inverse=True)
        v_back = oc.rotate(vq, vs, 256, inverse=True)
        kr = oc.rotate(k, ks, gk).reshape(6, -1, gk)
        k_step = np.abs(kr).max(axis=2) / (1 << (kb - 1))
        v_step = np.abs(oc.rotate(v, vs, 256)).max(axis=1) / (1 << (vb - 1))
        k_err = np.linalg.norm((k_back - k).reshape(6, -1, gk), axis=2)
        assert np.all(k_err <= math.sqrt(gk) * k_step * 0.5 * 1.01 + 1e-12)
        assert np.all(np.linalg.norm(v_back - v, axis=1) <= 16 * v_step * 0.5 * 1.01 + 1e-12)


def pin_attention_in_rotated_space(oc, rng):
    """Attention over the packed cache equals the plain oracle's attention
    over the dequantized rows with the rotations undone (the rotations are
    orthogonal, so q.k and the V average carry over): pins where the query
    and output rotations sit."""
    from oracle.attention import HND, decode_attention

    ks, vs = _signs(rng, 256), _signs(rng, 256)
    S, M, Hq, Hkv, P = 2, 3, 4, 2, 16
    lens = [37, 5]
    nb = 6
    kv = rng.standard_normal((nb, Hkv, P, 2, 256))
    table = np.array([[0, 1, 2], [3, 4, 5]])
    q = rng.standard_normal((S, M, Hq, 256))
    for fmt in oc.FORMATS:
        kb, vb, compact = oc.FORMATS[fmt]
        gk = 256 if compact else 64
        cache = oc.encode_rows(kv[..., 0, :], kv[..., 1, :], ks, vs, fmt)
        got = oc.decode_attention_quant(q, cache, table, lens, 0.0625, HND, fmt, ks, vs)
        kq, vq = oc.decode_rows(cache, fmt)
        plain = np.stack([oc.rotate(kq, ks, gk, inverse=True), oc.rotate(vq, vs, 256, inverse=True)], axis=-2)
        want = decode_attention(q, plain, table, lens, 0.0625, 0, HND)
        assert np.allclose(got, want, atol=1e-12)


ALL = [pin_hadamard_closed_form, pin_rotation, pin_sign_bits, pin_quantizer, pin_packing, pin_encode_unit_key,
       pin_encode_error_bound, pin_attention_in_rotated_space]
