"""The fp64 oracle against its pins (closed forms, brute force, a library
routine, hand-derived fixtures).  CPU only."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oa
import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture
def rng():
    return np.random.default_rng(1234)


def test_context_one(rng):
    pins.pin_context_one(oracle.decode_attention, rng)


def test_constant_keys(rng):
    pins.pin_constant_keys(oracle.decode_attention, rng)


def test_window_one(rng):
    pins.pin_window_one(oracle.decode_attention, rng)


def test_brute_force(rng):
    pins.pin_brute_force(oracle.decode_attention, rng)


def test_split_merge(rng):
    pins.pin_split_merge(oracle.decode_attention, oracle.split_decode_attention, rng)


def test_merge_formula(rng):
    pins.pin_merge_formula(oracle.merge_states, rng)


def test_causal_consistency(rng):
    pins.pin_causal_consistency(oracle.decode_attention, rng)


def test_block_permutation_and_layouts(rng):
    pins.pin_block_permutation(oracle.decode_attention, rng)


def test_planted_keys(rng):
    pins.pin_planted_keys(oracle.decode_attention, rng)


def test_gqa(rng):
    pins.pin_gqa(oracle.decode_attention, rng)


def test_sdpa_crosscheck(rng):
    pins.pin_sdpa(oracle.decode_attention, rng)


def test_padding(rng):
    pins.pin_padding(oracle.decode_attention, rng)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _cache_from_rows(k, v, P, Hkv=1):
    """One-block HND cache holding the given K/V rows at offsets 0..n-1."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, D = k.shape
    kv = np.zeros((1, Hkv, P, 2, D))
    kv[0, 0, :n, 0] = k
    kv[0, 0, :n, 1] = v
    return kv


@pytest.mark.parametrize("name", ["softmax_weights_123.json", "causal_rows.json", "window_rows.json"])
def test_golden_rows(name):
    g = _load(name)
    kv = _cache_from_rows(g["k"], g["v"], g["page_size"])
    out = oracle.decode_attention(
        np.asarray(g["q"]), kv, np.asarray(g["block_table"]), g["seq_lens"], g["scale"], g["window"], g["layout"]
    )
    np.testing.assert_allclose(out, np.asarray(g["expected"]), rtol=0, atol=1e-14)


def test_golden_gqa():
    g = _load("gqa_map.json")
    kp, vp = np.asarray(g["k_per_head"]), np.asarray(g["v_per_head"])
    Hkv, n, D = kp.shape
    kv = np.zeros((1, Hkv, g["page_size"], 2, D))
    kv[0, :, :n, 0] = kp
    kv[0, :, :n, 1] = vp
    out = oracle.decode_attention(
        np.asarray(g["q"]), kv, np.asarray(g["block_table"]), g["seq_lens"], g["scale"], g["window"], g["layout"]
    )
    np.testing.assert_array_equal(out, np.asarray(g["expected"]))


def test_golden_paged_gather():
    g = _load("paged_gather.json")
    P = g["page_size"]
    table = np.asarray(g["block_table"])
    kv = np.zeros((2, 1, P, 2, 1))
    for pos, b in enumerate(table[0]):
        kv[b, 0, :, 1, 0] = P * pos + np.arange(P)
    out = oracle.decode_attention(np.asarray(g["q"]), kv, table, g["seq_lens"], g["scale"], g["window"], g["layout"])
    np.testing.assert_array_equal(out, np.asarray(g["expected"]))


def test_golden_key_bounds():
    g = _load("key_bounds.json")
    for L, M, m, W, lo, hi, empty in g["rows"]:
        got = oa.key_bounds(L, M, m, W)
        assert (got[1] < got[0]) == empty, (L, M, m, W, got)
        if not empty:
            assert got == (lo, hi), (L, M, m, W, got)


def test_golden_merge():
    g = _load("merge_example.json")
    parts = [(np.asarray(a, dtype=np.float64), -math.inf if m == "-inf" else m, l) for a, m, l in g["partials"]]
    np.testing.assert_allclose(oracle.merge_states(parts), g["expected"], rtol=0, atol=1e-15)


def test_varlen_maps():
    pins.pin_varlen_maps(oracle.query_maps)


def test_varlen_brute_force(rng):
    pins.pin_varlen_brute_force(oracle.decode_attention_varlen, rng)


def test_varlen_uniform(rng):
    pins.pin_varlen_uniform(oracle.decode_attention_varlen, oracle.decode_attention, rng)
