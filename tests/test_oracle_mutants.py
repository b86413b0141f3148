"""Negative controls for the oracle's pins: an oracle copy with one planted
mistake must fail at least one pin.  The mistakes are planted in the
oracle's source text, on the CPU; the real oracle is untouched."""

import inspect
import types

import numpy as np
import pytest

from oracle import attention as oa
import oracle_pins as pins

# (name, original text, planted mistake)
MUTATIONS = [
    ("causal_off_by_one", "return lo, qpos\n", "return lo, qpos - 1\n"),
    ("window_one_too_many", "lo = max(0, qpos - window + 1)", "lo = max(0, qpos - window)"),
    ("gqa_modulo_map", "h = kvh * G + g\n                    out[s, m, h] = _softmax", "h = g * Hkv + kvh\n                    out[s, m, h] = _softmax"),
    ("k_v_swapped", "return np.asarray(slots[:, 0], dtype=np.float64), np.asarray(slots[:, 1], dtype=np.float64)",
     "return np.asarray(slots[:, 1], dtype=np.float64), np.asarray(slots[:, 0], dtype=np.float64)"),
    ("scale_dropped", "z = scale * (K @ qrow)\n    w = np.exp", "z = (K @ qrow)\n    w = np.exp"),
    ("merge_no_rescale", "f = math.exp(m - m_star)", "f = 1.0"),
    ("segment_no_max", "m = float(z.max())", "m = 0.0"),
    ("nhd_axes_swapped", "return kv[block, offset, kv_head]", "return kv[block, kv_head, offset]"),
    ("page_offset_wrong", "offsets = keys % P", "offsets = (keys // P) % P"),
    ("first_key_dropped", "K, V = K_all[lo : hi + 1], V_all[lo : hi + 1]", "K, V = K_all[lo + 1 : hi + 1], V_all[lo + 1 : hi + 1]"),
    ("varlen_klen_off_by_one", "max(0, L - q_len + i + 1) if L > 0", "max(0, L - q_len + i) if L > 0"),
    ("varlen_window_one_too_few", "lo = max(0, k - window) if window > 0 else 0", "lo = max(0, k - window + 1) if window > 0 else 0"),
    ("varlen_request_shifted", "K, V = gather_kv(kv, layout, block_table[r], kvh, range(lo, k))",
     "K, V = gather_kv(kv, layout, block_table[max(r - 1, 0)], kvh, range(lo, k))"),
]


def _mutant(old, new):
    src = inspect.getsource(oa)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _all_pins(mod):
    rng = np.random.default_rng(99)
    yield lambda: pins.pin_context_one(mod.decode_attention, rng)
    yield lambda: pins.pin_constant_keys(mod.decode_attention, rng)
    yield lambda: pins.pin_window_one(mod.decode_attention, rng)
    yield lambda: pins.pin_split_merge(mod.decode_attention, mod.split_decode_attention, rng)
    yield lambda: pins.pin_merge_formula(mod.merge_states, rng)
    yield lambda: pins.pin_causal_consistency(mod.decode_attention, rng)
    yield lambda: pins.pin_block_permutation(mod.decode_attention, rng)
    yield lambda: pins.pin_planted_keys(mod.decode_attention, rng)
    yield lambda: pins.pin_gqa(mod.decode_attention, rng)
    yield lambda: pins.pin_sdpa(mod.decode_attention, rng)
    yield lambda: pins.pin_padding(mod.decode_attention, rng)
    yield lambda: pins.pin_brute_force(mod.decode_attention, rng)
    yield lambda: pins.pin_varlen_maps(mod.query_maps)
    yield lambda: pins.pin_varlen_uniform(mod.decode_attention_varlen, mod.decode_attention, rng)
    yield lambda: pins.pin_varlen_brute_force(mod.decode_attention_varlen, rng)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(name, old, new):
    mod = _mutant(old, new)
    for pin in _all_pins(mod):
        try:
            pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return  # caught
    pytest.fail(f"planted mistake {name!r} passed every pin")
