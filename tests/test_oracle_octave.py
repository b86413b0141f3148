"""The quantized-cache oracle against its pins, and planted mistakes that
the pins must catch (CPU only; the mistakes are planted in a copy of the
oracle's source text)."""

import inspect
import types

import numpy as np
import pytest

from oracle import octave as oc
import octave_pins as pins


@pytest.mark.parametrize("pin", pins.ALL, ids=[p.__name__ for p in pins.ALL])
def test_pin(pin):
    pin(oc, np.random.default_rng(7))


MUTATIONS = [
    ("rotation_not_normalised", "h = hadamard(block) / math.sqrt(block)", "h = hadamard(block)"),
    ("inverse_in_forward_order", "(xb @ h.T) * s", "(s * xb) @ h.T"),
    ("sign_bits_reversed", "(int(w[i // 32]) >> (i % 32)) & 1", "(int(w[i // 32]) >> (31 - i % 32)) & 1"),
    ("round_not_floor", "np.floor(x / safe)", "np.round(x / safe)"),
    ("no_half_step", "- half + 0.5)", "- half)"),
    ("step_not_fp16", "delta = fp16_round(np.abs(x).max(axis=-1) / half)", "delta = np.abs(x).max(axis=-1) / half"),
    ("groups_kc_major", "c = np.swapaxes(c, -2, -3)  # [..., g, kc, e]: groups in g-major order", "c = c"),
    ("codes_big_endian", "out = (word[..., None] >> (8 * np.arange(bits))) & 0xFF  # little-endian bytes",
     "out = (word[..., None] >> (8 * np.arange(bits)[::-1])) & 0xFF"),
    ("k_whole_head", "k_group = D if compact else ROPE_DIM", "k_group = D"),
    ("v_with_k_signs", "vr = rotate(v, v_signs, D)", "vr = rotate(v, k_signs, D)"),
    ("query_not_rotated", "q_rot = rotate(q, k_signs, k_group)", "q_rot = q"),
    ("output_not_rotated_back", "return rotate(o_rot, v_signs, D, inverse=True)", "return o_rot"),
    ("output_rotated_with_k_blocks", "return rotate(o_rot, v_signs, D, inverse=True)",
     "return rotate(o_rot, v_signs, k_group, inverse=True)"),
]


def _mutant(old, new):
    src = inspect.getsource(oc)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("octave_mutant")
    exec(compile(src.replace(old, new, 1), "octave_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(name, old, new):
    mod = _mutant(old, new)
    for pin in pins.ALL:
        try:
            pin(mod, np.random.default_rng(7))
        except (AssertionError, ValueError, IndexError):
            return  # caught
    pytest.fail(f"planted mistake {name!r} passed every pin")
