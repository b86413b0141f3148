"""fp64 oracle of the KV-cache write with a rotary embedding.

TEST INFRASTRUCTURE ONLY -- imported by ``tests/`` and ``bench.py``'s CPU
baseline; never by the product path.

Sources (page titles and the part of each):

* rocm_octave_attn docs page (``vllm.v1.attention.backends.rocm_octave_attn``):
  ``RocmOctaveAttentionImpl.do_kv_cache_update`` (the first
  ``slot_mapping.shape[0]`` tokens of key and value go to their slots; an
  empty mapping writes nothing), ``customize_spec`` (one packed K+V slot per
  token and kv head), ``supported_kv_cache_layouts`` (HND and NHD), and the
  rotary width carried per head size (``registered_rope_dim``).
* ROCm/vllm pull request 1330, "Summary": the fused rotary / KV-cache write
  is its own step before attention.

Readings where the pages are silent (listed in the design doc): a slot is
``block * page_size + offset``; negative slots are skipped; the rotation
pairs element ``i`` with ``i + rope_dim / 2`` (first and second half of the
rotary width) using ``cos = table[p, i]`` and ``sin = table[p, rope_dim/2 + i]``
of a caller-supplied table; elements from ``rope_dim`` on are not rotated.

Parity status: every function is pinned (tests/test_oracle_rope.py).
"""

from __future__ import annotations

import numpy as np

NHD = 0
HND = 1


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate the first ``2 * len(cos)`` elements of the last axis of ``x``
    in pairs ``(i, i + r/2)``: ``(x1, x2) -> (x1 cos - x2 sin, x2 cos + x1 sin)``.
    ``cos`` and ``sin`` broadcast against ``x[..., :r/2]``."""
    x = np.asarray(x, dtype=np.float64)
    half = np.shape(cos)[-1]
    y = x.copy()
    x1, x2 = x[..., :half], x[..., half : 2 * half]
    y[..., :half] = x1 * cos - x2 * sin
    y[..., half : 2 * half] = x2 * cos + x1 * sin
    return y


def cache_write(
    kv: np.ndarray,
    layout: int,
    key: np.ndarray,
    value: np.ndarray,
    slot_mapping,
    positions=None,
    cos_sin: np.ndarray | None = None,
    rope_dim: int = 0,
    q: np.ndarray | None = None,
):
    """Return ``(kv_out, q_out)`` in fp64: ``kv`` with token ``t``'s rotated
    K and its V written into slot ``slot_mapping[t]`` of every kv head
    (tokens with a negative slot skipped), and the rotated query rows
    (``None`` without ``q``)."""
    kv_out = np.array(kv, dtype=np.float64, copy=True)
    P = kv.shape[2] if layout == HND else kv.shape[1]
    n = len(slot_mapping)
    half = rope_dim // 2

    def rot(x, t):
        if rope_dim == 0:
            return np.asarray(x, dtype=np.float64)
        row = np.asarray(cos_sin[int(positions[t])], dtype=np.float64)
        return rope(x, row[:half], row[half:rope_dim])

    for t in range(n):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        b, o = s // P, s % P
        for h in range(key.shape[1]):
            k = rot(key[t, h], t)
            if layout == HND:
                kv_out[b, h, o, 0] = k
                kv_out[b, h, o, 1] = value[t, h]
            else:
                kv_out[b, o, h, 0] = k
                kv_out[b, o, h, 1] = value[t, h]
    q_out = None
    if q is not None:
        q_out = np.stack([rot(q[t], t) for t in range(n)]) if n else np.zeros_like(q, dtype=np.float64)
    return kv_out, q_out
