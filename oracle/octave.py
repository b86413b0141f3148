"""fp64 oracle of the quantized ("octave") packed KV cache and of decode
attention over it -- TEST INFRASTRUCTURE ONLY (imported by ``tests/``,
``smoke()`` and the CPU baseline of ``bench.py``; never by the product
path, with which it shares no code).

What the pages fix (vllm.v1.attention.backends.rocm_octave_attn docs page):
* ``RocmOctaveAttentionBackend.supported_kv_cache_dtypes``: three formats,
  ``octave_k3v4``, ``octave_k3v3`` and ``octave_k3v3_compact`` -- keys at 3
  bits, values at 4 or 3 bits, and a compact variant;
  ``customize_spec``: one packed K+V slot per (token, kv head) of
  ``fmt.slot_bytes`` bytes; ``get_supported_head_sizes``: head size 256
  with 64 rotary dimensions (``RocmOctaveAttentionImpl.__init__``).
* ``RocmOctaveAttentionImpl._signs`` / ``do_kv_cache_update`` / ``_decode``
  / ``_prefill``: a vector of sign bits per head size is passed to the
  store and decode kernels for K and for V; queries and keys are rotated
  with the K signs and, unless the format is compact, "in blocks"; values
  with the V signs over the whole head; the attention runs in the rotated
  space and its output is rotated back with the V signs (the inverse
  flag of ``octave_rotate``).

The pages print no rotation, block size, quantizer or bit layout.  The
readings below (listed in the design doc with reasons) are the plainest ones
the rest supports:
* rotation = sign flip then the Sylvester Walsh-Hadamard transform,
  normalised: ``R x = H_n (s * x) / sqrt(n)``; its inverse is
  ``s * (H_n y) / sqrt(n)`` (H_n is symmetric with H_n H_n = n I);
* K blocks: the 64-dim blocks of the rotary width (head size 256 = four
  blocks, each rotated with its own 64 signs); the compact format rotates
  K over the whole head; V is always rotated over the whole head;
* quantizer: uniform mid-rise with ``2^b`` levels per scale group,
  ``delta = fp16(absmax / 2^(b-1))``, code ``c = clamp(floor(x / delta),
  -2^(b-1), 2^(b-1) - 1) + 2^(b-1)`` and value ``(c - 2^(b-1) + 1/2) *
  delta``; K scale groups are the K rotation blocks (one per 64 dims, or
  one per head when compact), V has one scale per head;
* sign bits: bit ``i % 32`` of word ``i // 32`` set means element i is
  negated;
* slot layout (bytes, head size D, b_K = 3, b_V = 4 or 3): the K codes,
  then the V codes, then the K scales and the V scale as fp16, zero-padded
  to a multiple of 16.  Codes go in groups of 8 elements packed into b
  bytes, little-endian, code e of a group at bits ``b e .. b e + b - 1``;
  element ``d = 32 kc + 8 g + e`` (kc < D/32, g < 4, e < 8) is code e of
  group ``g * D/32 + kc``: each of the four 16-lane groups of an MFMA tile
  finds its elements in its own contiguous bytes.

Parity status: every function here is pinned in tests/test_oracle_octave.py
(closed forms, brute force, exactly representable caches, hand-checked
fixtures under tests/golden/ and planted mistakes).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import HND, NHD, decode_attention

HEAD_SIZE = 256
ROPE_DIM = 64  # K rotation blocks (non-compact formats) and K scale groups

# name -> (K bits, V bits, compact)
FORMATS = {
    "octave_k3v4": (3, 4, False),
    "octave_k3v3": (3, 3, False),
    "octave_k3v3_compact": (3, 3, True),
}


def hadamard(n: int) -> np.ndarray:
    """Sylvester Walsh-Hadamard matrix of order n (a power of two):
    H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def signs_from_bits(words: np.ndarray, n: int) -> np.ndarray:
    """+-1 vector of length n from packed sign bits (bit set = negative)."""
    w = np.asarray(words, dtype=np.uint32)
    bits = np.array([(int(w[i // 32]) >> (i % 32)) & 1 for i in range(n)])
    return np.where(bits == 1, -1.0, 1.0)


def rotate(x: np.ndarray, signs: np.ndarray, block: int, inverse: bool = False) -> np.ndarray:
    """Rotate the last axis of x in blocks of ``block`` elements.

    Forward: each block b becomes ``H (s_b * x_b) / sqrt(block)``;
    inverse: ``s_b * (H y_b) / sqrt(block)``, the transpose of the forward
    map (orthogonal).  ``signs`` has the full length of the axis.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % block:
        raise ValueError("block must divide the axis")
    h = hadamard(block) / math.sqrt(block)
    out = np.empty_like(x)
    for b0 in range(0, n, block):
        s = signs[b0 : b0 + block]
        xb = x[..., b0 : b0 + block]
        out[..., b0 : b0 + block] = (s * xb) @ h.T if not inverse else (xb @ h.T) * s
    return out


def fp16_round(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def quantize(x: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Codes (0 .. 2^bits - 1) and fp16 steps of scale groups along the
    last axis of x (one group per row; fp64 decisions).  A group of zeros
    gets step 0 and the middle code."""
    half = 1 << (bits - 1)
    x = np.asarray(x, dtype=np.float64)
    delta = fp16_round(np.abs(x).max(axis=-1) / half)
    safe = np.where(delta > 0, delta, 1.0)[..., None]
    c = np.clip(np.floor(x / safe), -half, half - 1).astype(np.int64) + half
    c = np.where(delta[..., None] > 0, c, half)
    return c, delta


def dequantize(codes: np.ndarray, delta, bits: int) -> np.ndarray:
    half = 1 << (bits - 1)
    return (np.asarray(codes, dtype=np.float64) - half + 0.5) * np.asarray(delta, dtype=np.float64)[..., None]


def _groups(fmt: str, D: int):
    kb, vb, compact = FORMATS[fmt]
    k_group = D if compact else ROPE_DIM
    return kb, vb, compact, k_group


def slot_bytes(fmt: str, D: int = HEAD_SIZE) -> int:
    kb, vb, compact, k_group = _groups(fmt, D)
    raw = kb * D // 8 + vb * D // 8 + 2 * (D // k_group) + 2
    return -(-raw // 16) * 16


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Codes (last axis D) packed in groups of 8 into ``bits`` bytes each:
    element 32 kc + 8 g + e is code e (bits bits*e ..) of group g * D/32 + kc."""
    codes = np.asarray(codes, dtype=np.int64)
    D = codes.shape[-1]
    nkc = D // 32
    c = codes.reshape(codes.shape[:-1] + (nkc, 4, 8))  # [..., kc, g, e]
    c = np.swapaxes(c, -2, -3)  # [..., g, kc, e]: groups in g-major order
    word = (c << (bits * np.arange(8))).sum(axis=-1)  # [..., g, kc]: 8 codes in 8 * bits bits
    out = (word[..., None] >> (8 * np.arange(bits))) & 0xFF  # little-endian bytes
    return out.reshape(codes.shape[:-1] + (bits * D // 8,)).astype(np.uint8)


def unpack_codes(raw: np.ndarray, bits: int, D: int) -> np.ndarray:
    raw = np.asarray(raw, dtype=np.uint8).astype(np.int64)
    nkc = D // 32
    r = raw.reshape(raw.shape[:-1] + (4, nkc, bits))  # [..., g, kc, byte]
    word = (r << (8 * np.arange(bits))).sum(axis=-1)  # [..., g, kc]
    c = (word[..., None] >> (bits * np.arange(8))) & ((1 << bits) - 1)  # [..., g, kc, e]
    return np.swapaxes(c, -2, -3).reshape(raw.shape[:-1] + (D,))


def encode_rows(k: np.ndarray, v: np.ndarray, k_signs: np.ndarray, v_signs: np.ndarray, fmt: str) -> np.ndarray:
    """Packed slot bytes of K and V rows (last axis D; any leading shape):
    rotate, quantize per scale group, pack (module docstring layout)."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    D = k.shape[-1]
    kb, vb, compact, k_group = _groups(fmt, D)
    lead = k.shape[:-1]
    kr = rotate(k, k_signs, k_group).reshape(lead + (D // k_group, k_group))
    vr = rotate(v, v_signs, D)
    kc, k_scales = quantize(kr, kb)  # [..., ng, k_group], [..., ng]
    vc, v_scale = quantize(vr, vb)  # [..., D], [...]
    scales = np.concatenate([k_scales, v_scale[..., None]], axis=-1).astype(np.float16).view(np.uint8)
    body = np.concatenate([pack_codes(kc.reshape(lead + (D,)), kb), pack_codes(vc, vb), scales], axis=-1)
    out = np.zeros(lead + (slot_bytes(fmt, D),), dtype=np.uint8)
    out[..., : body.shape[-1]] = body
    return out


def decode_rows(raw: np.ndarray, fmt: str, D: int = HEAD_SIZE) -> tuple[np.ndarray, np.ndarray]:
    """Dequantized K and V rows of packed slots (last axis slot bytes),
    still in the rotated space."""
    kb, vb, compact, k_group = _groups(fmt, D)
    raw = np.asarray(raw, dtype=np.uint8)
    lead = raw.shape[:-1]
    nk, nv = kb * D // 8, vb * D // 8
    kc = unpack_codes(raw[..., :nk], kb, D)
    vc = unpack_codes(raw[..., nk : nk + nv], vb, D)
    ng = D // k_group
    scales = np.ascontiguousarray(raw[..., nk + nv : nk + nv + 2 * (ng + 1)]).view(np.float16).astype(np.float64)
    kq = dequantize(kc.reshape(lead + (ng, k_group)), scales[..., :ng], kb).reshape(lead + (D,))
    vq = dequantize(vc, scales[..., ng], vb)
    return kq, vq


def dequantize_cache(cache: np.ndarray, fmt: str, D: int = HEAD_SIZE) -> np.ndarray:
    """fp64 cache of dequantized rotated (K, V) rows, shape (..., 2, D),
    from a packed cache of shape (..., slot_bytes)."""
    kq, vq = decode_rows(cache, fmt, D)
    return np.stack([kq, vq], axis=-2)


def decode_attention_quant(
    q: np.ndarray,
    cache: np.ndarray,
    block_table: np.ndarray,
    seq_lens,
    scale: float,
    layout: int,
    fmt: str,
    k_signs: np.ndarray,
    v_signs: np.ndarray,
) -> np.ndarray:
    """Decode attention over a packed quantized cache, fp64.

    The queries are rotated with the K rotation, attention (the plain
    gather-then-softmax oracle, ``decode_attention``) runs over the
    dequantized rotated keys and values, and the output is rotated back
    with the inverse V rotation -- the order of ``_decode`` / ``_prefill``
    on the octave page.  ``cache`` is (blocks, kv_heads, page, slot_bytes)
    for HND or (blocks, page, kv_heads, slot_bytes) for NHD; no sliding
    window (the octave backend has none).
    """
    D = q.shape[-1]
    kb, vb, compact, k_group = _groups(fmt, D)
    q_rot = rotate(q, k_signs, k_group)
    kv = dequantize_cache(cache, fmt, D)
    o_rot = decode_attention(q_rot, kv, block_table, seq_lens, scale, 0, layout)
    return rotate(o_rot, v_signs, D, inverse=True)
