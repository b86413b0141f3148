"""fp64 oracle: gather-then-softmax paged-KV decode attention.

TEST INFRASTRUCTURE ONLY -- imported by ``tests/``, ``smoke()`` and the CPU
baseline of ``bench.py``; never by the product path.

Sources (titles of the pages this follows, and the part of each):

* rocm_rdna_hip docs page (``vllm.v1.attention.ops.rocm_rdna_hip``):
  ``expected_kv_cache_strides`` (HND block/head/token strides, one packed
  2*D row per token and head), ``KernelVariant`` (window 0 = full causal
  attention; G = num_q_heads // num_kv_heads), ``plan_prefill`` (the window
  start of a query position is ``pos - window + 1``) and
  ``prefill_batch_features`` (a token sees at most ``window`` keys).
* rocm_octave_attn docs page (``vllm.v1.attention.backends.rocm_octave_attn``):
  ``RocmOctaveMetadataBuilder._fill_query_maps`` (query i of a request with
  q_len queries and seq_len tokens attends to K length
  ``seq_len - q_len + i + 1``; padding queries get K length 0),
  ``RocmOctaveAttentionBackend.supported_kv_cache_layouts`` (LBHNC / LBNHC:
  HND and NHD), ``customize_spec`` (one packed K+V slot per token and head),
  ``RocmOctaveAttentionImpl.forward`` (no metadata: output zero-filled),
  ``_mid_o_shape`` (split partials are D values plus 2 scalars per split).
* ROCm/vllm pull request 1330 (HIP decode attention for gfx1151), "Summary":
  decode and speculative decode over M <= 8 query tokens, split-KV with an
  in-kernel merge, sliding windows, batched decode.

Readings where the pages are silent (listed with reasons in the design doc):
K occupies elements 0..D-1 of the packed slot and V elements D..2D-1; NHD
is ``[block, token, kv_head, 2, D]``; q head h uses kv head ``h // G``;
the window counts the current key; a row with no visible key (sequence
length 0, or a position before the first key) outputs zeros.

Parity status: every function below is pinned (tests/test_oracle.py,
tests/oracle_pins.py, tests/test_oracle_mutants.py, tests/golden/).  No function
is "parity unpinned".
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

NHD = 0
HND = 1


def key_bounds(seq_len: int, query_len: int, m: int, window: int) -> tuple[int, int]:
    """Inclusive key range ``(lo, hi)`` visible to query token ``m``.

    The token's position is ``qpos = seq_len - query_len + m``; by the K
    length rule of ``_fill_query_maps`` (octave page) it sees keys
    ``0 .. qpos``.  A window ``W > 0`` keeps the last ``W`` of them, ending
    at the token itself (``plan_prefill`` window start ``qpos - W + 1``,
    rdna_hip page).  The range is empty when ``hi < lo`` (sequence length 0,
    or fewer tokens than queries).
    """
    qpos = seq_len - query_len + m
    lo = 0
    if window > 0:
        lo = max(0, qpos - window + 1)
    if seq_len <= 0:
        return 0, -1
    return lo, qpos


def slot(kv: np.ndarray, layout: int, block, kv_head: int, offset) -> np.ndarray:
    """The packed ``(2, D)`` K+V slot of one token of one kv head
    (``block`` and ``offset`` may be index arrays of equal length).

    HND cache ``[blocks, kv_heads, page, 2, D]`` (strides of
    ``expected_kv_cache_strides``, rdna_hip page); NHD swaps the page and
    head axes (LBNHC of ``supported_kv_cache_layouts``, octave page).
    """
    if layout == HND:
        return kv[block, kv_head, offset]
    if layout == NHD:
        return kv[block, offset, kv_head]
    raise ValueError(f"unknown layout {layout}")


def gather_kv(
    kv: np.ndarray, layout: int, table_row: np.ndarray, kv_head: int, keys: Iterable[int]
) -> tuple[np.ndarray, np.ndarray]:
    """Gather the K and V rows of logical ``keys`` of one sequence.

    Key ``t`` lives in physical block ``table_row[t // P]`` at offset
    ``t % P``; K is the first half of its slot, V the second.
    """
    P = kv.shape[2] if layout == HND else kv.shape[1]
    keys = np.asarray(list(keys), dtype=np.int64)
    blocks = np.asarray(table_row, dtype=np.int64)[keys // P]
    offsets = keys % P
    slots = slot(kv, layout, blocks, kv_head, offsets)  # [n, 2, D]
    return np.asarray(slots[:, 0], dtype=np.float64), np.asarray(slots[:, 1], dtype=np.float64)


def _softmax_attend(qrow: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """``softmax(scale * K q) @ V`` for one query row (fp64)."""
    z = scale * (K @ qrow)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def decode_attention(
    q: np.ndarray,
    kv: np.ndarray,
    block_table: np.ndarray,
    seq_lens: Sequence[int],
    scale: float,
    window: int,
    layout: int,
) -> np.ndarray:
    """Reference output ``[S, M, Hq, D]`` in fp64.

    For every sequence, query token and q head: gather the visible keys of
    kv head ``h // G``, take ``softmax(scale * q.k)`` over them and average
    the V rows with those weights.  Rows with no visible key are zero (the
    zero fill of padded queries, ``_fill_query_maps`` / ``forward`` on the
    octave page).
    """
    q = np.asarray(q, dtype=np.float64)
    S, M, Hq, D = q.shape
    Hkv = kv.shape[1] if layout == HND else kv.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    out = np.zeros((S, M, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        for kvh in range(Hkv):
            K_all, V_all = gather_kv(kv, layout, block_table[s], kvh, range(L))
            for m in range(M):
                lo, hi = key_bounds(L, M, m, window)
                if hi < lo:
                    continue
                K, V = K_all[lo : hi + 1], V_all[lo : hi + 1]
                for g in range(G):
                    h = kvh * G + g
                    out[s, m, h] = _softmax_attend(q[s, m, h], K, V, scale)
    return out


def query_maps(q_start: Sequence[int], seq_lens: Sequence[int]) -> tuple[np.ndarray, np.ndarray]:
    """Per packed query token: its request and its K length.

    ``RocmOctaveMetadataBuilder._fill_query_maps`` (octave page): the
    tokens of request ``s`` are ``q_start[s] .. q_start[s + 1] - 1``; query
    ``i`` of a request with ``q_len`` queries and ``seq_len`` tokens attends
    to K length ``seq_len - q_len + i + 1``, and padding (``seq_len`` 0)
    gets K length 0.  Tokens before ``q_start[0]`` belong to no request
    (request -1, K length 0).
    """
    S = len(q_start) - 1
    T = int(q_start[S])
    q_to_req = np.full(T, -1, dtype=np.int64)
    q_to_klen = np.zeros(T, dtype=np.int64)
    for s in range(S):
        a, b = int(q_start[s]), int(q_start[s + 1])
        q_len, L = b - a, int(seq_lens[s])
        for i in range(q_len):
            q_to_req[a + i] = s
            q_to_klen[a + i] = max(0, L - q_len + i + 1) if L > 0 else 0
    return q_to_req, q_to_klen


def decode_attention_varlen(
    q: np.ndarray,
    q_start: Sequence[int],
    kv: np.ndarray,
    block_table: np.ndarray,
    seq_lens: Sequence[int],
    scale: float,
    window: int,
    layout: int,
) -> np.ndarray:
    """Reference output ``[T, Hq, D]`` in fp64 for packed queries with a
    query count per request (mixed decode and speculative verify).

    Token ``t`` of request ``r = q_to_req[t]`` with K length ``k =
    q_to_klen[t]`` (``query_maps``) sees keys ``lo .. k - 1`` of its
    request, ``lo = 0`` or, with a window ``W > 0``, ``max(0, k - W)``
    (the window ends at the token itself: ``plan_prefill``, rdna_hip page).
    Tokens with K length 0 output zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = kv.shape[1] if layout == HND else kv.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    q_to_req, q_to_klen = query_maps(q_start, seq_lens)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for t in range(T):
        r, k = int(q_to_req[t]), int(q_to_klen[t])
        if r < 0 or k <= 0:
            continue
        lo = max(0, k - window) if window > 0 else 0
        for kvh in range(Hkv):
            K, V = gather_kv(kv, layout, block_table[r], kvh, range(lo, k))
            for g in range(G):
                h = kvh * G + g
                out[t, h] = _softmax_attend(q[t, h], K, V, scale)
    return out


def segment_state(
    qrow: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float
) -> tuple[np.ndarray, float, float]:
    """Split-KV partial of one query row over one key segment.

    Returns ``(acc, m, l)``: ``m`` the largest logit, ``l`` the sum of
    ``exp(z - m)`` and ``acc`` the unnormalised ``sum exp(z - m) v``.  These
    are the per-split (acc, m/l) partials of ``KernelVariant.scratch_shapes``
    (rdna_hip page) and the D + 2 values per split of ``_mid_o_shape``
    (octave page).  An empty segment is ``(0, -inf, 0)``.
    """
    D = V.shape[1]
    if K.shape[0] == 0:
        return np.zeros(D), -math.inf, 0.0
    z = scale * (K @ qrow)
    m = float(z.max())
    w = np.exp(z - m)
    return w @ V, m, float(w.sum())


def merge_states(states: Sequence[tuple[np.ndarray, float, float]]) -> np.ndarray:
    """Log-sum-exp merge of split partials into the attention output.

    ``m* = max m_j``, ``l* = sum l_j exp(m_j - m*)``,
    ``o = sum acc_j exp(m_j - m*) / l*`` -- the in-kernel merge of split-KV
    segments (pull request 1330, "Summary").  Empty segments contribute
    nothing; if every segment is empty the row is zero.
    """
    ms = [m for _, m, _ in states]
    D = states[0][0].shape[0]
    m_star = max(ms)
    if m_star == -math.inf:
        return np.zeros(D)
    acc = np.zeros(D)
    l_star = 0.0
    for a, m, l in states:
        if m == -math.inf:
            continue
        f = math.exp(m - m_star)
        acc += f * a
        l_star += f * l
    return acc / l_star


def split_decode_attention(
    q: np.ndarray,
    kv: np.ndarray,
    block_table: np.ndarray,
    seq_lens: Sequence[int],
    scale: float,
    window: int,
    layout: int,
    boundaries: Sequence[int],
) -> np.ndarray:
    """Same output as ``decode_attention``, computed as split segments.

    ``boundaries`` are key positions ``b_0 < b_1 < ...``; segment ``j``
    holds keys ``[b_j, b_{j+1})`` (the first segment starts at 0 and the
    last ends at the sequence length).  Each segment yields a partial via
    ``segment_state`` restricted to the row's visible keys; the partials
    are combined with ``merge_states``.
    """
    q = np.asarray(q, dtype=np.float64)
    S, M, Hq, D = q.shape
    Hkv = kv.shape[1] if layout == HND else kv.shape[2]
    G = Hq // Hkv
    out = np.zeros((S, M, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        cuts = sorted({0, L, *[b for b in boundaries if 0 < b < L]})
        for kvh in range(Hkv):
            K_all, V_all = gather_kv(kv, layout, block_table[s], kvh, range(L))
            for m in range(M):
                lo, hi = key_bounds(L, M, m, window)
                if hi < lo:
                    continue
                for g in range(G):
                    h = kvh * G + g
                    states = []
                    for a, b in zip(cuts[:-1], cuts[1:]):
                        a2, b2 = max(a, lo), min(b, hi + 1)
                        states.append(
                            segment_state(q[s, m, h], K_all[a2:b2], V_all[a2:b2], scale)
                            if b2 > a2
                            else segment_state(q[s, m, h], K_all[:0], V_all[:0], scale)
                        )
                    out[s, m, h] = merge_states(states)
    return out
