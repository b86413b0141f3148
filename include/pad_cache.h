/*
 * pad_cache.h -- KV-cache write (with an optional rotary embedding) of
 * libpad_attn.so: the step before decode attention, writing the packed
 * K+V slots that pad_decode_attn reads (include/pad_attn.h).
 *
 * What it computes.  For every new token t < num_tokens with slot
 * s = slot_mapping[t] >= 0, and every kv head h:
 *
 *     cache slot (block s / page_size, offset s % page_size, head h):
 *         K half = rope(key[t, h, :], positions[t])
 *         V half = value[t, h, :]
 *
 * and, when q is given, q[t, hq, :] = rope(q[t, hq, :], positions[t]) in
 * place for every query head hq.  rope() rotates the first rope_dim
 * elements in pairs (i, i + rope_dim / 2), i < rope_dim / 2:
 *
 *     y[i]                = x[i] * cos - x[i + rope_dim/2] * sin
 *     y[i + rope_dim / 2] = x[i + rope_dim/2] * cos + x[i] * sin
 *
 * with cos = cos_sin_cache[p][i] and sin = cos_sin_cache[p][rope_dim/2 + i]
 * for position p; elements from rope_dim on are copied.  rope_dim = 0 is a
 * plain store.  Arithmetic in fp32, each result rounded to nearest even
 * into the cache dtype.
 *
 * Sources (page titles and sections):
 *   - vllm.v1.attention.backends.rocm_octave_attn docs page:
 *     `RocmOctaveAttentionImpl.do_kv_cache_update` (the first
 *     slot_mapping.shape[0] tokens of key and value are stored at their
 *     slot; an empty mapping stores nothing), `customize_spec` (one packed
 *     K+V slot per token and kv head), `supported_kv_cache_layouts` (HND
 *     and NHD), `forward_includes_kv_cache_update = False` (the write is
 *     its own step before attention), and the rotary dimension carried
 *     per head size (`registered_rope_dim`, 64 rotary dims at head size
 *     256).
 *   - ROCm/vllm pull request 1330, "Summary": the fused rotary / KV-cache
 *     write is a separate step stacked on the decode kernel.
 *   The pages do not print the rotation itself; the pairing above (first
 *   and second half of the rotary dims) with a caller-supplied cos/sin
 *   table is the reading this library takes.
 *
 * Layouts (dense, row-major; key, value, q and the cache share the dtype):
 *   key, value      [num_tokens, num_kv_heads, head_size]
 *   q               [num_tokens, num_q_heads, head_size] (optional, in place)
 *   slot_mapping    int64 [num_tokens]; slot = block * page_size + offset;
 *                   negative slots (padding tokens) are skipped
 *   positions       int64 [num_tokens] (needed when rope_dim > 0)
 *   cos_sin_cache   fp32 [max_position, rope_dim]: cos then sin
 *   kv_cache        as in pad_attn.h, HND or NHD, num_blocks blocks
 *
 * Ownership, threading and errors as in pad_attn.h: device pointers owned
 * by the caller, one kernel on `stream`, no allocation or synchronisation;
 * host-visible facts are validated.  Device contract: positions in
 * [0, max_position) -- values outside are clamped into it -- and slots
 * below num_blocks * page_size -- larger slots are skipped.
 */
#ifndef PAD_CACHE_H
#define PAD_CACHE_H

#include <stddef.h>
#include <stdint.h>

#include "pad_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pad_cache_shape {
  int32_t num_tokens;    /* >= 0 (0: nothing to do)                           */
  int32_t num_q_heads;   /* >= 1, a multiple of num_kv_heads (with q)          */
  int32_t num_kv_heads;  /* >= 1                                              */
  int32_t head_size;     /* 64, 128, 256 or 512                               */
  int32_t page_size;     /* >= 1                                              */
  int32_t num_blocks;    /* >= 1, blocks in kv_cache                          */
  int32_t dtype;         /* pad_dtype                                         */
  int32_t layout;        /* pad_layout                                        */
  int32_t rope_dim;      /* 0, or a multiple of 16 up to head_size            */
  int32_t max_position;  /* rows of cos_sin_cache (>= 1 when rope_dim > 0)    */
} pad_cache_shape;

/* Write new tokens' K (rotated) and V into their cache slots and rotate q
 * in place (q may be NULL).  key, value, q and kv_cache 16-byte aligned;
 * slot_mapping, positions 8-byte aligned; cos_sin_cache 4-byte aligned.
 * positions and cos_sin_cache may be NULL when rope_dim is 0. */
pad_status pad_rope_cache_write(const pad_cache_shape* shape, void* q, const void* key, const void* value,
                                const int64_t* slot_mapping, const int64_t* positions,
                                const float* cos_sin_cache, void* kv_cache, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAD_CACHE_H */
