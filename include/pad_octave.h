/*
 * pad_octave.h -- the quantized ("octave") packed KV cache of
 * libpad_attn.so: writing new tokens into it and decode attention over it.
 *
 * Source: vllm.v1.attention.backends.rocm_octave_attn docs page --
 * RocmOctaveAttentionBackend.supported_kv_cache_dtypes (formats
 * octave_k3v4, octave_k3v3, octave_k3v3_compact), customize_spec (one
 * packed K+V slot per token and kv head), get_supported_head_sizes (head
 * size 256, 64 rotary dims), RocmOctaveAttentionImpl._signs /
 * do_kv_cache_update / _decode (sign bits for K and V handed to the store
 * and decode kernels; queries and keys rotated with the K signs, in blocks
 * unless compact; values with the V signs; the output rotated back).  The
 * pages print no rotation, quantizer or bit layout; this library's reading:
 *
 *   rotation   R x = H (s * x) / sqrt(n), H the Sylvester Walsh-Hadamard
 *              matrix of order n, s = +-1 from the sign bits (bit i % 32 of
 *              word i / 32 set: element i negated); K in four 64-dim blocks
 *              (one 256-dim block when compact), V in one 256-dim block
 *   quantizer  per scale group: step = fp16(max |x| / 2^(b-1)), code =
 *              clamp(floor(x / step), -2^(b-1), 2^(b-1) - 1) + 2^(b-1),
 *              value (code - 2^(b-1) + 1/2) * step; K groups = K blocks,
 *              V one group; b = 3 for K, 4 (k3v4) or 3 for V
 *   slot       K codes, V codes, K steps, V step (fp16), zero pad to 16 B:
 *              240 B (k3v4) or 208 B; codes in groups of 8 packed into b
 *              bytes little-endian (code e at bits b*e); element
 *              d = 32 kc + 8 g + e (kc < 8, g < 4, e < 8) is code e of
 *              group 8 g + kc
 *   cache      HND [num_blocks, num_kv_heads, page_size, slot_bytes] or NHD
 *              [num_blocks, page_size, num_kv_heads, slot_bytes] bytes
 *
 * Ownership, streams and errors as in pad_attn.h: device pointers owned by
 * the caller, no allocation, no synchronisation; host-visible facts are
 * validated and reported as a pad_status.
 */
#ifndef PAD_OCTAVE_H
#define PAD_OCTAVE_H

#include <stddef.h>
#include <stdint.h>

#include "pad_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pad_kv_format {
  PAD_KV_OCTAVE_K3V4 = 1,
  PAD_KV_OCTAVE_K3V3 = 2,
  PAD_KV_OCTAVE_K3V3_COMPACT = 3,
} pad_kv_format;

/* Head size of the packed formats. */
#define PAD_OCTAVE_HEAD_SIZE 256

/* Bytes of one packed slot of `format` at `head_size` (only 256 is
 * supported: PAD_EUNSUPPORTED otherwise; PAD_EINVAL for an unknown format). */
pad_status pad_octave_slot_bytes(int32_t format, int32_t head_size, int32_t* bytes);

/* Shape of a cache write. */
typedef struct pad_octave_cache_shape {
  int32_t num_tokens;   /* T >= 0 new tokens                                  */
  int32_t num_kv_heads; /* Hkv >= 1                                           */
  int32_t head_size;    /* 256                                                */
  int32_t page_size;    /* P >= 1 slots per block                             */
  int32_t num_blocks;   /* blocks in the cache                                */
  int32_t dtype;        /* pad_dtype of key and value                         */
  int32_t layout;       /* pad_layout of the cache                            */
  int32_t format;       /* pad_kv_format                                      */
} pad_octave_cache_shape;

/* Rotate, quantize and pack new tokens' K and V rows into their slots
 * (do_kv_cache_update on the octave page).  key, value: [T, Hkv, 256] of
 * `dtype`; slot_mapping: int64 [T], slot = block * page_size + offset,
 * negative = skip (padding), at or past num_blocks * page_size = skip;
 * k_signs, v_signs: uint32 [8] sign bits; cache: 16-byte aligned bytes of
 * the shape above.  Slots of skipped tokens, and every other slot, are left
 * as they are.  One kernel on `stream`. */
pad_status pad_octave_cache_write(const pad_octave_cache_shape* shape, const void* key, const void* value,
                                  const int64_t* slot_mapping, const uint32_t* k_signs, const uint32_t* v_signs,
                                  void* cache, void* stream);

/* Workspace bytes for pad_decode_attn_octave calls of `shape` (as
 * pad_decode_attn_workspace_size, for the packed format's bytes per key). */
pad_status pad_decode_attn_octave_workspace_size(const pad_shape* shape, int32_t format, size_t* bytes);

/* Decode attention (the rule of pad_decode_attn, no sliding window: the
 * octave backend has none) over a packed cache.  shape->head_size must be
 * 256; shape->dtype is the type of q and out (the cache holds codes);
 * shape->layout the cache layout; shape->path AUTO or MFMA.  The queries
 * are rotated with the K rotation inside the kernel, the products run on
 * the codes in the rotated space, and the output is rotated back with the
 * inverse V rotation before it is written, so q and out are in the model's
 * space.  k_signs and v_signs: device uint32 [8], 4-byte aligned.  Other
 * arguments, workspace rules (zeroed once, left zero) and errors as
 * pad_decode_attn; one kernel on `stream`. */
pad_status pad_decode_attn_octave(const pad_shape* shape, int32_t format, const void* q, const void* cache,
                                  const int32_t* block_table, const int32_t* seq_lens, const uint32_t* k_signs,
                                  const uint32_t* v_signs, float scale, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* pad_decode_attn_octave with a query count per sequence: the per-request
 * query maps of RocmOctaveMetadataBuilder._fill_query_maps on the octave
 * page, given as offsets.  q and out are packed [T, num_q_heads, 256] rows;
 * sequence s owns rows q_start[s] .. q_start[s + 1] - 1, its M_s query
 * tokens at positions L_s - M_s + m.  q_start: device int32 [num_seqs + 1],
 * 4-byte aligned, read only on the device; shape->query_len bounds every
 * M_s; the device-value contract and the clamping are those of
 * pad_decode_attn_varlen (pad_attn.h).  Every other argument, the
 * workspace rules and the errors as pad_decode_attn_octave (PAD_EINVAL for
 * a missing or misaligned q_start). */
pad_status pad_decode_attn_octave_varlen(const pad_shape* shape, int32_t format, const void* q,
                                         const int32_t* q_start, const void* cache, const int32_t* block_table,
                                         const int32_t* seq_lens, const uint32_t* k_signs, const uint32_t* v_signs,
                                         float scale, void* out, void* workspace, size_t workspace_bytes,
                                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAD_OCTAVE_H */
