/*
 * pad_calib.h -- read-bandwidth calibration kernels of libpad_attn.so.
 *
 * These are measurement tools, not part of the attention computation: they
 * give the practical HBM read ceiling that a decode-attention launch is
 * compared against.  They compute nothing but an XOR of the bytes they read
 * (so the loads cannot be removed), and write one int32 to `sink` only when
 * that XOR hits a fixed 32-bit value (practically never).
 *
 * Source: ROCm/vllm pull request 1330, "Summary" -- the kernel is treated
 * as an HBM-bound stream and reported as a fraction of peak bandwidth; the
 * gather kernel below walks pages exactly as the attention kernel does
 * (same block table, same key range per query window), so its rate is the
 * best any gather of those pages reaches on this device.
 *
 * Ownership and errors as in pad_attn.h: device pointers owned by the
 * caller, one kernel enqueued on `stream` per call, no allocation, no
 * synchronisation; host-visible facts are validated and reported as a
 * pad_status.
 */
#ifndef PAD_CALIB_H
#define PAD_CALIB_H

#include <stddef.h>
#include <stdint.h>

#include "pad_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read the K+V rows of every key a decode call of `shape` would attend
 * (keys max(0, L - M - window + 1) .. L - 1 of each sequence and kv head,
 * rounded out to whole 16-key tiles, which stay inside their page), with
 * 16-byte loads in the same page walk as the attention kernel.
 *   waves            4 or 8 waves per workgroup; each wave takes every
 *                    waves-th tile of its segment
 *   tiles_in_flight  1 or 2 tiles loaded per wave before they are consumed
 *                    (1 only for head size 512)
 *   segments         1..256 workgroups per (sequence, kv head); the grid is
 *                    (num_kv_heads * segments, num_seqs)
 *   sink             device int32, written only on the improbable XOR hit
 * shape->path, num_segments and schedule are ignored.  Sequences whose
 * length is <= 0 read nothing; lengths above the table capacity are
 * clamped to it. */
pad_status pad_calib_gather_read(const pad_shape* shape, const void* kv_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t window, int32_t waves,
                                 int32_t tiles_in_flight, int32_t segments, int32_t* sink, void* stream);

/* Read `bytes` contiguous bytes from `src` (16-byte aligned, bytes a
 * multiple of 16) with 16-byte loads over a grid of `blocks` workgroups
 * (1..65536) of `threads` threads (256, 512 or 1024); each workgroup reads
 * one contiguous range with `loads_in_flight` loads per thread issued
 * before any is consumed (4, 8 or 16).  Other values: PAD_EINVAL. */
pad_status pad_calib_stream_read(const void* src, size_t bytes, int32_t blocks, int32_t threads,
                                 int32_t loads_in_flight, int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAD_CALIB_H */
