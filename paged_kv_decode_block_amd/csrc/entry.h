// Host entry helpers shared by the library's extern "C" sources.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/pad_attn.h"

namespace pad {

// Compute units of the current device (cached per device; 256 when no
// device can be queried).
int device_cus();

// The buffer and scale checks of a decode call (host-visible facts only):
// a finite scale and, unless the batch is empty, present and aligned q,
// kv_cache, out (16 bytes), block_table and seq_lens (4 bytes).
pad_status check_buffers(const pad_shape* shape, const void* q, const void* kv_cache, const int32_t* block_table,
                         const int32_t* seq_lens, float scale, const void* out);

// Validate, plan and enqueue one decode launch on `stream` (the body of
// pad_decode_attn, of pad_decode_attn_varlen when q_start is not null, and
// of pad_decode_attn_octave when format is a pad_kv_format).
pad_status decode(const pad_shape* shape, const void* q, const int32_t* q_start, const void* kv_cache,
                  const int32_t* block_table, const int32_t* seq_lens, float scale, int32_t window, void* out,
                  void* workspace, size_t workspace_bytes, void* stream, int format = 0,
                  const uint32_t* k_signs = nullptr, const uint32_t* v_signs = nullptr);

// Bytes of one packed slot of `format` at `head_size` (0: not built).
int octave_slot_bytes(int format, int head_size);

}  // namespace pad
