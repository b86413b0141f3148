// Device-side parameters and launchers of the decode-attention kernels.
#pragma once

#include <cstdint>

#include "plan.h"

namespace pad {

// Everything a decode-attention workgroup needs; passed by value.
struct Params {
  const void* q;              // [S, M, Hq, D], or packed [T, Hq, D] with q_start
  const int32_t* q_start;     // packed layout: first query token of each sequence
                              // [S + 1] (device); null: uniform M = query_len
  const void* kv;             // packed K+V cache (HND or NHD)
  const int32_t* block_table; // [S, max_blocks]
  const int32_t* seq_lens;    // [S]
  void* out;                  // same layout as q
  int32_t* ws_cnt;            // merge control [S, Hkv, row_groups, merge_slices]
  float* ws_ml;               // partial (m, l) [slots, slot_rows, 2]
  float* ws_acc;              // partial acc     [slots, slot_rows, D]
  int64_t block_stride;       // elements between physical blocks
  int64_t head_stride;        // elements between kv heads of a block
  int64_t token_stride;       // elements between tokens of a block
  int32_t num_seqs, query_len, num_q_heads, num_kv_heads, group, page_size, max_blocks;
  int32_t rows;               // G * M query rows per (sequence, kv head)
  int32_t window;             // 0 = full causal
  int32_t nseg;               // segments per (sequence, kv head, row group)
  int32_t seg_tiles;          // planned 16-key tiles per segment
  int32_t row_groups;         // workgroups splitting the rows
  int32_t group_rows;         // query rows per row group (row tiles * 16)
  int32_t merge_slices;       // slices of the merged output (merging workgroups)
  int32_t slot_rows;          // rows of one partial slot (see Plan::slot_rows)
  uint32_t merge_wait_ticks;  // helpers' wait bound (100 MHz real-time ticks)
  int32_t persistent;         // 1: balanced persistent grid (one workgroup per CU, two for a packed cache)
  int32_t unit_lead;          // balanced grid: lead positions per unit
  float scale_log2;           // scale * log2(e): logits are kept in the exp2 domain
  const uint32_t* k_signs;    // packed cache: sign bits of the K rotation [8]
  const uint32_t* v_signs;    // packed cache: sign bits of the V rotation [8]
};

// Enqueue the decode kernel the plan selects.  Returns a HIP error code
// (0 = success).
int launch_decode(const Plan& plan, const Params& params, int dtype, int head_size, void* stream);

// The same for one head size D (64, 128, 256 or 512).
template <int D>
int launch_decode_hs(const Plan& plan, const Params& params, int dtype, void* stream);

// Enqueue the prefill kernel (head size 64 or 128; path PAD_PATH_PREFILL).
int launch_prefill(const Plan& plan, const Params& params, int dtype, int head_size, void* stream);

// Enqueue the packed-cache decode kernel (head size 256) for `format`
// (pad_kv_format).  Returns a HIP error code.
int launch_decode_octave(const Plan& plan, const Params& params, int dtype, int format, void* stream);

// Enqueue a fill of `words` 32-bit zeros at `ptr`.
int launch_zero(void* ptr, size_t words, void* stream);

}  // namespace pad
