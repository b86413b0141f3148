// Host-side launch planning for paged-KV decode attention.
//
// A "unit" is one (sequence, kv head) pair: all G*M query rows of the kv
// head share one read of its K/V pages (ROCm/vllm pull request 1330,
// "Summary": one workgroup per kv head, row group and KV segment).  The
// key range of a unit is split into segments; each segment is one
// workgroup whose partial (acc, m, l) is merged in-kernel once every
// segment has arrived: the merged output is cut into slices, and the last
// arriver and the workgroups that arrived just before it merge one slice
// each.  The planner picks the row tiling (16-row MFMA tiles,
// the rows_padded rule of KernelVariant on the rocm_rdna_hip page), the
// number of segments (enough workgroups to fill the device, cf. the
// split cap of 256 "to fill its CUs with one query" of _mid_o_shape on the
// rocm_octave_attn page) and the workspace layout.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/pad_attn.h"

namespace pad {

constexpr int kTileKeys = 16;    // keys per MFMA tile (page sizes are multiples of 16)
// Query tokens per sequence and GQA-packed query rows per kv head of one
// call: decode and speculative verify use M <= 8; longer prefill chunks
// take one row group per 16-row tiles of a workgroup, each reading only
// the keys its own tokens reach.
constexpr int kMaxQueryLen = 4096;
constexpr int kMaxRows = 32768;
constexpr int kMaxSegments = 256;
// Longest segment in tiles: a workgroup stages its segment's block ids
// (one int32 per tile) in LDS.
constexpr int kMaxSegTiles = 4096;
// Merge slices per unit: about kSliceBytes of partial accumulators each,
// at most kMaxSlices (one control word per slice in the counter prefix).
constexpr int kMaxSlices = 32;
constexpr size_t kSliceBytes = size_t(32) << 10;
// Merge control words are spaced one 128-byte line apart (in int32s).
constexpr int kCtlWordStride = 32;
// The dot-product family serves up to this many query rows per kv head at
// head sizes up to kDotMaxHeadSize, with kDotWaves waves per workgroup.
constexpr int kDotMaxRows = 4;
constexpr int kDotMaxHeadSize = 128;
constexpr int kDotWaveCount = 4;
// The prefill family (head sizes 64 and 128): workgroups of kPrefillWaves
// waves (two per 32-row slab) take kPrefillRows GQA-packed query rows of a
// kv head and stream its keys in LDS tiles of kPrefillKeys; a segment
// spans at most
// kPrefillMaxSegTiles 16-key tiles (its block ids are staged in LDS).  The
// planner picks the family for at least kPrefillMinRows rows per kv head
// and kPrefillMinWork query rows x keys per kv head (see make_plan).
constexpr int kPrefillWaves = 8;
constexpr int kPrefillRows = 128;
// 128 keys per LDS tile (each wave two 32-key blocks per step, half the
// barriers of 64-key tiles): 256-token chunk over 4096 keys 418 -> 426
// TFLOP/s, 2048-token prompt 555 -> 569, 4096-token prompt 703 -> 738; the
// two tile buffers then fill 151.5 KB of LDS, the kernel 253 VGPRs.
constexpr int kPrefillKeys = 128;
constexpr int kPrefillMaxSegTiles = 1024;
constexpr int kPrefillMinRows = 128;
constexpr int64_t kPrefillMinWork = int64_t(1) << 20;  // query rows x keys per kv head
// Merge control words live in a fixed-size prefix of the workspace, so
// calls of different shapes can share one workspace: partials never land
// where any shape keeps control words, and every call leaves them zero.
constexpr size_t kCounterBytes = size_t(1) << 20;
// Balanced persistent grid (batched decode): at most this many sequences
// (its LDS tables).
constexpr int kPersistMaxSeqs = 1024;
// Balanced persistent grid: each unit also counts as this many tiles of
// work when the batch is cut into equal shares, for the fixed cost of an
// item (its first cold loads, combine, publish, arrival and merge) that a
// share pays once per unit it meets.  Batch workload (64 sequences of
// 512..16384 keys, head size 256), graph-timed: 229.4 us at 0, 225.9 at 3,
// 223.2 at 6, 222.7 at 8, 219-221 from 10 to 24.  The same batch at other
// head sizes (M = 4) keeps 12: 32/8 heads of 128 389.3 us against 394.4 /
// 390.4 / 395.3 at 6 / 24 / 48; 16/2 heads of 512 736.5 against 738.4 /
// 744.8 / 756.2.
constexpr int kUnitLeadTiles = 12;
// The same for a packed (quantized) cache: its 16-key tiles carry about a
// quarter of the bytes, while an item's fixed cost does not shrink (it
// adds the query rotation and the output's inverse rotation).  Batch
// workload, k3v4 / k3v3 compact, event-timed: 12 lead tiles 155 / 152 us,
// 24 142 / 141, 40 138 / 139, 64 135 / 134, 96 139 / 141, 140 147 / 146.
constexpr int kUnitLeadTilesPacked = 64;
// Workgroups per CU for a packed cache.  Its per-tile chain (loads,
// unpack, products, softmax) is latency-bound at one wave per SIMD; with
// one 16-row tile per wave a workgroup fits 256 registers per lane and 74
// KiB of LDS, so two share a CU and one's chain overlaps the other's
// (batch workload, k3v4: 193-199 us with two row tiles, one workgroup per
// CU and 12 lead tiles; 155-160 us with one row tile, two per CU).
constexpr int kPackedWgPerCu = 2;
constexpr int64_t kLdsPerCu = 160 << 10;  // LDS bytes of a gfx950 CU

// Waves per workgroup.  Four for every shape: on one bf16 sequence with
// 32 query / 8 kv heads of size 128 and 16-key pages, 4 waves with one
// tile in flight beyond the one computed beat 8 waves with two (32k keys:
// 31.9 vs 36.1 us; 4k keys: 12.4 vs 16.6 us) -- more loads in flight per
// CU only queue longer.
constexpr int waves_for(int head_size, int row_tiles) { return (void)head_size, (void)row_tiles, 4; }

struct Plan {
  int path;          // PAD_PATH_MFMA / PAD_PATH_DOT / PAD_PATH_PREFILL
  int rows;          // G*M rows per unit
  int row_tiles;     // 16-row tiles handled by each workgroup (per wave)
  int row_groups;    // workgroups splitting a unit's rows
  int waves;         // waves per workgroup
  int nseg;          // segments per (unit, row group)
  int seg_tiles;     // planned tiles per segment
  int merge_slices;  // slices the merged output is cut into (1..kMaxSlices)
  int ws_nseg;       // segment slots the workspace holds (>= nseg, the same for every window)
  int persistent;    // 1: one workgroup per CU (two for a packed cache) takes an equal share of the batch's tiles
  int lean;          // 1: the grid fills the device (single-copy tile loop)
  int grid_x, grid_y;
  int slot_rows;     // rows of one partial slot: G*M (grid) or row_tiles*16 (balanced grid)
  int unit_lead;     // balanced grid: lead positions per unit (kUnitLeadTiles or kUnitLeadTilesPacked)
  // Workspace layout (byte offsets; all 256-byte aligned): the counter
  // prefix (kCounterBytes; per (unit, row group) merge_slices words, one
  // 128-byte line apart: the arrival counter, then one hand-over word per
  // slice after the first), then the partial slots of (m, l) and of acc:
  // per unit nseg slots of all G*M rows on the grid schedule, 2 per
  // workgroup of row_tiles*16 rows on the balanced grid.  ws_bytes covers
  // every schedule the shape may take under any window.
  size_t ws_counters, ws_ml, ws_acc, ws_bytes;
};

// Validates the shape fields (not pointers) and fills `plan`.  key_bytes:
// K/V bytes per key of one kv head that the segment sizing assumes (0: the
// 2 * head_size elements of an fp16/bf16 cache).
pad_status make_plan(const pad_shape& shape, int window, int num_cus, Plan* plan, int key_bytes = 0);

// Largest row tiles per wave that fit the accumulator budget at head size D.
int max_row_tiles(int head_size);

}  // namespace pad
