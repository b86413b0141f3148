// Host-side launch planning (see plan.h).
#include "plan.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

namespace pad {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool known_head_size(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

// Planner decisions go to stderr, one line per plan that differs from the
// previous one logged on the calling thread, when the environment variable
// PAD_LOG is set to anything but "" or "0" (read once per process).
bool log_plans() {
  static const bool on = [] {
    const char* v = std::getenv("PAD_LOG");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
  }();
  return on;
}

const char* path_name(int path) {
  switch (path) {
    case PAD_PATH_MFMA: return "mfma";
    case PAD_PATH_DOT: return "dot";
    case PAD_PATH_PREFILL: return "prefill";
  }
  return "?";
}

void log_plan(const pad_shape& sh, int window, int num_cus, const Plan& p) {
  char line[512];
  std::snprintf(line, sizeof(line),
                "pad plan: S=%d M=%d Hq=%d Hkv=%d D=%d page=%d max_seq_len=%d window=%d dtype=%d layout=%d cus=%d"
                " -> path=%s rows=%d row_tiles=%d row_groups=%d waves=%d segments=%dx%d tiles grid=%dx%d"
                " merge_slices=%d persistent=%d lead=%d workspace=%zu\n",
                sh.num_seqs, sh.query_len, sh.num_q_heads, sh.num_kv_heads, sh.head_size, sh.page_size,
                sh.max_seq_len, window, sh.dtype, sh.layout, num_cus, path_name(p.path), p.rows, p.row_tiles,
                p.row_groups, p.waves, p.nseg, p.seg_tiles, p.grid_x, p.grid_y, p.merge_slices, p.persistent,
                p.unit_lead, p.ws_bytes);
  thread_local std::string last;
  if (last == line) return;
  last = line;
  std::fputs(line, stderr);
}

}  // namespace

int max_row_tiles(int head_size) {
  // The fp32 accumulator of one 16-row tile costs head_size/4 registers per
  // lane; keep it at or below 128 per wave.
  return std::max(1, std::min(4, 512 / head_size));
}

pad_status make_plan(const pad_shape& sh, int window, int num_cus, Plan* pl, int key_bytes) {
  if (sh.num_seqs < 0 || sh.query_len < 1 || sh.num_q_heads < 1 || sh.num_kv_heads < 1 ||
      sh.head_size < 1 || sh.page_size < 1 || sh.max_blocks_per_seq < 1 || sh.max_seq_len < 0 ||
      sh.num_segments < 0 || window < 0 || num_cus < 1)
    return PAD_EINVAL;
  if (sh.num_q_heads % sh.num_kv_heads != 0) return PAD_EINVAL;
  if (sh.dtype != PAD_F16 && sh.dtype != PAD_BF16) return PAD_EINVAL;
  if (sh.layout != PAD_NHD && sh.layout != PAD_HND) return PAD_EINVAL;
  if (sh.path < PAD_PATH_AUTO || sh.path > PAD_PATH_PREFILL) return PAD_EINVAL;
  if (sh.schedule < PAD_SCHED_AUTO || sh.schedule > PAD_SCHED_PERSISTENT) return PAD_EINVAL;
  const int64_t table_keys = int64_t(sh.max_blocks_per_seq) * sh.page_size;
  if (sh.max_seq_len > table_keys) return PAD_EINVAL;
  // Key and tile indices are 32-bit on the device.
  if (table_keys > (int64_t(1) << 30)) return PAD_EUNSUPPORTED;
  // Decode and speculative verify (M <= 8) and prefill chunks up to
  // kMaxQueryLen tokens (kMaxRows GQA-packed rows); other head sizes and
  // page sizes that are not multiples of the 16-key tile are not built.
  if (sh.query_len > kMaxQueryLen || !known_head_size(sh.head_size) || sh.page_size % kTileKeys != 0)
    return PAD_EUNSUPPORTED;
  if (sh.num_seqs > 65535) return PAD_EUNSUPPORTED;
  // The decode kernel takes the cache strides (at most one block's
  // elements) as 32-bit values.
  if (int64_t(sh.num_kv_heads) * sh.page_size * 2 * sh.head_size > INT32_MAX) return PAD_EUNSUPPORTED;
  const int G = sh.num_q_heads / sh.num_kv_heads;
  const int rows = G * sh.query_len;
  if (rows > kMaxRows) return PAD_EUNSUPPORTED;
  const bool dot_ok = rows <= kDotMaxRows && sh.head_size <= kDotMaxHeadSize;
  if (sh.path == PAD_PATH_DOT && !dot_ok) return PAD_EUNSUPPORTED;
  // The prefill family: head sizes 64 and 128, one workgroup per item.
  const bool prefill_ok = (sh.head_size == 64 || sh.head_size == 128) && sh.schedule != PAD_SCHED_PERSISTENT;
  if (sh.path == PAD_PATH_PREFILL && !prefill_ok) return PAD_EUNSUPPORTED;
  const int tiles_total = int(ceil_div(rows, 16));

  Plan p{};
  // The key-split MFMA family serves every shape and is the automatic
  // choice up to kPrefillMinRows rows per kv head; from there on (prefill
  // chunks) the prefill family, whose workgroups share each K/V tile among
  // 128 rows.  The per-head dot-product family is used when asked for.
  // AUTO takes it where its 128-row blocks fill a quarter of the device
  // and a kv head has at least 2^20 query rows x keys of work (32/8 heads
  // of 128, bf16, graph-timed, prefill family against the key-split one:
  // 256 tokens over 4096 keys 42 against 65 us, a 1024-token prompt 28.4
  // against 56.6, 768 tokens 31.6 against 42.9, 640 tokens 27.4 against
  // 36.6, 512 tokens over 384 keys of context 27.1 against 30.6; a
  // 512-token prompt (2^20) ties at 23.1 / 23.3 and 256 tokens over 512
  // keys (0.75 x 2^20) at 23.6; a 384-token prompt, 25.0 against 19.2, and
  // short chunks over long contexts, whose row blocks do not fill the
  // device (64 tokens over 8192 keys 86.8 against 38.9), stay with the
  // key-split family).
  {
    const int64_t pf_units = int64_t(std::max(1, sh.num_seqs)) * sh.num_kv_heads * ceil_div(rows, kPrefillRows);
    const int64_t keys = sh.max_seq_len ? sh.max_seq_len : int64_t(sh.max_blocks_per_seq) * sh.page_size;
    const bool pf_wins = rows >= kPrefillMinRows && 4 * pf_units >= num_cus && rows * keys >= kPrefillMinWork;
    if (sh.path == PAD_PATH_AUTO)
      p.path = prefill_ok && pf_wins ? PAD_PATH_PREFILL : PAD_PATH_MFMA;
    else
      p.path = sh.path;
  }
  p.rows = rows;
  if (p.path == PAD_PATH_DOT) {
    p.row_tiles = 1;
    p.row_groups = 1;
    p.waves = kDotWaveCount;
  } else if (p.path == PAD_PATH_PREFILL) {
    p.row_tiles = kPrefillRows / 16;
    p.row_groups = int(ceil_div(rows, kPrefillRows));
    p.waves = kPrefillWaves;
  } else {
    // A packed cache takes one row tile per wave, so two workgroups fit a
    // CU (kPackedWgPerCu).
    int rt = std::min(tiles_total, key_bytes > 0 ? 1 : max_row_tiles(sh.head_size));
    p.row_groups = int(ceil_div(tiles_total, rt));
    p.row_tiles = int(ceil_div(tiles_total, p.row_groups));
    p.waves = waves_for(sh.head_size, p.row_tiles);
  }

  // Tiles one unit may have to read: the whole length bound, or the window
  // span (window + M - 1 keys) plus one tile of alignment slack -- never
  // more than the whole bound, so no window plans more than window 0.
  const int64_t max_len = sh.max_seq_len ? sh.max_seq_len : table_keys;
  const int64_t all_tiles = std::max<int64_t>(1, ceil_div(max_len, kTileKeys));
  int64_t span_tiles = all_tiles;
  if (window > 0)
    span_tiles = std::min(all_tiles, ceil_div(int64_t(window) + sh.query_len - 1, kTileKeys) + 1);

  const int64_t units = int64_t(sh.num_seqs) * sh.num_kv_heads * p.row_groups;
  // One workgroup per CU: its 4 waves keep enough loads in flight; two
  // for a packed cache, whose workgroups are smaller.  The grid
  // schedule's segment fill still counts one per CU (grid_fill): a packed
  // cache's shorter segments at two per CU cost more in partials and merges
  // than the pairing gains (k3v4, 16/2 heads of 256, event-timed: one
  // sequence of 32k keys at M = 1 20.4 against 26.6 us, at M = 4 27.5
  // against 35.2; 8 sequences of 4k keys at M = 4 27.5 against 73.4).
  const int64_t slots = int64_t(num_cus) * (key_bytes > 0 ? kPackedWgPerCu : 1);
  const int64_t grid_fill = num_cus;
  p.unit_lead = key_bytes > 0 ? kUnitLeadTilesPacked : kUnitLeadTiles;
  // K/V bytes of one 16-key tile of one kv head: two fp16/bf16 rows per key,
  // or the packed slot of a quantized cache.
  const int64_t tile_bytes = int64_t(kTileKeys) * (key_bytes > 0 ? key_bytes : 2 * sh.head_size * 2);
  // A batch whose lengths may differ runs on the balanced persistent grid
  // when one round of about 3 MiB per workgroup would not cover its
  // planned K/V: the lengths are only known on the device, where a static
  // grid (or a queue of fixed-size items) leaves CUs idle behind short,
  // dead or late items, while the balanced grid gives every CU the same
  // number of tiles (64 bf16 sequences of 512..16384 keys, 16/2 heads of
  // 256: a queue of 3 MiB items took 239 us, with the schedule alone
  // costing about 50 us over an even split).  It needs the batch's tiles to
  // count in 32 bits, its sequences to fit the LDS tables and one control
  // word per unit to fit the counter prefix.
  const int64_t seg_persist = std::max<int64_t>(4, (int64_t(3) << 20) / tile_bytes);
  // The dot and prefill families are built for one workgroup per item only.
  const bool can_persist = p.path == PAD_PATH_MFMA && sh.num_seqs <= kPersistMaxSeqs &&
                           units * (ceil_div(table_keys, kTileKeys) + 1 + p.unit_lead) < (int64_t(1) << 31) &&
                           units * kCtlWordStride * int64_t(sizeof(int32_t)) <= int64_t(kCounterBytes);
  if (sh.schedule == PAD_SCHED_PERSISTENT && !can_persist) return PAD_EUNSUPPORTED;
  p.persistent = sh.schedule == PAD_SCHED_PERSISTENT ||
                 (sh.schedule == PAD_SCHED_AUTO && can_persist && sh.num_seqs > 1 &&
                  units * std::max<int64_t>(1, sh.num_segments > 0 ? sh.num_segments : ceil_div(span_tiles, seg_persist)) >
                      slots);
  // Prefill: about one workgroup per CU (one fits: 300 registers per
  // lane; 256 tokens over 4096 keys in 4 segments 56.8 us, in 8 81.2 us)
  // over the units' row blocks, segments of at least one LDS tile
  // (kPrefillKeys keys) and a multiple of one.  Computed from the window-free
  // span as well, so the workspace bound below covers every window.
  auto prefill_nseg = [&](int64_t tiles) {
    const int64_t want = ceil_div(slots, std::max<int64_t>(1, units));
    return std::max<int64_t>(1, std::min(want, ceil_div(tiles, kPrefillKeys / kTileKeys)));
  };
  int64_t nseg;
  if (sh.num_segments > 0) {
    nseg = sh.num_segments;
  } else if (p.path == PAD_PATH_PREFILL) {
    nseg = prefill_nseg(span_tiles);
  } else if (p.persistent) {
    nseg = 1;  // the balanced grid splits units by share, not by segment
  } else {
    // One full round of workgroups for a single sequence; two rounds when a
    // batch's lengths may differ, so short sequences leave no idle CUs.
    const int64_t target = sh.num_seqs > 1 ? 2 * grid_fill : grid_fill;
    const int64_t fill = std::max<int64_t>(1, target / std::max<int64_t>(1, units));
    // About 64 KiB of K/V per segment, 4 to 8 tiles (two tiles per wave at
    // head size 128, one at 512), 4 tiles while that leaves fewer than 16
    // segments, and 2 where that makes at most 16 (a 512-key window of head
    // size 256 at M=4 took 12.1 us in 17 two-tile segments against 11.4 in
    // 7 longer ones): short contexts are latency-bound, and more,
    // shorter segments overlap more of their dependent round trips (one
    // bf16 sequence, 32/8 heads of 128, M=1: 256 keys in 8 segments 7.5 us
    // against 8.3 in 4; 1k keys in 16 segments 9.1 us against 11.2 us in 4;
    // 2k keys in 16 segments 10.2 against 11.3 us in 8; 4k keys in 32
    // segments 12.0 against 12.6 us in 16).  At least 4 segments while the
    // device has room.
    int64_t seg_target = std::max<int64_t>(4, std::min<int64_t>(8, (int64_t(64) << 10) / tile_bytes));
    if (span_tiles / seg_target < 16) seg_target = 4;
    if (span_tiles / seg_target < 16 && ceil_div(span_tiles, 2) <= 16) seg_target = 2;
    const int64_t wg_rows = std::min(rows, p.row_tiles * 16);
    // Strided key rows (NHD with several kv heads: consecutive keys of one
    // head sit a token stride apart) make each tile's loads slower, and
    // short spans gain from two-tile segments up to twice that count while
    // a segment's partial stays within a quarter of its K/V bytes (a
    // 512-key window, head size 256, fp16, 8/2 heads: M = 1, 4 rows, 10.07
    // us in 7 segments against 8.90 in 17; M = 4, 16 rows, 11.4 in 7
    // against 12.1 in 17).
    const bool strided = sh.layout == PAD_NHD && sh.num_kv_heads > 1;
    const bool two_tile = strided && seg_target > 2 && span_tiles / seg_target < 16 &&
                          ceil_div(span_tiles, 2) <= 32 &&
                          4 * wg_rows * (sh.head_size + 2) * int64_t(sizeof(float)) <= 2 * tile_bytes;
    if (two_tile) seg_target = 2;
    // Where that still leaves 32 or more segments, a segment also keeps its
    // partial (wg_rows rows of D + 2 floats, written and read back) below a
    // sixth of its K/V bytes: wide heads with many live rows otherwise spend
    // more on the merge than the extra workgroups save (head size 512, 16
    // rows per workgroup: 32 segments against 64 at 4k keys, 19.8 against
    // 21.3 us; 64 against 128 at 8k keys, 24.8 against 27.5 us).  Shorter
    // contexts keep the smaller segments (there 16 segments of 1k keys beat
    // 8, 15.5 against 18.0 us).
    const int64_t part_min = ceil_div(6 * wg_rows * (sh.head_size + 2) * int64_t(sizeof(float)), tile_bytes);
    if (part_min > seg_target && span_tiles / part_min >= 32) seg_target = part_min;
    const int64_t work = std::max<int64_t>(1, span_tiles / seg_target);
    nseg = std::min<int64_t>(fill, std::max<int64_t>(work, std::min<int64_t>(4, fill)));
    if (two_tile) nseg = std::min<int64_t>(fill, ceil_div(span_tiles, 2));
    // A unit of at most 64 KiB of K/V runs as one segment: its loop is a
    // single round of loads, shorter than the split-KV epilogue (one bf16
    // sequence, 32/8 heads of 128, 128 keys: 6.4 us against 7.2 us at the
    // best split; fp16, 4/1 heads of 64, 256 keys: 5.5 against 6.5 us).
    if (span_tiles * tile_bytes <= (int64_t(64) << 10)) nseg = 1;
  }
  nseg = std::min<int64_t>(nseg, span_tiles);
  nseg = std::min<int64_t>(nseg, kMaxSegments);
  nseg = std::max<int64_t>(1, nseg);
  p.seg_tiles = int(ceil_div(span_tiles, nseg));
  if (p.path == PAD_PATH_PREFILL && sh.num_segments == 0)
    p.seg_tiles = int(ceil_div(p.seg_tiles, kPrefillKeys / kTileKeys) * (kPrefillKeys / kTileKeys));
  p.nseg = int(ceil_div(span_tiles, p.seg_tiles));
  // The row groups of one (kv head, segment) read the same tiles; the
  // kernel places them on one XCD (sharing its L2) when segments x kv
  // heads is a multiple of the 8 XCDs.  An automatic count keeps that
  // (measured at head size 512, M = 5, three row groups, 16k keys: 41
  // segments 45.0 us, 32 segments 41.6 us).
  if (sh.num_segments == 0 && !p.persistent && p.path == PAD_PATH_MFMA && p.row_groups > 1 &&
      (int64_t(p.nseg) * sh.num_kv_heads) % 8 != 0) {
    for (int64_t n = p.nseg - 1; n >= 1; --n) {
      const int64_t st = ceil_div(span_tiles, n);
      const int64_t n2 = ceil_div(span_tiles, st);
      if ((n2 * sh.num_kv_heads) % 8 == 0) {
        p.seg_tiles = int(st);
        p.nseg = int(n2);
        break;
      }
    }
  }
  // A workgroup stages its segment's block ids in LDS, so no segment may
  // exceed kMaxSegTiles tiles -- also for device lengths beyond
  // max_seq_len, up to the table's capacity (the kernel clamps to it and
  // splits the tiles it finds over the planned segments).
  // A window's span may straddle one more tile than its keys fill, but no
  // unit reads more tiles than the table holds (so every window plans
  // within the window-free bound the workspace is sized for).
  // (The prefill family's id area holds kPrefillMaxSegTiles.)
  const int64_t seg_cap = p.path == PAD_PATH_PREFILL ? kPrefillMaxSegTiles : kMaxSegTiles;
  int64_t max_tiles = ceil_div(table_keys, kTileKeys);
  if (window > 0) max_tiles = std::min(max_tiles, ceil_div(int64_t(window) + sh.query_len - 1, kTileKeys) + 1);
  if (p.persistent) {
    // Items on the balanced grid are shares of the batch's tiles; one
    // longer than the LDS id area is walked in chunks.
    p.nseg = 1;
    p.seg_tiles = int(span_tiles);
  } else if (ceil_div(max_tiles, p.nseg) > seg_cap || p.seg_tiles > seg_cap) {
    const int64_t need = ceil_div(max_tiles, seg_cap);
    if (need > kMaxSegments) return PAD_EUNSUPPORTED;
    p.nseg = int(std::max<int64_t>(p.nseg, need));
    p.seg_tiles = int(ceil_div(span_tiles, p.nseg));
  }

  if (p.persistent) {
    // One workgroup per CU: the key-split family fills a CU's registers
    // and most of its LDS (two per CU for a packed cache).
    p.grid_x = int(slots);
    p.grid_y = 1;
  } else {
    p.grid_x = p.nseg * sh.num_kv_heads * p.row_groups;
    p.grid_y = std::max(1, sh.num_seqs);
  }
  // A grid with a workgroup for every CU is bandwidth-bound: with one row
  // tile per wave it runs the tile loop with a single copy of its body
  // (fewer cold instruction fetches); smaller grids, and waves with more
  // row tiles (more compute per tile), keep a tile of lead (one sequence
  // of 32k keys, 48/8 heads of 128, M=8: 37.5 against 42.3 us).  The
  // persistent grid takes the lean loop too (batch workload 246 -> 239 us).
  p.lean = p.persistent || (p.row_tiles == 1 && int64_t(p.grid_x) * p.grid_y >= num_cus);

  // The workspace holds partial slots for whichever schedule the shape
  // may take under any window, so one pad_decode_attn_workspace_size
  // serves every call of the shape.  Grid: per unit a segment count that
  // bounds what any window plans (forced, the static grid's fill and the
  // LDS block-id bound, all at the window-free span); the slot stride of a
  // call is its own count.  Balanced grid: two slots per workgroup.
  const bool may_persist = can_persist && (sh.schedule == PAD_SCHED_PERSISTENT ||
                                           (sh.schedule == PAD_SCHED_AUTO && sh.num_seqs > 1));
  const bool may_grid = sh.schedule != PAD_SCHED_PERSISTENT;
  int64_t ws_nseg;
  if (sh.num_segments > 0) {
    ws_nseg = sh.num_segments;
  } else if (p.path == PAD_PATH_PREFILL) {
    ws_nseg = prefill_nseg(all_tiles);
  } else {
    const int64_t target = sh.num_seqs > 1 ? 2 * grid_fill : grid_fill;
    // A window-free span of at most 64 KiB per unit plans one segment
    // (and so does every window, which only shortens it).
    const bool one_seg = all_tiles * tile_bytes <= (int64_t(64) << 10);
    ws_nseg = one_seg ? 1 : std::max<int64_t>(1, target / std::max<int64_t>(1, units));
  }
  ws_nseg = std::min(ws_nseg, std::min<int64_t>(all_tiles, kMaxSegments));
  ws_nseg = std::max<int64_t>(ws_nseg, ceil_div(ceil_div(table_keys, kTileKeys), seg_cap));
  if (!p.persistent) ws_nseg = std::max<int64_t>(ws_nseg, p.nseg);
  p.ws_nseg = int(ws_nseg);
  const size_t S = size_t(sh.num_seqs), H = size_t(sh.num_kv_heads), D = size_t(sh.head_size);
  const size_t grid_rows = may_grid && ws_nseg > 1 ? S * H * size_t(ws_nseg) * size_t(rows) : 0;
  const size_t bal_slot_rows = size_t(std::min(rows, p.row_tiles * 16));
  const size_t bal_rows = may_persist ? 2 * size_t(slots) * bal_slot_rows : 0;
  auto bytes_for = [&](size_t r) { return r ? kCounterBytes + align_up(r * 2 * sizeof(float)) + align_up(r * D * sizeof(float)) : 0; };
  p.ws_bytes = std::max(bytes_for(grid_rows), bytes_for(bal_rows));
  p.ws_counters = 0;
  p.ws_ml = p.ws_bytes ? kCounterBytes : 0;
  if (p.persistent) {
    p.slot_rows = int(bal_slot_rows);
    p.ws_acc = p.ws_ml + align_up(bal_rows * 2 * sizeof(float));
  } else {
    p.slot_rows = rows;
    p.ws_acc = p.ws_ml + align_up(grid_rows * 2 * sizeof(float));
  }
  if (p.persistent) {
    // The last arriving item of a unit merges alone: items start as
    // workgroups reach them, so a helper could wait for a whole share.
    p.merge_slices = 1;
  } else if (p.nseg > 1) {
    // Slices: about kSliceBytes of partial accumulators each, limited by
    // the segments (each merging workgroup must have arrived) and by the
    // control words the counter prefix holds.
    const size_t wg_rows = size_t(std::min(rows, p.row_tiles * 16));
    const size_t vol = size_t(p.nseg) * wg_rows * D * sizeof(float);
    // Helpers wait for their unit's last segment, so they are used only
    // when every workgroup of the grid can be resident at once.  On a grid
    // larger than one workgroup per CU the last segment may only start
    // once a waiting helper's CU frees up (measured: 48 segments of a
    // 512-wide head with 4 row groups, 384 workgroups, took 425 us with
    // helpers against 73 us at 32 segments): the last arriver merges alone
    // there.
    const bool resident = int64_t(p.grid_x) * p.grid_y <= slots;
    int64_t k = resident ? int64_t((vol + kSliceBytes - 1) / kSliceBytes) : 1;
    k = std::max<int64_t>(1, std::min<int64_t>(k, std::min(p.nseg, kMaxSlices)));
    const size_t ctl_units = S * H * size_t(p.row_groups);
    k = std::min<int64_t>(k, int64_t(kCounterBytes / (sizeof(int32_t) * kCtlWordStride * std::max<size_t>(1, ctl_units))));
    if (k < 1) return PAD_EUNSUPPORTED;  // more units than the control prefix holds
    p.merge_slices = int(k);
  } else {
    p.merge_slices = 1;
  }
  *pl = p;
  if (log_plans()) log_plan(sh, window, num_cus, p);
  return PAD_OK;
}

}  // namespace pad
