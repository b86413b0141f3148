// Paged-KV decode / speculative-verify attention for gfx950 (CDNA4).
//
// One workgroup serves one (sequence, kv head, row group, KV segment): it
// packs the G*M query rows of the kv head into 16-row MFMA tiles so the
// kv head's K/V pages are read once for all of them, walks its segment's
// 16-key tiles, and either writes the output directly (one segment) or
// writes a partial (acc, m, l) that the last segment to arrive merges
// (ROCm/vllm pull request 1330, "Summary"; split partials and counters as
// in KernelVariant.scratch_shapes / make_scratch on the rocm_rdna_hip
// page).
//
// Inside a workgroup the waves take interleaved 16-key tiles of the
// segment, each with its own online-softmax state over all rows, and are
// combined through LDS at the end.  Per tile a wave:
//   * loads the K and V rows of the tile straight into registers with
//     16-byte loads (lane = key c, 8 consecutive head-dim elements), one
//     tile ahead of the tile it computes;
//   * computes S^T = K Q^T with v_mfma_f32_16x16x32_{bf16,f16}: K is the
//     A operand as loaded, the query tile is the B operand, and the result
//     leaves each lane with 4 keys of one query row (row = lane % 16), so
//     row max and sum need only the 4 lane groups (two cross-lane steps);
//   * stages V in LDS and reads it back transposed with ds_read_b64_tr_b16
//     (4 keys of one head-dim column per lane) as the A operand of
//     v_mfma_f32_16x16x16 for O^T += V^T P^T, whose B operand (P rounded to
//     the input dtype) is exactly the softmax lane layout.
// Logits live in the exp2 domain (scale * log2 e folded in).
//
// Split partials are written with device-coherent (write-through) stores,
// so publishing them costs no L2 write-back: each wave waits for its own
// stores, then one atomic per workgroup counts the arrival.  The merge is
// shared: the output is cut into slices, merged by the last arriver and by
// the workgroups that arrived just before it, which wait (bounded) for the
// last arriver's go; a slice whose helper stopped waiting falls back to the
// last arriver.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "decode_common.h"
#include "kernels.h"
#include "octave_dev.h"

#ifndef PAD_HEAD_SIZE
#error "compile once per head size with -DPAD_HEAD_SIZE=64|128|256|512"
#endif

namespace pad {
namespace {

using namespace dev;


// Workgroup shape (waves per workgroup from waves_for) and LDS layout.
// LEAN selects the tile loop with a single copy of its body (below).
template <int D, int RT, bool LEAN = false>
struct Shape {
  static constexpr int NW = waves_for(D, RT);
  static constexpr int kThreads = NW * 64;
  static constexpr int KC = D / 32;  // 32-wide head-dim chunks (QK^T MFMA steps)
  static constexpr int DT = D / 16;  // 16-wide head-dim tiles of the output
  static constexpr int kVStride = D + 8;    // elements per staged V row (16-byte padded)
  static constexpr int kAccStride = D + 4;  // floats per accumulator row in LDS
  static constexpr int kRows = RT * 16;
  // Tiles in flight beyond the one being computed: one while the register
  // budget allows it (a second one measured slower).  The ring of PF + 1
  // register tiles unrolls the loop body PF + 1 times, and the first pass
  // through each copy is fetched cold; the lean loop (PF = 0: a tile's
  // successor is issued once its scores have consumed it) keeps one copy.
  // The planner picks it for grids that fill the device with one row tile
  // per wave, and for the persistent grid (batch workload 246 -> 239 us,
  // one sequence of 32k keys 33.2 -> 32.9 us); latency-bound grids and
  // waves with several row tiles keep the ring.
  static constexpr int PF = !LEAN && D * RT <= 512 && D < 512 ? 1 : 0;
  // LDS: V staging and the segment's block ids during the tile loop,
  // afterwards the wave-combine area; then the persistent grid's tables.
  // The last 16 bytes hold the merge role, hand-over and queue words.
  static constexpr int kVBytes = NW * 16 * kVStride * 2;
  // The segment's block ids, one per tile, follow the V staging area.
  static constexpr int kIdsBytes = kMaxSegTiles * 4;
  static constexpr int kLoopBytes = kVBytes + kIdsBytes;
  static constexpr int kCombineBytes = Combine<D, RT, NW>::kBytes;
  // Then the balanced persistent grid's tables: clamped lengths and the
  // first tile of each sequence.
  static constexpr int kPersistOff = kLoopBytes > kCombineBytes ? kLoopBytes : kCombineBytes;
  static constexpr int kBytes = kPersistOff + (2 * kPersistMaxSeqs + 1) * 4 + 16;
  static_assert(kLoopBytes >= kPersistMaxSeqs * 4, "the per-sequence tile counts fit the tile-loop area");
};

// The tile a lane holds: its key's K and V rows (eight elements of every
// 32-wide chunk, per its lane group), or its share of a packed slot.
template <int KC>
struct PlainTile {
  i32x4 k[KC];
  i32x4 v[KC];
};

// One work item of (sequence s, kv head kvh, row group rg).  On the grid
// schedule (PERSIST = false) it is segment `seg` of the unit's key range,
// found once the length is known; on the balanced persistent grid the
// caller passes the item (its tiles, partial slot and merge layout) in `fr`.
// FMT: 0 for an fp16/bf16 cache, else the packed format (pad_kv_format) of
// a quantized cache (head size 256): the products then run on codes in the
// rotated space (octave_dev.h).
template <typename T, int D, int RT, bool LEAN, bool PERSIST, int FMT = 0>
__device__ __forceinline__ void decode_unit(const Params& p, unsigned char* lds, int s, int kvh, int rg, int seg,
                                            Frag fr) {
  // The products' element type: the input's, or fp16 for a packed cache
  // (codes as 1024 + c, the rotated queries and the step-scaled weights in
  // fp16, whatever the type of q and out -- the octave page's kernels run
  // in fp16).
  using MF = std::conditional_t<FMT == 0, Mfma<T>, Mfma<_Float16>>;
  using SH = Shape<D, RT, LEAN>;
  constexpr int NW = SH::NW, KC = SH::KC, DT = SH::DT;
  static_assert(FMT == 0 || D == kOctD, "packed formats are built for head size 256");
  static_assert(FMT == 0 || SH::kBytes * kPackedWgPerCu <= kLdsPerCu,
                "kPackedWgPerCu packed-cache workgroups share one CU's LDS");
  // Tiles in flight beyond the one computed: a packed tile carries a
  // quarter of the bytes of a bf16 one in a few registers per lane, so the
  // packed path keeps a deeper ring.
  constexpr int PF = FMT ? kOctRing : SH::PF;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  // The length is read first and used last in this prologue: the loads
  // that do not depend on it (the query rows and, without a window, the
  // segment's block ids) are in flight at the same time.  It and the first
  // block id are read before the query count is known (both reads are in
  // range for any sequence), so they depend on preloaded arguments only.
  const int L_dev = p.seq_lens[s];
  const int32_t* table = p.block_table + int64_t(s) * p.max_blocks;
  // The item's block ids (one per tile) go to LDS, so a tile's page
  // address costs an LDS read instead of a scalar load that may miss.  At
  // most kMaxSegTiles ids are staged at a time: a longer item (only a
  // persistent share can be) is walked in chunks.  On the grid without a
  // window a segment starts at tile seg * seg_tiles whatever the length
  // (unless a length past the planning bound stretches the segments), so
  // its planned tiles are staged before the length is known; entries past
  // the sequence's end are staged but never used.  A thread stages the
  // same slots in both passes, so a second pass needs no barrier first.
  int* sm_ids = reinterpret_cast<int*>(lds + SH::kVBytes);
  const bool spec_ids = !PERSIST && p.window == 0;
  // The block id of each wave's first tile by one wave-uniform load beside
  // the length, issued before the staging loads: an in-range read of the
  // table row, used only once the length shows the tile exists, so the
  // first K/V loads wait neither for the staged ids nor for the barrier.
  int blk_first = 0;
  if (PERSIST) {
    const int b = ((fr.ts + wave) * 16) / p.page_size;
    blk_first = __builtin_amdgcn_readfirstlane(table[min(b, p.max_blocks - 1)]);
    const int n = min(fr.te - fr.ts, kMaxSegTiles);
    for (int t = tid; t < n; t += SH::kThreads) sm_ids[t] = table[((fr.ts + t) * 16) / p.page_size];
  } else if (spec_ids) {
    const int b = ((seg * p.seg_tiles + wave) * 16) / p.page_size;
    blk_first = __builtin_amdgcn_readfirstlane(table[min(b, p.max_blocks - 1)]);
  }
  const SeqQ sq = seq_queries(p, s);
  const int M = sq.m;
  const int rows = p.group * M;  // this sequence's query rows
  const int row0 = rg * RT * 16;
  const int wg_rows = min(RT * 16, rows - row0);
  if (wg_rows <= 0) return;  // no query token, or a row group past this sequence's rows

  if (spec_ids) {
    const int ts0 = seg * p.seg_tiles;
    for (int t = tid; t < p.seg_tiles; t += SH::kThreads) {
      const int b = ((ts0 + t) * 16) / p.page_size;
      if (b < p.max_blocks) sm_ids[t] = table[b];
    }
  }

  // Per-lane query row (row = lane % 16 of each row tile); rows past G*M
  // see nothing.
  i32x4 qop[RT][KC];
  const T* Q = static_cast<const T*>(p.q);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int ru = row0 + rt * 16 + c;
    if (ru < rows) {
      const int m = ru / p.group, gq = ru % p.group;
      const T* qrow = Q + ((int64_t(sq.first) + m) * p.num_q_heads + kvh * p.group + gq) * D;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) qop[rt][kc] = *reinterpret_cast<const i32x4*>(qrow + 32 * kc + 8 * g);
    } else {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) qop[rt][kc] = i32x4{0, 0, 0, 0};
    }
  }

  // Packed cache: the query rows go to the rotated space of the keys,
  // q' = H (s * q) / sqrt(n) over each K block (64 dims, or 256 when
  // compact), in fp32, rounded back to T for the MFMA; qsum[rt][b] is the
  // sum of the rounded q' over K block b of the lane's row (the offset of
  // the code operand is taken off with it).  Element 32 kc + 8 g + e has
  // index bits e (this lane), g (lane groups: lane bits 4 and 5) and kc.
  constexpr int KG = FMT ? Oct<FMT>::KG : 1;
  float qsum[RT][KG];
  if constexpr (FMT != 0) {
    using OT = OctType<T>;     // the input queries
    using OF = OctType<_Float16>;  // the rotated ones
    uint32_t ksw[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) ksw[kc] = p.k_signs[kc];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float f[KC][8];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint32_t w = uint32_t(qop[rt][kc][q4]);
          f[kc][2 * q4] = OT::lo(w);
          f[kc][2 * q4 + 1] = OT::hi(w);
        }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((ksw[kc] >> (8 * g + e)) & 1u) f[kc][e] = -f[kc][e];
#pragma unroll
      for (int st = 1; st < 8; st <<= 1)  // index bits 0-2: e
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!(e & st)) {
              const float a = f[kc][e], b = f[kc][e | st];
              f[kc][e] = a + b;
              f[kc][e | st] = a - b;
            }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)  // index bits 3-4: g
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          f[kc][e] = wht_lane_stage(f[kc][e], 16, (g & 1) != 0);
          f[kc][e] = wht_lane_stage(f[kc][e], 32, (g & 2) != 0);
        }
      constexpr int kSpan = KG == 4 ? 2 : KC;  // chunks per K block
#pragma unroll
      for (int st = 1; st < kSpan; st <<= 1)  // index bits from 5 on: kc within the block
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          if (!(kc & st))
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float a = f[kc][e], b = f[kc | st][e];
              f[kc][e] = a + b;
              f[kc | st][e] = a - b;
            }
      constexpr float kNorm = KG == 4 ? 0.125f : 0.0625f;  // 1 / sqrt(block)
      float qs[KG];
#pragma unroll
      for (int b = 0; b < KG; ++b) qs[b] = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint32_t lo = MF::bits(f[kc][2 * q4] * kNorm), hi = MF::bits(f[kc][2 * q4 + 1] * kNorm);
          const uint32_t w = lo | (hi << 16);
          qop[rt][kc][q4] = int(w);
          qs[kc / kSpan] += OF::lo(w) + OF::hi(w);
        }
#pragma unroll
      for (int b = 0; b < KG; ++b) {
        qs[b] += __shfl_xor(qs[b], 16);
        qs[b] += __shfl_xor(qs[b], 32);
        qsum[rt][b] = qs[b];
      }
    }
  }

  // Lengths past the block table's capacity are clamped to it.
  const int L = min(L_dev, p.max_blocks * p.page_size);
  bool early;
  if constexpr (PERSIST) {
    early = true;  // the item's first ids are staged and each wave's first block id is known
  } else {
    if (L <= 0) {
      if (seg == 0) zero_rows<T, D>(p, s, kvh, row0, wg_rows, SH::kThreads);
      return;
    }
    const SegSplit sp = split_of(p, L, M, rg);
    if (seg >= sp.n_live) return;
    fr.ts = sp.t_lo + seg * sp.seg_tiles;
    fr.te = min(fr.ts + sp.seg_tiles, sp.t_hi);
    fr.n_parts = sp.n_live;
    fr.merge_slices = p.merge_slices;
    const int64_t slot0 = (int64_t(s) * p.num_kv_heads + kvh) * p.nseg;
    fr.slot = slot0 + seg;
    fr.parts.first = slot0;
    fr.parts.last = slot0 + sp.n_live - 1;
    fr.parts.n = sp.n_live;
    fr.parts.row0 = row0;
    fr.ctl = p.ws_cnt + ((int64_t(s) * p.num_kv_heads + kvh) * p.row_groups + rg) * p.merge_slices * kCtlStride;
    // Without a window (and unless a length past the planning bound
    // stretched the segments) the ids staged above are the segment's.
    early = spec_ids && sp.seg_tiles == p.seg_tiles && fr.ts == seg * p.seg_tiles;
    if (!early)
      for (int t = tid; t < fr.te - fr.ts; t += SH::kThreads) sm_ids[t] = table[((fr.ts + t) * 16) / p.page_size];
  }
  const int ts = fr.ts, te = fr.te;
  const int k_lo = p.window > 0 ? max(0, L - M - p.window + 1) : 0;
  // Tiles needing no mask: every key visible to every row.
  const int lo_last = p.window > 0 ? max(0, L - p.window) : 0;
  const int qpos_first = L - M;

  // Per-lane query row: position and window start (rows past G*M see
  // nothing).
  int qpos_r[RT], lo_r[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int ru = row0 + rt * 16 + c;
    qpos_r[rt] = ru < rows ? L - M + ru / p.group : -1;
    lo_r[rt] = ru < rows && p.window > 0 ? max(0, qpos_r[rt] - p.window + 1) : 0;
  }

  float m_run[RT], l_run[RT];
  f32x4 acc[RT][DT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const unsigned char* KVh =
      static_cast<const unsigned char*>(p.kv) + int64_t(kvh) * p.head_stride * int64_t(sizeof(T));
  // Byte offset of this lane's 16-byte chunk inside a tile: key row c,
  // head-dim elements 8g..8g+7 of chunk 0 (32-bit, per lane); the tile base
  // itself is wave-uniform, so the loads take a scalar base address.  A
  // packed slot is read as this lane group's K and V codes and the key's
  // step area.
  const uint32_t lane_off = FMT ? uint32_t(c * p.token_stride) * uint32_t(sizeof(T))
                                : uint32_t(c * p.token_stride + 8 * g) * uint32_t(sizeof(T));
  uint16_t* vs = reinterpret_cast<uint16_t*>(lds) + wave * 16 * SH::kVStride;
  // Transposed-read address of this lane: row 4g + c/4, columns 4(c%4).. of
  // each 16-column tile (ds_read_b64_tr_b16 returns column c of the 4x16
  // block its 16-lane group addresses, i.e. 4 keys of one head-dim column).
  const uint16_t* vtr = vs + (4 * g + (c >> 2)) * SH::kVStride + 4 * (c & 3);

  using Tile = std::conditional_t<FMT == 0, PlainTile<KC>, OctTile>;
  // Packed cache: the row sums of the rounded step-scaled weights that
  // multiply the V codes, as one more PV product against an operand of
  // ones (every lane of the row holds its row's sum); the V offset is taken
  // off the accumulator with them after the last tile.
  f32x4 psum[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) psum[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue_tile = [&](Tile& tl, int t, int blk) {
    const int key0 = t * 16;
    const unsigned char* base =
        KVh + (int64_t(blk) * p.block_stride + int64_t(key0 % p.page_size) * p.token_stride) * int64_t(sizeof(T));
    const unsigned char* row = base + lane_off;
    if constexpr (FMT == 0) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) tl.k[kc] = *reinterpret_cast<const i32x4*>(row + 64 * kc);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) tl.v[kc] = *reinterpret_cast<const i32x4*>(row + 2 * D + 64 * kc);
    } else {
      using SL = OctSlot<FMT>;
      const unsigned char* kp = row + SL::kKBytesPerGroup * g;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const uint2 w = *reinterpret_cast<const uint2*>(kp + 8 * i);
        tl.k[2 * i] = w.x;
        tl.k[2 * i + 1] = w.y;
      }
      const unsigned char* vp = row + SL::kVOff + SL::kVBytesPerGroup * g;
      if constexpr (Oct<FMT>::VB == 4) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 w = *reinterpret_cast<const uint4*>(vp + 16 * i);
          tl.v[4 * i] = w.x;
          tl.v[4 * i + 1] = w.y;
          tl.v[4 * i + 2] = w.z;
          tl.v[4 * i + 3] = w.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const uint2 w = *reinterpret_cast<const uint2*>(vp + 8 * i);
          tl.v[2 * i] = w.x;
          tl.v[2 * i + 1] = w.y;
        }
      }
      const uint4 sw = *reinterpret_cast<const uint4*>(row + SL::kSOff);
      tl.sc[0] = sw.x;
      tl.sc[1] = sw.y;
      tl.sc[2] = sw.z;
      tl.sc[3] = sw.w;
    }
  };

  // Scores of tile t: stage its V rows in LDS, S^T = K Q^T, mask, online
  // softmax; leaves P (input dtype, MFMA B layout) in pb.  After it the
  // tile's registers are free.
  auto score_tile = [&](Tile& tl, int t, uint64_t (&pb)[RT]) {
    const int key0 = t * 16;
    const bool edge = !(key0 >= lo_last && key0 + 15 <= qpos_first);
    // Packed cache: each lane's four scores belong to keys 4g + j; their
    // K steps (one per K block) and V step come from the lanes that loaded
    // those keys' step areas (lane 4g + j).
    float kstep[KG][4], vstep[4];
    i32x4 kop[FMT ? KC : 1];
    if constexpr (FMT == 0) {
      if (edge) {
        // Keys outside [k_lo, L) may hold anything (even NaN); they must not
        // reach the PV product, where 0 * NaN would poison the sum.
        const int key = key0 + c;
        if (key < k_lo || key >= L) {
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) tl.v[kc] = i32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        *reinterpret_cast<i32x4*>(vs + c * SH::kVStride + 32 * kc + 8 * g) = tl.v[kc];
    } else {
      // V codes as operands (finite whatever the slot holds: keys outside
      // [k_lo, L) get a weight of exactly 0 below).
      constexpr int VB = Oct<FMT>::VB;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        i32x4 vv;
        if constexpr (VB == 4)
          vv = codes8_nibbles(tl.v[kc]);
        else
          vv = codes8<3>(bits_window(tl.v, 24 * kc));
        *reinterpret_cast<i32x4*>(vs + c * SH::kVStride + 32 * kc + 8 * g) = vv;
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kop[kc] = codes8<3>(bits_window(tl.k, 24 * kc));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int src = 4 * g + j;
        if constexpr (KG == 4) {
          const uint32_t w0 = uint32_t(__shfl(int(tl.sc[0]), src)), w1 = uint32_t(__shfl(int(tl.sc[1]), src));
          const uint32_t w2 = uint32_t(__shfl(int(tl.sc[2]), src));
          kstep[0][j] = half_bits_to_float(w0);
          kstep[1][j] = half_bits_to_float(w0 >> 16);
          kstep[2][j] = half_bits_to_float(w1);
          kstep[3][j] = half_bits_to_float(w1 >> 16);
          vstep[j] = half_bits_to_float(w2);
        } else {
          const uint32_t w0 = uint32_t(__shfl(int(tl.sc[0]), src));
          kstep[0][j] = half_bits_to_float(w0);
          vstep[j] = half_bits_to_float(w0 >> 16);
        }
      }
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float x[4];
      if constexpr (FMT == 0) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) sc = MF::qk(tl.k[kc], qop[rt][kc], sc);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = sc[j] * p.scale_log2;
      } else {
        // Per K block: codes x q' (scaled back by 2^24), minus the level
        // offset times the block's q' sum, times the block's step.
        constexpr float kOff = float(1 << (Oct<FMT>::KB - 1)) - 0.5f;
        constexpr int kSpan = KC / KG;
        float sj[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < KG; ++b) {
          f32x4 sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = b * kSpan; kc < (b + 1) * kSpan; ++kc) sb = MF::qk(kop[kc], qop[rt][kc], sb);
          const float corr = kOff * qsum[rt][b];
#pragma unroll
          for (int j = 0; j < 4; ++j) sj[j] += kstep[b][j] * fmaf(sb[j], kCodeScale, -corr);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = sj[j] * p.scale_log2;
      }
      // One wave-uniform branch per row tile, selects inside it.
      if (edge) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = key0 + 4 * g + j;
          if (key < lo_r[rt] || key > qpos_r[rt]) x[j] = kNegInf;
        }
      }
      float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      // The row's reference maximum moves only when a tile exceeds it by
      // more than kMaxSlack (weights then stay below 2^kMaxSlack), so the
      // accumulator is rescaled rarely -- and skipped by the whole wave
      // when none of its rows moved.  m, l and acc stay consistent with
      // the reference, which is all the combine and the merge need.
      const bool move = tmax > m_run[rt] + kMaxSlack;
      const float m_new = move ? tmax : m_run[rt];
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = move ? fast_exp2(m_run[rt] - m_use) : 1.f;
      float pj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pj[j] = fast_exp2(x[j] - m_use);
      l_run[rt] = l_run[rt] * alpha + ((pj[0] + pj[1]) + (pj[2] + pj[3]));
      m_run[rt] = m_new;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= alpha;
        if constexpr (FMT != 0) psum[rt] *= alpha;
      }
      if constexpr (FMT == 0) {
        pb[rt] = pack4(MF::bits(pj[0]), MF::bits(pj[1]), MF::bits(pj[2]), MF::bits(pj[3]));
      } else {
        // The V step goes into the weight; on edge tiles keys outside
        // [k_lo, L) weigh exactly 0 (their step may be anything).
        float w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pj[j] * vstep[j];
        if (edge) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = key0 + 4 * g + j;
            if (key < k_lo || key >= L) w[j] = 0.f;
          }
        }
        pb[rt] = pack4(MF::bits(w[0]), MF::bits(w[1]), MF::bits(w[2]), MF::bits(w[3]));
      }
    }
  };

  // O^T += V^T P^T from the V rows staged in LDS.
  constexpr int kPvAhead = DT < 4 ? DT : 4;
  auto pv_tile = [&](const uint64_t (&pb)[RT]) {
    // The staged V rows were written by other lanes of this wave; LDS
    // operations of a wave complete in order, the fences keep the compiler
    // from moving the reads above the writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint64_t va[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      va[dt] = __builtin_bit_cast(
          uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vtr + 16 * dt)));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][dt] = MF::pv(va[dt], pb[rt], acc[rt][dt]);
    if constexpr (FMT != 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) psum[rt] = MF::pv(kOnes4, pb[rt], psum[rt]);
    }
    // Order: kPvAhead reads, then per column the RT products and the read
    // kPvAhead columns on, so several LDS round trips overlap instead of
    // one read waiting before each column's products.
    __builtin_amdgcn_sched_group_barrier(0x100, kPvAhead, 0);
#pragma unroll
    for (int dt = 0; dt < DT - kPvAhead; ++dt) {
      __builtin_amdgcn_sched_group_barrier(0x008, RT, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, RT * kPvAhead + (FMT != 0 ? RT : 0), 0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // The item's tiles in chunks of at most kMaxSegTiles staged ids (one
  // chunk on the grid schedule).  Within a chunk, tile i of this wave is
  // cs + wave + i * NW.
  Tile ring[PF + 1];
  int cs = ts;
  {
    const int ce = min(te, cs + kMaxSegTiles);
    // The first tile's loads go out before the barrier that publishes the
    // staged ids when its block id is already known.
    if (early && cs + wave < ce) issue_tile(ring[0], cs + wave, blk_first);
  }
  __syncthreads();
  for (;;) {
    const int ce = min(te, cs + kMaxSegTiles);
    const int first_t = cs + wave;
    const int n_w = first_t < ce ? (ce - first_t + NW - 1) / NW : 0;
    // Physical block of tile t (wave-uniform).
    auto block_of = [&](int t) { return __builtin_amdgcn_readfirstlane(sm_ids[t - cs]); };
    if ((!early || cs != ts) && n_w > 0) issue_tile(ring[0], first_t, block_of(first_t));

    // PF tiles are in flight beyond the one being computed (a ring of PF + 1
    // register buffers, the first issued above), and each tile's block id is
    // read one tile before its loads are issued.  The prefetch index is
    // clamped to the wave's last tile instead of being skipped, so every
    // iteration has the same loads in flight and the compiler's wait counts
    // stay exact (the clamped re-reads of the last tile hit in cache).
    auto tile_at = [&](int i) { return first_t + min(i, n_w - 1) * NW; };
    if constexpr (PF == 0) {
      // No register room for a second tile: the next tile's loads go out as
      // soon as the scores have consumed the current one, so they overlap
      // the PV product (whose V operand is already in LDS).
      Tile& tl = ring[0];
      for (int i = 0; i < n_w; ++i) {
        uint64_t pb[RT];
        score_tile(tl, first_t + i * NW, pb);
        if (i + 1 < n_w) issue_tile(tl, first_t + (i + 1) * NW, block_of(first_t + (i + 1) * NW));
        pv_tile(pb);
      }
    } else if (n_w > 0) {
      // (Reloading a tile's registers right after its scores, which keeps
      // PF + 1 tiles in flight through the PV product, measured slower.)
#pragma unroll
      for (int u = 1; u < PF; ++u) issue_tile(ring[u], tile_at(u), block_of(tile_at(u)));
      int blk_next = block_of(tile_at(PF));
      for (int i = 0;; i += PF + 1) {
#pragma unroll
        for (int u = 0; u <= PF; ++u) {
          uint64_t pb[RT];
          issue_tile(ring[(u + PF) % (PF + 1)], tile_at(i + u + PF), blk_next);
          blk_next = block_of(tile_at(i + u + PF + 1));
          score_tile(ring[u], first_t + (i + u) * NW, pb);
          pv_tile(pb);
          if (i + u + 1 >= n_w) goto chunk_done;
        }
      }
    }
  chunk_done:
    if (ce >= te) break;
    // Next chunk: every wave has read its last id of this one.
    __syncthreads();
    cs = ce;
    for (int t = tid; t < min(te - cs, kMaxSegTiles); t += SH::kThreads)
      sm_ids[t] = table[((cs + t) * 16) / p.page_size];
    __syncthreads();
  }

  // Packed cache: the V codes entered the products as offset + code, with
  // the step in the weight; the offset times the row's sum of the rounded
  // weights comes off every column.
  if constexpr (FMT != 0) {
    constexpr float kOff = float(1 << (Oct<FMT>::VB - 1)) - 0.5f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float corr = kOff * psum[rt][0];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[rt][dt][e] = fmaf(acc[rt][dt][e], kCodeScale, -corr);
    }
  }

  // ---- combine the waves (one LDS slot per wave, summed in wave order:
  //      deterministic) ----
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_run[rt] += __shfl_xor(l_run[rt], 16);
    l_run[rt] += __shfl_xor(l_run[rt], 32);
  }
  __syncthreads();  // V staging area is reused below
  using CB = Combine<D, RT, NW>;
  float* sm_m = CB::m(lds);      // [NW][kRows]
  float* sm_l = CB::l(lds);      // [NW][kRows]
  float* sm_ms = CB::ms(lds);    // [kRows] merged max
  float* sm_ls = CB::ls(lds);    // [kRows] merged sum
  float* sm_acc = CB::acc(lds);  // [NW][kRows][kAccStride]
  if (g == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      sm_m[wave * SH::kRows + rt * 16 + c] = m_run[rt];
      sm_l[wave * SH::kRows + rt * 16 + c] = l_run[rt];
    }
  }
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + c;
    float ms = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) ms = fmaxf(ms, sm_m[w * SH::kRows + r]);
    const float mu = ms == kNegInf ? 0.f : ms;
    const float f = fast_exp2(m_run[rt] - mu);
    float* slot = sm_acc + (wave * SH::kRows + r) * CB::kAccStride + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(slot + 16 * dt) = acc[rt][dt] * f;
    if (wave == 0 && g == 0) {
      float ls = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) ls += sm_l[w * SH::kRows + r] * fast_exp2(sm_m[w * SH::kRows + r] - mu);
      sm_ms[r] = ms;
      sm_ls[r] = ls;
    }
  }
  __syncthreads();
  if constexpr (FMT != 0) {
    // Packed cache: the summed rows leave the rotated space of the values,
    // o = s * (H o') / 16, before they are written or published (the merge
    // is linear, so it may combine rotated-back partials).  A wave takes a
    // row at a time, four consecutive columns per lane: index bits 0-1 in
    // the lane, bits 2-7 across lanes.
    const uint32_t vsw = p.v_signs[lane >> 3];
    for (int r = wave; r < wg_rows; r += NW) {
      float* rowp = sm_acc + r * CB::kAccStride + 4 * lane;
      f32x4 a = *reinterpret_cast<const f32x4*>(rowp);
#pragma unroll
      for (int w = 1; w < NW; ++w) a += *reinterpret_cast<const f32x4*>(rowp + w * CB::kRows * CB::kAccStride);
      float v[4] = {a[0] + a[1], a[0] - a[1], a[2] + a[3], a[2] - a[3]};
      float u[4] = {v[0] + v[2], v[1] + v[3], v[0] - v[2], v[1] - v[3]};
#pragma unroll
      for (int o = 1; o < 64; o <<= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = wht_lane_stage(u[i], o, (lane & o) != 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = u[i] * 0.0625f;
        a[i] = ((vsw >> ((4 * lane + i) & 31)) & 1u) ? -x : x;
      }
      *reinterpret_cast<f32x4*>(rowp) = a;
    }
    __syncthreads();
  }
  finish<T, D, RT, NW, FMT ? 1 : NW>(p, lds, s, kvh, row0, wg_rows, fr, SH::kBytes);
}

// PERSIST selects the grid: one workgroup per item, or the persistent
// grid (separate instantiations, so each inlines the item body once).
// The arguments the prologue's first loads depend on (the length, the first
// block id and the first K/V tile's address) lead the argument list as
// scalars, and the build preloads the first 11 arguments -- the three
// pointers and seq_lens .. head_stride, 14 dwords; the token stride, needed
// only once the length has arrived, is not among them -- into scalar
// registers before the waves start (the compiler option
// -amdgpu-kernarg-preload-count counts arguments): those loads then wait
// for no kernel-argument fetch.  The other fields stay in the Params block; the
// host keeps the three strides within 32 bits.  (One sequence of 32k
// keys: 31.35 -> 31.03 us; 4k keys: 12.89 -> 12.65 us.)
// A packed cache's kernels are held to two waves per SIMD (at most 256
// registers per lane), so kPackedWgPerCu workgroups share a CU.
template <typename T, int D, int RT, bool PERSIST, bool LEAN, int FMT = 0>
__global__ __launch_bounds__((Shape<D, RT>::kThreads))
__attribute__((amdgpu_waves_per_eu(FMT != 0 ? kPackedWgPerCu : 1))) void decode_mfma_kernel(
    const int32_t* seq_lens, const int32_t* block_table, const void* kv, int32_t row_groups, int32_t num_kv_heads,
    int32_t max_blocks, int32_t seg_tiles, int32_t page_size, int32_t window, int32_t block_stride,
    int32_t head_stride, int32_t token_stride, Params params) {
  Params p = params;
  p.seq_lens = seq_lens;
  p.block_table = block_table;
  p.kv = kv;
  p.row_groups = row_groups;
  p.num_kv_heads = num_kv_heads;
  p.max_blocks = max_blocks;
  p.seg_tiles = seg_tiles;
  p.page_size = page_size;
  p.window = window;
  p.block_stride = block_stride;
  p.head_stride = head_stride;
  p.token_stride = token_stride;
  using SH = Shape<D, RT, LEAN>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[SH::kBytes];
  if constexpr (!PERSIST) {
    // One workgroup per item.  Workgroups are dealt to the 8 XCDs
    // round-robin by index; when a kv head's rows take several row groups,
    // the row groups of one (kv head, segment) are given consecutive
    // indices on one XCD, so they run together and all but the first find
    // the K/V tiles in that XCD's L2.
    int kvh, rg, seg;
    if (p.row_groups > 1 && gridDim.x % (kXcds * p.row_groups) == 0) {
      const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
      rg = local % p.row_groups;
      const int pair = (local / p.row_groups) * kXcds + xcd;
      kvh = pair % p.num_kv_heads;
      seg = pair / p.num_kv_heads;
    } else {
      const int units = p.num_kv_heads * p.row_groups;
      const int unit = blockIdx.x % units;
      seg = blockIdx.x / units;
      kvh = unit % p.num_kv_heads;
      rg = unit / p.num_kv_heads;
    }
    decode_unit<T, D, RT, LEAN, false, FMT>(p, lds, blockIdx.y, kvh, rg, seg, Frag{});
  } else {
    balanced_loop(
        p, lds, SH::kPersistOff, SH::kThreads,
        [&](int s, int kvh, int rg, const Frag& f) { decode_unit<T, D, RT, LEAN, true, FMT>(p, lds, s, kvh, rg, 0, f); },
        [&](int s, int kvh, int rg, int M) {
          const int row0 = rg * RT * 16, n = min(RT * 16, p.group * M - row0);
          if (n > 0) zero_rows<T, D>(p, s, kvh, row0, n, SH::kThreads);
        });
  }
}

// ---------------------------------------------------------------------------
// Per-head dot-product family for small GQA (G*M <= 4 query rows per kv
// head, head size <= 128): no MFMA and no row padding.  The K/V loads, the
// tile loop, the combine and the split-KV epilogue are those of the MFMA
// kernel; per 16-key tile a wave
//   * forms each row's q.k with v_dot2_f32_{bf16,f16} over the eight
//     head-dim elements a lane holds, then sums the four lane groups that
//     split the head dimension (two cross-lane steps);
//   * takes the online softmax over the tile's 16 keys (one key per lane);
//   * accumulates p * v in fp32 per lane, i.e. per key slot; the key slots
//     are summed once, after the last tile.
template <typename T>
struct Dot;

template <>
struct Dot<__bf16> {
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ float dot2(int a, int b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(x2, a), __builtin_bit_cast(x2, b), c, false);
  }
  static __device__ __forceinline__ float lo(int w) { return __builtin_bit_cast(float, uint32_t(w) << 16); }
  static __device__ __forceinline__ float hi(int w) { return __builtin_bit_cast(float, uint32_t(w) & 0xffff0000u); }
};

template <>
struct Dot<_Float16> {
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ float dot2(int a, int b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(x2, a), __builtin_bit_cast(x2, b), c, false);
  }
  static __device__ __forceinline__ float lo(int w) { return float(__builtin_bit_cast(x2, w)[0]); }
  static __device__ __forceinline__ float hi(int w) { return float(__builtin_bit_cast(x2, w)[1]); }
};

constexpr int kDotWaves = kDotWaveCount;
constexpr int kDotRows = kDotMaxRows;

template <int D>
struct DotShape {
  static constexpr int NW = kDotWaves;
  static constexpr int kThreads = NW * 64;
  static constexpr int KC = D / 32;
  static constexpr int PF = 1;
  static constexpr int kBytes = Combine<D, 1, NW>::kBytes + 16;
};

template <typename T, int D>
__global__ __launch_bounds__(kDotWaves * 64) void decode_dot_kernel(Params p) {
  using DT2 = Dot<T>;
  using SH = DotShape<D>;
  using CB = Combine<D, 1, SH::NW>;
  constexpr int NW = SH::NW, KC = SH::KC, R = kDotRows;
  __shared__ __attribute__((aligned(16))) unsigned char lds[SH::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int s = blockIdx.y;
  const int kvh = blockIdx.x % p.num_kv_heads;
  const int seg = blockIdx.x / p.num_kv_heads;
  const SeqQ sq = seq_queries(p, s);
  const int M = sq.m;
  const int rows = p.group * M;  // <= kDotRows
  if (rows == 0) return;

  // Lengths past the block table's capacity are clamped to it.
  const int L = min(p.seq_lens[s], p.max_blocks * p.page_size);
  if (L <= 0) {
    if (seg == 0) zero_rows<T, D>(p, s, kvh, 0, rows, SH::kThreads);
    return;
  }
  const int k_lo = p.window > 0 ? max(0, L - M - p.window + 1) : 0;
  const int t_lo = k_lo >> 4, t_hi = (L + 15) >> 4;
  const int n_tiles = t_hi - t_lo;
  const int seg_tiles = max(p.seg_tiles, (n_tiles + p.nseg - 1) / p.nseg);
  const int n_live = (n_tiles + seg_tiles - 1) / seg_tiles;
  if (seg >= n_live) return;
  const int ts = t_lo + seg * seg_tiles, te = min(ts + seg_tiles, t_hi);
  const int lo_last = p.window > 0 ? max(0, L - p.window) : 0;
  const int qpos_first = L - M;

  // Query rows (row = m * G + head in group), each lane holding the eight
  // head-dim elements 32 kc + 8 g .. of every chunk kc.
  int qpos_r[R], lo_r[R];
  i32x4 q[R][KC];
  const T* Q = static_cast<const T*>(p.q);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rows) {
      const int m = r / p.group, gq = r % p.group;
      qpos_r[r] = L - M + m;
      lo_r[r] = p.window > 0 ? max(0, qpos_r[r] - p.window + 1) : 0;
      const T* qrow = Q + ((int64_t(sq.first) + m) * p.num_q_heads + kvh * p.group + gq) * D;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) q[r][kc] = *reinterpret_cast<const i32x4*>(qrow + 32 * kc + 8 * g);
    } else {
      qpos_r[r] = -1;
      lo_r[r] = 0;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) q[r][kc] = i32x4{0, 0, 0, 0};
    }
  }

  float m_run[R], l_run[R];       // l_run: this lane's key slot only
  float acc[R][KC][8];            // this lane's key slot, head-dim 32 kc + 8 g + e
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m_run[r] = kNegInf;
    l_run[r] = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][kc][e] = 0.f;
  }

  const unsigned char* KVh =
      static_cast<const unsigned char*>(p.kv) + int64_t(kvh) * p.head_stride * int64_t(sizeof(T));
  const int32_t* table = p.block_table + int64_t(s) * p.max_blocks;
  const uint32_t lane_off = uint32_t(c * p.token_stride + 8 * g) * uint32_t(sizeof(T));

  struct Tile {
    i32x4 k[KC];
    i32x4 v[KC];
  };
  auto block_of = [&](int t) { return table[(t * 16) / p.page_size]; };
  auto issue_tile = [&](Tile& tl, int t, int blk) {
    const int key0 = t * 16;
    const unsigned char* row =
        KVh + (int64_t(blk) * p.block_stride + int64_t(key0 % p.page_size) * p.token_stride) * int64_t(sizeof(T)) +
        lane_off;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) tl.k[kc] = *reinterpret_cast<const i32x4*>(row + 64 * kc);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) tl.v[kc] = *reinterpret_cast<const i32x4*>(row + 2 * D + 64 * kc);
  };

  auto compute_tile = [&](Tile& tl, int t) {
    const int key0 = t * 16;
    const int key = key0 + c;  // this lane's key
    const bool edge = !(key0 >= lo_last && key0 + 15 <= qpos_first);
    if (edge && (key < k_lo || key >= L)) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) tl.v[kc] = i32x4{0, 0, 0, 0};
    }
    float vf[KC][8];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vf[kc][2 * w] = DT2::lo(tl.v[kc][w]);
        vf[kc][2 * w + 1] = DT2::hi(tl.v[kc][w]);
      }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r >= rows) continue;
      float dotp = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int w = 0; w < 4; ++w) dotp = DT2::dot2(tl.k[kc][w], q[r][kc][w], dotp);
      dotp += __shfl_xor(dotp, 16);
      dotp += __shfl_xor(dotp, 32);
      float x = dotp * p.scale_log2;
      if (edge && (key < lo_r[r] || key > qpos_r[r])) x = kNegInf;
      float tmax = x;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
      const float m_new = fmaxf(m_run[r], tmax);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[r] - m_use);
      const float pr = fast_exp2(x - m_use);
      l_run[r] = l_run[r] * alpha + pr;
      m_run[r] = m_new;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][kc][e] = acc[r][kc][e] * alpha + pr * vf[kc][e];
    }
  };

  // Same tile schedule as the MFMA kernel (interleaved tiles, one tile of
  // prefetch, clamped prefetch index).
  const int first_t = ts + wave;
  const int n_w = first_t < te ? (te - first_t + NW - 1) / NW : 0;
  auto tile_at = [&](int i) { return first_t + min(i, n_w - 1) * NW; };
  if (n_w > 0) {
    Tile ring[SH::PF + 1];
#pragma unroll
    for (int u = 0; u < SH::PF; ++u) issue_tile(ring[u], tile_at(u), block_of(tile_at(u)));
    int blk_next = block_of(tile_at(SH::PF));
    for (int i = 0;; i += SH::PF + 1) {
#pragma unroll
      for (int u = 0; u <= SH::PF; ++u) {
        issue_tile(ring[(u + SH::PF) % (SH::PF + 1)], tile_at(i + u + SH::PF), blk_next);
        blk_next = block_of(tile_at(i + u + SH::PF + 1));
        compute_tile(ring[u], first_t + (i + u) * NW);
        if (i + u + 1 >= n_w) goto tiles_done;
      }
    }
  }
tiles_done:

  // Sum the 16 key slots of each lane group (fixed butterfly order).
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) l_run[r] += __shfl_xor(l_run[r], off);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) acc[r][kc][e] += __shfl_xor(acc[r][kc][e], off);
  }

  // Combine the waves through LDS, as in the MFMA kernel.
  float* sm_m = CB::m(lds);
  float* sm_l = CB::l(lds);
  float* sm_ms = CB::ms(lds);
  float* sm_ls = CB::ls(lds);
  float* sm_acc = CB::acc(lds);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (lane == 0) {
      sm_m[wave * CB::kRows + r] = m_run[r];
      sm_l[wave * CB::kRows + r] = l_run[r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= rows) continue;
    float ms = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) ms = fmaxf(ms, sm_m[w * CB::kRows + r]);
    const float mu = ms == kNegInf ? 0.f : ms;
    const float f = fast_exp2(m_run[r] - mu);
    if (c == 0) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        float* dst = sm_acc + (wave * CB::kRows + r) * CB::kAccStride + 32 * kc + 8 * g;
        *reinterpret_cast<f32x4*>(dst) = f32x4{acc[r][kc][0], acc[r][kc][1], acc[r][kc][2], acc[r][kc][3]} * f;
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[r][kc][4], acc[r][kc][5], acc[r][kc][6], acc[r][kc][7]} * f;
      }
    }
    if (wave == 0 && lane == 0) {
      float ls = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) ls += sm_l[w * CB::kRows + r] * fast_exp2(sm_m[w * CB::kRows + r] - mu);
      sm_ms[r] = ms;
      sm_ls[r] = ls;
    }
  }
  __syncthreads();
  Frag fr;
  fr.ts = ts;
  fr.te = te;
  fr.n_parts = n_live;
  fr.merge_slices = p.merge_slices;
  const int64_t slot0 = (int64_t(s) * p.num_kv_heads + kvh) * p.nseg;
  fr.slot = slot0 + seg;
  fr.parts.first = slot0;
  fr.parts.last = slot0 + n_live - 1;
  fr.parts.n = n_live;
  fr.parts.row0 = 0;
  fr.ctl = p.ws_cnt + (int64_t(s) * p.num_kv_heads + kvh) * p.merge_slices * kCtlStride;
  finish<T, D, 1, NW>(p, lds, s, kvh, 0, rows, fr, SH::kBytes);
}

// The persistent grid always fills the device and runs the lean loop; a
// grid of one workgroup per item takes it when the plan says it fills the
// device.  Where the ring has one tile anyway, one variant serves both.
// A packed cache (FMT > 0) keeps the two-tile ring on both schedules: its
// tiles take a few registers per lane.
template <typename T, int D, int RT, int FMT = 0>
int launch_t(const Plan& pl, const Params& pr, hipStream_t st) {
  constexpr bool kTwo = FMT == 0 && Shape<D, RT, false>::PF != Shape<D, RT, true>::PF;
  const dim3 grid(pl.grid_x, pl.grid_y), block(Shape<D, RT>::kThreads);
  const auto kernel = pl.persistent      ? decode_mfma_kernel<T, D, RT, true, kTwo, FMT>
                      : kTwo && pl.lean ? decode_mfma_kernel<T, D, RT, false, kTwo, FMT>
                                        : decode_mfma_kernel<T, D, RT, false, false, FMT>;
  // The strides fit in 32 bits (checked by the planner).
  hipLaunchKernelGGL(kernel, grid, block, 0, st, pr.seq_lens, pr.block_table, pr.kv, pr.row_groups, pr.num_kv_heads,
                     pr.max_blocks, pr.seg_tiles, pr.page_size, pr.window, int32_t(pr.block_stride),
                     int32_t(pr.head_stride), int32_t(pr.token_stride), pr);
  return int(hipGetLastError());
}

#ifndef PAD_OCTAVE
template <typename T, int D>
int launch_d(const Plan& pl, const Params& pr, hipStream_t st) {
  switch (pl.row_tiles) {
    case 1: return launch_t<T, D, 1>(pl, pr, st);
    case 2: if constexpr (D <= 256) return launch_t<T, D, 2>(pl, pr, st); break;
    case 3: if constexpr (D <= 128) return launch_t<T, D, 3>(pl, pr, st); break;
    case 4: if constexpr (D <= 128) return launch_t<T, D, 4>(pl, pr, st); break;
  }
  return int(hipErrorInvalidValue);
}

template <typename T, int D>
int launch_dtype(const Plan& pl, const Params& pr, hipStream_t st) {
  if (pl.path == PAD_PATH_DOT) {
    if constexpr (D <= kDotMaxHeadSize) {
      hipLaunchKernelGGL((decode_dot_kernel<T, D>), dim3(pl.grid_x, pl.grid_y), dim3(DotShape<D>::kThreads), 0, st,
                         pr);
      return int(hipGetLastError());
    }
    return int(hipErrorInvalidValue);
  }
  return launch_d<T, D>(pl, pr, st);
}
#else
// The planner gives a packed cache one row tile per wave.
template <typename T, int FMT>
int launch_octave_t(const Plan& pl, const Params& pr, hipStream_t st) {
  if (pl.row_tiles == 1) return launch_t<T, kOctD, 1, FMT>(pl, pr, st);
  return int(hipErrorInvalidValue);
}

template <typename T>
int launch_octave_dtype(const Plan& pl, const Params& pr, int format, hipStream_t st) {
  switch (format) {
    case PAD_KV_OCTAVE_K3V4: return launch_octave_t<T, PAD_KV_OCTAVE_K3V4>(pl, pr, st);
    case PAD_KV_OCTAVE_K3V3: return launch_octave_t<T, PAD_KV_OCTAVE_K3V3>(pl, pr, st);
    case PAD_KV_OCTAVE_K3V3_COMPACT: return launch_octave_t<T, PAD_KV_OCTAVE_K3V3_COMPACT>(pl, pr, st);
  }
  return int(hipErrorInvalidValue);
}
#endif

}  // namespace

#ifndef PAD_OCTAVE
// This source is compiled once per head size (PAD_HEAD_SIZE), so the
// instantiations of the four sizes build in parallel.
template <>
int launch_decode_hs<PAD_HEAD_SIZE>(const Plan& plan, const Params& params, int dtype, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == PAD_BF16) return launch_dtype<__bf16, PAD_HEAD_SIZE>(plan, params, st);
  return launch_dtype<_Float16, PAD_HEAD_SIZE>(plan, params, st);
}
#else
// A further build of this source (head size 256, PAD_OCTAVE) holds the
// packed-cache kernels only.
int launch_decode_octave(const Plan& plan, const Params& params, int dtype, int format, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == PAD_BF16) return launch_octave_dtype<__bf16>(plan, params, format, st);
  return launch_octave_dtype<_Float16>(plan, params, format, st);
}
#endif

}  // namespace pad
