// Prefill chunks for gfx950: attention of a chunk of query tokens (its
// own keys included, causal) over the paged cache, as the prefill work
// items of plan_prefill and PrefillVariant (block_rows, key_tile,
// double_buffer) on the rocm_rdna_hip docs page describe it: a workgroup
// takes a block of query rows of one kv head and streams the key range in
// shared key tiles.
//
// One workgroup serves one (sequence, kv head, 128-row block, key
// segment): the kv head's G * M query rows are GQA-packed (row = token * G
// + head) and cut into blocks of 128.  Its eight waves form four slabs of
// 32 rows; the two waves of a slab take the two 64-key halves of every
// 128-key tile (two independent waves per SIMD, so one's softmax overlaps
// the other's products) and are combined at the end.  Per tile, staged
// once in LDS for all eight waves (double-buffered, its loads issued two
// tiles ahead into registers), a wave
//   * forms S^T = K Q^T with v_mfma_f32_32x32x16 (K rows from LDS as the A
//     operand, its query rows as the B operand, kept in registers), which
//     leaves each lane 16 keys of one query row per 32-key block -- the row
//     maximum needs one cross-lane step;
//   * takes the online softmax in the exp2 domain with the decode kernel's
//     lazy rescale;
//   * accumulates O^T += V^T P^T with the same instruction: P^T is the B
//     operand exactly as the scores left it, once the keys of a 16-key step
//     are taken in the order the score layout holds them (keys 4h..4h+3 and
//     8+4h..8+4h+3 of the step in lane half h), and V^T is read in that
//     order from LDS by two transposed reads (ds_read_b64_tr_b16: four
//     consecutive keys of one head-dim column per lane).
// A block's key range is split into segments that fill the device; their
// partials are merged by the split-KV epilogue of the decode kernel.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "decode_common.h"
#include "kernels.h"

namespace pad {
namespace {

using namespace dev;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T>
struct Mfma32;
template <>
struct Mfma32<__bf16> {
  static __device__ __forceinline__ f32x16 mma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  }
};
template <>
struct Mfma32<_Float16> {
  static __device__ __forceinline__ f32x16 mma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
};

template <int D>
struct PfShape {
  static constexpr int NW = kPrefillWaves;
  static constexpr int kThreads = NW * 64;
  static constexpr int kHalves = NW / 4;   // waves per 32-row slab (key halves of a tile)
  static constexpr int kRows = kPrefillRows;   // query rows of a workgroup
  static constexpr int kKeys = kPrefillKeys;   // keys of an LDS tile
  static constexpr int kGroups = kKeys / 16;   // 16-key groups of a tile
  static constexpr int KB = kKeys / 32 / kHalves;  // 32-key blocks of a tile per wave
  // Elements per LDS row.  K rows are read 16 bytes per lane, 32
  // consecutive rows at a time: a 4-dword pad puts them on distinct banks.
  // V rows are read transposed, 8 bytes per lane from four consecutive
  // rows and two 16-column groups: a 16-dword pad puts a 32-lane read on
  // all 64 banks once.
  static constexpr int kStride = D + 8;
  static constexpr int kVStride = D + 32;
  static constexpr int kTileElems = kKeys * kStride;  // the K rows; the V rows follow
  static constexpr int kBufBytes = (kTileElems + kKeys * kVStride) * 2;  // the K and V rows of one tile
  static constexpr int kIdsOff = 2 * kBufBytes;         // after two buffers
  static constexpr int kLoopBytes = kIdsOff + kPrefillMaxSegTiles * 8;
  using CB = Combine<D, kRows / 16, 1>;
  static constexpr int kBytes = (kLoopBytes > CB::kBytes ? kLoopBytes : CB::kBytes) + 16;
  static constexpr int DS = D / 16;  // 16-element steps of QK^T
  static constexpr int DB = D / 32;  // 32-column blocks of the output
  static constexpr int kChunksPerKey = 2 * D / 8;  // 16-byte chunks of a key's K and V rows
  static constexpr int kPerThread = kKeys * kChunksPerKey / kThreads;
  static_assert(kPerThread * kThreads == kKeys * kChunksPerKey, "tile chunks split evenly over the threads");
  static_assert(NW == 4 || NW == 8, "four slabs of 32 rows, one or two waves each");
  // The pair exchange (running max and sum of each half) after the loop
  // uses the block-id area, past the combine area.
  static_assert(kIdsOff >= CB::kBytes && kPrefillMaxSegTiles >= 4 * kRows, "exchange area");
};

template <typename T, int D>
__global__ __launch_bounds__(kPrefillWaves * 64, 1) void prefill_kernel(Params p) {
  using SH = PfShape<D>;
  using MM = Mfma32<T>;
  using MF = Mfma<T>;
  using CB = typename SH::CB;
  constexpr int DS = SH::DS, DB = SH::DB, NT = SH::kThreads;
  __shared__ __attribute__((aligned(16))) unsigned char lds[SH::kBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;  // this lane's query row in the wave, its lane half
  const int slab = wave & 3, half = wave >> 2;  // the wave's 32 rows, its 32-key blocks of a tile

  // Work item: the row blocks of the latest tokens (the longest key ranges)
  // first.
  const int per_rg = p.num_kv_heads * p.nseg;
  const int rg = p.row_groups - 1 - int(blockIdx.x) / per_rg;
  const int rest = int(blockIdx.x) % per_rg;
  const int kvh = rest % p.num_kv_heads, seg = rest / p.num_kv_heads;
  const int s = blockIdx.y;
  const SeqQ sq = seq_queries(p, s);
  const int M = sq.m;
  const int rows = p.group * M;
  const int row0 = rg * SH::kRows;
  const int wg_rows = min(SH::kRows, rows - row0);
  if (wg_rows <= 0) return;
  const int L = clamped_len(p, s);
  if (L <= 0) {
    if (seg == 0) zero_rows<T, D>(p, s, kvh, row0, wg_rows, NT);
    return;
  }
  const SegSplit sp = split_of(p, L, M, rg);
  if (seg >= sp.n_live) return;
  Frag fr;
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
  const int ts = fr.ts, te = fr.te;

  // Where each 16-key tile of the segment starts: the element offset of
  // its first key's K row in the kv head's cache (page and in-page token),
  // once per tile here rather than per load (the planner keeps a segment
  // within kPrefillMaxSegTiles tiles).
  const int32_t* table = p.block_table + int64_t(s) * p.max_blocks;
  int64_t* sm_off = reinterpret_cast<int64_t*>(lds + SH::kIdsOff);
  for (int t = tid; t < te - ts; t += NT) {
    const int key = (t + ts) * 16;
    sm_off[t] = int64_t(table[key / p.page_size]) * p.block_stride + int64_t(key % p.page_size) * p.token_stride;
  }

  // This lane's query row: its B operand chunks (head-dim 16 st + 8 h ..
  // + 7 of step st), position and window start; rows past G*M see nothing.
  // The scale's sign goes into the query rows (an exact sign flip), so
  // the scores' exp2-domain values are x * |scale log2 e|: the largest raw
  // score of a row gives the largest scaled one.
  const int r = row0 + slab * 32 + n;
  const float sl2 = fabsf(p.scale_log2);
  const int qsign = p.scale_log2 < 0.f ? int(0x80008000u) : 0;
  i32x4 qop[DS];
  if (r < rows) {
    const T* qrow = static_cast<const T*>(p.q) +
                    ((int64_t(sq.first) + r / p.group) * p.num_q_heads + kvh * p.group + r % p.group) * D + 8 * h;
#pragma unroll
    for (int st = 0; st < DS; ++st) qop[st] = *reinterpret_cast<const i32x4*>(qrow + 16 * st) ^ qsign;
  } else {
#pragma unroll
    for (int st = 0; st < DS; ++st) qop[st] = i32x4{0, 0, 0, 0};
  }
  const int qpos = r < rows ? L - M + r / p.group : -1;
  const int lo_r = r < rows && p.window > 0 ? max(0, qpos - p.window + 1) : 0;
  // Keys every row of the workgroup sees, inside the segment: tiles within
  // [full_lo, full_hi] need no mask.  Keys outside [key_lo, key_hi) are not
  // loaded (their rows are zero: they may hold anything, even NaN).
  const int qpos_min = L - M + row0 / p.group;
  const int qpos_max = L - M + (row0 + wg_rows - 1) / p.group;
  const int lo_min = p.window > 0 ? max(0, qpos_min - p.window + 1) : 0;
  const int lo_max = p.window > 0 ? max(0, qpos_max - p.window + 1) : 0;
  const int key_lo = max(16 * ts, lo_min), key_hi = min(16 * te, L);
  const int full_lo = max(16 * ts, lo_max), full_hi = min(min(16 * te, L) - 1, qpos_min);
  // This row's visible keys in the segment: [vis_lo, vis_hi), empty for a
  // row past the query rows.
  const int vis_lo = max(lo_r, key_lo), vis_hi = min(qpos + 1, key_hi);
  const uint32_t vis_span = uint32_t(max(vis_hi - vis_lo, 0));

  const unsigned char* KVh =
      static_cast<const unsigned char*>(p.kv) + int64_t(kvh) * p.head_stride * int64_t(sizeof(T));
  auto kbuf = [&](int b) { return reinterpret_cast<uint16_t*>(lds + b * SH::kBufBytes); };
  // Chunk u of this thread in a tile: key kKeysPerU u + key_t of the tile,
  // its K row (part 0) or V row, 16 bytes at column chunk col.  A tile's
  // four 16-key groups each lie in one page: their offsets are
  // wave-uniform (a group outside the segment is clamped to one inside it;
  // such keys are zeroed when the tile is stored), and a chunk sits at a
  // fixed byte offset from its group's first K row.
  constexpr int kKeysPerU = NT / (D / 4);
  static_assert(kKeysPerU == 16 || kKeysPerU == 32, "a thread's chunk u covers one or two 16-key groups");
  const int key_t = tid / (D / 4), part = (tid / (D / 8)) & 1, col = tid % (D / 8);
  const uint32_t chunk_off =
      (uint32_t(key_t & 15) * uint32_t(p.token_stride) + uint32_t(part * D)) * uint32_t(sizeof(T)) + 16u * col;
  // Two register stages: a tile's loads go out two tiles ahead of its
  // products, every chunk loaded (a fixed count per tile keeps the
  // compiler's wait counts exact, so storing a tile waits only for its own
  // loads).
  i32x4 stage[2][SH::kPerThread];
  auto load_tile = [&](int kt, int sl) {
    const unsigned char* gbase[SH::kGroups];
#pragma unroll
    for (int g = 0; g < SH::kGroups; ++g) {
      const int t16 = min(max(SH::kGroups * kt + g, ts), te - 1);
      const int64_t off = sm_off[t16 - ts];
      const uint32_t lo = __builtin_amdgcn_readfirstlane(int(uint32_t(uint64_t(off))));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(int(uint32_t(uint64_t(off) >> 32)));
      gbase[g] = KVh + int64_t((uint64_t(hi) << 32) | lo) * int64_t(sizeof(T));
    }
#pragma unroll
    for (int u = 0; u < SH::kPerThread; ++u) {
      // the key's 16-key group: u (16 keys per u) or one of u's two groups
      const unsigned char* gb =
          kKeysPerU == 16 ? gbase[u] : gbase[2 * u + (key_t >> 4)];
      stage[sl][u] = *reinterpret_cast<const i32x4*>(gb + chunk_off);
    }
  };
  // Keys outside [key_lo, key_hi) may hold anything (even NaN): zeros go to
  // LDS instead.
  auto store_tile = [&](int kt, int b, int sl) {
    const int key0 = kt * SH::kKeys;
    const bool full = key0 >= key_lo && key0 + SH::kKeys <= key_hi;
#pragma unroll
    for (int u = 0; u < SH::kPerThread; ++u) {
      const int key = kKeysPerU * u + key_t;
      i32x4 v = stage[sl][u];
      if (!full && (key0 + key < key_lo || key0 + key >= key_hi)) v = i32x4{0, 0, 0, 0};
      *reinterpret_cast<i32x4*>(kbuf(b) + part * SH::kTileElems + key * (part ? SH::kVStride : SH::kStride) +
                                8 * col) = v;
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;

  __syncthreads();  // the block ids
  const int kt0 = ts / SH::kGroups, kt1 = (te + SH::kGroups - 1) / SH::kGroups;
  load_tile(kt0, 0);
  store_tile(kt0, 0, 0);
  load_tile(min(kt0 + 1, kt1 - 1), 1);
  __syncthreads();
  // Tile kt is in LDS buffer b; tile kt + 1 in register stage b ^ 1 goes to
  // LDS buffer b ^ 1 after the products; tile kt + 2 is loaded into stage
  // b (free once tile kt was stored) -- the last tile again past the end,
  // so every iteration has the same loads in flight.  Unrolled by two so
  // the stage indices are constants.
  auto step = [&](int kt, int b) {
    load_tile(min(kt + 2, kt1 - 1), b);
    const uint16_t* kt_lds = kbuf(b);
    const uint16_t* vt_lds = kbuf(b) + SH::kTileElems;
    const int key0 = kt * SH::kKeys;
    // S^T of this wave's 32-key blocks kb = half * KB + j (independent
    // product chains).
    constexpr int KB = SH::KB;
    f32x16 sc[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[j][v] = 0.f;
      const uint16_t* kr = kt_lds + ((half * KB + j) * 32 + n) * SH::kStride + 8 * h;
#pragma unroll
      for (int st = 0; st < DS; ++st) sc[j] = MM::mma(*reinterpret_cast<const i32x4*>(kr + 16 * st), qop[st], sc[j]);
    }
    // Value v of block kb is key key0 + 32 kb + 8 (v / 4) + 4 h + v % 4.
    // The online softmax; on tiles with a key some row may not see
    // (wave-uniform), with those scores masked: -inf for the maximum and
    // a zero weight whatever the scale.  p = 2^(x |scale log2 e| - m).
    // The two variants are separate code, so the unmasked tiles run no
    // mask arithmetic.
    float alpha = 1.f, psum = 0.f;
    bool moved = false;
    i32x4 pb[KB][2];
    auto softmax = [&](auto masked_t) {
      constexpr bool kMasked = decltype(masked_t)::value;
      if constexpr (kMasked) {
        // The row sees keys [vis_lo, vis_hi); relative to this lane's first
        // key, a key is visible when its offset is below the span.
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          const int base = key0 + 32 * (half * KB + j) + 4 * h - vis_lo;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (uint32_t(base + 8 * (v >> 2) + (v & 3)) >= vis_span) sc[j][v] = kNegInf;
        }
      }
      float tmax = kNegInf;
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sc[j][v]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      tmax = tmax == kNegInf ? kNegInf : tmax * sl2;
      const bool move = tmax > m_run + kMaxSlack;
      const float m_new = move ? tmax : m_run;
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      alpha = move ? fast_exp2(m_run - m_use) : 1.f;
      m_run = m_new;
      moved = __builtin_amdgcn_ballot_w64(move) != 0;
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = sc[j][8 * sub + 2 * e], x1 = sc[j][8 * sub + 2 * e + 1];
            float p0 = fast_exp2(fmaf(x0, sl2, -m_use));
            float p1 = fast_exp2(fmaf(x1, sl2, -m_use));
            if constexpr (kMasked) {
              p0 = x0 == kNegInf ? 0.f : p0;
              p1 = x1 == kNegInf ? 0.f : p1;
            }
            psum += p0 + p1;
            pb[j][sub][e] = int(MF::pack2(p0, p1));
          }
    };
    const bool edge =
        __builtin_amdgcn_readfirstlane(int(!(key0 >= full_lo && key0 + SH::kKeys - 1 <= full_hi))) != 0;
    if (edge)
      softmax(std::true_type{});
    else
      softmax(std::false_type{});
    l_run = l_run * alpha + psum;
    if (moved) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    // O^T += V^T P^T: for 16-key step (kb, sub) the A operand of lane
    // (column d, half h) is V of keys 32 kb + 16 sub + 4 h + 0..3 and
    // + 8 + 0..3, two transposed reads (lane group g4 = lane / 16 addresses
    // rows 4 h + i / 4, columns 16 (g4 % 2) + 4 (i % 4) of the block).
    // The wave issuing its PV products runs at a raised priority, so the
    // other wave of its SIMD fills the gaps with its softmax (medians of six
    // graph-timed runs on two boxes, TFLOP/s: chunk 463 / 442 against 458 /
    // 438, 2048-token prompt 612 / 594 against 611 / 586, 4096-token prompt
    // 763 / 728 against 750 / 723; raised for the QK^T products too:
    // slower; for the softmax instead: no gain).
    __builtin_amdgcn_s_setprio(1);
    const int g4 = lane >> 4, i16 = lane & 15;
    const uint16_t* vtr = vt_lds + (4 * h + (i16 >> 2)) * SH::kVStride + 16 * (g4 & 1) + 4 * (i16 & 3);
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint16_t* a = vtr + (32 * (half * KB + j) + 16 * sub) * SH::kVStride + 32 * db;
          const uint64_t lo = __builtin_bit_cast(
              uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a)));
          const uint64_t hi = __builtin_bit_cast(
              uint64_t,
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a + 8 * SH::kVStride)));
          const i32x4 va = {int(uint32_t(lo)), int(uint32_t(lo >> 32)), int(uint32_t(hi)), int(uint32_t(hi >> 32))};
          acc[db] = MM::mma(va, pb[j][sub], acc[db]);
        }
    __builtin_amdgcn_s_setprio(0);
    if (kt + 1 < kt1) store_tile(kt + 1, b ^ 1, b ^ 1);
    __syncthreads();
  };
  for (int kt = kt0; kt < kt1; kt += 2) {
    step(kt, 0);
    if (kt + 1 >= kt1) break;
    step(kt + 1, 1);
  }

  // Rows of this wave: the running sum over both lane halves; with two key
  // halves per slab, the pair's maxima and sums meet in the block-id area
  // (dead now) and each wave rescales its accumulator to the pair's
  // maximum.  Then the accumulator columns (value v of block db is column
  // 32 db + 8 (v / 4) + 4 h + v % 4) go to slot 0 of the combine area,
  // which overlays the tile buffers: the second half's rows first, added
  // into the first half's in fixed order.
  l_run += __shfl_xor(l_run, 32);
  const int rr = slab * 32 + n;
  float* slot = CB::acc(lds) + rr * CB::kAccStride + 4 * h;
  auto put = [&]() {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(slot + 32 * db + 8 * q4) =
            f32x4{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]};
  };
  if constexpr (SH::kHalves == 1) {
    put();
    if (h == 0) {
      CB::ms(lds)[rr] = m_run;
      CB::ls(lds)[rr] = l_run;
    }
  } else {
    float* xm = reinterpret_cast<float*>(lds + SH::kIdsOff);  // [2][kRows]
    float* xl = xm + 2 * SH::kRows;                          // [2][kRows]
    if (h == 0) {
      xm[half * SH::kRows + rr] = m_run;
      xl[half * SH::kRows + rr] = l_run;
    }
    __syncthreads();
    const float m0 = xm[rr], m1 = xm[SH::kRows + rr];
    const float ms = fmaxf(m0, m1);
    const float mu = ms == kNegInf ? 0.f : ms;
    const float f = fast_exp2(m_run - mu);
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= f;
    if (half == 0 && h == 0) {
      CB::ms(lds)[rr] = ms;
      CB::ls(lds)[rr] = xl[rr] * fast_exp2(m0 - mu) + xl[SH::kRows + rr] * fast_exp2(m1 - mu);
    }
    if (half == 1) put();
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(slot + 32 * db + 8 * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][4 * q4 + e] += o[e];
        }
      put();
    }
  }
  __syncthreads();
  finish<T, D, SH::kRows / 16, 1, 1, NT>(p, lds, s, kvh, row0, wg_rows, fr, SH::kBytes);
}

template <typename T, int D>
int launch_prefill_t(const Plan& pl, const Params& pr, hipStream_t st) {
  hipLaunchKernelGGL((prefill_kernel<T, D>), dim3(pl.grid_x, pl.grid_y), dim3(PfShape<D>::kThreads), 0, st, pr);
  return int(hipGetLastError());
}

}  // namespace

int launch_prefill(const Plan& plan, const Params& params, int dtype, int head_size, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = dtype == PAD_BF16;
  switch (head_size) {
    case 64: return bf ? launch_prefill_t<__bf16, 64>(plan, params, st) : launch_prefill_t<_Float16, 64>(plan, params, st);
    case 128:
      return bf ? launch_prefill_t<__bf16, 128>(plan, params, st) : launch_prefill_t<_Float16, 128>(plan, params, st);
  }
  return int(hipErrorInvalidValue);
}

}  // namespace pad
