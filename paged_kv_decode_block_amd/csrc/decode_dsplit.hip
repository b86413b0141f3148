// Paged-KV decode attention for kv heads with many query rows (gfx950):
// the head-dimension-split family.
//
// When the G*M query rows of a kv head take two or more 16-row MFMA tiles
// (wide heads, speculative verify), one workgroup of four waves serves up
// to four row tiles and reads every 16-key K/V tile of its segment once
// (ROCm/vllm pull request 1330, "Summary": one read of a kv head's pages
// for all of its query rows; the accumulator split across waves along the
// head dimension).  Per tile:
//   * the workgroup stages K in LDS (16-byte loads spread over all
//     threads); each wave stages its own quarter of the head dimension of
//     V in a wave-private LDS buffer;
//   * wave r computes S^T = K Q_r^T for row tile r, masks it, updates the
//     online softmax of those rows and leaves P_r (input dtype) and the
//     rows' rescale factors in LDS;
//   * after one barrier every wave accumulates O^T += V^T P^T for every
//     row tile over its quarter of the head dimension.
// A wave's accumulator is rows x D/4, so several tiles of loads stay in
// flight in registers, and no cross-wave combine is needed at the end:
// each wave writes its own columns.  The split-KV arrival, the sliced merge and the persistent grid
// are those of the key-split kernel.
//
// LDS layout of K (and of each V quarter): 16-byte chunks of a key's row,
// the chunk index XORed with the key's low bits, so the 16 keys a 16-lane
// group reads at one head-dim offset fall in distinct banks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_common.h"
#include "kernels.h"

namespace pad {
namespace {

using namespace dev;

template <int D, int RT>
struct SplitShape {
  static constexpr int NW = 4;                  // waves; wave w owns head-dim quarter w
  static constexpr int kThreads = NW * 64;
  static constexpr int KC = D / 32;             // 32-wide head-dim chunks (QK^T MFMA steps)
  static constexpr int DQ = D / NW;             // head-dim columns per wave
  static constexpr int DTQ = DQ / 16;           // 16-wide output tiles per wave
  static constexpr int kKRow = 2 * D;           // bytes of one key's K row
  static constexpr int kKChunks = D / 8;        // 16-byte chunks of a K row
  static constexpr int kVRow = 2 * DQ;          // bytes of one key's V quarter
  static constexpr int kVChunks = DQ / 8;       // 16-byte chunks of a V quarter
  static constexpr int kKBytes = 16 * kKRow;    // K of one tile
  static constexpr int kVBytes = 16 * kVRow;    // one wave's V quarter of one tile
  static constexpr int KL = kKBytes / 16 / kThreads;  // K loads per thread per tile
  static constexpr int VL = kVBytes / 16 / 64;        // V loads per lane per tile
  // Tiles in flight (register stages): eight up to head size 256, four at
  // 512 with two row tiles, two where the query operand and a
  // four-row-tile accumulator at 512 leave no room.
  static constexpr int NS = D <= 256 ? 8 : (RT <= 2 ? 4 : 2);
  static constexpr int kKSwz = kKChunks < 16 ? kKChunks - 1 : 15;
  static constexpr int kVSwz = kVChunks < 16 ? kVChunks - 1 : 15;
  static_assert(KL >= 1 && KL * 16 * kThreads == kKBytes, "whole K chunks per thread");
  static_assert(VL >= 1 && VL * 16 * 64 == kVBytes, "whole V chunks per lane");
  static_assert(kKChunks >= 16, "the K swizzle spans 16 chunks");
  // LDS: K double buffer, per-wave V double buffers, P and rescale double
  // buffers, the final (m, l) of each row, the segment's block ids; then
  // the persistent grid's tables and 16 bytes of flags.
  static constexpr int kKOff = 0;
  static constexpr int kVOff = kKOff + 2 * kKBytes;
  static constexpr int kPOff = kVOff + NW * 2 * kVBytes;
  static constexpr int kPBytes = RT * 64 * 8;           // P of every row tile, one tile of keys
  static constexpr int kAOff = kPOff + 2 * kPBytes;
  static constexpr int kABytes = RT * 16 * 4;           // rescale factor per row
  static constexpr int kMLOff = kAOff + 2 * kABytes;
  static constexpr int kIdsOff = kMLOff + RT * 16 * 8;
  static constexpr int kPersistOff = kIdsOff + kMaxSegTiles * 4;
  static constexpr int kBytes = kPersistOff + (2 * kPersistMaxSeqs + 1) * 4 + 16;
  static_assert(kIdsOff >= 2 * kPersistMaxSeqs * 4, "persistent prologue scratch fits the tile area");
};

// One work item: segment `seg` of (sequence s, kv head kvh, row group rg).
template <typename T, int D, int RT>
__device__ __forceinline__ void split_unit(const Params& p, unsigned char* lds, int s, int kvh, int rg, int seg) {
  using MF = Mfma<T>;
  using SH = SplitShape<D, RT>;
  constexpr int KC = SH::KC, DTQ = SH::DTQ, NT = SH::kThreads, NS = SH::NS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int row0 = rg * RT * 16;
  const int wg_rows = min(RT * 16, p.rows - row0);
  const int M = p.query_len;

  const int L = clamped_len(p, s);
  if (L <= 0) {
    if (seg == 0) zero_rows<T, D>(p, s, kvh, row0, wg_rows, NT);
    return;
  }
  const int k_lo = p.window > 0 ? max(0, L - M - p.window + 1) : 0;
  const SegSplit sp = split_of(p, L);
  const int n_live = sp.n_live;
  if (seg >= n_live) return;
  const int ts = sp.t_lo + seg * sp.seg_tiles, te = min(ts + sp.seg_tiles, sp.t_hi);
  const int n_t = te - ts;
  const int lo_last = p.window > 0 ? max(0, L - p.window) : 0;
  const int qpos_first = L - M;

  // QK^T rows of this wave: row tile `wave` (if the workgroup has it and
  // it holds a live row); lane row c.
  const bool qk_wave = wave < RT && row0 + wave * 16 < p.rows;
  const int ru = row0 + wave * 16 + c;
  int qpos = -1, lo = 0;
  i32x4 qop[KC];
  {
    const T* Q = static_cast<const T*>(p.q);
    if (qk_wave && ru < p.rows) {
      const int m = ru / p.group, gq = ru % p.group;
      qpos = L - M + m;
      lo = p.window > 0 ? max(0, qpos - p.window + 1) : 0;
      const T* qrow = Q + ((int64_t(s) * M + m) * p.num_q_heads + kvh * p.group + gq) * D;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) qop[kc] = *reinterpret_cast<const i32x4*>(qrow + 32 * kc + 8 * g);
    } else {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) qop[kc] = i32x4{0, 0, 0, 0};
    }
  }

  // The segment's block ids (one per tile) in LDS.
  const int32_t* table = p.block_table + int64_t(s) * p.max_blocks;
  int* sm_ids = reinterpret_cast<int*>(lds + SH::kIdsOff);
  for (int t = tid; t < n_t; t += NT) sm_ids[t] = table[((ts + t) * 16) / p.page_size];
  __syncthreads();

  const unsigned char* KVh =
      static_cast<const unsigned char*>(p.kv) + int64_t(kvh) * p.head_stride * int64_t(sizeof(T));
  const uint32_t tok_bytes = uint32_t(p.token_stride) * uint32_t(sizeof(T));
  // K chunk u of thread tid: q = u * NT + tid -> key q / kKChunks, chunk
  // q % kKChunks of its K row.  V chunk u of this lane: q = u * 64 + lane
  // -> key q / kVChunks, chunk q % kVChunks of its V quarter.
  auto k_key = [&](int u) { return (u * NT + tid) / SH::kKChunks; };
  auto k_x = [&](int u) { return (u * NT + tid) % SH::kKChunks; };
  auto v_key = [&](int u) { return (u * 64 + lane) / SH::kVChunks; };
  auto v_x = [&](int u) { return (u * 64 + lane) % SH::kVChunks; };
  const uint32_t v_col_bytes = uint32_t(2 * D + wave * 2 * SH::DQ);  // V half, then this wave's quarter

  struct Stage {
    i32x4 k[SH::KL];
    i32x4 v[SH::VL];
  };
  auto tile_of = [&](int i) { return ts + min(i, n_t - 1); };
  auto issue = [&](Stage& st, int i) {
    const int t = tile_of(i);
    const int blk = __builtin_amdgcn_readfirstlane(sm_ids[t - ts]);
    const unsigned char* base = KVh + (int64_t(blk) * p.block_stride +
                                       int64_t((t * 16) % p.page_size) * p.token_stride) * int64_t(sizeof(T));
#pragma unroll
    for (int u = 0; u < SH::KL; ++u)
      st.k[u] = *reinterpret_cast<const i32x4*>(base + (uint32_t(k_key(u)) * tok_bytes + uint32_t(k_x(u)) * 16u));
#pragma unroll
    for (int u = 0; u < SH::VL; ++u)
      st.v[u] = *reinterpret_cast<const i32x4*>(
          base + (uint32_t(v_key(u)) * tok_bytes + v_col_bytes + uint32_t(v_x(u)) * 16u));
  };
  // Copy a staged tile to LDS buffer `buf`.  V rows of keys outside
  // [k_lo, L) become zero: they may hold anything, even NaN, and would
  // otherwise reach PV as 0 * NaN.
  auto put = [&](const Stage& st, int i, int buf) {
    const int key0 = tile_of(i) * 16;
    unsigned char* kd = lds + SH::kKOff + buf * SH::kKBytes;
    unsigned char* vd = lds + SH::kVOff + (wave * 2 + buf) * SH::kVBytes;
#pragma unroll
    for (int u = 0; u < SH::KL; ++u) {
      const int key = k_key(u);
      *reinterpret_cast<i32x4*>(kd + key * SH::kKRow + ((k_x(u) ^ (key & SH::kKSwz)) * 16)) = st.k[u];
    }
#pragma unroll
    for (int u = 0; u < SH::VL; ++u) {
      const int key = v_key(u);
      const int kabs = key0 + key;
      const i32x4 v = (kabs < k_lo || kabs >= L) ? i32x4{0, 0, 0, 0} : st.v[u];
      *reinterpret_cast<i32x4*>(vd + key * SH::kVRow + ((v_x(u) ^ (key & SH::kVSwz)) * 16)) = v;
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[RT][DTQ];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int dt = 0; dt < DTQ; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Scores of tile i for this wave's row tile: P and the rows' rescale
  // factor go to LDS buffer `buf`.
  auto scores = [&](int i, int buf) {
    uint64_t* pdst = reinterpret_cast<uint64_t*>(lds + SH::kPOff + buf * SH::kPBytes) + wave * 64 + lane;
    float* adst = reinterpret_cast<float*>(lds + SH::kAOff + buf * SH::kABytes) + wave * 16 + c;
    if (!qk_wave) {
      if (wave < RT) {  // a row tile with no live row: no weight, no rescale of zeros
        *pdst = 0;
        if (g == 0) *adst = 0.f;
      }
      return;
    }
    const unsigned char* kb = lds + SH::kKOff + buf * SH::kKBytes;
    const int key0 = tile_of(i) * 16;
    // S^T = K Q^T: lane (g, c) holds K[key c][32 kc + 8 g .. + 8].
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const i32x4 k = *reinterpret_cast<const i32x4*>(kb + c * SH::kKRow + (((4 * kc + g) ^ (c & SH::kKSwz)) * 16));
      sc = MF::qk(k, qop[kc], sc);
    }
    const bool edge = !(key0 >= lo_last && key0 + 15 <= qpos_first);
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = sc[j] * p.scale_log2;
      if (edge) {
        const int key = key0 + 4 * g + j;
        if (key < lo || key > qpos) x[j] = kNegInf;
      }
    }
    float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float pj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pj[j] = fast_exp2(x[j] - m_use);
    l_run = l_run * alpha + ((pj[0] + pj[1]) + (pj[2] + pj[3]));
    m_run = m_new;
    *pdst = pack4(MF::bits(pj[0]), MF::bits(pj[1]), MF::bits(pj[2]), MF::bits(pj[3]));
    if (g == 0) *adst = alpha;
  };

  // O^T += V^T P^T over this wave's head-dim quarter, for every row tile.
  // The transposed V read of lane (g, c) addresses key 4 g + c / 4,
  // columns 16 dt + 4 (c % 4) .. + 3 of the quarter.
  const int vkey = 4 * g + (c >> 2);
  auto pv = [&](int buf) {
    const uint64_t* psrc = reinterpret_cast<const uint64_t*>(lds + SH::kPOff + buf * SH::kPBytes) + lane;
    const float* asrc = reinterpret_cast<const float*>(lds + SH::kAOff + buf * SH::kABytes) + c;
    uint64_t pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      pb[rt] = psrc[rt * 64];
      const float a = asrc[rt * 16];
#pragma unroll
      for (int dt = 0; dt < DTQ; ++dt) acc[rt][dt] *= a;
    }
    const unsigned char* vrow =
        lds + SH::kVOff + (wave * 2 + buf) * SH::kVBytes + vkey * SH::kVRow + (c & 1) * 8;
#pragma unroll
    for (int dt = 0; dt < DTQ; ++dt) {
      const int x8 = 2 * dt + ((c & 3) >> 1);
      const uint64_t va = __builtin_bit_cast(
          uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(vrow + ((x8 ^ (vkey & SH::kVSwz)) * 16))));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][dt] = MF::pv(va, pb[rt], acc[rt][dt]);
    }
  };

  // Tile i's loads go out NS iterations ahead into stage i % NS; one
  // iteration ahead the stage is copied to LDS buffer (i + 1) % 2.  The
  // barrier of iteration i orders: this iteration's copies and scores
  // before the next iteration's scores and before the PV of this one; the
  // previous iteration's PV before this iteration's copies.
  Stage stage[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) issue(stage[u], u);
  put(stage[0], 0, 0);
  issue(stage[0], NS);
  __syncthreads();
  for (int i = 0;; i += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int it = i + u;
      put(stage[(u + 1) % NS], it + 1, (u + 1) & 1);
      issue(stage[(u + 1) % NS], it + 1 + NS);
      scores(it, u & 1);
      __syncthreads();
      pv(u & 1);
      if (it + 1 >= n_t) goto tiles_done;
    }
  }
tiles_done:

  // Row sums of the QK^T waves over the four lane groups that split a
  // tile's keys; (m, l) of every row to LDS for the output or the partial.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float* sm_ml = reinterpret_cast<float*>(lds + SH::kMLOff);
  if (wave < RT && g == 0) {
    sm_ml[(wave * 16 + c) * 2] = m_run;
    sm_ml[(wave * 16 + c) * 2 + 1] = l_run;
  }
  __syncthreads();

  // This wave's columns of row (rt, c): O^T[16 dt + 4 g + j][c].
  const int col0 = wave * SH::DQ + 4 * g;
  T* out_s = static_cast<T*>(p.out) + int64_t(s) * M * p.num_q_heads * D;
  if (n_live == 1) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = rt * 16 + c;
      if (r >= wg_rows) continue;
      const float l = sm_ml[r * 2 + 1];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      T* orow = out_row(p, out_s, kvh, row0 + r, D);
#pragma unroll
      for (int dt = 0; dt < DTQ; ++dt) {
        uint2 o;
        o.x = uint32_t(MF::bits(acc[rt][dt][0] * inv)) | (uint32_t(MF::bits(acc[rt][dt][1] * inv)) << 16);
        o.y = uint32_t(MF::bits(acc[rt][dt][2] * inv)) | (uint32_t(MF::bits(acc[rt][dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + col0 + 16 * dt) = o;
      }
    }
    return;
  }
  // Publish this wave's columns of the partial (device-coherent stores).
  const int64_t slot_row0 = ((int64_t(s) * p.num_kv_heads + kvh) * p.nseg + seg) * p.rows + row0;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + c;
    if (r >= wg_rows) continue;
#pragma unroll
    for (int dt = 0; dt < DTQ; ++dt) store_coherent(p.ws_acc + (slot_row0 + r) * D + col0 + 16 * dt, acc[rt][dt]);
  }
  for (int r = tid; r < wg_rows; r += NT) store_coherent2(p.ws_ml + (slot_row0 + r) * 2, sm_ml[r * 2], sm_ml[r * 2 + 1]);
  arrive_and_merge<T, D, NT>(p, reinterpret_cast<int*>(lds + SH::kBytes - 16), s, kvh, rg, row0, wg_rows, n_live);
}

// PERSIST selects the grid: one workgroup per item, or the persistent grid.
// One wave per SIMD: the compiler schedules for latency hiding within a
// wave instead of for occupancy.
template <typename T, int D, int RT, bool PERSIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_split_kernel(Params p) {
  using SH = SplitShape<D, RT>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[SH::kBytes];
  if constexpr (!PERSIST) {
    const int units = p.num_kv_heads * p.row_groups;
    const int unit = blockIdx.x % units;
    split_unit<T, D, RT>(p, lds, blockIdx.y, unit % p.num_kv_heads, unit / p.num_kv_heads, blockIdx.x / units);
  } else {
    persistent_loop(p, lds, SH::kPersistOff, SH::kBytes, SH::kThreads,
                    [&](int s, int kvh, int rg, int seg) { split_unit<T, D, RT>(p, lds, s, kvh, rg, seg); });
  }
}

template <typename T, int D, int RT>
int launch_r(const Plan& pl, const Params& pr, hipStream_t st) {
  if (pl.persistent)
    hipLaunchKernelGGL((decode_split_kernel<T, D, RT, true>), dim3(pl.grid_x, pl.grid_y), dim3(256), 0, st, pr);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, RT, false>), dim3(pl.grid_x, pl.grid_y), dim3(256), 0, st, pr);
  return int(hipGetLastError());
}

template <typename T, int D>
int launch_d(const Plan& pl, const Params& pr, hipStream_t st) {
  switch (pl.row_tiles) {
    case 2: return launch_r<T, D, 2>(pl, pr, st);
    case 4: return launch_r<T, D, 4>(pl, pr, st);
  }
  return int(hipErrorInvalidValue);
}

template <typename T>
int launch_t(const Plan& pl, const Params& pr, int head_size, hipStream_t st) {
  switch (head_size) {
    case 128: return launch_d<T, 128>(pl, pr, st);
    case 256: return launch_d<T, 256>(pl, pr, st);
    case 512: return launch_d<T, 512>(pl, pr, st);
  }
  return int(hipErrorInvalidValue);
}

}  // namespace

int launch_split(const Plan& plan, const Params& params, int dtype, int head_size, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == PAD_BF16) return launch_t<__bf16>(plan, params, head_size, st);
  return launch_t<_Float16>(plan, params, head_size, st);
}

}  // namespace pad
