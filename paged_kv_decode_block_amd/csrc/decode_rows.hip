// Paged-KV decode attention for kv heads with many query rows (gfx950).
//
// When the G*M query rows of a kv head take two or more 16-row MFMA tiles
// (wide heads, speculative verify), each wave of a workgroup owns one row
// tile and the workgroup shares every 16-key K/V tile through LDS: the tile
// is read from HBM once, by all waves together, and every wave runs QK^T,
// the online softmax and PV for its own rows on it.  Each wave thus sees
// the whole segment for its rows, so no cross-wave combine is needed at the
// end -- a wave publishes its rows' partial (or output) straight from
// registers.  The split-KV arrival, the sliced merge and the persistent
// grid are those of the key-split kernel (ROCm/vllm pull request 1330,
// "Summary": one read of a kv head's pages for all of its query rows).
//
// Tile staging: a 16-key tile of K and V (16 * 4 * D bytes, contiguous per
// token slot) is loaded with 16-byte loads, thread t taking chunks t,
// t + threads, ... so each load instruction reads consecutive bytes; the
// registers of the next two tiles are in flight while the current one is
// computed.  In LDS each K (and V) row is kept in 16-byte chunks whose
// index is XORed with the key's low four bits, so the sixteen keys a
// 16-lane group reads at one head-dim offset (the A operand of the QK^T
// MFMA, or four keys of the transposed V read) fall in distinct banks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_common.h"
#include "kernels.h"

namespace pad {
namespace {

using namespace dev;

template <int D, int NWR>
struct RowsShape {
  static constexpr int NW = NWR;  // waves = row tiles per workgroup
  static constexpr int kThreads = NW * 64;
  static constexpr int KC = D / 32;            // 32-wide head-dim chunks (QK^T MFMA steps)
  static constexpr int DT = D / 16;            // 16-wide head-dim tiles of the output
  static constexpr int kRowChunks = D / 8;     // 16-byte chunks of one K (or V) row
  static constexpr int kRowBytes = D * 2;      // bytes of one K (or V) row
  static constexpr int kHalfBytes = 16 * kRowBytes;   // K (or V) rows of one tile
  static constexpr int kTileBytes = 2 * kHalfBytes;   // K and V of 16 keys
  static constexpr int kLoads = kTileBytes / 16 / kThreads;  // 16-byte loads per thread per tile
  static_assert(kLoads >= 1 && kLoads * 16 * kThreads == kTileBytes, "whole 16-byte chunks per thread");
  static_assert(kRowChunks >= 16, "the XOR swizzle spans 16 chunks");
  // LDS: two tile buffers and the segment's block ids; the persistent
  // grid's tables after them; 16 bytes of flags at the end.
  static constexpr int kIdsOff = 2 * kTileBytes;
  static constexpr int kPersistOff = kIdsOff + kMaxSegTiles * 4;
  static constexpr int kBytes = kPersistOff + (2 * kPersistMaxSeqs + 1) * 4 + 16;
  static_assert(kPersistOff >= 2 * kPersistMaxSeqs * 4, "persistent prologue scratch fits the tile area");
};

// One work item: segment `seg` of (sequence s, kv head kvh, row group rg).
template <typename T, int D, int NWR>
__device__ __forceinline__ void rows_unit(const Params& p, unsigned char* lds, int s, int kvh, int rg, int seg) {
  using MF = Mfma<T>;
  using SH = RowsShape<D, NWR>;
  constexpr int KC = SH::KC, DT = SH::DT, NT = SH::kThreads;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int row0 = rg * NWR * 16;                 // first row of the workgroup
  const int wg_rows = min(NWR * 16, p.rows - row0);
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

  // This wave's rows: lane row c of row tile `wave`.
  const int ru = row0 + wave * 16 + c;
  const bool row_ok = ru < p.rows;
  int qpos = -1, lo = 0;
  i32x4 qop[KC];
  {
    const T* Q = static_cast<const T*>(p.q);
    if (row_ok) {
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
  // Thread t's chunks of a tile: q = u * NT + t -> token q / (D / 4) of the
  // tile, chunk y = q % (D / 4) of the token's K|V slot (powers of two:
  // recomputed where used rather than held in registers).
  const uint32_t tok_bytes = uint32_t(p.token_stride) * uint32_t(sizeof(T));
  auto chunk_tok = [&](int u) { return (u * NT + tid) / (D / 4); };
  auto chunk_y = [&](int u) { return (u * NT + tid) % (D / 4); };

  struct Stage {
    i32x4 v[SH::kLoads];
  };
  auto tile_of = [&](int i) { return ts + min(i, n_t - 1); };
  auto issue = [&](Stage& st, int i) {
    const int t = tile_of(i);
    const int blk = __builtin_amdgcn_readfirstlane(sm_ids[t - ts]);
    const unsigned char* base = KVh + (int64_t(blk) * p.block_stride +
                                       int64_t((t * 16) % p.page_size) * p.token_stride) * int64_t(sizeof(T));
#pragma unroll
    for (int u = 0; u < SH::kLoads; ++u)
      st.v[u] = *reinterpret_cast<const i32x4*>(base + (uint32_t(chunk_tok(u)) * tok_bytes + uint32_t(chunk_y(u)) * 16u));
  };
  // Copy a staged tile to LDS buffer `buf`; V rows of keys outside
  // [k_lo, L) become zero (they may hold anything, even NaN, and would
  // otherwise reach PV as 0 * NaN).
  auto put = [&](Stage& st, int i, int buf) {
    const int key0 = tile_of(i) * 16;
    unsigned char* dst = lds + buf * SH::kTileBytes;
#pragma unroll
    for (int u = 0; u < SH::kLoads; ++u) {
      const int tok = chunk_tok(u), y = chunk_y(u);
      const int part = y / SH::kRowChunks, x = y % SH::kRowChunks;
      const int key = key0 + tok;
      i32x4 v = st.v[u];
      if (part == 1 && (key < k_lo || key >= L)) v = i32x4{0, 0, 0, 0};
      *reinterpret_cast<i32x4*>(dst + part * SH::kHalfBytes + tok * SH::kRowBytes + ((x ^ (tok & 15)) * 16)) = v;
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A wave whose row tile lies past the kv head's rows only loads.
  const bool wave_live = row0 + wave * 16 < p.rows;
  auto compute = [&](int i, int buf) {
    if (!wave_live) return;
    const unsigned char* kb = lds + buf * SH::kTileBytes;
    const unsigned char* vb = kb + SH::kHalfBytes;
    const int key0 = tile_of(i) * 16;
    // S^T = K Q^T: lane (g, c) holds K[key c][32 kc + 8 g .. + 8].
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const i32x4 k = *reinterpret_cast<const i32x4*>(kb + c * SH::kRowBytes + (((4 * kc + g) ^ c) * 16));
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
    const uint64_t pb = pack4(MF::bits(pj[0]), MF::bits(pj[1]), MF::bits(pj[2]), MF::bits(pj[3]));
    // O^T += V^T P^T: lane (g, c) addresses key 4 g + c / 4, head-dim
    // columns 16 dt + 4 (c % 4) .. + 3 (8 bytes of a 16-byte chunk).
    const int vkey = 4 * g + (c >> 2);
    const unsigned char* vrow = vb + vkey * SH::kRowBytes + (c & 1) * 8;
    const int vsw = vkey & 15;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt] *= alpha;
      const int x8 = 2 * dt + ((c & 3) >> 1);
      const uint64_t va = __builtin_bit_cast(
          uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(vrow + ((x8 ^ vsw) * 16))));
      acc[dt] = MF::pv(va, pb, acc[dt]);
    }
  };

  // Two tiles in flight: stage r[t % 2] holds tile t until it is copied to
  // LDS buffer t % 2 one iteration before it is computed.
  Stage r0, r1;
  issue(r0, 0);
  issue(r1, 1);
  put(r0, 0, 0);
  issue(r0, 2);
  __syncthreads();
  for (int i = 0; i < n_t; ++i) {
    compute(i, i & 1);
    if (i & 1) {
      put(r0, i + 1, 0);
      issue(r0, i + 3);
    } else {
      put(r1, i + 1, 1);
      issue(r1, i + 3);
    }
    __syncthreads();
  }

  // Row sum over the four lane groups that split a tile's keys.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  T* out_s = static_cast<T*>(p.out) + int64_t(s) * M * p.num_q_heads * D;
  if (n_live == 1) {
    if (row_ok) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      T* orow = out_row(p, out_s, kvh, ru, D);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint2 o;
        o.x = uint32_t(MF::bits(acc[dt][0] * inv)) | (uint32_t(MF::bits(acc[dt][1] * inv)) << 16);
        o.y = uint32_t(MF::bits(acc[dt][2] * inv)) | (uint32_t(MF::bits(acc[dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = o;
      }
    }
    return;
  }
  // Publish this wave's rows of the partial (device-coherent stores).
  if (row_ok) {
    const int64_t slot = ((int64_t(s) * p.num_kv_heads + kvh) * p.nseg + seg) * p.rows + ru;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) store_coherent(p.ws_acc + slot * D + 16 * dt + 4 * g, acc[dt]);
    if (g == 0) store_coherent2(p.ws_ml + slot * 2, m_run, l_run);
  }
  arrive_and_merge<T, D, NT>(p, reinterpret_cast<int*>(lds + SH::kBytes - 16), s, kvh, rg, row0, wg_rows, n_live);
}

// PERSIST selects the grid: one workgroup per item, or the persistent grid.
// Waves per SIMD the compiler may assume: one for 2- and 4-wave workgroups
// (a CU holds one or two of them), two for 8-wave workgroups; it then
// schedules for latency hiding within a wave instead of for occupancy.
template <typename T, int D, int NWR, bool PERSIST>
__global__ __launch_bounds__(NWR * 64) __attribute__((amdgpu_waves_per_eu(NWR <= 4 ? 1 : 2, NWR <= 4 ? 1 : 2)))
void decode_rows_kernel(Params p) {
  using SH = RowsShape<D, NWR>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[SH::kBytes];
  if constexpr (!PERSIST) {
    const int units = p.num_kv_heads * p.row_groups;
    const int unit = blockIdx.x % units;
    rows_unit<T, D, NWR>(p, lds, blockIdx.y, unit % p.num_kv_heads, unit / p.num_kv_heads, blockIdx.x / units);
  } else {
    persistent_loop(p, lds, SH::kPersistOff, SH::kBytes, SH::kThreads,
                    [&](int s, int kvh, int rg, int seg) { rows_unit<T, D, NWR>(p, lds, s, kvh, rg, seg); });
  }
}

template <typename T, int D, int NWR>
int launch_w(const Plan& pl, const Params& pr, hipStream_t st) {
  if (pl.persistent)
    hipLaunchKernelGGL((decode_rows_kernel<T, D, NWR, true>), dim3(pl.grid_x, pl.grid_y), dim3(NWR * 64), 0, st, pr);
  else
    hipLaunchKernelGGL((decode_rows_kernel<T, D, NWR, false>), dim3(pl.grid_x, pl.grid_y), dim3(NWR * 64), 0, st, pr);
  return int(hipGetLastError());
}

template <typename T, int D>
int launch_r(const Plan& pl, const Params& pr, hipStream_t st) {
  switch (pl.waves) {
    case 2: if constexpr (D < 512) return launch_w<T, D, 2>(pl, pr, st); break;
    case 4: return launch_w<T, D, 4>(pl, pr, st);
    case 8: if constexpr (D == 128) return launch_w<T, D, 8>(pl, pr, st); break;
  }
  return int(hipErrorInvalidValue);
}

template <typename T>
int launch_rt(const Plan& pl, const Params& pr, int head_size, hipStream_t st) {
  switch (head_size) {
    case 128: return launch_r<T, 128>(pl, pr, st);
    case 256: return launch_r<T, 256>(pl, pr, st);
    case 512: return launch_r<T, 512>(pl, pr, st);
  }
  return int(hipErrorInvalidValue);
}

}  // namespace

int launch_rows(const Plan& plan, const Params& params, int dtype, int head_size, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == PAD_BF16) return launch_rt<__bf16>(plan, params, head_size, st);
  return launch_rt<_Float16>(plan, params, head_size, st);
}

}  // namespace pad
