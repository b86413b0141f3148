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

#include "kernels.h"

namespace pad {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  typedef short x4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4 qk(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(x8, a), __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(uint64_t a, uint64_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(x4, a), __builtin_bit_cast(x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t bits(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }
};

template <>
struct Mfma<_Float16> {
  typedef _Float16 x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 x4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4 qk(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(x8, a), __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(uint64_t a, uint64_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(x4, a), __builtin_bit_cast(x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t bits(float x) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x)); }
};

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint64_t pack4(uint16_t a, uint16_t b, uint16_t c, uint16_t d) {
  return uint64_t(a) | (uint64_t(b) << 16) | (uint64_t(c) << 32) | (uint64_t(d) << 48);
}

// Device-coherent store of 16 bytes (two 8-byte write-through stores).
__device__ __forceinline__ void store_coherent(float* dst, f32x4 v) {
  uint64_t* d = reinterpret_cast<uint64_t*>(dst);
  __hip_atomic_store(d, __builtin_bit_cast(uint64_t, __builtin_shufflevector(v, v, 0, 1)), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, __builtin_bit_cast(uint64_t, __builtin_shufflevector(v, v, 2, 3)), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent2(float* dst, float a, float b) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(dst),
                     uint64_t(__builtin_bit_cast(uint32_t, a)) | (uint64_t(__builtin_bit_cast(uint32_t, b)) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS layout of the wave combine: per wave its running max and sum per row
// and its rescaled accumulator rows, plus the workgroup's merged max/sum.
template <int D, int RT, int NW>
struct Combine {
  static constexpr int kRows = RT * 16;
  static constexpr int kAccStride = D + 4;
  static constexpr int kBytes = (2 * NW * kRows + 2 * kRows) * 4 + NW * kRows * kAccStride * 4;
  static __device__ float* m(unsigned char* lds) { return reinterpret_cast<float*>(lds); }
  static __device__ float* l(unsigned char* lds) { return m(lds) + NW * kRows; }
  static __device__ float* ms(unsigned char* lds) { return l(lds) + NW * kRows; }
  static __device__ float* ls(unsigned char* lds) { return ms(lds) + kRows; }
  static __device__ float* acc(unsigned char* lds) { return ls(lds) + kRows; }
};

// Workgroup shape (waves per workgroup from waves_for) and LDS layout.
template <int D, int RT>
struct Shape {
  static constexpr int NW = waves_for(D, RT);
  static constexpr int kThreads = NW * 64;
  static constexpr int KC = D / 32;  // 32-wide head-dim chunks (QK^T MFMA steps)
  static constexpr int DT = D / 16;  // 16-wide head-dim tiles of the output
  static constexpr int kVStride = D + 8;    // elements per staged V row (16-byte padded)
  static constexpr int kAccStride = D + 4;  // floats per accumulator row in LDS
  static constexpr int kRows = RT * 16;
  // Tiles in flight beyond the one being computed: one while the register
  // budget allows it (a second one measured slower).
  static constexpr int PF = D * RT <= 512 && D < 512 ? 1 : 0;
  // LDS: V staging and the segment's block ids during the tile loop,
  // afterwards the wave-combine area; then the persistent grid's tables.
  // The last 16 bytes hold the merge role, hand-over and queue words.
  static constexpr int kVBytes = NW * 16 * kVStride * 2;
  // The segment's block ids, one per tile, follow the V staging area.
  static constexpr int kIdsBytes = kMaxSegTiles * 4;
  static constexpr int kLoopBytes = kVBytes + kIdsBytes;
  static constexpr int kCombineBytes = Combine<D, RT, NW>::kBytes;
  // Then the persistent grid's rank order and item prefix.
  static constexpr int kPersistOff = kLoopBytes > kCombineBytes ? kLoopBytes : kCombineBytes;
  static constexpr int kBytes = kPersistOff + (2 * kPersistMaxSeqs + 1) * 4 + 16;
  static_assert(kLoopBytes >= 2 * kPersistMaxSeqs * 4, "persistent prologue scratch fits the tile-loop area");
};

template <typename T>
__device__ __forceinline__ T* out_row(const Params& p, T* out_s, int kvh, int ru, int D) {
  const int m = ru / p.group, gq = ru % p.group;
  return out_s + (int64_t(m) * p.num_q_heads + kvh * p.group + gq) * D;
}

// ---- split-KV merge ----
// The merged output of a unit is rows x D floats, cut into items (row r,
// four head-dim columns d4): item = r * (D / 4) + d4.  Merge slice `slice`
// of `nslices` covers items [slice * I / nslices, (slice + 1) * I / nslices).
// LN lanes serve one item; lane `sub` takes slots sub, sub + LN, ... in
// chunks of LN * U slots (U per lane), keeping a running (m, l, acc) in the
// exp2 domain:  m* = max m_j,  l* = sum l_j 2^(m_j - m*),
// acc* = sum acc_j 2^(m_j - m*)  (the log-sum-exp merge of split
// partials); the LN lanes then combine in a fixed butterfly.  Each item's
// sums follow one fixed order for a given (slot count, LN, U), whichever
// workgroup merges it.  Every load is unconditional (item and slot indices
// clamped, extra slots weighted zero) so the wait counts stay exact, and
// the (pass, chunk) work of a thread is one stream with the next unit's
// loads in flight while the current one is consumed.
template <int U>
struct MergeChunk {
  f32x4 acc[U];
  float2 ml[U];
};

template <int D, int NT, int LN, int U>
__device__ __forceinline__ void merge_load(const Params& p, MergeChunk<U>& b, int64_t slot0, int row0, int i0, int i1,
                                           int n, int nch, int w) {
  constexpr int IPP = NT / LN, CH = LN * U;
  const int pass = w / nch, ch = w - pass * nch;
  const int it = min(i0 + pass * IPP + int(threadIdx.x) / LN, i1 - 1);
  const int r = it / (D / 4), d4 = it % (D / 4);
  const float* acc0 = p.ws_acc + (slot0 * p.rows + row0 + r) * D + 4 * d4;
  const float* ml0 = p.ws_ml + (slot0 * p.rows + row0 + r) * 2;
  const int first = ch * CH + int(threadIdx.x) % LN;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = min(first + LN * u, n - 1);
    b.acc[u] = *reinterpret_cast<const f32x4*>(acc0 + int64_t(j) * p.rows * D);
    b.ml[u] = *reinterpret_cast<const float2*>(ml0 + int64_t(j) * p.rows * 2);
  }
}

template <typename T, int D, int NT, int LN, int U>
__device__ __forceinline__ void merge_consume(const Params& p, const MergeChunk<U>& b, int i0, int i1, int n, int nch,
                                              int w, int row0, T* out_s, int kvh, float& m_run, float& l_run,
                                              f32x4& a_run) {
  using MF = Mfma<T>;
  constexpr int IPP = NT / LN, CH = LN * U;
  const int pass = w / nch, ch = w - pass * nch;
  const int sub = int(threadIdx.x) % LN;
  if (ch == 0) {
    m_run = kNegInf;
    l_run = 0.f;
    a_run = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int first = ch * CH + sub;
  float mj[U];
  float mloc = kNegInf;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    mj[u] = first + LN * u < n ? b.ml[u].x : kNegInf;
    mloc = fmaxf(mloc, mj[u]);
  }
  const float m_new = fmaxf(m_run, mloc);
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  const float sc = fast_exp2(m_run - m_use);
  l_run *= sc;
  a_run *= sc;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float wgt = fast_exp2(mj[u] - m_use);
    l_run += wgt * b.ml[u].y;
    a_run += wgt * b.acc[u];
  }
  m_run = m_new;
  if (ch != nch - 1) return;
  // Last chunk of the pass: combine the item's lanes and write it.
  float m_all = m_run;
#pragma unroll
  for (int o = 1; o < LN; o <<= 1) m_all = fmaxf(m_all, __shfl_xor(m_all, o));
  const float f = fast_exp2(m_run - (m_all == kNegInf ? 0.f : m_all));
  float l = l_run * f;
  f32x4 a = a_run * f;
#pragma unroll
  for (int o = 1; o < LN; o <<= 1) {
    l += __shfl_xor(l, o);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += __shfl_xor(a[e], o);
  }
  const int it = i0 + pass * IPP + int(threadIdx.x) / LN;
  if (sub == 0 && it < i1) {
    const int r = it / (D / 4), d4 = it % (D / 4);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint2 o;
    o.x = uint32_t(MF::bits(a[0] * inv)) | (uint32_t(MF::bits(a[1] * inv)) << 16);
    o.y = uint32_t(MF::bits(a[2] * inv)) | (uint32_t(MF::bits(a[3] * inv)) << 16);
    *reinterpret_cast<uint2*>(out_row(p, out_s, kvh, row0 + r, D) + 4 * d4) = o;
  }
}

template <typename T, int D, int NT, int LN, int U>
__device__ __forceinline__ void merge_items(const Params& p, int64_t slot0, int n, int row0, int i0, int i1, T* out_s,
                                         int kvh) {
  constexpr int IPP = NT / LN, CH = LN * U;
  const int nch = (n + CH - 1) / CH;
  const int W = (i1 - i0 + IPP - 1) / IPP * nch;
  float m_run = kNegInf, l_run = 0.f;
  f32x4 a_run = {0.f, 0.f, 0.f, 0.f};
  MergeChunk<U> b0, b1;
  merge_load<D, NT, LN, U>(p, b0, slot0, row0, i0, i1, n, nch, 0);
  if (W == 1) {
    merge_consume<T, D, NT, LN, U>(p, b0, i0, i1, n, nch, 0, row0, out_s, kvh, m_run, l_run, a_run);
    return;
  }
  for (int w = 0; w < W; w += 2) {
    merge_load<D, NT, LN, U>(p, b1, slot0, row0, i0, i1, n, nch, min(w + 1, W - 1));
    merge_consume<T, D, NT, LN, U>(p, b0, i0, i1, n, nch, w, row0, out_s, kvh, m_run, l_run, a_run);
    merge_load<D, NT, LN, U>(p, b0, slot0, row0, i0, i1, n, nch, min(w + 2, W - 1));
    if (w + 1 < W)
      merge_consume<T, D, NT, LN, U>(p, b1, i0, i1, n, nch, w + 1, row0, out_s, kvh, m_run, l_run, a_run);
  }
}

// Merge slice `slice` of `nslices` of the n partials of a unit (slots
// slot0 .. slot0 + n - 1, rows row0 .. row0 + wg_rows - 1 of each) into
// the output.  Lanes per item and slots per lane follow the slot count
// only, so an item's sums take the same order whatever the slicing and
// whichever workgroup merges it: the output bits depend on the sequence
// and the segment split alone.  The caller has acquired the partials.
template <typename T, int D, int NT>
__device__ __forceinline__ void merge_slice(const Params& p, int64_t slot0, int n, int row0, int wg_rows, int slice,
                                            int nslices, T* out_s, int kvh) {
  const int items = wg_rows * (D / 4);
  const int i0 = slice * items / nslices, i1 = (slice + 1) * items / nslices;
  if (i1 <= i0) return;
  const int ln = n >= 24 ? 4 : (n >= 8 ? 2 : 1);
  const int per = (n + ln - 1) / ln;
  const int u = per <= 2 ? 2 : (per <= 4 ? 4 : 8);
  switch (ln * 16 + u) {
    case 4 * 16 + 2: merge_items<T, D, NT, 4, 2>(p, slot0, n, row0, i0, i1, out_s, kvh); break;
    case 4 * 16 + 4: merge_items<T, D, NT, 4, 4>(p, slot0, n, row0, i0, i1, out_s, kvh); break;
    case 4 * 16 + 8: merge_items<T, D, NT, 4, 8>(p, slot0, n, row0, i0, i1, out_s, kvh); break;
    case 2 * 16 + 2: merge_items<T, D, NT, 2, 2>(p, slot0, n, row0, i0, i1, out_s, kvh); break;
    case 2 * 16 + 4: merge_items<T, D, NT, 2, 4>(p, slot0, n, row0, i0, i1, out_s, kvh); break;
    case 2 * 16 + 8: merge_items<T, D, NT, 2, 8>(p, slot0, n, row0, i0, i1, out_s, kvh); break;
    case 1 * 16 + 2: merge_items<T, D, NT, 1, 2>(p, slot0, n, row0, i0, i1, out_s, kvh); break;
    case 1 * 16 + 4: merge_items<T, D, NT, 1, 4>(p, slot0, n, row0, i0, i1, out_s, kvh); break;
    default: merge_items<T, D, NT, 1, 8>(p, slot0, n, row0, i0, i1, out_s, kvh); break;
  }
}

// Hand-over word of a merge slice (one per slice after the first).  The
// helper merging slice s (the s-th workgroup to arrive before the last)
// and the last arriver each act on it once or twice:
//   helper:  idle -> waiting, then waits (bounded) until the unit's arrival
//            count is complete or the word says go; then waiting -> done
//            (if the word already says go, the helper resets it to idle);
//            on timeout waiting -> gave_up, leaving the slice to the last
//            arriver (if go got there first, it merges after all).
//   last:    -> go; finding done or gave_up, it resets the word to idle (and
//            for gave_up merges the slice itself).
// Whoever acts second leaves the word idle, so every launch starts clean.
constexpr int kSliceIdle = 0, kSliceWaiting = 1, kSliceGo = 2, kSliceGaveUp = 3, kSliceDone = 4;
// Control words of a unit sit one cache line (128 bytes) apart: the
// helpers poll their own words while the last arriver updates them.
constexpr int kCtlStride = kCtlWordStride;

// A helper's side of the exchange (one thread): whether it merges its
// slice.  Every path ends: the wait is bounded by wait_ticks of the
// 100 MHz real-time counter.
__device__ __forceinline__ bool helper_wait(int* word, const int* counter, int n, uint32_t wait_ticks) {
  int seen = kSliceIdle;
  if (!__hip_atomic_compare_exchange_strong(word, &seen, kSliceWaiting, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)) {
    // The last arriver came first (go): this is the word's last use.
    __hip_atomic_store(word, kSliceIdle, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + wait_ticks;
  while (__builtin_amdgcn_s_memrealtime() < t_end) {
    if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n ||
        __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kSliceGo) {
      if (__hip_atomic_exchange(word, kSliceDone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kSliceGo)
        __hip_atomic_store(word, kSliceIdle, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return true;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  seen = kSliceWaiting;
  if (__hip_atomic_compare_exchange_strong(word, &seen, kSliceGaveUp, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT))
    return false;
  __hip_atomic_store(word, kSliceIdle, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // go came first
  return true;
}

// After the waves of a workgroup have left their results in LDS -- per
// wave w: sm_m/sm_l[w][row] (running max and sum) and the accumulator
// rows, already rescaled to the workgroup maximum, in slot w of sm_acc; and
// the workgroup's merged max/sum in sm_ms/sm_ls -- sum the slots in wave
// order (deterministic) and either write the output (single segment) or
// publish this segment's partial and count its arrival.  Of the n arrivals
// of a unit, the last one and the k - 1 before it (k = merge slices) merge
// one slice of the output each; the rest are done.
template <typename T, int D, int RT, int NW>
__device__ __forceinline__ void finish(const Params& p, unsigned char* lds, int s, int kvh, int rg, int seg, int row0,
                                       int wg_rows, int n_live, int lds_bytes) {
  using MF = Mfma<T>;
  using CB = Combine<D, RT, NW>;
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x;
  const float* sm_acc = CB::acc(lds);
  const float* sm_ms = CB::ms(lds);
  const float* sm_ls = CB::ls(lds);
  // Thread-distributed result: item (row r, 4 head-dim columns d4).
  auto combined = [&](int r, int d4) {
    const float* col = sm_acc + r * CB::kAccStride + 4 * d4;
    f32x4 a = *reinterpret_cast<const f32x4*>(col);
#pragma unroll
    for (int w = 1; w < NW; ++w) a += *reinterpret_cast<const f32x4*>(col + w * CB::kRows * CB::kAccStride);
    return a;
  };

  T* out_s = static_cast<T*>(p.out) + int64_t(s) * p.query_len * p.num_q_heads * D;
  if (n_live == 1) {
    for (int it = tid; it < wg_rows * (D / 4); it += NT) {
      const int r = it / (D / 4), d4 = it % (D / 4);
      const f32x4 a = combined(r, d4);
      const float ls = sm_ls[r];
      const float inv = ls > 0.f ? 1.f / ls : 0.f;
      uint2 o;
      o.x = uint32_t(MF::bits(a[0] * inv)) | (uint32_t(MF::bits(a[1] * inv)) << 16);
      o.y = uint32_t(MF::bits(a[2] * inv)) | (uint32_t(MF::bits(a[3] * inv)) << 16);
      *reinterpret_cast<uint2*>(out_row(p, out_s, kvh, row0 + r, D) + 4 * d4) = o;
    }
    return;
  }

  // Publish the partial with device-coherent stores.
  const int64_t slot0 = (int64_t(s) * p.num_kv_heads + kvh) * p.nseg;
  {
    const int64_t base = (slot0 + seg) * p.rows + row0;
    for (int it = tid; it < wg_rows * (D / 4); it += NT) {
      const int r = it / (D / 4), d4 = it % (D / 4);
      store_coherent(p.ws_acc + (base + r) * D + 4 * d4, combined(r, d4));
    }
    for (int r = tid; r < wg_rows; r += NT) store_coherent2(p.ws_ml + (base + r) * 2, sm_ms[r], sm_ls[r]);
  }
  int* ctl = p.ws_cnt + ((int64_t(s) * p.num_kv_heads + kvh) * p.row_groups + rg) * p.merge_slices * kCtlStride;
  int* sm_flag = reinterpret_cast<int*>(lds + lds_bytes - 16);
  const int k = min(p.merge_slices, n_live);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  __syncthreads();
  if (tid == 0) {
    // Role: 0 = last arriver, 1 .. k-1 = helper merging that slice, -1 = done.
    const int rank = __hip_atomic_fetch_add(ctl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int role = -1;
    if (rank == n_live - 1) {
      role = 0;
    } else if (rank >= n_live - k) {
      const int sl = n_live - 1 - rank;
      if (helper_wait(ctl + sl * kCtlStride, ctl, n_live, p.merge_wait_ticks)) role = sl;
    }
    // Acquire: the other workgroups' partials are visible from here on.
    if (role >= 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    sm_flag[0] = role;
  }
  __syncthreads();
  const int role = sm_flag[0];
  if (role < 0) return;
  if (role > 0) {
    merge_slice<T, D, NT>(p, slot0, n_live, row0, wg_rows, role, k, out_s, kvh);
    return;
  }
  // Last arriver: say go to the helpers (lanes 1 .. k-1 of wave 0), merge
  // slice 0 while those exchanges are in flight, then settle each word and
  // take over the slices whose helpers gave up.
  int old = kSliceIdle;
  if (tid >= 1 && tid < k)
    old = __hip_atomic_exchange(ctl + tid * kCtlStride, kSliceGo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  merge_slice<T, D, NT>(p, slot0, n_live, row0, wg_rows, 0, k, out_s, kvh);
  if (tid < 64) {
    const bool mine = old == kSliceGaveUp;
    if (mine || old == kSliceDone)
      __hip_atomic_store(ctl + tid * kCtlStride, kSliceIdle, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t own = __ballot(mine);
    if (tid == 0) {
      sm_flag[1] = int(uint32_t(own));
      // The arrival counter's last use in this launch: helpers that still
      // poll it have the go word.
      __hip_atomic_store(ctl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  for (uint32_t own = uint32_t(sm_flag[1]); own != 0; own &= own - 1)
    merge_slice<T, D, NT>(p, slot0, n_live, row0, wg_rows, __builtin_ctz(own), k, out_s, kvh);
}

template <typename T, int D>
__device__ __forceinline__ void zero_rows(const Params& p, int s, int kvh, int row0, int nrows, int nthreads) {
  T* out_s = static_cast<T*>(p.out) + int64_t(s) * p.query_len * p.num_q_heads * D;
  const int items = nrows * (D / 8);
  for (int it = threadIdx.x; it < items; it += nthreads) {
    const int r = it / (D / 8), d8 = it % (D / 8);
    *reinterpret_cast<i32x4*>(out_row(p, out_s, kvh, row0 + r, D) + 8 * d8) = i32x4{0, 0, 0, 0};
  }
}

// Segments of a sequence of (clamped) length L: its visible key range in
// 16-key tiles [t_lo, t_hi), split into n_live segments of seg_tiles tiles
// (at least the planned count, stretched when a device length exceeds the
// planning bound).
struct SegSplit {
  int t_lo, t_hi, seg_tiles, n_live;
};

__device__ __forceinline__ int clamped_len(const Params& p, int s) {
  // Lengths past the block table's capacity are clamped to it.
  return min(p.seq_lens[s], p.max_blocks * p.page_size);
}

__device__ __forceinline__ SegSplit split_of(const Params& p, int L) {
  SegSplit r;
  const int k_lo = p.window > 0 ? max(0, L - p.query_len - p.window + 1) : 0;
  r.t_lo = k_lo >> 4;
  r.t_hi = (L + 15) >> 4;
  const int n_tiles = r.t_hi - r.t_lo;
  r.seg_tiles = max(p.seg_tiles, (n_tiles + p.nseg - 1) / p.nseg);
  r.n_live = (n_tiles + r.seg_tiles - 1) / r.seg_tiles;
  return r;
}

// Persistent grid (batched decode): one workgroup per CU takes work items
// from a queue in the workspace until none are left.  Items are the live
// segments of every (sequence, kv head, row group), longest sequences
// first (ties by index; up to kPersistSortSeqs sequences, else in index
// order) and, within a sequence, unit-major so the segments of a unit run
// together and its merge helpers wait little.  An item's work does not
// depend on which workgroup takes it, so results stay bitwise the same.
// Sequences of length <= 0 get one item per unit (its zero output).
// Every workgroup ends with one failed take; the last of those resets the
// queue for the next launch.
template <typename Body>
__device__ __forceinline__ void persistent_loop(const Params& p, unsigned char* lds, int persist_off, int lds_bytes,
                                               int nt, Body body) {
  const int tid = threadIdx.x;
  const int S = p.num_seqs;
  const int units = p.num_kv_heads * p.row_groups;
  int* sm_order = reinterpret_cast<int*>(lds + persist_off);  // [S]: sequence of rank r
  int* sm_pref = sm_order + kPersistMaxSeqs;                   // [S + 1]: first item of rank r
  // Scratch before the first item (the tile-loop area): lengths and item
  // counts per rank.
  int* sm_len = reinterpret_cast<int*>(lds);                   // [S]
  int* sm_cnt = sm_len + kPersistMaxSeqs;                      // [S]
  int* sm_take = reinterpret_cast<int*>(lds + lds_bytes - 16) + 2;
  for (int i = tid; i < S; i += nt) sm_len[i] = clamped_len(p, i);
  __syncthreads();
  const bool sort = S <= kPersistSortSeqs;
  for (int i = tid; i < S; i += nt) {
    const int li = sm_len[i];
    int rank = i;
    if (sort) {
      rank = 0;
      for (int j = 0; j < S; ++j) {
        const int lj = sm_len[j];
        rank += (lj > li) || (lj == li && j < i);
      }
    }
    sm_order[rank] = i;
  }
  __syncthreads();
  // Items per rank, then an exclusive prefix (wave 0: lanes own
  // contiguous chunks of ranks).
  for (int r = tid; r < S; r += nt) {
    const int L = sm_len[sm_order[r]];
    sm_cnt[r] = L <= 0 ? units : units * split_of(p, L).n_live;
  }
  __syncthreads();
  if (tid < 64) {
    const int chunk = (S + 63) / 64;
    const int r0 = min(S, tid * chunk), r1 = min(S, r0 + chunk);
    int sum = 0;
    for (int r = r0; r < r1; ++r) sum += sm_cnt[r];
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (tid >= o) incl += v;
    }
    int run = incl - sum;
    for (int r = r0; r < r1; ++r) {
      sm_pref[r] = run;
      run += sm_cnt[r];
    }
    if (tid == 63) sm_pref[S] = incl;
  }
  __syncthreads();
  const int total = sm_pref[S];
  int* queue = p.ws_cnt + kQueueWord;
  for (;;) {
    if (tid == 0) sm_take[0] = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int item = sm_take[0];
    __syncthreads();
    if (item >= total) {
      if (tid == 0 && item == total + int(gridDim.x) - 1)
        __hip_atomic_store(queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    // Rank holding the item: the last r with sm_pref[r] <= item.
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sm_pref[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int s = sm_order[lo];
    const int local = item - sm_pref[lo];
    const int L = clamped_len(p, s);
    const int per_unit = L <= 0 ? 1 : split_of(p, L).n_live;
    const int unit = local / per_unit, seg = local % per_unit;
    body(s, unit % p.num_kv_heads, unit / p.num_kv_heads, seg);
    __syncthreads();  // LDS is reused by the next item
  }
}

// One work item: segment `seg` of (sequence s, kv head kvh, row group rg).
template <typename T, int D, int RT>
__device__ __forceinline__ void decode_unit(const Params& p, unsigned char* lds, int s, int kvh, int rg, int seg) {
  using MF = Mfma<T>;
  using SH = Shape<D, RT>;
  constexpr int NW = SH::NW, KC = SH::KC, DT = SH::DT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const int row0 = rg * RT * 16;
  const int wg_rows = min(RT * 16, p.rows - row0);
  const int M = p.query_len;

  const int L = clamped_len(p, s);
  if (L <= 0) {
    if (seg == 0) zero_rows<T, D>(p, s, kvh, row0, wg_rows, SH::kThreads);
    return;
  }
  const int k_lo = p.window > 0 ? max(0, L - M - p.window + 1) : 0;
  const SegSplit sp = split_of(p, L);
  const int t_hi = sp.t_hi, seg_tiles = sp.seg_tiles, n_live = sp.n_live;
  if (seg >= n_live) return;
  const int ts = sp.t_lo + seg * seg_tiles, te = min(ts + seg_tiles, t_hi);
  // Tiles needing no mask: every key visible to every row.
  const int lo_last = p.window > 0 ? max(0, L - p.window) : 0;
  const int qpos_first = L - M;

  // Per-lane query row (row = lane % 16 of each row tile): position and
  // window start; rows past G*M see nothing.
  int qpos_r[RT], lo_r[RT];
  i32x4 qop[RT][KC];
  const T* Q = static_cast<const T*>(p.q);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int ru = row0 + rt * 16 + c;
    if (ru < p.rows) {
      const int m = ru / p.group, gq = ru % p.group;
      qpos_r[rt] = L - M + m;
      lo_r[rt] = p.window > 0 ? max(0, qpos_r[rt] - p.window + 1) : 0;
      const T* qrow = Q + ((int64_t(s) * M + m) * p.num_q_heads + kvh * p.group + gq) * D;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) qop[rt][kc] = *reinterpret_cast<const i32x4*>(qrow + 32 * kc + 8 * g);
    } else {
      qpos_r[rt] = -1;
      lo_r[rt] = 0;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) qop[rt][kc] = i32x4{0, 0, 0, 0};
    }
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
  const int32_t* table = p.block_table + int64_t(s) * p.max_blocks;
  // Byte offset of this lane's 16-byte chunk inside a tile: key row c,
  // head-dim elements 8g..8g+7 of chunk 0 (32-bit, per lane); the tile base
  // itself is wave-uniform, so the loads take a scalar base address.
  const uint32_t lane_off = uint32_t(c * p.token_stride + 8 * g) * uint32_t(sizeof(T));
  uint16_t* vs = reinterpret_cast<uint16_t*>(lds) + wave * 16 * SH::kVStride;
  // Transposed-read address of this lane: row 4g + c/4, columns 4(c%4).. of
  // each 16-column tile (ds_read_b64_tr_b16 returns column c of the 4x16
  // block its 16-lane group addresses, i.e. 4 keys of one head-dim column).
  const uint16_t* vtr = vs + (4 * g + (c >> 2)) * SH::kVStride + 4 * (c & 3);

  struct Tile {
    i32x4 k[KC];
    i32x4 v[KC];
  };

  // The segment's block ids (one per tile) go to LDS once, so a tile's
  // page address costs an LDS read instead of a scalar load that may miss.
  // The planner keeps segments within kMaxSegTiles tiles.
  int* sm_ids = reinterpret_cast<int*>(lds + SH::kVBytes);
  for (int t = tid; t < te - ts; t += SH::kThreads) sm_ids[t] = table[((ts + t) * 16) / p.page_size];
  __syncthreads();
  // Physical block of tile t (wave-uniform).
  auto block_of = [&](int t) { return __builtin_amdgcn_readfirstlane(sm_ids[t - ts]); };

  auto issue_tile = [&](Tile& tl, int t, int blk) {
    const int key0 = t * 16;
    const unsigned char* base =
        KVh + (int64_t(blk) * p.block_stride + int64_t(key0 % p.page_size) * p.token_stride) * int64_t(sizeof(T));
    const unsigned char* row = base + lane_off;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) tl.k[kc] = *reinterpret_cast<const i32x4*>(row + 64 * kc);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) tl.v[kc] = *reinterpret_cast<const i32x4*>(row + 2 * D + 64 * kc);
  };

  auto compute_tile = [&](Tile& tl, int t) {
    const int key0 = t * 16;
    const bool edge = !(key0 >= lo_last && key0 + 15 <= qpos_first);
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

    uint64_t pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) sc = MF::qk(tl.k[kc], qop[rt][kc], sc);
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = sc[j] * p.scale_log2;
        if (edge) {
          const int key = key0 + 4 * g + j;
          if (key < lo_r[rt] || key > qpos_r[rt]) x[j] = kNegInf;
        }
      }
      float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run[rt], tmax);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[rt] - m_use);
      float pj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pj[j] = fast_exp2(x[j] - m_use);
      l_run[rt] = l_run[rt] * alpha + ((pj[0] + pj[1]) + (pj[2] + pj[3]));
      m_run[rt] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= alpha;
      pb[rt] = pack4(MF::bits(pj[0]), MF::bits(pj[1]), MF::bits(pj[2]), MF::bits(pj[3]));
    }

    // The staged V rows were written by other lanes of this wave; LDS
    // operations of a wave complete in order, the fences keep the compiler
    // from moving the reads above the writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint64_t va = __builtin_bit_cast(
          uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vtr + 16 * dt)));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][dt] = MF::pv(va, pb[rt], acc[rt][dt]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Interleaved tiles per wave: tile i of this wave is ts + wave + i * NW.
  // PF tiles are in flight beyond the one being computed (a ring of PF + 1
  // register buffers), and each tile's block id is read one tile before
  // its loads are issued.  The prefetch index is clamped to the wave's last
  // tile instead of being skipped, so every iteration has the same loads in
  // flight and the compiler's wait counts stay exact (the clamped re-reads
  // of the last tile hit in cache).
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
  finish<T, D, RT, NW>(p, lds, s, kvh, rg, seg, row0, wg_rows, n_live, SH::kBytes);
}

// PERSIST selects the grid: one workgroup per item, or the persistent
// grid (separate instantiations, so each inlines the item body once).
template <typename T, int D, int RT, bool PERSIST>
__global__ __launch_bounds__((Shape<D, RT>::kThreads)) void decode_mfma_kernel(Params p) {
  using SH = Shape<D, RT>;
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
    decode_unit<T, D, RT>(p, lds, blockIdx.y, kvh, rg, seg);
  } else {
    persistent_loop(p, lds, SH::kPersistOff, SH::kBytes, SH::kThreads,
                    [&](int s, int kvh, int rg, int seg) { decode_unit<T, D, RT>(p, lds, s, kvh, rg, seg); });
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
  const int rows = p.rows;  // <= kDotRows
  const int M = p.query_len;

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
      const T* qrow = Q + ((int64_t(s) * M + m) * p.num_q_heads + kvh * p.group + gq) * D;
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
  finish<T, D, 1, NW>(p, lds, s, kvh, 0, seg, 0, rows, n_live, SH::kBytes);
}

__global__ void zero_kernel(uint32_t* p, size_t n) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

template <typename T, int D, int RT>
int launch_t(const Plan& pl, const Params& pr, hipStream_t st) {
  if (pl.persistent)
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, RT, true>), dim3(pl.grid_x, pl.grid_y), dim3(Shape<D, RT>::kThreads),
                       0, st, pr);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, RT, false>), dim3(pl.grid_x, pl.grid_y), dim3(Shape<D, RT>::kThreads),
                       0, st, pr);
  return int(hipGetLastError());
}

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
int launch_dot(const Plan& pl, const Params& pr, hipStream_t st) {
  hipLaunchKernelGGL((decode_dot_kernel<T, D>), dim3(pl.grid_x, pl.grid_y), dim3(DotShape<D>::kThreads), 0, st, pr);
  return int(hipGetLastError());
}

template <typename T>
int launch_dtype(const Plan& pl, const Params& pr, int head_size, hipStream_t st) {
  if (pl.path == PAD_PATH_DOT) {
    switch (head_size) {
      case 64: return launch_dot<T, 64>(pl, pr, st);
      case 128: return launch_dot<T, 128>(pl, pr, st);
    }
    return int(hipErrorInvalidValue);
  }
  switch (head_size) {
    case 64: return launch_d<T, 64>(pl, pr, st);
    case 128: return launch_d<T, 128>(pl, pr, st);
    case 256: return launch_d<T, 256>(pl, pr, st);
    case 512: return launch_d<T, 512>(pl, pr, st);
  }
  return int(hipErrorInvalidValue);
}

}  // namespace

int launch_decode(const Plan& plan, const Params& params, int dtype, int head_size, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == PAD_BF16) return launch_dtype<__bf16>(plan, params, head_size, st);
  return launch_dtype<_Float16>(plan, params, head_size, st);
}

int launch_zero(void* ptr, size_t words, void* stream) {
  if (words == 0) return 0;
  const size_t blocks = (words + 255) / 256;
  const unsigned grid = unsigned(blocks < 1024 ? blocks : 1024);
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(ptr), words);
  return int(hipGetLastError());
}

}  // namespace pad
