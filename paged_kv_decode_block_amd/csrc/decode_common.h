// Device code shared by the decode-attention kernels (gfx950): MFMA
// traits, stores, the split-KV merge and its hand-over protocol, segment
// splits and the balanced persistent grid's work loop.  Included by the kernel
// sources only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace pad {
namespace dev {

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
  // Two values rounded to bf16 and packed (a in the low half): one
  // conversion instruction for the pair.
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, b2));
  }
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
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
  }
};

constexpr float kNegInf = -__builtin_huge_valf();
// Slack of a row's reference maximum in the exp2 domain: scores up to this
// far above it keep it (softmax weights up to 2^8 before normalisation).
constexpr float kMaxSlack = 8.f;
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

template <typename T>
__device__ __forceinline__ T* out_row(const Params& p, T* out_s, int kvh, int ru, int D) {
  const int m = ru / p.group, gq = ru % p.group;
  return out_s + (int64_t(m) * p.num_q_heads + kvh * p.group + gq) * D;
}

// Query tokens of sequence s (at most query_len) and the index of its first
// token in q and out: the uniform layout, or the packed one whose tokens
// of sequence s start at q_start[s] (per-request query counts, as the
// query maps of the octave page's metadata builder give them).  Counts
// outside [0, query_len] are clamped into it.
struct SeqQ {
  int m, first;
};
__device__ __forceinline__ SeqQ seq_queries(const Params& p, int s) {
  if (p.q_start == nullptr) return SeqQ{p.query_len, s * p.query_len};
  const int a = p.q_start[s];
  return SeqQ{min(max(p.q_start[s + 1] - a, 0), p.query_len), a};
}

// Output rows of sequence s.
template <typename T>
__device__ __forceinline__ T* seq_out(const Params& p, int s, int D) {
  return static_cast<T*>(p.out) + int64_t(seq_queries(p, s).first) * p.num_q_heads * D;
}

// ---- split-KV merge ----
// The merged output of a unit is rows x D floats, cut into items (row r,
// four head-dim columns d4): item = r * (D / 4) + d4.  Merge slice `slice`
// of `nslices` covers items [slice * I / nslices, (slice + 1) * I / nslices).
// LN = 2^lg lanes serve one item, enough that kMergeU slots per lane cover
// all n slots (n <= 256): lane `sub` takes slots sub, sub + LN, ..., so an
// item costs one round of loads.  Each lane forms the log-sum-exp merge of
// its slots in the exp2 domain,  m* = max m_j,  l* = sum l_j 2^(m_j - m*),
// acc* = sum acc_j 2^(m_j - m*),  and the LN lanes then combine in a fixed
// butterfly.  Each item's sums follow one fixed order for a given slot
// count, whichever workgroup merges it.  Every load is unconditional (item
// and slot indices clamped, extra slots weighted zero) so the wait counts
// stay exact, and the passes of a thread form one stream with the next
// pass's loads in flight while the current one is consumed.  LN is a
// run-time value: one compiled body serves every slot count, which keeps
// this once-per-launch code small (as several unrolled variants it cost
// the merge about a microsecond of instruction fetch; a variant taking
// several items per thread when n <= 8 -- a quarter of the passes for two
// partials -- measured no faster on the batch workload and 1.2-1.4 us
// slower on one sequence of 4k and 32k keys).
constexpr int kMergeU = 8;
struct MergeChunk {
  f32x4 acc[kMergeU];
  float2 ml[kMergeU];
};

// Where a unit's n partials live.  Partial j (0 <= j < n) is in slot
// first + j for j < n - 1 and in slot `last` for j = n - 1: on the grid
// schedule the unit's slots are consecutive (last = first + n - 1); on the
// balanced persistent grid the last one may sit in the other half of the
// slot array.  A slot holds Params::slot_rows rows of (m, l) and of acc;
// the unit's rows start at row `row0` of each slot.
struct Parts {
  int64_t first, last;
  int n, row0;
};

// One work item: tiles [ts, te) of one unit's key range, its partial slot
// and where the unit's other partials and control words are.
struct Frag {
  int ts, te;          // 16-key tiles of this item
  int n_parts;         // partials of the unit (1: the item is the whole unit and writes the output)
  int merge_slices;    // workgroups sharing the unit's merge
  int64_t slot;        // this item's partial slot (n_parts > 1)
  Parts parts;         // the unit's partials, in merge order
  int* ctl;            // the unit's arrival counter, then one hand-over word per slice
};

// The unit's first partial slot starts at a wave-uniform 64-bit base; a
// slot and an item are 32-bit byte offsets from it: below 2^32 for up to
// 255 consecutive slots of 4096 rows x 512 columns x 4 bytes (grid), or
// 511 slots of at most 64 rows (balanced grid).
template <int D, int NT>
__device__ __forceinline__ void merge_load(const Params& p, MergeChunk& b, const unsigned char* acc_base,
                                           const unsigned char* ml_base, uint32_t last_rel, int i0, int i1, int n,
                                           int lg, int pass) {
  const int it = min(i0 + pass * (NT >> lg) + (int(threadIdx.x) >> lg), i1 - 1);
  const int r = it / (D / 4), d4 = it % (D / 4);
  const uint32_t acc_item = uint32_t(r * D + 4 * d4) * 4u;
  const uint32_t ml_item = uint32_t(r) * 8u;
  const uint32_t acc_slot = uint32_t(p.slot_rows) * uint32_t(D) * 4u, ml_slot = uint32_t(p.slot_rows) * 8u;
  const int sub = int(threadIdx.x) & ((1 << lg) - 1);
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) {
    const uint32_t j = uint32_t(min(sub + (u << lg), n - 1));
    const uint32_t jr = j == uint32_t(n - 1) ? last_rel : j;
    b.acc[u] = *reinterpret_cast<const f32x4*>(acc_base + (jr * acc_slot + acc_item));
    b.ml[u] = *reinterpret_cast<const float2*>(ml_base + (jr * ml_slot + ml_item));
  }
}

template <typename T, int D, int NT>
__device__ __forceinline__ void merge_consume(const Params& p, const MergeChunk& b, int i0, int i1, int n, int lg,
                                              int pass, int row0, T* out_s, int kvh) {
  using MF = Mfma<T>;
  const int sub = int(threadIdx.x) & ((1 << lg) - 1);
  float mj[kMergeU];
  float mloc = kNegInf;
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) {
    mj[u] = sub + (u << lg) < n ? b.ml[u].x : kNegInf;
    mloc = fmaxf(mloc, mj[u]);
  }
  const float m_use = mloc == kNegInf ? 0.f : mloc;
  float l_loc = 0.f;
  f32x4 a_loc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) {
    const float wgt = fast_exp2(mj[u] - m_use);
    l_loc += wgt * b.ml[u].y;
    a_loc += wgt * b.acc[u];
  }
  // Combine the item's lanes and write it.
  float m_all = mloc;
  for (int o = 1; o < (1 << lg); o <<= 1) m_all = fmaxf(m_all, __shfl_xor(m_all, o));
  const float f = fast_exp2(mloc - (m_all == kNegInf ? 0.f : m_all));
  float l = l_loc * f;
  f32x4 a = a_loc * f;
  for (int o = 1; o < (1 << lg); o <<= 1) {
    l += __shfl_xor(l, o);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += __shfl_xor(a[e], o);
  }
  const int it = i0 + pass * (NT >> lg) + (int(threadIdx.x) >> lg);
  if (sub == 0 && it < i1) {
    const int r = it / (D / 4), d4 = it % (D / 4);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint2 o;
    o.x = uint32_t(MF::bits(a[0] * inv)) | (uint32_t(MF::bits(a[1] * inv)) << 16);
    o.y = uint32_t(MF::bits(a[2] * inv)) | (uint32_t(MF::bits(a[3] * inv)) << 16);
    *reinterpret_cast<uint2*>(out_row(p, out_s, kvh, row0 + r, D) + 4 * d4) = o;
  }
}

// Merge slice `slice` of `nslices` of a unit's partials (rows
// pt.row0 .. pt.row0 + wg_rows - 1 of each slot) into output rows
// out_row0 .. out_row0 + wg_rows - 1.  Lanes per item follow the partial
// count only, so an item's sums take the same order whatever the slicing
// and whichever workgroup merges it: the output bits depend on the
// partials alone.  The caller has acquired the partials.
template <typename T, int D, int NT>
__device__ __forceinline__ void merge_slice(const Params& p, const Parts& pt, int out_row0, int wg_rows, int slice,
                                            int nslices, T* out_s, int kvh) {
  const int n = pt.n;
  const int items = wg_rows * (D / 4);
  const int i0 = slice * items / nslices, i1 = (slice + 1) * items / nslices;
  if (i1 <= i0) return;
  const int lg = n <= 8 ? 0 : (n <= 16 ? 1 : (n <= 32 ? 2 : (n <= 64 ? 3 : (n <= 128 ? 4 : 5))));
  const int ipp = NT >> lg;
  const int W = (i1 - i0 + ipp - 1) / ipp;
  const int64_t row_base = pt.first * p.slot_rows + pt.row0;
  const unsigned char* acc_base = reinterpret_cast<const unsigned char*>(p.ws_acc + row_base * D);
  const unsigned char* ml_base = reinterpret_cast<const unsigned char*>(p.ws_ml + row_base * 2);
  const uint32_t last_rel = uint32_t(pt.last - pt.first);
  MergeChunk b0, b1;
  merge_load<D, NT>(p, b0, acc_base, ml_base, last_rel, i0, i1, n, lg, 0);
  if (W == 1) {
    merge_consume<T, D, NT>(p, b0, i0, i1, n, lg, 0, out_row0, out_s, kvh);
    return;
  }
  for (int w = 0; w < W; w += 2) {
    merge_load<D, NT>(p, b1, acc_base, ml_base, last_rel, i0, i1, n, lg, min(w + 1, W - 1));
    merge_consume<T, D, NT>(p, b0, i0, i1, n, lg, w, out_row0, out_s, kvh);
    merge_load<D, NT>(p, b0, acc_base, ml_base, last_rel, i0, i1, n, lg, min(w + 2, W - 1));
    if (w + 1 < W) merge_consume<T, D, NT>(p, b1, i0, i1, n, lg, w + 1, out_row0, out_s, kvh);
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
// slice, and whether its word still needs the helper's second action.
// Every path ends: the wait is bounded by wait_ticks of the 100 MHz
// real-time counter.  Seeing the unit complete, the helper merges at once
// and posts "done" alongside its merge loads (kHelperSettle): the exchange
// only settles who resets the word, so it need not delay the merge.
constexpr int kHelperGaveUp = 0, kHelperMerge = 1, kHelperSettle = 2;
__device__ __forceinline__ int helper_wait(int* word, const int* counter, int n, uint32_t wait_ticks) {
  int seen = kSliceIdle;
  if (!__hip_atomic_compare_exchange_strong(word, &seen, kSliceWaiting, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)) {
    // The last arriver came first (go): this is the word's last use.
    __hip_atomic_store(word, kSliceIdle, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return kHelperMerge;
  }
  const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + wait_ticks;
  for (;;) {
    // Both words are read in one round trip.
    const int cnt = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int w = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (cnt == n || w == kSliceGo) return kHelperSettle;
    if (__builtin_amdgcn_s_memrealtime() >= t_end) break;
    __builtin_amdgcn_s_sleep(1);
  }
  seen = kSliceWaiting;
  if (__hip_atomic_compare_exchange_strong(word, &seen, kSliceGaveUp, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT))
    return kHelperGaveUp;
  __hip_atomic_store(word, kSliceIdle, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // go came first
  return kHelperMerge;
}

// Count this workgroup's arrival for its unit (its partial rows are
// published with device-coherent stores) and take part in the merge: of
// the n arrivals of a unit, the last one and the k - 1 before it (k = merge
// slices) merge one slice of the output each; the rest are done.  `flags`
// are 16 bytes of LDS (words 0 and 1).
template <typename T, int D, int NT>
__device__ __forceinline__ void arrive_and_merge(const Params& p, int* flags, int s, int kvh, int row0, int wg_rows,
                                                 const Frag& f) {
  const int tid = threadIdx.x;
  T* out_s = seq_out<T>(p, s, D);
  int* ctl = f.ctl;
  const int n_live = f.n_parts;
  int* sm_flag = flags;
  const int k = min(f.merge_slices, n_live);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  __syncthreads();
  // Thread 0 of a helper that saw the unit complete still posts "done" on
  // its word (kHelperSettle).
  bool settle = false;
  if (tid == 0) {
    // Role: 0 = last arriver, 1 .. k-1 = helper merging that slice, -1 = done.
    const int rank = __hip_atomic_fetch_add(ctl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int role = -1;
    if (rank == n_live - 1) {
      role = 0;
    } else if (rank >= n_live - k) {
      const int sl = n_live - 1 - rank;
      const int h = helper_wait(ctl + sl * kCtlStride, ctl, n_live, p.merge_wait_ticks);
      if (h != kHelperGaveUp) role = sl;
      settle = h == kHelperSettle;
    }
    // Acquire: the other workgroups' partials are visible from here on.
    // (Device-coherent loads of the partials instead of this fence, which
    // invalidates the die's L2, measured slower.)
    if (role >= 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    sm_flag[0] = role;
  }
  __syncthreads();
  const int role = sm_flag[0];
  if (role < 0) return;
  // Slices this workgroup merges: its own (slice 0 for the last arriver),
  // and for the last arriver those whose helpers gave up -- known once its
  // "go" exchanges (issued before its own slice) return.  A settling
  // helper's "done" exchange is likewise issued before its merge loads and
  // read after them.  One merge call site keeps the kernel's code and
  // register use small.
  int old = kSliceIdle;
  if (role == 0 && tid >= 1 && tid < k)
    old = __hip_atomic_exchange(ctl + tid * kCtlStride, kSliceGo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (settle)
    old = __hip_atomic_exchange(ctl + role * kCtlStride, kSliceDone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t todo = 1u << role;
  bool settled = role > 0;
  while (todo != 0) {
    const int sl = __builtin_ctz(todo);
    todo &= todo - 1;
    merge_slice<T, D, NT>(p, f.parts, row0, wg_rows, sl, k, out_s, kvh);
    if (!settled) {
      settled = true;
      if (tid < 64) {
        const bool mine = old == kSliceGaveUp;
        if (mine || old == kSliceDone)
          __hip_atomic_store(ctl + tid * kCtlStride, kSliceIdle, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t own = __ballot(mine);
        if (tid == 0) {
          sm_flag[1] = int(uint32_t(own));
          // The arrival counter's last use in this launch: helpers that
          // still poll it have the go word.
          __hip_atomic_store(ctl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
      todo |= uint32_t(sm_flag[1]);
    }
  }
  // A settling helper that finds go on its word acts second: it resets it.
  if (settle && old == kSliceGo)
    __hip_atomic_store(ctl + role * kCtlStride, kSliceIdle, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int D>
__device__ __forceinline__ void zero_rows(const Params& p, int s, int kvh, int row0, int nrows, int nthreads) {
  T* out_s = seq_out<T>(p, s, D);
  const int items = nrows * (D / 8);
  for (int it = threadIdx.x; it < items; it += nthreads) {
    const int r = it / (D / 8), d8 = it % (D / 8);
    *reinterpret_cast<i32x4*>(out_row(p, out_s, kvh, row0 + r, D) + 8 * d8) = i32x4{0, 0, 0, 0};
  }
}

// Segments of row group rg of a sequence of (clamped) length L with M query
// tokens: the key range its rows can see, in 16-key tiles [t_lo, t_hi),
// split into n_live segments of seg_tiles tiles (at least the planned
// count, stretched when a device length exceeds the planning bound).  The
// group's rows (row = m * G + head) hold tokens first_m .. last_m, which
// see keys below L - M + last_m + 1 and, with a window W, from
// L - M + first_m - W + 1 on: a tile of a prefill chunk reads only the
// keys its own tokens reach (the work list entries of plan_prefill on the
// rdna_hip page).  A group with no row has no segment; one whose tokens
// all sit before the first key keeps one tile (all masked: zero rows).
struct SegSplit {
  int t_lo, t_hi, seg_tiles, n_live;
};

__device__ __forceinline__ int clamped_len(const Params& p, int s) {
  // Lengths past the block table's capacity are clamped to it.
  return min(p.seq_lens[s], p.max_blocks * p.page_size);
}

__device__ __forceinline__ SegSplit split_of(const Params& p, int L, int M, int rg) {
  SegSplit r;
  const int rows = p.group * M;
  const int r0 = rg * p.group_rows;
  if (r0 >= rows) {
    r.t_lo = r.t_hi = r.seg_tiles = r.n_live = 0;
    return r;
  }
  const int first_m = r0 / p.group, last_m = (min(rows, r0 + p.group_rows) - 1) / p.group;
  const int k_end = min(L, L - M + last_m + 1);
  const int k_lo = p.window > 0 ? max(0, L - M + first_m - p.window + 1) : 0;
  r.t_lo = k_lo >> 4;
  r.t_hi = max((k_end + 15) >> 4, r.t_lo + 1);
  const int n_tiles = r.t_hi - r.t_lo;
  r.seg_tiles = max(p.seg_tiles, (n_tiles + p.nseg - 1) / p.nseg);
  r.n_live = (n_tiles + r.seg_tiles - 1) / r.seg_tiles;
  return r;
}

// Balanced persistent grid (batched decode).  Every unit -- (sequence, row
// group, kv head) in that order -- takes p.unit_lead lead positions (its
// item's fixed cost, in tiles) and then one position per 16-key tile of its
// key range [t_lo, t_hi) of split_of; the units are laid end to end, T
// positions in all, and workgroup b of the Gs = min(G, T) first of the G =
// gridDim.x workgroups (one per CU, or two for a packed cache) takes the
// contiguous share [b T / Gs, (b + 1) T / Gs): every workgroup gets the same
// work, tiles plus item costs, whatever the lengths.  A share computes the tiles among its positions; lead positions
// alone make no item.  A unit inside one share is computed
// whole and written directly.  A unit cut by share boundaries is computed
// as one work item per share it meets; each item publishes a partial and
// the last to arrive merges them in share order (fixed, so the result is
// deterministic for a given batch).  A workgroup publishes at most two
// partials: slot b for the item that reaches its share's end, slot G + b
// for an item that starts at its share's start and ends inside it
// (b < Gs <= G, so the two halves never meet).  So a
// unit met by shares b0..b1 has its partials in slots b0 .. b1 - 1 and
// then b1 (its end is b1's share end) or G + b1.
// Sequences of length <= 0 with query tokens get zero rows (written by
// workgroup s % G); those without query tokens have nothing to do.  The
// planner keeps T below 2^31.
template <typename Body, typename Zero>
__device__ __forceinline__ void balanced_loop(const Params& p, unsigned char* lds, int tables_off, int nt,
                                              Body body, Zero zero) {
  const int tid = threadIdx.x;
  const int S = p.num_seqs;
  int* sm_len = reinterpret_cast<int*>(lds + tables_off);  // [S]: clamped lengths
  int* sm_pref = sm_len + kPersistMaxSeqs;                   // [S + 1]: first tile of sequence s
  // Before the first item the tile-loop area holds the tile counts.
  int* sm_cnt = reinterpret_cast<int*>(lds);  // [S]
  for (int i = tid; i < S; i += nt) {
    const int L = clamped_len(p, i);
    sm_len[i] = L;
    int n = 0;
    const int M = seq_queries(p, i).m;
    if (L > 0 && M > 0) {
      for (int rg = 0; rg < p.row_groups; ++rg) {
        const SegSplit sp = split_of(p, L, M, rg);
        if (sp.n_live > 0) n += p.unit_lead + sp.t_hi - sp.t_lo;
      }
    }
    sm_cnt[i] = n * p.num_kv_heads;
  }
  __syncthreads();
  // Exclusive prefix over the sequences (wave 0: lanes own contiguous
  // chunks of sequences).
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
  const int G = int(gridDim.x), b = int(blockIdx.x);
  // Zero rows of padded sequences.
  for (int s = b; s < S; s += G) {
    if (sm_len[s] > 0) continue;
    const int M = seq_queries(p, s).m;
    if (M == 0) continue;
    for (int rg = 0; rg < p.row_groups; ++rg)
      for (int kvh = 0; kvh < p.num_kv_heads; ++kvh) zero(s, kvh, rg, M);
  }
  const int T = sm_pref[S];
  // Shares of the first min(G, T) workgroups, each at least one position.
  // A share meets a unit when it holds one of the unit's tiles (not only
  // lead positions); each share a unit meets has an item that arrives.
  const int Gs = min(G, T);
  if (b >= Gs) return;
  const int start = int(int64_t(b) * T / Gs), end = int(int64_t(b + 1) * T / Gs);
  // Share holding position t: the largest b' with floor(b' T / Gs) <= t.
  auto owner = [&](int t) { return int((int64_t(t + 1) * Gs - 1) / T); };
  auto share_end = [&](int bb) { return int(int64_t(bb + 1) * T / Gs); };
  // Sequence holding position `start`: the last s with sm_pref[s] <= start.
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sm_pref[mid] <= start) lo = mid; else hi = mid - 1;
  }
  int pos = start;
  for (int s = lo; s < S && pos < end; ++s) {
    const int L = sm_len[s];
    const int M = L > 0 ? seq_queries(p, s).m : 0;
    if (M == 0) continue;
    int ub = sm_pref[s];  // first position of the unit being visited
    for (int rg = 0; rg < p.row_groups && pos < end; ++rg) {
      const SegSplit sp = split_of(p, L, M, rg);
      if (sp.n_live == 0) continue;
      const int nu = sp.t_hi - sp.t_lo;
      for (int kvh = 0; kvh < p.num_kv_heads && pos < end; ++kvh, ub += p.unit_lead + nu) {
        // Positions [ub, ub + lead) stand for the item's fixed cost; the
        // unit's tiles are positions [rb, ue).
        const int rb = ub + p.unit_lead, ue = rb + nu;
        if (ue <= pos) continue;
        const int f0 = max(rb, pos), f1 = min(ue, end);
        if (f0 >= f1) {  // the share ends among the lead positions
          pos = end;
          break;
        }
        const int b0 = owner(rb), b1 = owner(ue - 1);
        Frag f;
        f.ts = sp.t_lo + (f0 - rb);
        f.te = sp.t_lo + (f1 - rb);
        f.n_parts = b1 - b0 + 1;
        f.merge_slices = 1;
        f.slot = f1 == end ? b : G + b;
        f.parts.first = b0;
        f.parts.last = ue == share_end(b1) ? b1 : G + b1;
        f.parts.n = f.n_parts;
        f.parts.row0 = 0;
        f.ctl = p.ws_cnt + ((int64_t(s) * p.num_kv_heads + kvh) * p.row_groups + rg) * kCtlStride;
        body(s, kvh, rg, f);
        __syncthreads();  // LDS is reused by the next item
        pos = f1;
      }
    }
  }
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

// After the waves of a workgroup have left their results in LDS -- per
// wave w: sm_m/sm_l[w][row] (running max and sum) and the accumulator
// rows, already rescaled to the workgroup maximum, in slot w of sm_acc; and
// the workgroup's merged max/sum in sm_ms/sm_ls -- sum the slots in wave
// order (deterministic) and either write the output (single segment) or
// publish this segment's partial and take part in the merge.  NSUM slots
// are summed (1 when the rows were already summed and rotated into slot 0).
// NT threads take part (NW * 64 by default).
template <typename T, int D, int RT, int NW, int NSUM = NW, int NT = NW * 64>
__device__ __forceinline__ void finish(const Params& p, unsigned char* lds, int s, int kvh, int row0, int wg_rows,
                                       const Frag& f, int lds_bytes) {
  using MF = Mfma<T>;
  using CB = Combine<D, RT, NW>;
  const int tid = threadIdx.x;
  const float* sm_acc = CB::acc(lds);
  const float* sm_ms = CB::ms(lds);
  const float* sm_ls = CB::ls(lds);
  // Thread-distributed result: item (row r, 4 head-dim columns d4).
  auto combined = [&](int r, int d4) {
    const float* col = sm_acc + r * CB::kAccStride + 4 * d4;
    f32x4 a = *reinterpret_cast<const f32x4*>(col);
#pragma unroll
    for (int w = 1; w < NSUM; ++w) a += *reinterpret_cast<const f32x4*>(col + w * CB::kRows * CB::kAccStride);
    return a;
  };

  T* out_s = seq_out<T>(p, s, D);
  if (f.n_parts == 1) {
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
  {
    const int64_t base = f.slot * p.slot_rows + f.parts.row0;
    for (int it = tid; it < wg_rows * (D / 4); it += NT) {
      const int r = it / (D / 4), d4 = it % (D / 4);
      store_coherent(p.ws_acc + (base + r) * D + 4 * d4, combined(r, d4));
    }
    for (int r = tid; r < wg_rows; r += NT) store_coherent2(p.ws_ml + (base + r) * 2, sm_ms[r], sm_ls[r]);
  }
  arrive_and_merge<T, D, NT>(p, reinterpret_cast<int*>(lds + lds_bytes - 16), s, kvh, row0, wg_rows, f);
}

}  // namespace dev
}  // namespace pad
