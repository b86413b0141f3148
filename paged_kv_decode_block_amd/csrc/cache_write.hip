// KV-cache write with an optional rotary embedding (declared in
// include/pad_cache.h): the step before decode attention, storing each new
// token's K (rotated) and V into its packed K+V cache slot and rotating the
// query rows in place (vllm.v1.attention.backends.rocm_octave_attn docs
// page: `do_kv_cache_update` stores key/value at `slot_mapping`;
// `customize_spec`: one packed K+V slot per token and kv head).
//
// One workgroup per token; a thread owns 16-byte chunks (eight elements)
// of the token's head rows.  A rotated pair (i, i + rope_dim / 2) lies in
// two chunks half the rotary width apart, and the thread owning the first
// computes and stores both, so every element is read and written once.
// The work is a stream of 16-byte loads and stores: HBM-bound.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/pad_cache.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Cvt;
template <>
struct Cvt<__bf16> {
  static __device__ __forceinline__ float f(uint32_t b) { return __builtin_bit_cast(float, b << 16); }
  static __device__ __forceinline__ uint32_t b(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }
};
template <>
struct Cvt<_Float16> {
  static __device__ __forceinline__ float f(uint32_t b) { return float(__builtin_bit_cast(_Float16, uint16_t(b))); }
  static __device__ __forceinline__ uint32_t b(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
};

struct WriteArgs {
  unsigned char* q;            // [T, Hq, D] or null
  const unsigned char* key;    // [T, Hkv, D]
  const unsigned char* value;  // [T, Hkv, D]
  const int64_t* slots;        // [T]
  const int64_t* positions;    // [T] (rotation only)
  const float* cos_sin;        // [max_pos, rope_dim] (rotation only)
  unsigned char* kv;           // packed cache
  int64_t token_stride, head_stride, block_stride;  // bytes
  int64_t capacity;            // num_blocks * page_size slots
  int num_q_heads, num_kv_heads, page_size, rope_dim, max_pos;
};

// Element e of a chunk (eight 16-bit values in four 32-bit words).
__device__ __forceinline__ uint32_t elem(const i32x4& v, int e) { return (uint32_t(v[e >> 1]) >> (16 * (e & 1))) & 0xffffu; }

// Rotate the pair of chunks (lo: elements 8c.., hi: 8c + rope_dim/2 ..)
// with the cos/sin of this position.
template <typename T>
__device__ __forceinline__ void rotate(i32x4& lo, i32x4& hi, const float* cs, int c, int half) {
  i32x4 ol, oh;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t wl = 0, wh = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = 2 * w + k;
      const float x1 = Cvt<T>::f(elem(lo, e)), x2 = Cvt<T>::f(elem(hi, e));
      const float co = cs[8 * c + e], si = cs[half + 8 * c + e];
      wl |= Cvt<T>::b(x1 * co - x2 * si) << (16 * k);
      wh |= Cvt<T>::b(x2 * co + x1 * si) << (16 * k);
    }
    ol[w] = int(wl);
    oh[w] = int(wh);
  }
  lo = ol;
  hi = oh;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void cache_write_kernel(WriteArgs a) {
  constexpr int CH = D / 8;  // 16-byte chunks per head row
  const int t = blockIdx.x;
  const int64_t slot = a.slots[t];
  const bool store = slot >= 0 && slot < a.capacity;
  const int half = a.rope_dim / 2;  // elements
  const int rot = a.rope_dim / 8;   // rotated chunks (pairs: rot / 2)
  const float* cs = nullptr;
  if (a.rope_dim > 0) {
    int64_t p = a.positions[t];
    p = p < 0 ? 0 : (p >= a.max_pos ? a.max_pos - 1 : p);
    cs = a.cos_sin + p * a.rope_dim;
  }
  const int64_t blk = store ? slot / a.page_size : 0, off = store ? slot % a.page_size : 0;
  unsigned char* dst_tok = a.kv + blk * a.block_stride + off * a.token_stride;

  // K and V of every kv head.
  if (store) {
    for (int w = threadIdx.x; w < a.num_kv_heads * CH; w += 256) {
      const int h = w / CH, c = w % CH;
      const int64_t src = (int64_t(t) * a.num_kv_heads + h) * D * 2 + c * 16;
      unsigned char* dst = dst_tok + h * a.head_stride;
      *reinterpret_cast<i32x4*>(dst + 2 * D + c * 16) = *reinterpret_cast<const i32x4*>(a.value + src);
      if (c < rot / 2) {
        i32x4 lo = *reinterpret_cast<const i32x4*>(a.key + src);
        i32x4 hi = *reinterpret_cast<const i32x4*>(a.key + src + 2 * half);
        rotate<T>(lo, hi, cs, c, half);
        *reinterpret_cast<i32x4*>(dst + c * 16) = lo;
        *reinterpret_cast<i32x4*>(dst + c * 16 + 2 * half) = hi;
      } else if (c >= rot) {
        *reinterpret_cast<i32x4*>(dst + c * 16) = *reinterpret_cast<const i32x4*>(a.key + src);
      }
    }
  }
  // The query rows, in place (only the rotated pairs change).
  if (a.q != nullptr && rot > 0) {
    for (int w = threadIdx.x; w < a.num_q_heads * (rot / 2); w += 256) {
      const int h = w / (rot / 2), c = w % (rot / 2);
      unsigned char* row = a.q + (int64_t(t) * a.num_q_heads + h) * D * 2 + c * 16;
      i32x4 lo = *reinterpret_cast<const i32x4*>(row);
      i32x4 hi = *reinterpret_cast<const i32x4*>(row + 2 * half);
      rotate<T>(lo, hi, cs, c, half);
      *reinterpret_cast<i32x4*>(row) = lo;
      *reinterpret_cast<i32x4*>(row + 2 * half) = hi;
    }
  }
}

template <typename T>
int launch_t(int head_size, const WriteArgs& a, int tokens, hipStream_t st) {
  switch (head_size) {
    case 64: hipLaunchKernelGGL((cache_write_kernel<T, 64>), dim3(tokens), dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL((cache_write_kernel<T, 128>), dim3(tokens), dim3(256), 0, st, a); break;
    case 256: hipLaunchKernelGGL((cache_write_kernel<T, 256>), dim3(tokens), dim3(256), 0, st, a); break;
    case 512: hipLaunchKernelGGL((cache_write_kernel<T, 512>), dim3(tokens), dim3(256), 0, st, a); break;
    default: return -1;
  }
  return 0;
}

bool aligned(const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

}  // namespace

extern "C" pad_status pad_rope_cache_write(const pad_cache_shape* shape, void* q, const void* key,
                                           const void* value, const int64_t* slot_mapping, const int64_t* positions,
                                           const float* cos_sin_cache, void* kv_cache, void* stream) {
  if (!shape) return PAD_EINVAL;
  const pad_cache_shape& sh = *shape;
  if (sh.num_tokens < 0 || sh.num_kv_heads < 1 || sh.page_size < 1 || sh.num_blocks < 1 || sh.rope_dim < 0)
    return PAD_EINVAL;
  if (sh.dtype != PAD_F16 && sh.dtype != PAD_BF16) return PAD_EINVAL;
  if (sh.layout != PAD_NHD && sh.layout != PAD_HND) return PAD_EINVAL;
  if (sh.head_size != 64 && sh.head_size != 128 && sh.head_size != 256 && sh.head_size != 512)
    return PAD_EUNSUPPORTED;
  if (sh.rope_dim % 16 != 0 || sh.rope_dim > sh.head_size) return PAD_EUNSUPPORTED;
  if (q && (sh.num_q_heads < 1 || sh.num_q_heads % sh.num_kv_heads != 0)) return PAD_EINVAL;
  if (sh.rope_dim > 0 && sh.max_position < 1) return PAD_EINVAL;
  if (sh.num_tokens == 0) return PAD_OK;
  if (!key || !value || !slot_mapping || !kv_cache) return PAD_EINVAL;
  if (sh.rope_dim > 0 && (!positions || !cos_sin_cache)) return PAD_EINVAL;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(kv_cache, 16) || (q && !aligned(q, 16)) ||
      !aligned(slot_mapping, 8) || (positions && !aligned(positions, 8)) || (cos_sin_cache && !aligned(cos_sin_cache, 4)))
    return PAD_EINVAL;

  const int64_t D = sh.head_size, P = sh.page_size, H = sh.num_kv_heads, eb = 2;
  WriteArgs a{};
  a.q = static_cast<unsigned char*>(q);
  a.key = static_cast<const unsigned char*>(key);
  a.value = static_cast<const unsigned char*>(value);
  a.slots = slot_mapping;
  a.positions = positions;
  a.cos_sin = cos_sin_cache;
  a.kv = static_cast<unsigned char*>(kv_cache);
  if (sh.layout == PAD_HND) {
    a.token_stride = 2 * D * eb;
    a.head_stride = P * 2 * D * eb;
    a.block_stride = H * P * 2 * D * eb;
  } else {
    a.head_stride = 2 * D * eb;
    a.token_stride = H * 2 * D * eb;
    a.block_stride = P * H * 2 * D * eb;
  }
  a.capacity = int64_t(sh.num_blocks) * P;
  a.num_q_heads = q ? sh.num_q_heads : 0;
  a.num_kv_heads = sh.num_kv_heads;
  a.page_size = sh.page_size;
  a.rope_dim = sh.rope_dim;
  a.max_pos = sh.max_position;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int rc = sh.dtype == PAD_BF16 ? launch_t<__bf16>(sh.head_size, a, sh.num_tokens, st)
                                      : launch_t<_Float16>(sh.head_size, a, sh.num_tokens, st);
  if (rc != 0) return PAD_EUNSUPPORTED;
  return hipGetLastError() == hipSuccess ? PAD_OK : PAD_EHIP;
}
