// Writes new tokens' K and V rows into a quantized ("octave") packed cache
// (pad_octave_cache_write, include/pad_octave.h): rotate, quantize per
// scale group, pack -- the store kernel of do_kv_cache_update on the
// vllm.v1.attention.backends.rocm_octave_attn docs page, with the
// rotation, quantizer and layout this library reads into it (slot layout
// in include/pad_octave.h).
//
// One wave per (token, kv head), four consecutive elements d = 4 lane + i
// per lane: a rotation is the sign flip and a fast Walsh-Hadamard
// transform whose index bits 0-1 are in the lane and bits 2-7 across lanes
// (K in 64-dim blocks: lane bits 0-3 only, unless compact), in fp32; a
// scale group's absmax is a cross-lane maximum; steps are rounded to fp16
// before the codes are taken (code = clamp(floor(x / step)) + 2^(b-1)).
// The slot is assembled in LDS and written with 16-byte stores.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/pad_octave.h"
#include "entry.h"

namespace {

constexpr int kD = 256;
constexpr int kWaves = 4;
constexpr int kMaxSlot = 240;

struct StoreArgs {
  const void* key;
  const void* value;
  const int64_t* slots;
  const uint32_t* k_signs;
  const uint32_t* v_signs;
  unsigned char* cache;
  int64_t token_stride, head_stride, block_stride;  // bytes
  int64_t capacity;                                 // num_blocks * page_size
  int num_tokens, num_kv_heads, page_size, slot_bytes;
  int vbits, kgroups;                               // V code bits, K scale groups (4 or 1)
};

template <typename T>
__device__ __forceinline__ float elem(const void* p, int64_t i) {
  return float(static_cast<const T*>(p)[i]);
}

__device__ __forceinline__ float wht_stage(float v, int lane_xor, bool upper) {
  const float u = __shfl_xor(v, lane_xor);
  return upper ? u - v : v + u;
}

// Rotate the four elements of this lane: x = H (s * x) / sqrt(n) over
// blocks of 2^(2 + lane_bits) elements.
__device__ __forceinline__ void rotate4(float (&x)[4], uint32_t sign_word, int lane, int lane_bits) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if ((sign_word >> ((4 * lane + i) & 31)) & 1u) x[i] = -x[i];
  const float a0 = x[0] + x[1], a1 = x[0] - x[1], a2 = x[2] + x[3], a3 = x[2] - x[3];
  x[0] = a0 + a2;
  x[1] = a1 + a3;
  x[2] = a0 - a2;
  x[3] = a1 - a3;
  for (int o = 1; o < (1 << lane_bits); o <<= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = wht_stage(x[i], o, (lane & o) != 0);
  const float norm = lane_bits == 4 ? 0.125f : 0.0625f;  // 1 / sqrt(64) or 1 / sqrt(256)
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] *= norm;
}

// Codes of this lane's four elements in a scale group spread over
// 2^group_bits lanes; returns the group's fp16 step (as bits).
__device__ __forceinline__ uint32_t quantize4(const float (&x)[4], int bits, int group_bits, uint32_t (&code)[4]) {
  float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
  for (int o = 1; o < (1 << group_bits); o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const int half = 1 << (bits - 1);
  const _Float16 step16 = _Float16(amax / float(half));
  const float step = float(step16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (step > 0.f) {
      const float q = floorf(x[i] / step);
      code[i] = uint32_t(int(fminf(fmaxf(q, float(-half)), float(half - 1))) + half);
    } else {
      code[i] = uint32_t(half);
    }
  }
  return uint32_t(__builtin_bit_cast(uint16_t, step16));
}

// Put this lane's four codes (elements 4 lane .. 4 lane + 3) into the
// slot image in LDS: elements 8 j .. 8 j + 7 (j = lane / 2) form group
// g * 8 + kc (j = 4 kc + g) of `bits` bytes, code e at bits bits * e.
__device__ __forceinline__ void put_codes(unsigned char* img, const uint32_t (&code)[4], int bits, int lane) {
  uint32_t part = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) part |= code[i] << (bits * (4 * (lane & 1) + i));
  const uint32_t word = part | uint32_t(__shfl_xor(int(part), 1));
  if ((lane & 1) == 0) {
    const int j = lane >> 1;
    unsigned char* dst = img + ((j & 3) * 8 + (j >> 2)) * bits;
    for (int b = 0; b < bits; ++b) dst[b] = (unsigned char)(word >> (8 * b));
  }
}

template <typename T>
__global__ __launch_bounds__(kWaves * 64) void octave_store_kernel(StoreArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char img_all[kWaves][kMaxSlot];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int t = blockIdx.x;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.capacity) return;
  const int64_t blk = slot / a.page_size, off = slot % a.page_size;
  unsigned char* img = img_all[wave];
  const uint32_t ksw = a.k_signs[lane >> 3], vsw = a.v_signs[lane >> 3];
  const int kg_bits = a.kgroups == 4 ? 4 : 6;  // lanes per K group: 16 (64 dims) or 64
  for (int h = wave; h < a.num_kv_heads; h += kWaves) {
    const int64_t row = (int64_t(t) * a.num_kv_heads + h) * kD + 4 * lane;
    float k[4], v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k[i] = elem<T>(a.key, row + i);
      v[i] = elem<T>(a.value, row + i);
    }
    rotate4(k, ksw, lane, kg_bits);
    rotate4(v, vsw, lane, 6);
    uint32_t kc[4], vc[4];
    const uint32_t kstep = quantize4(k, 3, kg_bits, kc);
    const uint32_t vstep = quantize4(v, a.vbits, 6, vc);
    // the image: zero, then codes and steps
    for (int i = lane; i < a.slot_bytes; i += 64) img[i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    put_codes(img, kc, 3, lane);
    put_codes(img + 3 * kD / 8, vc, a.vbits, lane);
    const int soff = 3 * kD / 8 + a.vbits * kD / 8;
    uint16_t* steps = reinterpret_cast<uint16_t*>(img + soff);
    if (a.kgroups == 4) {
      if ((lane & 15) == 0) steps[lane >> 4] = uint16_t(kstep);
      if (lane == 0) steps[4] = uint16_t(vstep);
    } else if (lane == 0) {
      steps[0] = uint16_t(kstep);
      steps[1] = uint16_t(vstep);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    unsigned char* dst = a.cache + blk * a.block_stride + off * a.token_stride + int64_t(h) * a.head_stride;
    if (lane < a.slot_bytes / 16)
      *reinterpret_cast<uint4*>(dst + 16 * lane) = *reinterpret_cast<const uint4*>(img + 16 * lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

bool aligned_to(const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

}  // namespace

extern "C" pad_status pad_octave_cache_write(const pad_octave_cache_shape* shape, const void* key, const void* value,
                                             const int64_t* slot_mapping, const uint32_t* k_signs,
                                             const uint32_t* v_signs, void* cache, void* stream) {
  if (!shape) return PAD_EINVAL;
  const pad_octave_cache_shape& sh = *shape;
  if (sh.num_tokens < 0 || sh.num_kv_heads < 1 || sh.page_size < 1 || sh.num_blocks < 1) return PAD_EINVAL;
  if (sh.dtype != PAD_F16 && sh.dtype != PAD_BF16) return PAD_EINVAL;
  if (sh.layout != PAD_NHD && sh.layout != PAD_HND) return PAD_EINVAL;
  if (sh.format < PAD_KV_OCTAVE_K3V4 || sh.format > PAD_KV_OCTAVE_K3V3_COMPACT) return PAD_EINVAL;
  if (sh.head_size != PAD_OCTAVE_HEAD_SIZE) return PAD_EUNSUPPORTED;
  if (sh.num_tokens == 0) return PAD_OK;
  if (!key || !value || !slot_mapping || !k_signs || !v_signs || !cache) return PAD_EINVAL;
  if (!aligned_to(key, 8) || !aligned_to(value, 8) || !aligned_to(slot_mapping, 8) || !aligned_to(k_signs, 4) ||
      !aligned_to(v_signs, 4) || !aligned_to(cache, 16))
    return PAD_EINVAL;
  const int slot_bytes = pad::octave_slot_bytes(sh.format, sh.head_size);
  StoreArgs a{};
  a.key = key;
  a.value = value;
  a.slots = slot_mapping;
  a.k_signs = k_signs;
  a.v_signs = v_signs;
  a.cache = static_cast<unsigned char*>(cache);
  const int64_t P = sh.page_size, H = sh.num_kv_heads, sb = slot_bytes;
  if (sh.layout == PAD_HND) {
    a.token_stride = sb;
    a.head_stride = P * sb;
    a.block_stride = H * P * sb;
  } else {
    a.head_stride = sb;
    a.token_stride = H * sb;
    a.block_stride = P * H * sb;
  }
  a.capacity = int64_t(sh.num_blocks) * P;
  a.num_tokens = sh.num_tokens;
  a.num_kv_heads = sh.num_kv_heads;
  a.page_size = sh.page_size;
  a.slot_bytes = slot_bytes;
  a.vbits = sh.format == PAD_KV_OCTAVE_K3V4 ? 4 : 3;
  a.kgroups = sh.format == PAD_KV_OCTAVE_K3V3_COMPACT ? 1 : 4;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (sh.dtype == PAD_BF16)
    hipLaunchKernelGGL(octave_store_kernel<__bf16>, dim3(unsigned(sh.num_tokens)), dim3(kWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL(octave_store_kernel<_Float16>, dim3(unsigned(sh.num_tokens)), dim3(kWaves * 64), 0, st, a);
  return hipGetLastError() == hipSuccess ? PAD_OK : PAD_EHIP;
}
