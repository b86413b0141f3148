// Device helpers of the quantized ("octave") packed cache for the decode
// kernel at head size 256: slot geometry, code unpacking into MFMA
// operands and the Walsh-Hadamard rotations (vllm.v1.attention.backends.
// rocm_octave_attn docs page: formats octave_k3v4 / octave_k3v3 /
// octave_k3v3_compact, sign bits for K and V, queries and keys rotated with
// the K signs -- in 64-dim blocks unless compact -- and the output rotated
// back with the V signs).
//
// Slot of one (token, kv head), bytes: K codes (3 bits x 256 = 96), V codes
// (32 x VB), K steps (fp16, one per 64-dim block or one when compact), V step
// (fp16), zero pad to 16.  Codes go in groups of 8 packed into B bytes,
// little-endian, code e of a group at bits B e; element d = 32 kc + 8 g + e
// is code e of group g * 8 + kc, so the 16 lanes of MFMA lane group g (the
// lanes that hold elements 32 kc + 8 g .. + 7 of every chunk kc) read the
// lane-group's own 3 (K) or VB (V) bytes per chunk, 24 or 8 VB contiguous
// bytes.  A code c is used as the fp16 operand whose bits are c, the exact
// subnormal c * 2^-24: the products run on codes, and 2^24, the steps and
// the offset of the level (c - 2^(B-1) + 1/2) * step are applied
// afterwards.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/pad_octave.h"

namespace pad {
namespace dev {

constexpr int kOctD = 256;  // head size of the packed formats
// Packed tiles in flight per wave beyond the one being computed.
constexpr int kOctRing = 1;

template <int FMT>
struct Oct;
template <>
struct Oct<0> {  // an fp16/bf16 cache: no codes, one (unused) K group
  static constexpr int KB = 0, VB = 0, KG = 1;
};
template <>
struct Oct<PAD_KV_OCTAVE_K3V4> {
  static constexpr int KB = 3, VB = 4, KG = 4;  // bits of K and V codes, K scale groups
};
template <>
struct Oct<PAD_KV_OCTAVE_K3V3> {
  static constexpr int KB = 3, VB = 3, KG = 4;
};
template <>
struct Oct<PAD_KV_OCTAVE_K3V3_COMPACT> {
  static constexpr int KB = 3, VB = 3, KG = 1;
};

template <int FMT>
struct OctSlot {
  static constexpr int kVOff = 3 * kOctD / 8;                         // V codes
  static constexpr int kSOff = kVOff + Oct<FMT>::VB * kOctD / 8;      // steps (16-byte aligned)
  static constexpr int kKBytesPerGroup = 3 * kOctD / 32;              // 24: one lane group's K codes
  static constexpr int kVBytesPerGroup = Oct<FMT>::VB * kOctD / 32;   // 32 or 24
};

// One lane's share of a 16-key tile: its key's K and V codes for its lane
// group, and the key's 16-byte step area.
struct OctTile {
  uint32_t k[6];
  uint32_t v[8];
  uint32_t sc[4];
};

// 32 bits of a little-endian bit string held in N dwords, from bit `lo`
// on (only the bits that exist are meaningful; `lo` folds to a constant in
// the unrolled callers).
template <int N>
__device__ __forceinline__ uint32_t bits_window(const uint32_t (&w)[N], int lo) {
  const int i = lo >> 5, sh = lo & 31;
  return __builtin_amdgcn_alignbit(w[i + 1 < N ? i + 1 : N - 1], w[i], uint32_t(sh));
}

// Eight B-bit codes (code e at bits B e of x) as an fp16 MFMA operand:
// four dwords of two 16-bit values each whose bits are the code, i.e. the
// fp16 subnormal c * 2^-24 (exact; the products scale back by 2^24).
template <int B>
__device__ __forceinline__ i32x4 codes8(uint32_t x) {
  i32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = int(__builtin_amdgcn_ubfe(x, 2 * q * B, B) | (__builtin_amdgcn_ubfe(x, (2 * q + 1) * B, B) << 16));
  return r;
}

// The same for eight 4-bit codes: the even codes' nibbles and the odd
// codes' nibbles as bytes, interleaved with zero bytes by byte permutes.
__device__ __forceinline__ i32x4 codes8_nibbles(uint32_t x) {
  const uint32_t ev = x & 0x0f0f0f0fu, od = (x >> 4) & 0x0f0f0f0fu;
  i32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q)  // bytes: even code q, 0, odd code q, 0
    r[q] = int(__builtin_amdgcn_perm(od, ev, 0x0c040c00u + 0x00010001u * uint32_t(q)));
  return r;
}

// An fp16 MFMA operand of four ones.
constexpr uint64_t kOnes4 = 0x3c003c003c003c00ull;
// Scale of the products of subnormal code operands.
constexpr float kCodeScale = 16777216.f;  // 2^24

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return float(__builtin_bit_cast(_Float16, uint16_t(h & 0xffffu)));
}

// The two 16-bit halves of a dword of the element type as fp32.
template <typename T>
struct OctType;
template <>
struct OctType<__bf16> {
  static __device__ __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
};
template <>
struct OctType<_Float16> {
  static __device__ __forceinline__ float lo(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w))); }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16)));
  }
};

// One butterfly stage of the Walsh-Hadamard transform across lanes: the
// partner of this lane holds the element whose index differs in the bit
// that lane bit `lane_bit` stands for; the lane with that bit set keeps the
// difference (partner - own), the other the sum.
__device__ __forceinline__ float wht_lane_stage(float v, int lane_xor, bool upper) {
  const float u = __shfl_xor(v, lane_xor);
  return upper ? u - v : v + u;
}

}  // namespace dev
}  // namespace pad
