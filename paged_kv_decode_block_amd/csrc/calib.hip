// Read-bandwidth calibration kernels (declared in include/pad_calib.h).
//
// The gather kernel walks a decode call's pages the way the attention
// kernel does -- 16-key tiles, whole tiles inside one page, 16-byte loads,
// each wave taking every waves-th tile of its segment -- and only XORs what
// it reads.  Its rate is the ceiling a decode launch over the same pages
// can approach (ROCm/vllm pull request 1330, "Summary": the kernel is
// measured as an HBM stream).  The stream kernel reads one contiguous
// buffer for comparison.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/pad_calib.h"
#include "plan.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kSinkValue = 0x5EEDF00D;

struct GatherArgs {
  const unsigned char* kv;
  const int32_t* table;
  const int32_t* lens;
  int64_t token_stride, head_stride, block_stride;  // bytes
  int max_blocks, page_size, query_len, window, nseg, num_kv_heads;
  int* sink;
};

// CPL = 16-byte chunks per lane per tile: a tile is 16 keys of 4*D bytes
// (K and V rows of D two-byte elements), 4*D chunks over 64 lanes.
template <int NW, int U, int CPL>
__global__ __launch_bounds__(NW * 64) void gather_read_kernel(GatherArgs a) {
  constexpr int kRowChunks = 4 * CPL;  // 16-byte chunks in one key's K+V row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int s = blockIdx.y;
  const int h = blockIdx.x / a.nseg, seg = blockIdx.x % a.nseg;
  const int cap = a.max_blocks * a.page_size;
  int L = a.lens[s];
  L = L < cap ? L : cap;
  if (L <= 0) return;
  int lo = 0;
  if (a.window > 0) {
    lo = L - a.query_len - a.window + 1;
    lo = lo > 0 ? lo : 0;
  }
  const int t0 = lo / 16, t1 = (L + 15) / 16;
  const int per = (t1 - t0 + a.nseg - 1) / a.nseg;
  const int ts = t0 + seg * per;
  const int te = ts + per < t1 ? ts + per : t1;
  const int32_t* row = a.table + int64_t(s) * a.max_blocks;
  const unsigned char* head = a.kv + int64_t(h) * a.head_stride;

  uint32_t off[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int idx = j * 64 + lane;
    off[j] = uint32_t((idx / kRowChunks) * a.token_stride + (idx % kRowChunks) * 16);
  }
  i32x4 acc = {0, 0, 0, 0};
  for (int t = ts + wave; t < te; t += NW * U) {
    i32x4 v[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tt = t + u * NW;
      if (tt < te) {
        const int key0 = tt * 16;
        const int blk = row[key0 / a.page_size];
        const unsigned char* base = head + int64_t(blk) * a.block_stride + int64_t(key0 % a.page_size) * a.token_stride;
#pragma unroll
        for (int j = 0; j < CPL; ++j) v[u][j] = *reinterpret_cast<const i32x4*>(base + off[j]);
      } else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) v[u][j] = i32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < CPL; ++j) acc ^= v[u][j];
  }
  const int x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == kSinkValue) *a.sink = x;
}

// Each workgroup of NT threads reads one contiguous range with U 16-byte
// loads in flight per thread (NT * U * 16 bytes per step).
template <int NT, int U>
__global__ __launch_bounds__(NT) void stream_read_kernel(const i32x4* src, size_t n, int* sink) {
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t begin = size_t(blockIdx.x) * per;
  const size_t end = begin + per < n ? begin + per : n;
  i32x4 acc = {0, 0, 0, 0};
  for (size_t i = begin + threadIdx.x; i < end; i += size_t(U) * NT) {
    i32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const size_t j = i + size_t(k) * NT;
      v[k] = j < end ? src[j] : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k];
  }
  const int x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == kSinkValue) *sink = x;
}

template <int NT>
int launch_stream(int loads, const i32x4* src, size_t n, unsigned blocks, int* sink, hipStream_t st) {
  switch (loads) {
    case 4: hipLaunchKernelGGL((stream_read_kernel<NT, 4>), dim3(blocks), dim3(NT), 0, st, src, n, sink); return 0;
    case 8: hipLaunchKernelGGL((stream_read_kernel<NT, 8>), dim3(blocks), dim3(NT), 0, st, src, n, sink); return 0;
    case 16: hipLaunchKernelGGL((stream_read_kernel<NT, 16>), dim3(blocks), dim3(NT), 0, st, src, n, sink); return 0;
  }
  return -1;
}

template <int NW, int U, int CPL>
void launch_gather(const GatherArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((gather_read_kernel<NW, U, CPL>), grid, dim3(NW * 64), 0, st, a);
}

template <int NW, int U>
int launch_gather_d(int head_size, const GatherArgs& a, dim3 grid, hipStream_t st) {
  switch (head_size) {
    case 64: launch_gather<NW, U, 4>(a, grid, st); return 0;
    case 128: launch_gather<NW, U, 8>(a, grid, st); return 0;
    case 256: launch_gather<NW, U, 16>(a, grid, st); return 0;
    case 512:
      if constexpr (U == 1) {
        launch_gather<NW, 1, 32>(a, grid, st);
        return 0;
      }
      return -1;
  }
  return -1;
}

bool aligned(const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

}  // namespace

extern "C" {

pad_status pad_calib_gather_read(const pad_shape* shape, const void* kv_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t window, int32_t waves,
                                 int32_t tiles_in_flight, int32_t segments, int32_t* sink, void* stream) {
  if (!shape) return PAD_EINVAL;
  pad_shape sh = *shape;
  sh.path = PAD_PATH_AUTO;
  sh.num_segments = 0;
  sh.schedule = PAD_SCHED_AUTO;
  pad::Plan p;
  const pad_status st = pad::make_plan(sh, window, 256, &p);  // validates the shape fields and window
  if (st != PAD_OK) return st;
  if (waves != 4 && waves != 8) return PAD_EINVAL;
  if (tiles_in_flight != 1 && tiles_in_flight != 2) return PAD_EINVAL;
  if (tiles_in_flight == 2 && sh.head_size == 512) return PAD_EUNSUPPORTED;
  if (segments < 1 || segments > pad::kMaxSegments) return PAD_EINVAL;
  if (sh.num_seqs == 0) return PAD_OK;
  if (!kv_cache || !block_table || !seq_lens || !sink || !aligned(kv_cache, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(sink, 4))
    return PAD_EINVAL;
  if (int64_t(sh.num_kv_heads) * segments > 0x7fffffff || sh.num_seqs > 65535) return PAD_EUNSUPPORTED;

  const int64_t D = sh.head_size, P = sh.page_size, H = sh.num_kv_heads, eb = 2;
  GatherArgs a{};
  a.kv = static_cast<const unsigned char*>(kv_cache);
  a.table = block_table;
  a.lens = seq_lens;
  if (sh.layout == PAD_HND) {
    a.token_stride = 2 * D * eb;
    a.head_stride = P * 2 * D * eb;
    a.block_stride = H * P * 2 * D * eb;
  } else {
    a.head_stride = 2 * D * eb;
    a.token_stride = H * 2 * D * eb;
    a.block_stride = P * H * 2 * D * eb;
  }
  a.max_blocks = sh.max_blocks_per_seq;
  a.page_size = sh.page_size;
  a.query_len = sh.query_len;
  a.window = window;
  a.nseg = segments;
  a.num_kv_heads = sh.num_kv_heads;
  a.sink = sink;
  const dim3 grid(unsigned(sh.num_kv_heads * segments), unsigned(sh.num_seqs));
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  int rc;
  if (waves == 4)
    rc = tiles_in_flight == 1 ? launch_gather_d<4, 1>(sh.head_size, a, grid, hs)
                              : launch_gather_d<4, 2>(sh.head_size, a, grid, hs);
  else
    rc = tiles_in_flight == 1 ? launch_gather_d<8, 1>(sh.head_size, a, grid, hs)
                              : launch_gather_d<8, 2>(sh.head_size, a, grid, hs);
  if (rc != 0) return PAD_EUNSUPPORTED;
  return hipGetLastError() == hipSuccess ? PAD_OK : PAD_EHIP;
}

pad_status pad_calib_stream_read(const void* src, size_t bytes, int32_t blocks, int32_t threads,
                                 int32_t loads_in_flight, int32_t* sink, void* stream) {
  if (threads != 256 && threads != 512 && threads != 1024) return PAD_EINVAL;
  if (loads_in_flight != 4 && loads_in_flight != 8 && loads_in_flight != 16) return PAD_EINVAL;
  if (blocks < 1 || blocks > 65536) return PAD_EINVAL;
  if (bytes == 0) return PAD_OK;
  if (!src || !sink || !aligned(src, 16) || !aligned(sink, 4) || bytes % 16 != 0) return PAD_EINVAL;
  const i32x4* s = static_cast<const i32x4*>(src);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const unsigned g = unsigned(blocks);
  const int rc = threads == 256   ? launch_stream<256>(loads_in_flight, s, bytes / 16, g, sink, hs)
                 : threads == 512 ? launch_stream<512>(loads_in_flight, s, bytes / 16, g, sink, hs)
                                  : launch_stream<1024>(loads_in_flight, s, bytes / 16, g, sink, hs);
  if (rc != 0) return PAD_EINVAL;
  return hipGetLastError() == hipSuccess ? PAD_OK : PAD_EHIP;
}

}  // extern "C"
