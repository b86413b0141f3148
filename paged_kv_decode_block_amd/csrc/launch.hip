// Launch dispatch of the decode kernels by head size (each head size's
// kernels live in their own build of decode_mfma.hip), and the workspace
// fill: the split-KV control words start at zero once per workspace, and
// every decode launch leaves them zero.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace pad {
namespace {

__global__ void zero_kernel(uint32_t* p, size_t n) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

}  // namespace

int launch_zero(void* ptr, size_t words, void* stream) {
  if (words == 0) return 0;
  const size_t blocks = (words + 255) / 256;
  const unsigned grid = unsigned(blocks < 1024 ? blocks : 1024);
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(ptr), words);
  return int(hipGetLastError());
}

// The decode kernels of each head size live in their own build of
// decode_mfma.hip.
int launch_decode(const Plan& plan, const Params& params, int dtype, int head_size, void* stream) {
  if (plan.path == PAD_PATH_PREFILL) return launch_prefill(plan, params, dtype, head_size, stream);
  switch (head_size) {
    case 64: return launch_decode_hs<64>(plan, params, dtype, stream);
    case 128: return launch_decode_hs<128>(plan, params, dtype, stream);
    case 256: return launch_decode_hs<256>(plan, params, dtype, stream);
    case 512: return launch_decode_hs<512>(plan, params, dtype, stream);
  }
  return int(hipErrorInvalidValue);
}

}  // namespace pad
