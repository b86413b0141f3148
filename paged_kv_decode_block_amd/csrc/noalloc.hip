// pad_decode_attn_noalloc: the decode of pad_decode_attn with its
// workspace in a fixed device array of the library instead of a
// caller-supplied buffer, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Declared in include/pad_attn.h.
//
// The array is a file-scope __device__ variable: each GPU the library runs
// on holds its own copy (kNoallocScratchBytes) until the process ends.  Its
// name is a host-side stand-in in this file, not a device address: the
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is
// passed to kernels.  The array's first kCounterBytes hold the split-KV
// control words and the persistent grid's queue, which must start at zero:
// the first call on a device enqueues a fill kernel over them on the
// caller's stream (a kernel, not a memset node, so a captured graph that
// holds it replays correctly); every decode leaves them zero again.  The
// partial area needs no initial value (every slot is written before the
// merge reads it).  Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/pad_attn.h"
#include "entry.h"
#include "kernels.h"
#include "plan.h"

namespace {

// PAD_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU: the control prefix plus the
// split partials of every benchmark workload (the largest, 64 bf16
// sequences of up to 16384 keys with 32 query rows per kv head of size 256,
// needs about 27 MB).
constexpr size_t kNoallocScratchBytes = PAD_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocScratchBytes > pad::kCounterBytes, "the array holds the control prefix");

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

struct DeviceScratch {
  void* ptr = nullptr;  // device address of this GPU's copy of `scratch`
  bool zeroed = false;  // control prefix cleared by a fill that has run eagerly
};

std::mutex g_mu;
std::vector<DeviceScratch> g_dev;

// This device's copy of the array, looked up on the first call with the
// device current; its control prefix is cleared on `stream` until a fill
// has been enqueued outside graph capture.
pad_status device_scratch(void* stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PAD_EHIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (dev >= int(g_dev.size())) g_dev.resize(size_t(dev) + 1);
  DeviceScratch& d = g_dev[size_t(dev)];
  if (d.ptr == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PAD_EHIP;
    d.ptr = p;
  }
  if (!d.zeroed) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap) != hipSuccess) return PAD_EHIP;
    if (pad::launch_zero(d.ptr, pad::kCounterBytes / 4, stream) != 0) return PAD_EHIP;
    // A fill recorded into a graph runs only when the graph does; the next
    // eager call clears the prefix again.
    if (cap == hipStreamCaptureStatusNone) d.zeroed = true;
  }
  *out = d.ptr;
  return PAD_OK;
}

}  // namespace

extern "C" {

pad_status pad_decode_attn_noalloc(const pad_shape* shape, const void* q, const void* kv_cache,
                                   const int32_t* block_table, const int32_t* seq_lens, float scale,
                                   int32_t window, void* out, void* stream) {
  if (!shape) return PAD_EINVAL;
  pad::Plan p;
  const pad_status st = pad::make_plan(*shape, window, pad::device_cus(), &p);
  if (st != PAD_OK) return st;
  if (p.ws_bytes > kNoallocScratchBytes) return PAD_ESCRATCH;
  // Every host-visible check passes before anything is enqueued.
  const pad_status vb = pad::check_buffers(shape, q, kv_cache, block_table, seq_lens, scale, out);
  if (vb != PAD_OK) return vb;
  if (shape->num_seqs == 0) return PAD_OK;
  void* ws = nullptr;
  if (p.ws_bytes > 0) {
    const pad_status ss = device_scratch(stream, &ws);
    if (ss != PAD_OK) return ss;
  }
  return pad::decode(shape, q, nullptr, kv_cache, block_table, seq_lens, scale, window, out, ws,
                     p.ws_bytes > 0 ? kNoallocScratchBytes : 0, stream);
}

}  // extern "C"
