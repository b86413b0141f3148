// extern "C" entry points of libpad_attn.so (declared in include/pad_attn.h).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/pad_attn.h"
#include "entry.h"
#include "kernels.h"
#include "plan.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

namespace pad {

// Compute units of the current device (cached per device); 256 when no
// device can be queried.
int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= int(cache.size())) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

}  // namespace pad

namespace {

using pad::device_cus;

// Helpers' bound on waiting for the last segment, in ticks of the 100 MHz
// device real-time counter (see pad_set_merge_wait).
std::atomic<uint32_t> g_merge_wait_ticks{200 * 100};

}  // namespace

extern "C" {

pad_status pad_set_merge_wait(int32_t microseconds) {
  if (microseconds < 0 || microseconds > 1000000) return PAD_EINVAL;
  g_merge_wait_ticks.store(uint32_t(microseconds) * 100u);
  return PAD_OK;
}

int32_t pad_abi_version(void) { return PAD_ABI_VERSION; }

const char* pad_status_string(pad_status status) {
  switch (status) {
    case PAD_OK: return "ok";
    case PAD_EINVAL: return "invalid argument";
    case PAD_EUNSUPPORTED: return "unsupported shape";
    case PAD_EWORKSPACE: return "workspace missing, misaligned or too small";
    case PAD_EHIP: return "HIP runtime error";
    case PAD_ESCRATCH: return "the call needs more workspace than the library's fixed device array holds";
  }
  return "unknown status";
}

pad_status pad_decode_attn_plan(const pad_shape* shape, int32_t window, int32_t num_cus, pad_plan* plan) {
  if (!shape || !plan) return PAD_EINVAL;
  pad::Plan p;
  const pad_status st = pad::make_plan(*shape, window, num_cus, &p);
  if (st != PAD_OK) return st;
  plan->path = p.path;
  plan->rows = p.rows;
  plan->row_tiles = p.row_tiles;
  plan->row_groups = p.row_groups;
  plan->waves = p.waves;
  plan->num_segments = p.nseg;
  plan->segment_tiles = p.seg_tiles;
  plan->grid_x = p.grid_x;
  plan->grid_y = p.grid_y;
  plan->merge_slices = p.merge_slices;
  plan->persistent = p.persistent;
  plan->workspace_segments = p.ws_nseg;
  plan->workspace_bytes = p.ws_bytes;
  return PAD_OK;
}

pad_status pad_decode_attn_workspace_size(const pad_shape* shape, size_t* bytes) {
  if (!shape || !bytes) return PAD_EINVAL;
  pad::Plan p;
  // The planner sizes the workspace for a segment bound that does not
  // depend on the window, so any window's plan gives the same bytes.
  const pad_status st = pad::make_plan(*shape, 0, device_cus(), &p);
  if (st != PAD_OK) return st;
  *bytes = p.ws_bytes;
  return PAD_OK;
}

pad_status pad_decode_attn_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (bytes == 0) return PAD_OK;
  if (!workspace || !aligned(workspace, 256) || bytes % 4 != 0) return PAD_EINVAL;
  return pad::launch_zero(workspace, bytes / 4, stream) == 0 ? PAD_OK : PAD_EHIP;
}

}  // extern "C"

namespace pad {

pad_status check_buffers(const pad_shape* shape, const void* q, const void* kv_cache, const int32_t* block_table,
                         const int32_t* seq_lens, float scale, const void* out) {
  if (!std::isfinite(scale)) return PAD_EINVAL;
  if (shape->num_seqs == 0) return PAD_OK;
  if (!q || !kv_cache || !block_table || !seq_lens || !out) return PAD_EINVAL;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4))
    return PAD_EINVAL;
  return PAD_OK;
}

// One decode launch; q_start is null for the uniform [S, M, Hq, D] layout.
pad_status decode(const pad_shape* shape, const void* q, const int32_t* q_start, const void* kv_cache,
                  const int32_t* block_table, const int32_t* seq_lens, float scale, int32_t window, void* out,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape) return PAD_EINVAL;
  pad::Plan p;
  const pad_status st = pad::make_plan(*shape, window, device_cus(), &p);
  if (st != PAD_OK) return st;
  const pad_status vb = check_buffers(shape, q, kv_cache, block_table, seq_lens, scale, out);
  if (vb != PAD_OK) return vb;
  if (shape->num_seqs == 0) return PAD_OK;
  if (p.ws_bytes > 0 && (!workspace || !aligned(workspace, 256) || workspace_bytes < p.ws_bytes))
    return PAD_EWORKSPACE;

  const int64_t D = shape->head_size, P = shape->page_size, H = shape->num_kv_heads;
  pad::Params pr{};
  pr.q = q;
  pr.q_start = q_start;
  pr.kv = kv_cache;
  pr.block_table = block_table;
  pr.seq_lens = seq_lens;
  pr.out = out;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  pr.ws_cnt = p.ws_bytes ? reinterpret_cast<int32_t*>(ws + p.ws_counters) : nullptr;
  pr.ws_ml = p.ws_bytes ? reinterpret_cast<float*>(ws + p.ws_ml) : nullptr;
  pr.ws_acc = p.ws_bytes ? reinterpret_cast<float*>(ws + p.ws_acc) : nullptr;
  if (shape->layout == PAD_HND) {
    pr.token_stride = 2 * D;
    pr.head_stride = P * 2 * D;
    pr.block_stride = H * P * 2 * D;
  } else {
    pr.head_stride = 2 * D;
    pr.token_stride = H * 2 * D;
    pr.block_stride = P * H * 2 * D;
  }
  pr.num_seqs = shape->num_seqs;
  pr.query_len = shape->query_len;
  pr.num_q_heads = shape->num_q_heads;
  pr.num_kv_heads = shape->num_kv_heads;
  pr.group = shape->num_q_heads / shape->num_kv_heads;
  pr.page_size = shape->page_size;
  pr.max_blocks = shape->max_blocks_per_seq;
  pr.rows = p.rows;
  pr.window = window;
  pr.nseg = p.nseg;
  pr.seg_tiles = p.seg_tiles;
  pr.row_groups = p.row_groups;
  pr.group_rows = p.path == PAD_PATH_DOT ? p.rows : p.row_tiles * 16;
  pr.merge_slices = p.merge_slices;
  pr.slot_rows = p.slot_rows;
  pr.persistent = p.persistent;
  pr.merge_wait_ticks = g_merge_wait_ticks.load();
  pr.scale_log2 = float(double(scale) * 1.4426950408889634);  // log2(e)
  return pad::launch_decode(p, pr, shape->dtype, shape->head_size, stream) == 0 ? PAD_OK : PAD_EHIP;
}

}  // namespace pad

using pad::decode;

extern "C" {

pad_status pad_decode_attn(const pad_shape* shape, const void* q, const void* kv_cache,
                           const int32_t* block_table, const int32_t* seq_lens, float scale,
                           int32_t window, void* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return decode(shape, q, nullptr, kv_cache, block_table, seq_lens, scale, window, out, workspace,
                workspace_bytes, stream);
}

pad_status pad_decode_attn_varlen(const pad_shape* shape, const void* q, const int32_t* q_start,
                                  const void* kv_cache, const int32_t* block_table, const int32_t* seq_lens,
                                  float scale, int32_t window, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (shape && shape->num_seqs > 0 && (!q_start || !aligned(q_start, 4))) return PAD_EINVAL;
  return decode(shape, q, q_start, kv_cache, block_table, seq_lens, scale, window, out, workspace,
                workspace_bytes, stream);
}

}  // extern "C"
