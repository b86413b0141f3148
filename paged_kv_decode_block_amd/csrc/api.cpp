// extern "C" entry points of libpad_attn.so (declared in include/pad_attn.h).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/pad_attn.h"
#include "../../include/pad_octave.h"
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
int octave_slot_bytes(int format, int head_size) {
  if (head_size != 256) return 0;
  switch (format) {
    case PAD_KV_OCTAVE_K3V4: return 240;                // 96 + 128 + 10 -> 240
    case PAD_KV_OCTAVE_K3V3:                            // 96 + 96 + 10 -> 208
    case PAD_KV_OCTAVE_K3V3_COMPACT: return 208;        // 96 + 96 + 4 -> 208
  }
  return 0;
}

pad_status decode(const pad_shape* shape, const void* q, const int32_t* q_start, const void* kv_cache,
                  const int32_t* block_table, const int32_t* seq_lens, float scale, int32_t window, void* out,
                  void* workspace, size_t workspace_bytes, void* stream, int format, const uint32_t* k_signs,
                  const uint32_t* v_signs) {
  if (!shape) return PAD_EINVAL;
  int key_bytes = 0;
  if (format != 0) {
    if (format < PAD_KV_OCTAVE_K3V4 || format > PAD_KV_OCTAVE_K3V3_COMPACT) return PAD_EINVAL;
    if (shape->head_size != PAD_OCTAVE_HEAD_SIZE || shape->path == PAD_PATH_DOT) return PAD_EUNSUPPORTED;
    key_bytes = octave_slot_bytes(format, shape->head_size);
  }
  pad::Plan p;
  const pad_status st = pad::make_plan(*shape, window, device_cus(), &p, key_bytes);
  if (st != PAD_OK) return st;
  if (format != 0 && shape->num_seqs > 0 &&
      (!k_signs || !v_signs || !aligned(k_signs, 4) || !aligned(v_signs, 4)))
    return PAD_EINVAL;
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
  // Strides in 16-bit elements: a slot is 2 D elements, or the packed
  // slot's bytes / 2.
  const int64_t slot = format ? key_bytes / 2 : 2 * D;
  if (shape->layout == PAD_HND) {
    pr.token_stride = slot;
    pr.head_stride = P * slot;
    pr.block_stride = H * P * slot;
  } else {
    pr.head_stride = slot;
    pr.token_stride = H * slot;
    pr.block_stride = P * H * slot;
  }
  pr.k_signs = k_signs;
  pr.v_signs = v_signs;
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
  pr.unit_lead = p.unit_lead;
  pr.merge_wait_ticks = g_merge_wait_ticks.load();
  pr.scale_log2 = float(double(scale) * 1.4426950408889634);  // log2(e)
  const int rc = format ? pad::launch_decode_octave(p, pr, shape->dtype, format, stream)
                        : pad::launch_decode(p, pr, shape->dtype, shape->head_size, stream);
  return rc == 0 ? PAD_OK : PAD_EHIP;
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

extern "C" {

pad_status pad_octave_slot_bytes(int32_t format, int32_t head_size, int32_t* bytes) {
  if (!bytes) return PAD_EINVAL;
  if (format < PAD_KV_OCTAVE_K3V4 || format > PAD_KV_OCTAVE_K3V3_COMPACT) return PAD_EINVAL;
  const int b = pad::octave_slot_bytes(format, head_size);
  if (b == 0) return PAD_EUNSUPPORTED;
  *bytes = b;
  return PAD_OK;
}

pad_status pad_decode_attn_octave_workspace_size(const pad_shape* shape, int32_t format, size_t* bytes) {
  if (!shape || !bytes) return PAD_EINVAL;
  if (format < PAD_KV_OCTAVE_K3V4 || format > PAD_KV_OCTAVE_K3V3_COMPACT) return PAD_EINVAL;
  if (shape->head_size != PAD_OCTAVE_HEAD_SIZE || shape->path == PAD_PATH_DOT) return PAD_EUNSUPPORTED;
  pad::Plan p;
  const pad_status st = pad::make_plan(*shape, 0, device_cus(), &p, pad::octave_slot_bytes(format, shape->head_size));
  if (st != PAD_OK) return st;
  *bytes = p.ws_bytes;
  return PAD_OK;
}

pad_status pad_decode_attn_octave(const pad_shape* shape, int32_t format, const void* q, const void* cache,
                                  const int32_t* block_table, const int32_t* seq_lens, const uint32_t* k_signs,
                                  const uint32_t* v_signs, float scale, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!shape) return PAD_EINVAL;
  if (format < PAD_KV_OCTAVE_K3V4 || format > PAD_KV_OCTAVE_K3V3_COMPACT) return PAD_EINVAL;
  return decode(shape, q, nullptr, cache, block_table, seq_lens, scale, 0, out, workspace, workspace_bytes, stream,
                format, k_signs, v_signs);
}

pad_status pad_decode_attn_octave_varlen(const pad_shape* shape, int32_t format, const void* q,
                                         const int32_t* q_start, const void* cache, const int32_t* block_table,
                                         const int32_t* seq_lens, const uint32_t* k_signs, const uint32_t* v_signs,
                                         float scale, void* out, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  if (!shape) return PAD_EINVAL;
  if (format < PAD_KV_OCTAVE_K3V4 || format > PAD_KV_OCTAVE_K3V3_COMPACT) return PAD_EINVAL;
  if (shape->num_seqs > 0 && (!q_start || !aligned(q_start, 4))) return PAD_EINVAL;
  return decode(shape, q, q_start, cache, block_table, seq_lens, scale, 0, out, workspace, workspace_bytes, stream,
                format, k_signs, v_signs);
}

}  // extern "C"
