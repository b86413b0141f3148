// Host build of the C ABI's validation paths and of the launch planner
// (csrc/api.cpp, csrc/plan.cpp) for AddressSanitizer and
// UndefinedBehaviorSanitizer: a seeded sweep of valid and invalid call
// shapes through pad_decode_attn_plan, the workspace-size queries and the
// decode entry points.  No device is touched: the HIP runtime queries and
// the kernel launchers are stubbed here, and each stubbed launch checks the
// plan and parameters it receives against what the kernels assume (grid
// limits, partial slots and control words inside the workspace, 32-bit
// strides, segment bounds).  Exit status 0 and a summary line on success;
// the sanitizers abort on the first error.
#include <hip/hip_runtime_api.h>

#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "../../include/pad_attn.h"
#include "../../include/pad_octave.h"
#include "../../paged_kv_decode_block_amd/csrc/kernels.h"
#include "../../paged_kv_decode_block_amd/csrc/plan.h"

// ---- stubs: no device in this build ----
extern "C" hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
extern "C" hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }

namespace {

struct Call {
  pad_shape shape;
  int32_t window;
  size_t ws_bytes;
  int key_bytes;  // packed slot bytes (0: 2 D elements of 2 bytes)
};
Call g_call;
long g_launches = 0;

[[noreturn]] void fail(const char* what) {
  std::fprintf(stderr, "invariant failed: %s (S=%d M=%d Hq=%d Hkv=%d D=%d P=%d blocks=%d max_len=%d W=%d path=%d "
                       "sched=%d nseg=%d)\n",
               what, g_call.shape.num_seqs, g_call.shape.query_len, g_call.shape.num_q_heads, g_call.shape.num_kv_heads,
               g_call.shape.head_size, g_call.shape.page_size, g_call.shape.max_blocks_per_seq,
               g_call.shape.max_seq_len, g_call.window, g_call.shape.path, g_call.shape.schedule,
               g_call.shape.num_segments);
  std::abort();
}

void expect(bool ok, const char* what) {
  if (!ok) fail(what);
}

// What a launch may assume about its plan and parameters.
void check_launch(const pad::Plan& pl, const pad::Params& pr) {
  ++g_launches;
  const pad_shape& sh = g_call.shape;
  const int64_t S = sh.num_seqs, H = sh.num_kv_heads, D = sh.head_size;
  expect(pl.grid_x >= 1 && pl.grid_y >= 1 && pl.grid_y <= 65535, "grid within the launch limits");
  expect(pr.rows == sh.num_q_heads / sh.num_kv_heads * sh.query_len, "rows = G * M");
  expect(int64_t(pr.group_rows) * pr.row_groups >= pr.rows, "row groups cover the rows");
  if (pl.path == PAD_PATH_PREFILL) {
    expect(pl.row_tiles * 16 == pad::kPrefillRows && (sh.head_size == 64 || sh.head_size == 128),
           "prefill: 128-row blocks at head size 64 or 128");
    expect(!pl.persistent && pl.seg_tiles <= pad::kPrefillMaxSegTiles, "prefill: grid, segments within the id area");
  } else {
    expect(pl.row_tiles >= 1 && pl.row_tiles <= 4, "row tiles per wave");
  }
  expect(pr.block_stride > 0 && pr.block_stride <= INT32_MAX && pr.head_stride <= INT32_MAX &&
             pr.token_stride <= INT32_MAX,
         "strides fit the kernel's 32-bit arguments");
  expect(pl.merge_slices >= 1 && pl.merge_slices <= pad::kMaxSlices, "merge slices");
  if (pl.persistent) {
    expect(pl.grid_y == 1 && pl.nseg == 1, "balanced grid: one row of workgroups, no segments");
    expect(pl.merge_slices == 1, "balanced grid: the last arriver merges alone");
    const int64_t units = S * H * pl.row_groups;
    expect(units * pad::kCtlWordStride * 4 <= int64_t(pad::kCounterBytes), "balanced grid: control words fit");
    expect(sh.num_seqs <= pad::kPersistMaxSeqs, "balanced grid: sequences fit the LDS tables");
    const int64_t slots = 2 * int64_t(pl.grid_x);
    expect(pl.ws_ml >= pad::kCounterBytes, "partials after the control prefix");
    expect(pl.ws_ml + slots * pl.slot_rows * 2 * 4 <= pl.ws_acc, "(m, l) slots before the accumulators");
    expect(pl.ws_acc + slots * pl.slot_rows * D * 4 <= pl.ws_bytes, "accumulator slots inside the workspace");
  } else {
    expect(pl.nseg >= 1 && pl.nseg <= pad::kMaxSegments && pl.seg_tiles >= 1 && pl.seg_tiles <= pad::kMaxSegTiles,
           "segments within their bounds");
    expect(int64_t(pl.grid_x) == int64_t(pl.nseg) * H * pl.row_groups, "grid = segments x kv heads x row groups");
    if (pl.nseg > 1) {
      const int64_t slots = S * H * pl.nseg;
      expect(pl.nseg <= pl.ws_nseg, "segments within the workspace's slots");
      expect(pl.slot_rows == pr.rows, "grid slots hold every row");
      expect(pl.ws_ml >= pad::kCounterBytes, "partials after the control prefix");
      expect(pl.ws_ml + slots * pl.slot_rows * 2 * 4 <= pl.ws_acc, "(m, l) slots before the accumulators");
      expect(pl.ws_acc + slots * pl.slot_rows * D * 4 <= pl.ws_bytes, "accumulator slots inside the workspace");
      expect(S * H * pl.row_groups * pl.merge_slices * pad::kCtlWordStride * 4 <= int64_t(pad::kCounterBytes),
             "control words fit the prefix");
    }
  }
  expect(pl.ws_bytes <= g_call.ws_bytes, "the call's workspace covers the plan");
}

}  // namespace

namespace pad {
int launch_decode(const Plan& plan, const Params& params, int, int, void*) {
  check_launch(plan, params);
  return 0;
}
int launch_decode_octave(const Plan& plan, const Params& params, int, int, void*) {
  check_launch(plan, params);
  return 0;
}
int launch_zero(void*, size_t, void*) { return 0; }
}  // namespace pad

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 200000;
  std::mt19937_64 rng(20261203);
  auto pick = [&](std::initializer_list<int> v) {
    const size_t i = std::uniform_int_distribution<size_t>(0, v.size() - 1)(rng);
    return *(v.begin() + i);
  };
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  // Aligned stand-ins for device pointers: the stubbed launches never
  // dereference them.
  void* const dev = reinterpret_cast<void*>(uintptr_t(1) << 20);
  const int32_t* const dev_i = static_cast<const int32_t*>(dev);
  const uint32_t* const dev_u = static_cast<const uint32_t*>(dev);
  long counts[8] = {};
  for (long it = 0; it < iters; ++it) {
    // A valid shape, then in one draw of five a single field made invalid
    // or extreme.
    pad_shape sh{};
    sh.num_seqs = pick({0, 1, 2, 3, 65, 200, 1024, uni(1, 3000)});
    sh.query_len = pick({1, 1, 2, 4, 8, 16, 64, 256, 2048, 4096});
    sh.num_kv_heads = pick({1, 2, 4, 8, 64});
    sh.num_q_heads = sh.num_kv_heads * pick({1, 2, 4, 8, 16, 3});
    sh.head_size = pick({64, 128, 256, 512});
    sh.page_size = pick({16, 32, 48, 1056, 4096});
    sh.max_blocks_per_seq = pick({1, 2, 16, 64, 256, 2048, uni(1, 70000)});
    int64_t table_keys = int64_t(sh.max_blocks_per_seq) * sh.page_size;
    sh.max_seq_len = pick({0, 0, 1}) ? 0 : int32_t(std::min<int64_t>(table_keys, uni(1, 1 << 20)));
    sh.dtype = pick({PAD_F16, PAD_BF16});
    sh.layout = pick({PAD_NHD, PAD_HND});
    sh.num_segments = pick({0, 0, 0, 1, 7, 256});
    sh.path = pick({PAD_PATH_AUTO, PAD_PATH_AUTO, PAD_PATH_MFMA, PAD_PATH_DOT, PAD_PATH_PREFILL});
    sh.schedule = pick({PAD_SCHED_AUTO, PAD_SCHED_AUTO, PAD_SCHED_GRID, PAD_SCHED_PERSISTENT});
    int32_t window = pick({0, 0, 1, 100, 512, 4096, 100000});
    int32_t cus = pick({1, 80, 256, 304});
    if (uni(0, 4) == 0) {
      switch (uni(0, 13)) {
        case 0: sh.num_seqs = pick({-1, 65536, 70000}); break;
        case 1: sh.query_len = pick({0, -3, 4097, 100000}); break;
        case 2: sh.num_kv_heads = pick({0, -1}); break;
        case 3: sh.num_q_heads += pick({1, -1}); break;
        case 4: sh.head_size = pick({0, 96, 1024}); break;
        case 5: sh.page_size = pick({0, 8, 24, 32768}); break;
        case 6: sh.max_blocks_per_seq = pick({0, -5, 1 << 25}); break;
        case 7: sh.max_seq_len = int32_t(std::min<int64_t>(INT32_MAX, table_keys + 1)); break;
        case 8: sh.dtype = pick({2, -1}); break;
        case 9: sh.layout = pick({2, -1}); break;
        case 10: sh.num_segments = pick({-1, 257, 100000}); break;
        case 11: sh.path = pick({4, -1}); break;
        case 12: sh.schedule = pick({3, -1}); break;
        default: window = pick({-1, INT32_MAX}); break;
      }
    }
    table_keys = int64_t(sh.max_blocks_per_seq) * sh.page_size;
    pad_plan plan{};
    const pad_status ps = pad_decode_attn_plan(&sh, window, cus, &plan);
    counts[ps < 8 ? ps : 7]++;
    size_t ws = 0;
    const pad_status ws_st = pad_decode_attn_workspace_size(&sh, &ws);
    if (ps == PAD_OK && window == 0 && cus == 256) expect(ws_st == PAD_OK && ws == plan.workspace_bytes, "size query = plan");
    if (ws_st != PAD_OK) continue;
    // A call with exactly the queried workspace, and one with too little.
    g_call = Call{sh, window, ws, 0};
    const pad_status st = pad_decode_attn(&sh, dev, dev, dev_i, dev_i, 0.125f, window, dev, dev, ws, nullptr);
    if (st != PAD_OK && st != PAD_EUNSUPPORTED && st != PAD_EINVAL) fail("unexpected status with the queried workspace");
    if (ws > 0 && sh.num_seqs > 0) {
      const pad_status small = pad_decode_attn(&sh, dev, dev, dev_i, dev_i, 0.125f, window, dev, dev, ws - 4, nullptr);
      expect(small != PAD_OK, "too small a workspace is refused");
    }
    const pad_status vl =
        pad_decode_attn_varlen(&sh, dev, dev_i, dev, dev_i, dev_i, 0.125f, window, dev, dev, ws, nullptr);
    if (vl != PAD_OK && vl != PAD_EUNSUPPORTED && vl != PAD_EINVAL) fail("unexpected varlen status");
    // Packed-cache path (head size 256 only).
    const int32_t fmt = pick({0, 1, 2, 3, 4});
    size_t ows = 0;
    if (pad_decode_attn_octave_workspace_size(&sh, fmt, &ows) == PAD_OK) {
      int32_t sb = 0;
      if (pad_octave_slot_bytes(fmt, sh.head_size, &sb) == PAD_OK) {
        g_call = Call{sh, 0, ows, sb};
        const pad_status os = pad_decode_attn_octave(&sh, fmt, dev, dev, dev_i, dev_i, dev_u, dev_u, 0.0625f, dev, dev,
                                                     ows, nullptr);
        if (os != PAD_OK && os != PAD_EUNSUPPORTED && os != PAD_EINVAL) fail("unexpected packed-cache status");
      }
    }
  }
  // Null and non-finite arguments.
  pad_shape sh{};
  sh.num_seqs = 1;
  sh.query_len = 1;
  sh.num_q_heads = 8;
  sh.num_kv_heads = 2;
  sh.head_size = 128;
  sh.page_size = 16;
  sh.max_blocks_per_seq = 4;
  sh.dtype = PAD_BF16;
  sh.layout = PAD_HND;
  pad_plan plan{};
  expect(pad_decode_attn_plan(nullptr, 0, 256, &plan) == PAD_EINVAL, "null shape");
  expect(pad_decode_attn_plan(&sh, 0, 256, nullptr) == PAD_EINVAL, "null plan");
  expect(pad_decode_attn_plan(&sh, 0, 0, &plan) == PAD_EINVAL, "zero CUs");
  size_t ws = 0;
  expect(pad_decode_attn_workspace_size(&sh, &ws) == PAD_OK, "size query");
  g_call = Call{sh, 0, ws, 0};
  expect(pad_decode_attn(&sh, dev, dev, dev_i, dev_i, __builtin_nanf(""), 0, dev, dev, ws, nullptr) == PAD_EINVAL,
         "NaN scale refused");
  expect(pad_decode_attn(&sh, nullptr, dev, dev_i, dev_i, 1.f, 0, dev, dev, ws, nullptr) == PAD_EINVAL, "null q");
  expect(pad_decode_attn(&sh, static_cast<char*>(dev) + 2, dev, dev_i, dev_i, 1.f, 0, dev, dev, ws, nullptr) ==
             PAD_EINVAL,
         "misaligned q");
  expect(pad_decode_attn(nullptr, dev, dev, dev_i, dev_i, 1.f, 0, dev, dev, ws, nullptr) == PAD_EINVAL, "null shape");
  for (int s = -1; s <= 6; ++s) expect(pad_status_string(pad_status(s)) != nullptr, "status strings");
  std::printf("abi sweep ok: %ld shapes, %ld launches checked, plan statuses ok=%ld einval=%ld eunsupported=%ld\n",
              iters, g_launches, counts[PAD_OK], counts[PAD_EINVAL], counts[PAD_EUNSUPPORTED]);
  return 0;
}
