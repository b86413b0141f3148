/*
 * pad_attn.h -- C ABI of the paged-KV decode / speculative-verify attention
 * library (libpad_attn.so, HIP kernels for gfx950 / CDNA4).
 *
 * What it computes.  For every sequence s of a batch, every one of its M
 * newest query tokens m (M <= 8 for decode and speculative verify, up to
 * 256 for a prefill chunk) and every query head h, with L the
 * sequence's length (which already counts the M new tokens) and
 * qpos = L - M + m:
 *
 *     out[s,m,h,:] = sum_t softmax_t(scale * q[s,m,h,:] . K_t) * V_t
 *
 * over the keys t with lo <= t <= qpos, where lo = 0 without a window and
 * lo = max(0, qpos - window + 1) with one.  K_t and V_t are the two halves
 * of the packed K+V slot of token t of kv head h / (Hq / Hkv), found in
 * physical block block_table[s][t / page_size] at offset t % page_size.
 * A row with no visible key (L == 0 padding, or qpos < 0) is written as 0.
 *
 * Sources (page titles and sections):
 *   - ROCm/vllm pull request 1330, "Summary": decode and speculative decode
 *     attention over M <= 8 query tokens per sequence; all query rows of a
 *     kv head share one read of its K/V; split-KV segments with an
 *     in-kernel merge; sliding windows; batched decode; head sizes
 *     64/128/256/512.
 *   - vllm.v1.attention.ops.rocm_rdna_hip docs page: `KernelVariant`
 *     (layout codes 0 = NHD, 1 = HND; dtype flag 1 = bf16; window 0 = full
 *     causal), `expected_kv_cache_strides` (HND packed 2*D row strides),
 *     `KernelVariant.scratch_shapes` / `make_scratch` / `scratch_bytes`
 *     (fp32 split partials acc, m, l plus int32 counters that are zeroed
 *     once and left zeroed by every launch).
 *   - vllm.v1.attention.backends.rocm_octave_attn docs page:
 *     `RocmOctaveMetadataBuilder._fill_query_maps` (K length
 *     seq_len - q_len + i + 1, padding gets K length 0),
 *     `supported_kv_cache_layouts` (HND and NHD), `customize_spec` (one
 *     packed K+V slot per token and kv head), `RocmOctaveAttentionImpl`
 *     (`accept_output_buffer`: the caller owns the output; block sizes are
 *     multiples of 16).
 *
 * Layouts (all tensors dense, row-major, element type fp16 or bf16):
 *   q, out        [num_seqs, query_len, num_q_heads, head_size]
 *   kv_cache HND  [num_blocks, num_kv_heads, page_size, 2, head_size]
 *   kv_cache NHD  [num_blocks, page_size, num_kv_heads, 2, head_size]
 *                 (index 0 of the "2" axis is K, index 1 is V)
 *   block_table   int32 [num_seqs, max_blocks_per_seq]
 *   seq_lens      int32 [num_seqs]
 * Query head h uses kv head h / (num_q_heads / num_kv_heads).
 *
 * Ownership and threading.  Every pointer is a device pointer owned by the
 * caller; the library never allocates, frees or synchronises.  Each
 * pad_decode_attn call enqueues exactly one kernel on `stream` (a
 * hipStream_t, NULL = the null stream), so calls may be captured into a
 * HIP graph.  A workspace serves one in-flight call at a time; calls that
 * overlap on the same workspace race.  Calls made one after another on a
 * stream may share a workspace whatever their shapes.
 *
 * Errors.  Functions return a pad_status and never abort.  Only facts
 * visible on the host are validated (shape fields, pointer presence and
 * alignment, workspace size).  Device contents are the caller's contract:
 * block ids in the block table must address existing blocks for every page
 * a sequence's visible keys touch; violating it is undefined behaviour.  A
 * seq_lens[s] above max_blocks_per_seq * page_size is treated as that
 * capacity, and one <= 0 gives a zero output for the sequence.  The block
 * table must span [num_seqs, max_blocks_per_seq] int32 entries, all
 * readable: the kernel may read entries of pages no visible key touches
 * (before a window, past a sequence's end, the rows of length-0 sequences)
 * ahead of knowing the length, but never uses them, so their values are
 * don't-care (they need not name valid blocks).
 */
#ifndef PAD_ATTN_H
#define PAD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAD_ABI_VERSION 8

typedef enum pad_status {
  PAD_OK = 0,
  PAD_EINVAL = 1,        /* a shape field, pointer or alignment is invalid   */
  PAD_EUNSUPPORTED = 2,  /* valid but not built (e.g. head size 96)          */
  PAD_EWORKSPACE = 3,    /* workspace missing, misaligned or too small       */
  PAD_EHIP = 4,          /* the HIP runtime reported an error at launch      */
  PAD_ESCRATCH = 5       /* pad_decode_attn_noalloc: the call needs more than
                            the library's fixed PAD_NOALLOC_SCRATCH_BYTES     */
} pad_status;

/* Element type of q, kv_cache and out (same 0/1 flag as KernelVariant's
 * dtype field on the rocm_rdna_hip page). */
typedef enum pad_dtype { PAD_F16 = 0, PAD_BF16 = 1 } pad_dtype;

/* Cache layout codes of KernelVariant.layout (rocm_rdna_hip page). */
typedef enum pad_layout { PAD_NHD = 0, PAD_HND = 1 } pad_layout;

/* Which kernel family serves a call.  AUTO lets the planner choose; the
 * others force a family (tuning and tests).  MFMA: the waves of a workgroup
 * split a segment's keys and are combined at the end.  DOT: per-head dot
 * products (G*M <= 4, head size <= 128).  PREFILL: prefill chunks (head
 * size 64 or 128, one workgroup per item): 128 query rows of a kv head per
 * workgroup share each 128-key tile through LDS (the prefill work items of
 * plan_prefill on the rocm_rdna_hip page); AUTO takes it for chunks of at
 * least 128 rows per kv head whose row blocks fill a quarter of the device,
 * with at least 2^20 query rows x keys per kv head. */
typedef enum pad_path {
  PAD_PATH_AUTO = 0,
  PAD_PATH_MFMA = 1,
  PAD_PATH_DOT = 2,
  PAD_PATH_PREFILL = 3,
} pad_path;

/* Work schedule.  AUTO picks the balanced persistent grid for batches
 * whose K/V exceeds about 3 MiB per CU, else one workgroup per item.  Each
 * is deterministic (the same call gives the same bits); the two split the
 * keys differently, so they agree within rounding, not bit for bit.  On the
 * balanced grid a sequence's split -- and so the last bits of its output --
 * depends on the batch's total tile count (sequences of length 0 add none);
 * num_segments does not apply to it. */
typedef enum pad_schedule {  /* the dot family runs on the grid schedule only */
  PAD_SCHED_AUTO = 0,
  PAD_SCHED_GRID = 1,        /* one workgroup per (sequence, kv head, segment)  */
  PAD_SCHED_PERSISTENT = 2,  /* one workgroup per CU (two for a packed cache,
                                pad_octave.h), each taking an equal contiguous
                                share of the batch's 16-key tiles              */
} pad_schedule;

/* Shape of one call.  Every field is host data. */
typedef struct pad_shape {
  int32_t num_seqs;           /* S >= 0 (0: the call does nothing)                 */
  int32_t query_len;          /* M, 1..4096 query tokens per sequence; at most
                                 32768 rows G * M per kv head                    */
  int32_t num_q_heads;        /* Hq >= 1                                         */
  int32_t num_kv_heads;       /* Hkv >= 1, divides Hq                            */
  int32_t head_size;          /* D in {64, 128, 256, 512}                        */
  int32_t page_size;          /* P >= 16, a multiple of 16                       */
  int32_t max_blocks_per_seq; /* row stride of block_table, >= 1                 */
  int32_t max_seq_len;        /* host bound on seq_lens used to plan segments;
                                 0 = max_blocks_per_seq * page_size. A larger
                                 device length is still computed correctly.     */
  int32_t dtype;              /* pad_dtype                                       */
  int32_t layout;             /* pad_layout                                      */
  int32_t num_segments;       /* 0 = planner's choice; > 0 forces the split-KV
                                 segment count per (sequence, kv head)           */
  int32_t path;               /* pad_path                                        */
  int32_t schedule;           /* pad_schedule                                    */
} pad_shape;

/* The launch the planner chose (introspection, tests and tuning). */
typedef struct pad_plan {
  int32_t path;              /* PAD_PATH_MFMA, PAD_PATH_DOT or PAD_PATH_PREFILL   */
  int32_t rows;              /* query rows per (sequence, kv head) = G * M        */
  int32_t row_tiles;         /* rows of one workgroup in 16-row tiles             */
  int32_t row_groups;        /* workgroups splitting a kv head's rows             */
  int32_t waves;             /* waves (64 lanes) per workgroup                    */
  int32_t num_segments;      /* split-KV segments per (sequence, kv head, group)  */
  int32_t segment_tiles;     /* 16-key tiles per segment (planned)                */
  int32_t grid_x, grid_y;    /* launch grid                                       */
  int32_t merge_slices;      /* workgroups that share the merge of a split unit   */
  int32_t persistent;        /* 1: grid_x workgroups (one per CU) each take an
                                equal share of the batch's tiles (num_segments
                                is then 1); 0: one workgroup per item            */
  int32_t workspace_segments; /* segment slots per unit the workspace is sized for:
                                 a bound on num_segments over every window, so
                                 workspace_bytes is the same for every window  */
  uint64_t workspace_bytes;  /* bytes pad_decode_attn needs for this call         */
} pad_plan;

/* Version of this header the library was built from (PAD_ABI_VERSION). */
int32_t pad_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* pad_status_string(pad_status status);

/* Plan a call for a device with `num_cus` compute units (> 0).  Pure host
 * computation; no GPU needed.  `window` >= 0 as in pad_decode_attn.
 * Logging: with the environment variable PAD_LOG set to anything but "" or
 * "0" (read once per process), every plan the library makes -- here, for a
 * workspace size and for each decode call -- is printed to stderr as one
 * line "pad plan: <shape> -> <plan fields>", unless it equals the previous
 * line printed on the same thread. */
pad_status pad_decode_attn_plan(const pad_shape* shape, int32_t window, int32_t num_cus,
                                pad_plan* plan);

/* Workspace bytes that serve every call of this shape (any window) on the
 * current device.  0 means no workspace is needed (a single segment on a
 * grid of one workgroup per item).  The split partials are fp32
 * (acc[rows][D], m, l per row and slot), as in KernelVariant.scratch_shapes,
 * after a fixed 1 MiB prefix of int32 merge control words (per sequence,
 * kv head and row group: an arrival counter and one hand-over word per
 * merge slice after the first, each in its own 128-byte line).  Slots:
 * segment slots per (sequence, kv head) on the grid schedule, two per CU on
 * the balanced grid; the size covers every schedule the shape may take. */
pad_status pad_decode_attn_workspace_size(const pad_shape* shape, size_t* bytes);

/* Zero a workspace of `bytes` bytes (device pointer, 256-byte aligned) on
 * `stream`.  Needed once after allocation: every pad_decode_attn call
 * leaves the merge control words zero again. */
pad_status pad_decode_attn_workspace_init(void* workspace, size_t bytes, void* stream);

/* Paged-KV decode attention (see the top of this file).  `scale` multiplies
 * q.k before the softmax (finite); `window` is the sliding window in keys,
 * 0 for full causal attention.  q, kv_cache and out must be 16-byte
 * aligned, block_table and seq_lens 4-byte aligned, the workspace 256-byte
 * aligned with at least pad_decode_attn_workspace_size bytes (it may be
 * NULL when that size is 0).  out may not alias q or kv_cache. */
pad_status pad_decode_attn(const pad_shape* shape, const void* q, const void* kv_cache,
                           const int32_t* block_table, const int32_t* seq_lens, float scale,
                           int32_t window, void* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Paged-KV decode attention with a query count per sequence (mixed decode
 * and speculative-verify batches in one call).  The query rows are packed:
 * q and out are [T, num_q_heads, head_size] and sequence s owns tokens
 * q_start[s] .. q_start[s + 1] - 1, i.e. M_s = q_start[s + 1] - q_start[s]
 * query tokens whose positions are L_s - M_s + m, m < M_s, with the same
 * causal and window rule as above (query i of a request with q_len queries
 * and seq_len tokens sees K length seq_len - q_len + i + 1:
 * RocmOctaveMetadataBuilder._fill_query_maps on the octave page).
 * q_start is a device int32 array of num_seqs + 1 entries, read only on
 * the device (no host synchronisation; the call can be captured in a HIP
 * graph).  shape->query_len is the host bound on every M_s (1..4096; it sizes
 * the plan and the workspace like a uniform call of that M).  Contract on
 * the device values: q_start non-decreasing, q_start[0] >= 0, M_s <=
 * query_len, and q/out hold at least q_start[num_seqs] rows; a count
 * outside [0, query_len] is clamped into it (M_s = 0: the sequence is
 * skipped and its rows, if any, are left untouched).  Other arguments,
 * errors and ownership as pad_decode_attn; q_start must be 4-byte aligned
 * (PAD_EINVAL if missing or misaligned). */
pad_status pad_decode_attn_varlen(const pad_shape* shape, const void* q, const int32_t* q_start,
                                  const void* kv_cache, const int32_t* block_table, const int32_t* seq_lens,
                                  float scale, int32_t window, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Bytes of the fixed device array pad_decode_attn_noalloc uses as its
 * workspace, held by each GPU the library runs on until the process ends. */
#define PAD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the
 * decode of pad_decode_attn (same arguments, same kernels, same output
 * bits) with its workspace taken from a fixed array of
 * PAD_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU,
 * instead of a caller-supplied buffer.  The caller still owns q, kv_cache,
 * block_table, seq_lens and out.  It calls no hipMalloc or hipFree and
 * allocates nothing.  A call whose workspace (pad_decode_attn_workspace_size)
 * exceeds the array returns PAD_ESCRATCH before anything is enqueued.  On a
 * device's first call (and on every call until one is made outside graph
 * capture) a fill kernel clearing the array's 1 MiB control prefix is
 * enqueued on `stream` ahead of the decode; each decode leaves the prefix
 * zero again.  Every call on a GPU shares that GPU's array: calls that
 * overlap in time on one GPU (on different streams, or from different
 * threads without ordering) race and give undefined results. */
pad_status pad_decode_attn_noalloc(const pad_shape* shape, const void* q, const void* kv_cache,
                                   const int32_t* block_table, const int32_t* seq_lens, float scale,
                                   int32_t window, void* out, void* stream);

/* Bound, in microseconds, on how long a workgroup that shares the split-KV
 * merge waits for the last segment of its unit (process-wide; default 200;
 * 0 .. 1000000 accepted, else PAD_EINVAL).  A workgroup that stops waiting
 * leaves its merge slice to the last segment, so every value gives the
 * same output bits; 0 makes every such workgroup give up at once, which
 * lets tests exercise that hand-over.  Applies to calls enqueued after it
 * returns. */
pad_status pad_set_merge_wait(int32_t microseconds);

#ifdef __cplusplus
}
#endif

#endif /* PAD_ATTN_H */
