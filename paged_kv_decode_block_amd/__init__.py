"""Python binding of libpad_attn.so: paged-KV decode attention on gfx950.

Thin ctypes marshalling over the C ABI declared in ``include/pad_attn.h``;
the functions keep the C names.  PyTorch supplies device memory and the
current stream; every step of the computation runs in the library's HIP
kernels.  Importing this package fails if the library has not been built
(``python paged_kv_decode_block_amd/build.py``): there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "PAD_OK", "PAD_EINVAL", "PAD_EUNSUPPORTED", "PAD_EWORKSPACE", "PAD_EHIP", "PAD_ESCRATCH",
    "PAD_NOALLOC_SCRATCH_BYTES", "pad_decode_attn_noalloc",
    "PAD_KV_OCTAVE_K3V4", "PAD_KV_OCTAVE_K3V3", "PAD_KV_OCTAVE_K3V3_COMPACT", "OCTAVE_FORMATS",
    "pad_octave_cache_shape", "pad_octave_slot_bytes", "pad_octave_cache_write",
    "pad_decode_attn_octave_workspace_size", "pad_decode_attn_octave", "pad_decode_attn_octave_varlen",
    "PAD_F16", "PAD_BF16", "PAD_NHD", "PAD_HND",
    "PAD_PATH_AUTO", "PAD_PATH_MFMA", "PAD_PATH_DOT", "PAD_PATH_PREFILL",
    "PAD_SCHED_AUTO", "PAD_SCHED_GRID", "PAD_SCHED_PERSISTENT",
    "PadError", "pad_shape", "pad_plan", "lib", "LIB_PATH", "load_library",
    "pad_abi_version", "pad_status_string", "pad_decode_attn_plan",
    "pad_decode_attn_workspace_size", "pad_decode_attn_workspace_init", "pad_decode_attn",
    "pad_decode_attn_varlen", "pad_rope_cache_write", "pad_cache_shape",
    "pad_set_merge_wait", "pad_calib_gather_read", "pad_calib_stream_read",
    "make_shape", "Workspace",
]

PAD_OK, PAD_EINVAL, PAD_EUNSUPPORTED, PAD_EWORKSPACE, PAD_EHIP, PAD_ESCRATCH = 0, 1, 2, 3, 4, 5
# Bytes of the fixed device array pad_decode_attn_noalloc takes its workspace from.
PAD_NOALLOC_SCRATCH_BYTES = 64 << 20
PAD_F16, PAD_BF16 = 0, 1
PAD_NHD, PAD_HND = 0, 1
PAD_PATH_AUTO, PAD_PATH_MFMA, PAD_PATH_DOT, PAD_PATH_PREFILL = 0, 1, 2, 3
PAD_SCHED_AUTO, PAD_SCHED_GRID, PAD_SCHED_PERSISTENT = 0, 1, 2
PAD_KV_OCTAVE_K3V4, PAD_KV_OCTAVE_K3V3, PAD_KV_OCTAVE_K3V3_COMPACT = 1, 2, 3
OCTAVE_FORMATS = {"octave_k3v4": PAD_KV_OCTAVE_K3V4, "octave_k3v3": PAD_KV_OCTAVE_K3V3,
                  "octave_k3v3_compact": PAD_KV_OCTAVE_K3V3_COMPACT}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpad_attn.so")


class pad_shape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("query_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("path", ctypes.c_int32),
        ("schedule", ctypes.c_int32),
    ]


class pad_plan(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("row_tiles", ctypes.c_int32),
        ("row_groups", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("segment_tiles", ctypes.c_int32),
        ("grid_x", ctypes.c_int32),
        ("grid_y", ctypes.c_int32),
        ("merge_slices", ctypes.c_int32),
        ("persistent", ctypes.c_int32),
        ("workspace_segments", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_uint64),
    ]


class pad_cache_shape(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("max_position", ctypes.c_int32),
    ]


class pad_octave_cache_shape(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("format", ctypes.c_int32),
    ]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open a build of the library and declare its C signatures."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python paged_kv_decode_block_amd/build.py` "
            "(the decode-attention path has no non-HIP fallback)"
        )
    L = ctypes.CDLL(path)
    P = ctypes.POINTER
    L.pad_abi_version.restype = ctypes.c_int32
    L.pad_abi_version.argtypes = []
    L.pad_status_string.restype = ctypes.c_char_p
    L.pad_status_string.argtypes = [ctypes.c_int]
    L.pad_decode_attn_plan.restype = ctypes.c_int
    L.pad_decode_attn_plan.argtypes = [P(pad_shape), ctypes.c_int32, ctypes.c_int32, P(pad_plan)]
    L.pad_decode_attn_workspace_size.restype = ctypes.c_int
    L.pad_decode_attn_workspace_size.argtypes = [P(pad_shape), P(ctypes.c_size_t)]
    L.pad_decode_attn_workspace_init.restype = ctypes.c_int
    L.pad_decode_attn_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.pad_set_merge_wait.restype = ctypes.c_int
    L.pad_set_merge_wait.argtypes = [ctypes.c_int32]
    L.pad_decode_attn.restype = ctypes.c_int
    L.pad_decode_attn.argtypes = [
        P(pad_shape), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
    ]
    L.pad_decode_attn_noalloc.restype = ctypes.c_int
    L.pad_decode_attn_noalloc.argtypes = [
        P(pad_shape), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
    ]
    L.pad_octave_slot_bytes.restype = ctypes.c_int
    L.pad_octave_slot_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, P(ctypes.c_int32)]
    L.pad_octave_cache_write.restype = ctypes.c_int
    L.pad_octave_cache_write.argtypes = [P(pad_octave_cache_shape)] + [ctypes.c_void_p] * 7
    L.pad_decode_attn_octave_workspace_size.restype = ctypes.c_int
    L.pad_decode_attn_octave_workspace_size.argtypes = [P(pad_shape), ctypes.c_int32, P(ctypes.c_size_t)]
    L.pad_decode_attn_octave.restype = ctypes.c_int
    L.pad_decode_attn_octave.argtypes = [
        P(pad_shape), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p,
    ]
    L.pad_decode_attn_octave_varlen.restype = ctypes.c_int
    L.pad_decode_attn_octave_varlen.argtypes = [
        P(pad_shape), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_size_t, ctypes.c_void_p,
    ]
    L.pad_calib_gather_read.restype = ctypes.c_int
    L.pad_calib_gather_read.argtypes = [
        P(pad_shape), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
    ]
    L.pad_calib_stream_read.restype = ctypes.c_int
    L.pad_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.pad_rope_cache_write.restype = ctypes.c_int
    L.pad_rope_cache_write.argtypes = [
        P(pad_cache_shape), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ]
    L.pad_decode_attn_varlen.restype = ctypes.c_int
    L.pad_decode_attn_varlen.argtypes = [
        P(pad_shape), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
    ]
    return L


lib = load_library()


class PadError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {pad_status_string(status)} (status {status})")


def _check(status: int, where: str) -> None:
    if status != PAD_OK:
        raise PadError(status, where)


def pad_abi_version() -> int:
    return int(lib.pad_abi_version())


def pad_status_string(status: int) -> str:
    return lib.pad_status_string(int(status)).decode()


_DTYPE_CODE = {torch.float16: PAD_F16, torch.bfloat16: PAD_BF16}


def make_shape(
    q: torch.Tensor,
    kv_cache: torch.Tensor,
    block_table: torch.Tensor,
    layout: int,
    *,
    max_seq_len: int = 0,
    num_segments: int = 0,
    path: int = PAD_PATH_AUTO,
    schedule: int = PAD_SCHED_AUTO,
) -> pad_shape:
    """The ``pad_shape`` of a call, read off the tensors' sizes."""
    if q.dim() != 4 or kv_cache.dim() != 5 or block_table.dim() != 2:
        raise ValueError("expected q [S,M,Hq,D], kv_cache 5-d, block_table [S,max_blocks]")
    S, M, Hq, D = q.shape
    if layout == PAD_HND:
        _, Hkv, P, two, Dk = kv_cache.shape
    elif layout == PAD_NHD:
        _, P, Hkv, two, Dk = kv_cache.shape
    else:
        raise ValueError(f"unknown layout {layout}")
    if two != 2 or Dk != D:
        raise ValueError("kv_cache must hold packed (K, V) slots of the query head size")
    if q.dtype not in _DTYPE_CODE or kv_cache.dtype != q.dtype:
        raise ValueError("q and kv_cache must share dtype float16 or bfloat16")
    if block_table.shape[0] != S:
        raise ValueError("block_table must have one row per sequence")
    return pad_shape(
        num_seqs=S, query_len=M, num_q_heads=Hq, num_kv_heads=Hkv, head_size=D, page_size=P,
        max_blocks_per_seq=block_table.shape[1], max_seq_len=max_seq_len, dtype=_DTYPE_CODE[q.dtype],
        layout=layout, num_segments=num_segments, path=path, schedule=schedule,
    )


def pad_decode_attn_plan(shape: pad_shape, window: int = 0, num_cus: int | None = None) -> dict:
    """The planner's choice for ``shape`` (pure host computation)."""
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    plan = pad_plan()
    _check(lib.pad_decode_attn_plan(ctypes.byref(shape), int(window), int(num_cus), ctypes.byref(plan)),
           "pad_decode_attn_plan")
    return {name: getattr(plan, name) for name, _ in pad_plan._fields_}


def pad_decode_attn_workspace_size(shape: pad_shape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.pad_decode_attn_workspace_size(ctypes.byref(shape), ctypes.byref(n)),
           "pad_decode_attn_workspace_size")
    return int(n.value)


def _require_device(**tensors: torch.Tensor) -> None:
    """Every argument must be a contiguous device tensor."""
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def pad_decode_attn_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    _check(lib.pad_decode_attn_workspace_init(
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        ctypes.c_void_p(_stream_ptr(stream))), "pad_decode_attn_workspace_init")


class Workspace:
    """A zero-initialised device workspace (allocate it outside graph capture).

    ``get(shape, stream)`` returns a buffer of at least the bytes ``shape``
    needs, growing (and re-zeroing) it when a larger shape comes along.  The
    fill is enqueued on ``stream`` -- the stream the decode will run on --
    so the launch that follows sees the zeroed control words; a buffer
    allocated while another stream is current is recorded on ``stream``, so
    the caching allocator does not hand its memory out again while work on
    that stream may still use it (also when a larger shape replaces it).
    Calls on one workspace must be issued on one stream at a time.
    """

    def __init__(self, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.buf: torch.Tensor | None = None

    def get(self, shape: pad_shape, stream=None) -> torch.Tensor | None:
        need = pad_decode_attn_workspace_size(shape)
        if need == 0:
            return self.buf
        if self.buf is None or self.buf.numel() < need:
            buf = torch.empty(need, dtype=torch.uint8, device=self.device)
            _record_on(buf, stream)
            pad_decode_attn_workspace_init(buf, stream)
            self.buf = buf
        return self.buf


def _record_on(t: torch.Tensor, stream) -> None:
    """Tell the caching allocator that ``stream`` (None: the current one)
    uses ``t``, when that is not the stream it was allocated on."""
    if stream is not None and t.is_cuda and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)


def pad_set_merge_wait(microseconds: int) -> None:
    """Bound on a merge helper's wait for the last segment (process-wide)."""
    _check(lib.pad_set_merge_wait(int(microseconds)), "pad_set_merge_wait")


# Default workspaces, one per (device, stream): a workspace serves one
# in-flight call at a time, so calls on different streams get their own.
_default_ws: dict[tuple[int, int], Workspace] = {}


def _default_workspace(device: torch.device, shape: pad_shape, stream) -> torch.Tensor | None:
    key = (device.index, _stream_ptr(stream))
    ws = _default_ws.get(key)
    if ws is None:
        ws = _default_ws[key] = Workspace(device)
    return ws.get(shape, stream)


def pad_decode_attn(
    q: torch.Tensor,
    kv_cache: torch.Tensor,
    block_table: torch.Tensor,
    seq_lens: torch.Tensor,
    scale: float,
    window: int,
    out: torch.Tensor,
    *,
    layout: int = PAD_HND,
    workspace: torch.Tensor | None = None,
    max_seq_len: int = 0,
    num_segments: int = 0,
    path: int = PAD_PATH_AUTO,
    schedule: int = PAD_SCHED_AUTO,
    stream=None,
) -> torch.Tensor:
    """Paged-KV decode attention into ``out`` (see include/pad_attn.h).

    ``workspace`` must be a zero-initialised device buffer of at least
    ``pad_decode_attn_workspace_size`` bytes; when omitted, a per-device
    buffer is kept by this module (allocated on first use, so make one call
    before capturing a graph).
    """
    _require_device(q=q, kv_cache=kv_cache, block_table=block_table, seq_lens=seq_lens, out=out)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    if seq_lens.shape != (q.shape[0],):
        raise ValueError("seq_lens must have one entry per sequence")
    shape = make_shape(q, kv_cache, block_table, layout, max_seq_len=max_seq_len,
                       num_segments=num_segments, path=path, schedule=schedule)
    ws = _default_workspace(q.device, shape, stream) if workspace is None else workspace
    ws_ptr = ws.data_ptr() if ws is not None else 0
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib.pad_decode_attn(
        ctypes.byref(shape), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv_cache.data_ptr()),
        ctypes.c_void_p(block_table.data_ptr()), ctypes.c_void_p(seq_lens.data_ptr()),
        ctypes.c_float(scale), ctypes.c_int32(window), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_bytes), ctypes.c_void_p(_stream_ptr(stream)),
    ), "pad_decode_attn")
    return out


def pad_decode_attn_noalloc(
    q: torch.Tensor,
    kv_cache: torch.Tensor,
    block_table: torch.Tensor,
    seq_lens: torch.Tensor,
    scale: float,
    window: int,
    out: torch.Tensor,
    *,
    layout: int = PAD_HND,
    max_seq_len: int = 0,
    num_segments: int = 0,
    path: int = PAD_PATH_AUTO,
    schedule: int = PAD_SCHED_AUTO,
    stream=None,
) -> torch.Tensor:
    """``pad_decode_attn`` with its workspace in the library's fixed device
    array (include/pad_attn.h): nothing is allocated, by the library or
    here.  Calls that overlap on one GPU race."""
    _require_device(q=q, kv_cache=kv_cache, block_table=block_table, seq_lens=seq_lens, out=out)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    if seq_lens.shape != (q.shape[0],):
        raise ValueError("seq_lens must have one entry per sequence")
    shape = make_shape(q, kv_cache, block_table, layout, max_seq_len=max_seq_len,
                       num_segments=num_segments, path=path, schedule=schedule)
    _check(lib.pad_decode_attn_noalloc(
        ctypes.byref(shape), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv_cache.data_ptr()),
        ctypes.c_void_p(block_table.data_ptr()), ctypes.c_void_p(seq_lens.data_ptr()),
        ctypes.c_float(scale), ctypes.c_int32(window), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(_stream_ptr(stream)),
    ), "pad_decode_attn_noalloc")
    return out


def pad_decode_attn_varlen(
    q: torch.Tensor,
    q_start: torch.Tensor,
    kv_cache: torch.Tensor,
    block_table: torch.Tensor,
    seq_lens: torch.Tensor,
    scale: float,
    window: int,
    out: torch.Tensor,
    *,
    max_query_len: int = 8,
    layout: int = PAD_HND,
    workspace: torch.Tensor | None = None,
    max_seq_len: int = 0,
    num_segments: int = 0,
    path: int = PAD_PATH_AUTO,
    schedule: int = PAD_SCHED_AUTO,
    stream=None,
) -> torch.Tensor:
    """Decode attention with a query count per sequence (include/pad_attn.h).

    ``q`` and ``out`` are packed ``[T, Hq, D]``; sequence ``s`` owns rows
    ``q_start[s] .. q_start[s + 1] - 1`` (``q_start``: device int32,
    ``S + 1`` entries, never read on the host).  ``max_query_len`` bounds
    every per-sequence count (it sizes the plan and the workspace).
    """
    _require_device(q=q, q_start=q_start, kv_cache=kv_cache, block_table=block_table, seq_lens=seq_lens, out=out)
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must be packed [T, Hq, D] tensors of one dtype")
    S = block_table.shape[0]
    if q_start.dtype != torch.int32 or q_start.shape != (S + 1,):
        raise ValueError("q_start must be int32 with one entry per sequence plus one")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or seq_lens.shape != (S,):
        raise ValueError("block_table and seq_lens must be int32, one row / entry per sequence")
    T, Hq, D = q.shape
    q_like = torch.empty((S, max_query_len, Hq, D), dtype=q.dtype, device="meta")
    shape = make_shape(q_like, kv_cache, block_table, layout, max_seq_len=max_seq_len,
                       num_segments=num_segments, path=path, schedule=schedule)
    ws = _default_workspace(q.device, shape, stream) if workspace is None else workspace
    ws_ptr = ws.data_ptr() if ws is not None else 0
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib.pad_decode_attn_varlen(
        ctypes.byref(shape), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q_start.data_ptr()),
        ctypes.c_void_p(kv_cache.data_ptr()), ctypes.c_void_p(block_table.data_ptr()),
        ctypes.c_void_p(seq_lens.data_ptr()), ctypes.c_float(scale), ctypes.c_int32(window),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_bytes),
        ctypes.c_void_p(_stream_ptr(stream)),
    ), "pad_decode_attn_varlen")
    return out


def pad_rope_cache_write(
    key: torch.Tensor,
    value: torch.Tensor,
    kv_cache: torch.Tensor,
    slot_mapping: torch.Tensor,
    *,
    layout: int = PAD_HND,
    q: torch.Tensor | None = None,
    positions: torch.Tensor | None = None,
    cos_sin_cache: torch.Tensor | None = None,
    stream=None,
) -> None:
    """Store new tokens' K (rotated when a cos/sin table is given) and V in
    their cache slots, and rotate ``q`` in place (include/pad_cache.h).

    ``key``/``value`` ``[T, Hkv, D]``, ``q`` ``[T, Hq, D]``, ``slot_mapping``
    and ``positions`` int64 ``[T]``, ``cos_sin_cache`` fp32
    ``[max_position, rope_dim]`` (cos then sin).
    """
    tensors = [("key", key), ("value", value), ("kv_cache", kv_cache), ("slot_mapping", slot_mapping)]
    tensors += [(n, t) for n, t in (("q", q), ("positions", positions), ("cos_sin_cache", cos_sin_cache)) if t is not None]
    for name, t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if key.dim() != 3 or value.shape != key.shape or key.dtype not in _DTYPE_CODE or kv_cache.dtype != key.dtype:
        raise ValueError("key and value must be [T, Hkv, D] of the cache's dtype (float16 or bfloat16)")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (key.shape[0],):
        raise ValueError("slot_mapping must be int64 [T]")
    if layout == PAD_HND:
        nb, Hkv, P, two, D = kv_cache.shape
    else:
        nb, P, Hkv, two, D = kv_cache.shape
    if two != 2 or D != key.shape[2] or Hkv != key.shape[1]:
        raise ValueError("kv_cache must hold packed (K, V) slots of key's heads and head size")
    rope_dim, max_pos = 0, 0
    if cos_sin_cache is not None:
        if positions is None or positions.dtype != torch.int64 or positions.shape != (key.shape[0],):
            raise ValueError("a cos/sin table needs int64 positions [T]")
        if cos_sin_cache.dtype != torch.float32 or cos_sin_cache.dim() != 2:
            raise ValueError("cos_sin_cache must be float32 [max_position, rope_dim]")
        max_pos, rope_dim = cos_sin_cache.shape
    if q is not None and (q.dim() != 3 or q.shape[0] != key.shape[0] or q.shape[2] != D or q.dtype != key.dtype):
        raise ValueError("q must be [T, Hq, D] of key's dtype")
    shape = pad_cache_shape(
        num_tokens=key.shape[0], num_q_heads=q.shape[1] if q is not None else 0, num_kv_heads=Hkv, head_size=D,
        page_size=P, num_blocks=nb, dtype=_DTYPE_CODE[key.dtype], layout=layout, rope_dim=rope_dim,
        max_position=max_pos,
    )
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)  # noqa: E731
    _check(lib.pad_rope_cache_write(
        ctypes.byref(shape), ptr(q), ptr(key), ptr(value), ptr(slot_mapping), ptr(positions), ptr(cos_sin_cache),
        ptr(kv_cache), ctypes.c_void_p(_stream_ptr(stream))), "pad_rope_cache_write")


def pad_calib_gather_read(kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                          query_len: int, num_q_heads: int, window: int, sink: torch.Tensor, *,
                          layout: int = PAD_HND, waves: int = 4, tiles_in_flight: int = 1, segments: int = 32,
                          stream=None) -> None:
    """Read the pages a decode call would attend, computing nothing
    (include/pad_calib.h); ``sink`` is a device int32 tensor."""
    D = kv_cache.shape[-1]
    q_like = torch.empty((block_table.shape[0], query_len, num_q_heads, D), dtype=kv_cache.dtype, device="meta")
    shape = make_shape(q_like, kv_cache, block_table, layout)
    _check(lib.pad_calib_gather_read(
        ctypes.byref(shape), ctypes.c_void_p(kv_cache.data_ptr()), ctypes.c_void_p(block_table.data_ptr()),
        ctypes.c_void_p(seq_lens.data_ptr()), int(window), int(waves), int(tiles_in_flight), int(segments),
        ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(_stream_ptr(stream))), "pad_calib_gather_read")


def pad_calib_stream_read(src: torch.Tensor, sink: torch.Tensor, *, blocks: int = 2048, threads: int = 256,
                          loads_in_flight: int = 4, stream=None) -> None:
    """Read every byte of the contiguous device tensor ``src`` (include/pad_calib.h)."""
    _check(lib.pad_calib_stream_read(
        ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(), int(blocks), int(threads),
        int(loads_in_flight), ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(_stream_ptr(stream))),
        "pad_calib_stream_read")


def pad_octave_slot_bytes(fmt: int, head_size: int = 256) -> int:
    """Bytes of one packed slot (include/pad_octave.h)."""
    n = ctypes.c_int32(0)
    _check(lib.pad_octave_slot_bytes(int(fmt), int(head_size), ctypes.byref(n)), "pad_octave_slot_bytes")
    return int(n.value)


def _octave_cache_dims(cache: torch.Tensor, layout: int):
    if cache.dim() != 4 or cache.dtype != torch.uint8:
        raise ValueError("a packed cache is uint8 [blocks, kv_heads, page, slot] (HND) or [blocks, page, kv_heads, slot]")
    if layout == PAD_HND:
        nb, Hkv, P, sb = cache.shape
    elif layout == PAD_NHD:
        nb, P, Hkv, sb = cache.shape
    else:
        raise ValueError(f"unknown layout {layout}")
    return nb, Hkv, P, sb


def pad_octave_cache_write(key: torch.Tensor, value: torch.Tensor, cache: torch.Tensor, slot_mapping: torch.Tensor,
                           k_signs: torch.Tensor, v_signs: torch.Tensor, fmt: int, *, layout: int = PAD_HND,
                           stream=None) -> None:
    """Rotate, quantize and pack new tokens' K and V rows ``[T, Hkv, 256]``
    into their slots of a packed cache (include/pad_octave.h)."""
    _require_device(key=key, value=value, cache=cache, slot_mapping=slot_mapping, k_signs=k_signs, v_signs=v_signs)
    nb, Hkv, P, sb = _octave_cache_dims(cache, layout)
    if key.dim() != 3 or value.shape != key.shape or key.dtype not in _DTYPE_CODE or value.dtype != key.dtype:
        raise ValueError("key and value must be [T, Hkv, 256] of one dtype (float16 or bfloat16)")
    if key.shape[1] != Hkv or sb != pad_octave_slot_bytes(fmt, key.shape[2]):
        raise ValueError("the cache's kv heads and slot size must match key and the format")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (key.shape[0],):
        raise ValueError("slot_mapping must be int64 [T]")
    for n, t in (("k_signs", k_signs), ("v_signs", v_signs)):
        if t.dtype not in (torch.int32, torch.uint32) or t.numel() != key.shape[2] // 32:
            raise ValueError(f"{n} must hold head_size / 32 32-bit words")
    shape = pad_octave_cache_shape(num_tokens=key.shape[0], num_kv_heads=Hkv, head_size=key.shape[2], page_size=P,
                                   num_blocks=nb, dtype=_DTYPE_CODE[key.dtype], layout=layout, format=int(fmt))
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    _check(lib.pad_octave_cache_write(ctypes.byref(shape), ptr(key), ptr(value), ptr(slot_mapping), ptr(k_signs),
                                      ptr(v_signs), ptr(cache), ctypes.c_void_p(_stream_ptr(stream))),
           "pad_octave_cache_write")


def _octave_shape(q, cache, block_table, layout, fmt, **kw) -> pad_shape:
    nb, Hkv, P, sb = _octave_cache_dims(cache, layout)
    if q.dim() != 4 or q.dtype not in _DTYPE_CODE:
        raise ValueError("q must be [S, M, Hq, D] of float16 or bfloat16")
    S, M, Hq, D = q.shape
    if sb != pad_octave_slot_bytes(fmt, D):
        raise ValueError("the cache's slot size does not match the format")
    if block_table.shape[0] != S:
        raise ValueError("block_table must have one row per sequence")
    return pad_shape(num_seqs=S, query_len=M, num_q_heads=Hq, num_kv_heads=Hkv, head_size=D, page_size=P,
                     max_blocks_per_seq=block_table.shape[1], max_seq_len=kw.get("max_seq_len", 0),
                     dtype=_DTYPE_CODE[q.dtype], layout=layout, num_segments=kw.get("num_segments", 0),
                     path=kw.get("path", PAD_PATH_AUTO), schedule=kw.get("schedule", PAD_SCHED_AUTO))


def pad_decode_attn_octave_workspace_size(shape: pad_shape, fmt: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.pad_decode_attn_octave_workspace_size(ctypes.byref(shape), int(fmt), ctypes.byref(n)),
           "pad_decode_attn_octave_workspace_size")
    return int(n.value)


def _octave_workspace(device, shape: pad_shape, fmt: int, stream) -> torch.Tensor | None:
    """The default packed-cache workspace of (device, stream): grown and
    zeroed on that stream when a shape needs more."""
    key = (device.index, _stream_ptr(stream), "octave")
    ws_obj = _default_ws.get(key)
    if ws_obj is None:
        ws_obj = _default_ws[key] = Workspace(device)
    need = pad_decode_attn_octave_workspace_size(shape, fmt)
    if need and (ws_obj.buf is None or ws_obj.buf.numel() < need):
        buf = torch.empty(need, dtype=torch.uint8, device=device)
        _record_on(buf, stream)
        pad_decode_attn_workspace_init(buf, stream)
        ws_obj.buf = buf
    return ws_obj.buf


def pad_decode_attn_octave(q: torch.Tensor, cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                           k_signs: torch.Tensor, v_signs: torch.Tensor, scale: float, out: torch.Tensor, fmt: int, *,
                           layout: int = PAD_HND, workspace: torch.Tensor | None = None, max_seq_len: int = 0,
                           num_segments: int = 0, path: int = PAD_PATH_AUTO, schedule: int = PAD_SCHED_AUTO,
                           stream=None) -> torch.Tensor:
    """Decode attention over a packed quantized cache into ``out``
    (include/pad_octave.h): q and out in the model's space, no window."""
    _require_device(q=q, cache=cache, block_table=block_table, seq_lens=seq_lens, k_signs=k_signs, v_signs=v_signs,
                    out=out)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or seq_lens.shape != (q.shape[0],):
        raise ValueError("block_table and seq_lens must be int32, one row / entry per sequence")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    shape = _octave_shape(q, cache, block_table, layout, fmt, max_seq_len=max_seq_len, num_segments=num_segments,
                          path=path, schedule=schedule)
    ws = _octave_workspace(q.device, shape, fmt, stream) if workspace is None else workspace
    ws_ptr = ws.data_ptr() if ws is not None else 0
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    _check(lib.pad_decode_attn_octave(
        ctypes.byref(shape), int(fmt), ptr(q), ptr(cache), ptr(block_table), ptr(seq_lens), ptr(k_signs), ptr(v_signs),
        ctypes.c_float(scale), ptr(out), ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_bytes),
        ctypes.c_void_p(_stream_ptr(stream))), "pad_decode_attn_octave")
    return out


def pad_decode_attn_octave_varlen(q: torch.Tensor, q_start: torch.Tensor, cache: torch.Tensor,
                                  block_table: torch.Tensor, seq_lens: torch.Tensor, k_signs: torch.Tensor,
                                  v_signs: torch.Tensor, scale: float, out: torch.Tensor, fmt: int, *,
                                  max_query_len: int = 8, layout: int = PAD_HND, workspace: torch.Tensor | None = None,
                                  max_seq_len: int = 0, num_segments: int = 0, path: int = PAD_PATH_AUTO,
                                  schedule: int = PAD_SCHED_AUTO, stream=None) -> torch.Tensor:
    """Packed-cache decode with a query count per sequence
    (include/pad_octave.h): ``q`` and ``out`` are packed ``[T, Hq, 256]``;
    sequence ``s`` owns rows ``q_start[s] .. q_start[s + 1] - 1``
    (``q_start``: device int32, ``S + 1`` entries, never read on the host);
    ``max_query_len`` bounds every per-sequence count."""
    _require_device(q=q, q_start=q_start, cache=cache, block_table=block_table, seq_lens=seq_lens, k_signs=k_signs,
                    v_signs=v_signs, out=out)
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must be packed [T, Hq, D] tensors of one dtype")
    S = block_table.shape[0]
    if q_start.dtype != torch.int32 or q_start.shape != (S + 1,):
        raise ValueError("q_start must be int32 with one entry per sequence plus one")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or seq_lens.shape != (S,):
        raise ValueError("block_table and seq_lens must be int32, one row / entry per sequence")
    T, Hq, D = q.shape
    q_like = torch.empty((S, max_query_len, Hq, D), dtype=q.dtype, device="meta")
    shape = _octave_shape(q_like, cache, block_table, layout, fmt, max_seq_len=max_seq_len, num_segments=num_segments,
                          path=path, schedule=schedule)
    ws = _octave_workspace(q.device, shape, fmt, stream) if workspace is None else workspace
    ws_ptr = ws.data_ptr() if ws is not None else 0
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    _check(lib.pad_decode_attn_octave_varlen(
        ctypes.byref(shape), int(fmt), ptr(q), ptr(q_start), ptr(cache), ptr(block_table), ptr(seq_lens), ptr(k_signs),
        ptr(v_signs), ctypes.c_float(scale), ptr(out), ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_bytes),
        ctypes.c_void_p(_stream_ptr(stream))), "pad_decode_attn_octave_varlen")
    return out
