"""The C-ABI library on the CPU: it loads, exports every declared symbol,
plans shapes and rejects invalid calls before touching a GPU."""

import ctypes
import os
import re

import pytest

import paged_kv_decode_block_amd as pad

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pad_attn.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def _declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(pad_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert "pad_decode_attn" in names and "pad_decode_attn_workspace_size" in names
    assert "pad_calib_gather_read" in names and "pad_calib_stream_read" in names
    lib = ctypes.CDLL(pad.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"libpad_attn.so does not export {n}"


def test_abi_version_matches_header():
    m = re.search(r"#define PAD_ABI_VERSION (\d+)", open(HEADER).read())
    assert pad.pad_abi_version() == int(m.group(1))


def test_status_strings():
    for code in range(6):
        assert pad.pad_status_string(code) and pad.pad_status_string(code) != "unknown status"
    assert pad.pad_status_string(77) == "unknown status"


def shape(**kw):
    base = dict(num_seqs=1, query_len=4, num_q_heads=32, num_kv_heads=8, head_size=128, page_size=16,
                max_blocks_per_seq=2048, max_seq_len=0, dtype=pad.PAD_BF16, layout=pad.PAD_HND,
                num_segments=0, path=0, schedule=0)
    base.update(kw)
    return pad.pad_shape(**base)


def plan(sh, window=0, cus=256):
    return pad.pad_decode_attn_plan(sh, window, cus)


def _align(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize(
    "kw",
    [
        dict(),
        dict(query_len=1),
        dict(num_q_heads=4, num_kv_heads=1, head_size=64, max_blocks_per_seq=16, dtype=pad.PAD_F16),
        dict(num_q_heads=8, num_kv_heads=2, head_size=256, page_size=32, max_blocks_per_seq=512, layout=pad.PAD_NHD),
        dict(num_q_heads=16, num_kv_heads=2, head_size=512, page_size=32, max_blocks_per_seq=1024, query_len=8),
        dict(num_seqs=65, num_q_heads=16, num_kv_heads=2, head_size=256, page_size=1056, max_blocks_per_seq=16),
    ],
)
def test_plan_invariants(kw):
    sh = shape(**kw)
    p = plan(sh)
    G = sh.num_q_heads // sh.num_kv_heads
    rows = G * sh.query_len
    assert p["rows"] == rows
    # 16-row tiles per workgroup times workgroups per kv head cover the rows
    assert p["row_tiles"] * p["row_groups"] * 16 >= rows
    assert (p["row_tiles"] - 1) * p["row_groups"] * 16 < rows
    keys = sh.max_blocks_per_seq * sh.page_size
    tiles = -(-keys // 16)
    assert p["num_segments"] * p["segment_tiles"] >= tiles
    assert (p["num_segments"] - 1) * p["segment_tiles"] < tiles
    assert 1 <= p["num_segments"] <= 256
    D = sh.head_size
    if p["persistent"]:
        # one workgroup per CU, each taking an equal share of the batch's
        # tiles; two partial slots of one workgroup's rows per workgroup,
        # after the 1 MiB control prefix, and the last arriver merges alone
        assert p["grid_y"] == 1 and p["grid_x"] == 256 and p["num_segments"] == 1
        slot_rows = min(rows, p["row_tiles"] * 16)
        bal = (1 << 20) + _align(512 * slot_rows * 2 * 4) + _align(512 * slot_rows * D * 4)
        assert p["workspace_bytes"] >= bal
        assert p["merge_slices"] == 1
        return
    # segments stay within 4096 tiles (the LDS block-id stage) for any
    # device length up to the table's capacity
    assert p["segment_tiles"] <= 4096 and -(-tiles // p["num_segments"]) <= 4096
    assert p["grid_x"] == p["num_segments"] * sh.num_kv_heads * p["row_groups"]
    assert p["grid_y"] == sh.num_seqs
    S, H = sh.num_seqs, sh.num_kv_heads
    if p["num_segments"] == 1:
        assert p["merge_slices"] == 1
        if S == 1:
            assert p["workspace_bytes"] == 0
    else:
        # a fixed 1 MiB prefix of merge control words, then one (m, l) and one
        # acc slot per segment (or the balanced grid's slots, if larger, for a
        # batch that another window would put there)
        n = p["num_segments"]
        nw = p["workspace_segments"]
        assert nw >= n
        want = (1 << 20) + _align(S * H * nw * rows * 2 * 4) + _align(S * H * nw * rows * D * 4)
        assert p["workspace_bytes"] >= want
        if S == 1:
            assert p["workspace_bytes"] == want
        # about 32 KiB of partial accumulators per merge slice, at most 32
        # slices and no more than segments; control words fit the prefix
        k = p["merge_slices"]
        wg_rows = min(rows, p["row_tiles"] * 16)
        vol = n * wg_rows * D * 4
        assert 1 <= k <= min(32, n)
        # control words one 128-byte line apart; helpers only when the
        # whole grid is resident (one workgroup per CU)
        resident = p["grid_x"] * p["grid_y"] <= 256
        want_k = min(-(-vol // (32 << 10)), 32, n, (1 << 20) // (128 * S * H * p["row_groups"])) \
            if resident else 1
        assert k == want_k
        assert S * H * p["row_groups"] * k * 128 <= 1 << 20


def test_plan_bounds_segment_length():
    # a large table with a small planning bound: segments still cover the
    # whole table within 4096 tiles each
    p = plan(shape(max_blocks_per_seq=200000, max_seq_len=1000))
    tiles = 200000 * 16 // 16
    assert -(-tiles // p["num_segments"]) <= 4096 and p["segment_tiles"] <= 4096
    p = plan(shape(max_blocks_per_seq=200000, num_segments=1))
    assert p["num_segments"] >= 49
    with pytest.raises(pad.PadError) as e:
        plan(shape(max_blocks_per_seq=(1 << 30) // 16 + 1))
    assert e.value.status == pad.PAD_EUNSUPPORTED
    with pytest.raises(pad.PadError) as e:
        plan(shape(max_blocks_per_seq=(256 * 4096) + 1))
    assert e.value.status == pad.PAD_EUNSUPPORTED


def test_schedule_plan():
    batch = dict(num_seqs=65, num_q_heads=16, num_kv_heads=2, head_size=256, page_size=1056, max_blocks_per_seq=16)
    p = plan(shape(**batch))
    assert p["persistent"] == 1 and p["grid_x"] == 256 and p["grid_y"] == 1
    # the balanced grid splits by share: no segment count, the last arriver
    # merges alone, and a forced segment count does not change it
    assert p["num_segments"] == 1 and p["merge_slices"] == 1
    b = plan(shape(num_segments=8, schedule=pad.PAD_SCHED_PERSISTENT, **batch))
    assert (b["persistent"], b["num_segments"], b["grid_x"]) == (1, 1, 256)
    g = plan(shape(schedule=pad.PAD_SCHED_GRID, **batch))
    assert g["persistent"] == 0 and g["grid_y"] == 65
    # the automatic schedule's workspace also serves the grid the batch
    # takes under a window
    assert p["workspace_bytes"] >= g["workspace_bytes"]
    # a grid larger than one workgroup per CU: the last arriver merges alone
    a = plan(shape(num_segments=8, schedule=pad.PAD_SCHED_GRID, **batch))
    assert a["grid_x"] * a["grid_y"] > 256 and a["merge_slices"] == 1
    wide = dict(num_q_heads=16, num_kv_heads=2, head_size=512, page_size=32, max_blocks_per_seq=1024, query_len=8)
    assert plan(shape(num_segments=32, **wide))["merge_slices"] == 32  # 256 workgroups
    assert plan(shape(num_segments=48, **wide))["merge_slices"] == 1  # 384 workgroups
    # batch 1 stays on one workgroup per item unless asked
    assert plan(shape())["persistent"] == 0
    one = plan(shape(schedule=pad.PAD_SCHED_PERSISTENT, num_segments=1, max_blocks_per_seq=4))
    rows = 16
    assert one["persistent"] == 1 and one["num_segments"] == 1
    assert one["workspace_bytes"] == (1 << 20) + _align(512 * rows * 8) + _align(512 * rows * 128 * 4)
    # the balanced grid needs the batch's tiles to count in 32 bits and one
    # control word per unit in the 1 MiB prefix; otherwise a batch stays on
    # the grid, and asking for the balanced grid is rejected
    many = dict(num_seqs=1000, num_q_heads=64, num_kv_heads=16, head_size=128, max_blocks_per_seq=64)
    assert plan(shape(**many))["persistent"] == 0  # 16000 units of control words
    with pytest.raises(pad.PadError) as e:
        plan(shape(schedule=pad.PAD_SCHED_PERSISTENT, **many))
    assert e.value.status == pad.PAD_EUNSUPPORTED
    huge = dict(num_seqs=512, num_kv_heads=8, num_q_heads=8, max_blocks_per_seq=600000)
    assert plan(shape(**huge))["persistent"] == 0  # 4096 units x 600001 tiles >= 2^31
    # a long share is walked in chunks of staged block ids: no bound on the
    # tiles per workgroup
    long_batch = plan(shape(num_seqs=8, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=60000,
                            schedule=pad.PAD_SCHED_PERSISTENT))
    assert long_batch["persistent"] == 1 and long_batch["segment_tiles"] == 60000


def test_plan_fills_device():
    # batch 1, 8 kv heads, long context: enough workgroups for every CU
    p = plan(shape(), cus=256)
    assert p["grid_x"] * p["grid_y"] >= 256


@pytest.mark.parametrize("M", [3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("keys", [1024, 4096, 8192, 16384, 32768])
def test_plan_keeps_row_groups_on_one_xcd(M, keys):
    """With several row groups an automatic plan keeps segments x kv heads
    a multiple of the 8 XCDs, the condition under which the kernel places a
    (kv head, segment)'s row groups on one die."""
    p = plan(shape(num_q_heads=16, num_kv_heads=2, head_size=512, page_size=32,
                   max_blocks_per_seq=keys // 32, query_len=M))
    assert p["row_groups"] > 1
    assert (p["num_segments"] * 2) % 8 == 0, p
    assert p["grid_x"] <= 256  # resident: merge helpers take part


def test_plan_partial_bound_for_wide_heads():
    """Head size 512 with 16 live rows per workgroup: segments keep their
    partial below a sixth of their K/V bytes while 32 or more remain; short
    contexts keep the shorter segments that fill the device."""
    wide = dict(num_q_heads=16, num_kv_heads=2, head_size=512, page_size=32, query_len=2)
    part, tile = 16 * (512 + 2) * 4, 16 * 2 * 512 * 2
    for keys in (4096, 8192, 32768):
        p = plan(shape(max_blocks_per_seq=keys // 32, **wide))
        assert p["segment_tiles"] * tile >= 6 * part or p["num_segments"] < 32, (keys, p)
    short = plan(shape(max_blocks_per_seq=1024 // 32, **wide))
    assert short["num_segments"] == 16
    # the default workload's plan does not move
    assert plan(shape())["num_segments"] == 32


def test_plan_short_contexts_use_short_segments():
    """About 64 KiB of K/V per segment (8 tiles at head size 128), 4 and
    then 2 tiles while that leaves fewer than 16 segments, capped by one
    workgroup per CU; a unit of at most 64 KiB of K/V is one segment."""
    for keys, want in ((128, 1), (256, 8), (512, 16), (1024, 16), (2048, 16), (4096, 32), (8192, 32),
                       (32768, 32)):
        p = plan(shape(max_blocks_per_seq=keys // 16))
        assert p["num_segments"] == want, (keys, p)
        assert p["segment_tiles"] >= 2 or p["num_segments"] == 1
    one = plan(shape(num_q_heads=4, num_kv_heads=1, head_size=64, max_blocks_per_seq=16, dtype=pad.PAD_F16,
                     query_len=1))  # 256 keys of head size 64: 64 KiB per unit
    assert one["num_segments"] == 1 and one["workspace_bytes"] == 0


def test_forced_segments():
    for n in (1, 2, 7, 256):
        p = plan(shape(num_segments=n, max_blocks_per_seq=64))
        tiles = 64  # 1024 keys / 16
        assert p["num_segments"] <= n
        assert p["num_segments"] * p["segment_tiles"] >= tiles
        if n <= tiles:
            assert p["num_segments"] == -(-tiles // -(-tiles // n))


def test_dot_path_plan():
    p = plan(shape(query_len=1, path=pad.PAD_PATH_DOT))  # 4 rows, D=128
    assert p["path"] == pad.PAD_PATH_DOT and p["waves"] == 4 and p["row_groups"] == 1
    assert plan(shape(query_len=1))["path"] == pad.PAD_PATH_MFMA  # automatic choice
    p = plan(shape(num_q_heads=8, num_kv_heads=8, head_size=64, query_len=1, path=pad.PAD_PATH_DOT))
    assert p["rows"] == 1 and p["path"] == pad.PAD_PATH_DOT


def test_window_plan_is_smaller():
    full = plan(shape(max_blocks_per_seq=1024))
    win = plan(shape(max_blocks_per_seq=1024), window=512)
    assert win["workspace_bytes"] <= full["workspace_bytes"]
    assert win["num_segments"] * win["segment_tiles"] * 16 >= 512 + 4 - 1 + 15


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(query_len=0), pad.PAD_EINVAL),
        (dict(query_len=4097), pad.PAD_EUNSUPPORTED),
        (dict(query_len=2048, num_q_heads=256, num_kv_heads=8), pad.PAD_EUNSUPPORTED),  # 65536 rows
        (dict(head_size=96), pad.PAD_EUNSUPPORTED),
        (dict(head_size=0), pad.PAD_EINVAL),
        (dict(page_size=8), pad.PAD_EUNSUPPORTED),
        (dict(page_size=24), pad.PAD_EUNSUPPORTED),
        (dict(num_q_heads=30), pad.PAD_EINVAL),
        (dict(num_kv_heads=0), pad.PAD_EINVAL),
        (dict(dtype=2), pad.PAD_EINVAL),
        (dict(layout=5), pad.PAD_EINVAL),
        (dict(max_seq_len=2048 * 16 + 1), pad.PAD_EINVAL),
        (dict(num_segments=-1), pad.PAD_EINVAL),
        (dict(path=4), pad.PAD_EINVAL),
        (dict(path=-1), pad.PAD_EINVAL),
        (dict(path=pad.PAD_PATH_PREFILL, head_size=256), pad.PAD_EUNSUPPORTED),
        (dict(path=pad.PAD_PATH_PREFILL, schedule=pad.PAD_SCHED_PERSISTENT), pad.PAD_EUNSUPPORTED),
        (dict(schedule=3), pad.PAD_EINVAL),
        (dict(schedule=-1), pad.PAD_EINVAL),
        (dict(schedule=pad.PAD_SCHED_PERSISTENT, num_seqs=1025), pad.PAD_EUNSUPPORTED),
        (dict(path=pad.PAD_PATH_DOT), pad.PAD_EUNSUPPORTED),  # 16 rows: too many for the dot family
        (dict(path=pad.PAD_PATH_DOT, query_len=1, head_size=256), pad.PAD_EUNSUPPORTED),
        (dict(num_seqs=-1), pad.PAD_EINVAL),
        (dict(max_blocks_per_seq=0), pad.PAD_EINVAL),
        # one block of more than 2^31 - 1 elements (the kernel's strides are 32-bit)
        (dict(head_size=512, num_q_heads=64, num_kv_heads=64, page_size=32768, query_len=1, max_blocks_per_seq=4),
         pad.PAD_EUNSUPPORTED),
    ],
)
def test_plan_rejects(kw, status):
    with pytest.raises(pad.PadError) as e:
        plan(shape(**kw))
    assert e.value.status == status


def test_plan_accepts_largest_32bit_block():
    # 64 kv heads x 32752 tokens x 2 x 512 elements = 2,146,435,072 < 2^31.
    p = plan(shape(head_size=512, num_q_heads=64, num_kv_heads=64, page_size=32752, query_len=1, max_blocks_per_seq=4))
    assert p["num_segments"] >= 1


def test_plan_rejects_bad_window_and_cus():
    with pytest.raises(pad.PadError):
        plan(shape(), window=-1)
    with pytest.raises(pad.PadError):
        plan(shape(), cus=0)


def _call(sh, q=0x1000, kv=0x2000, bt=0x3000, sl=0x4000, out=0x5000, scale=1.0, window=0, ws=None, ws_bytes=0):
    P = ctypes.c_void_p
    return pad.lib.pad_decode_attn(ctypes.byref(sh) if sh is not None else None, P(q), P(kv), P(bt), P(sl),
                                   ctypes.c_float(scale), ctypes.c_int32(window), P(out), P(ws),
                                   ctypes.c_size_t(ws_bytes), None)


def test_decode_validates_before_launch():
    # None of these reaches the GPU: validation fails first (fake addresses).
    one_seg = shape(num_segments=1)
    assert _call(None) == pad.PAD_EINVAL
    assert _call(one_seg, scale=float("nan")) == pad.PAD_EINVAL
    assert _call(one_seg, scale=float("inf")) == pad.PAD_EINVAL
    assert _call(one_seg, q=0) == pad.PAD_EINVAL
    assert _call(one_seg, kv=0) == pad.PAD_EINVAL
    assert _call(one_seg, bt=0) == pad.PAD_EINVAL
    assert _call(one_seg, sl=0) == pad.PAD_EINVAL
    assert _call(one_seg, out=0) == pad.PAD_EINVAL
    assert _call(one_seg, q=0x1008) == pad.PAD_EINVAL  # 16-byte alignment
    assert _call(one_seg, kv=0x2004) == pad.PAD_EINVAL
    assert _call(one_seg, out=0x5002) == pad.PAD_EINVAL
    assert _call(one_seg, bt=0x3002) == pad.PAD_EINVAL  # 4-byte alignment
    assert _call(one_seg, window=-3) == pad.PAD_EINVAL
    assert _call(shape(query_len=4097)) == pad.PAD_EUNSUPPORTED
    split = shape(num_segments=4)
    need = plan(split)["workspace_bytes"]
    assert need > 0
    assert _call(split) == pad.PAD_EWORKSPACE
    assert _call(split, ws=0x10000, ws_bytes=need - 1) == pad.PAD_EWORKSPACE
    assert _call(split, ws=0x10010, ws_bytes=need) == pad.PAD_EWORKSPACE  # 256-byte alignment
    # an empty batch is a successful no-op, even with no buffers
    assert _call(shape(num_seqs=0), q=0, kv=0, bt=0, sl=0, out=0) == pad.PAD_OK


def test_workspace_size_and_init_validation():
    assert pad.pad_decode_attn_workspace_size(shape()) == plan(shape())["workspace_bytes"]
    P = ctypes.c_void_p
    assert pad.lib.pad_decode_attn_workspace_init(P(0), ctypes.c_size_t(0), None) == pad.PAD_OK
    assert pad.lib.pad_decode_attn_workspace_init(P(0), ctypes.c_size_t(256), None) == pad.PAD_EINVAL
    assert pad.lib.pad_decode_attn_workspace_init(P(0x1010), ctypes.c_size_t(256), None) == pad.PAD_EINVAL


def test_merge_wait_bounds():
    assert pad.lib.pad_set_merge_wait(-1) == pad.PAD_EINVAL
    assert pad.lib.pad_set_merge_wait(1000001) == pad.PAD_EINVAL
    assert pad.lib.pad_set_merge_wait(0) == pad.PAD_OK
    assert pad.lib.pad_set_merge_wait(200) == pad.PAD_OK


def test_calibration_validation():
    """The read-ceiling kernels reject bad arguments on the host (no launch)."""
    P = ctypes.c_void_p
    L = pad.lib

    def g(sh, waves=4, tif=1, segs=32, window=0, ptr=0x1000):
        return L.pad_calib_gather_read(ctypes.byref(sh), P(ptr), P(ptr), P(ptr), window, waves, tif, segs, P(ptr),
                                       None)

    assert g(shape(num_seqs=0)) == pad.PAD_OK  # nothing to read
    assert g(shape(num_seqs=0), waves=5) == pad.PAD_EINVAL
    assert g(shape(num_seqs=0), tif=3) == pad.PAD_EINVAL
    assert g(shape(num_seqs=0), segs=0) == pad.PAD_EINVAL
    assert g(shape(num_seqs=0), segs=257) == pad.PAD_EINVAL
    assert g(shape(num_seqs=0, head_size=96)) == pad.PAD_EUNSUPPORTED
    assert g(shape(num_seqs=0, head_size=512, num_q_heads=16, num_kv_heads=2), tif=2) == pad.PAD_EUNSUPPORTED
    assert g(shape(), window=-1) == pad.PAD_EINVAL
    assert g(shape(), ptr=0) == pad.PAD_EINVAL  # missing buffers
    assert g(shape(), ptr=0x1008) == pad.PAD_EINVAL  # kv_cache not 16-byte aligned
    assert L.pad_calib_stream_read(P(0), ctypes.c_size_t(0), 256, 256, 4, P(0), None) == pad.PAD_OK
    assert L.pad_calib_stream_read(P(0x1000), ctypes.c_size_t(24), 256, 256, 4, P(0x1000), None) == pad.PAD_EINVAL
    assert L.pad_calib_stream_read(P(0x1000), ctypes.c_size_t(32), 0, 256, 4, P(0x1000), None) == pad.PAD_EINVAL
    assert L.pad_calib_stream_read(P(0x1008), ctypes.c_size_t(32), 256, 256, 4, P(0x1000), None) == pad.PAD_EINVAL
    for threads, loads in ((128, 4), (256, 2), (2048, 8), (512, 32)):
        assert L.pad_calib_stream_read(P(0x1000), ctypes.c_size_t(32), 256, threads, loads, P(0x1000),
                                       None) == pad.PAD_EINVAL


def test_varlen_validation():
    """The packed-query entry point needs its q_start array (checked on the
    host before any launch); an empty batch needs nothing."""
    P = ctypes.c_void_p
    L = pad.lib

    def v(sh, qs):
        return L.pad_decode_attn_varlen(ctypes.byref(sh), P(0x1000), P(qs), P(0x1000), P(0x1000), P(0x1000),
                                        ctypes.c_float(0.1), 0, P(0x1000), P(0), ctypes.c_size_t(0), None)

    assert v(shape(num_seqs=0), 0) == pad.PAD_OK
    assert v(shape(), 0) == pad.PAD_EINVAL  # missing q_start
    assert v(shape(), 0x1002) == pad.PAD_EINVAL  # misaligned q_start
    assert v(shape(query_len=4097), 0x1000) == pad.PAD_EUNSUPPORTED  # bound on the per-sequence counts


def test_workspace_serves_every_window():
    """One workspace size per shape: every window's plan needs the same
    bytes, with at least as many segment slots as it uses (seeded shapes,
    forced and planned segment counts, all schedules)."""
    import numpy as np

    r = np.random.default_rng(11)
    for _ in range(300):
        D = int(r.choice([64, 128, 256, 512]))
        Hkv = int(r.choice([1, 2, 4, 8]))
        G = int(r.choice([1, 2, 4, 8, 16]))
        M = int(r.integers(1, 9))
        P = int(r.choice([16, 32, 48, 1056]))
        sh = shape(num_seqs=int(r.choice([1, 2, 5, 65, 1100])), query_len=M, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                   head_size=D, page_size=P, max_blocks_per_seq=int(r.integers(1, 600)),
                   num_segments=int(r.choice([0, 0, 1, 3, 16, 200])), schedule=int(r.choice([0, 1, 2])))
        try:
            base = pad.pad_decode_attn_workspace_size(sh)
        except pad.PadError:
            continue
        for w in (0, 1, 5, 16, 17, 100, 511, 512, 4000, 10 ** 6):
            p = plan(sh, w)
            assert p["workspace_bytes"] == base, (sh.num_seqs, D, Hkv, G, M, P, w, p)
            assert p["workspace_segments"] >= p["num_segments"]


def test_cache_write_validation():
    """Host checks of the cache write, before any launch."""
    P = ctypes.c_void_p
    L = pad.lib

    def w(ptr=0x1000, pos=0x1000, tab=0x1000, **kw):
        base = dict(num_tokens=4, num_q_heads=8, num_kv_heads=2, head_size=128, page_size=16, num_blocks=4,
                    dtype=pad.PAD_BF16, layout=pad.PAD_HND, rope_dim=64, max_position=100)
        base.update(kw)
        sh = pad.pad_cache_shape(**base)
        return L.pad_rope_cache_write(ctypes.byref(sh), P(ptr), P(ptr), P(ptr), P(ptr), P(pos), P(tab), P(ptr), None)

    assert w(num_tokens=0) == pad.PAD_OK
    assert w(head_size=96) == pad.PAD_EUNSUPPORTED
    assert w(rope_dim=40) == pad.PAD_EUNSUPPORTED  # not a multiple of 16
    assert w(rope_dim=256) == pad.PAD_EUNSUPPORTED  # wider than the head
    assert w(num_q_heads=3) == pad.PAD_EINVAL
    assert w(max_position=0) == pad.PAD_EINVAL
    assert w(pos=0) == pad.PAD_EINVAL  # rotation without positions
    assert w(ptr=0x1008) == pad.PAD_EINVAL  # misaligned tensors
    assert w(dtype=5) == pad.PAD_EINVAL


def test_dot_family_stays_on_the_grid():
    """The dot family has no persistent-grid build: a batch that would
    otherwise go persistent keeps one workgroup per item, and asking for the
    persistent schedule is rejected."""
    batch = dict(num_seqs=200, query_len=1, path=pad.PAD_PATH_DOT)
    p = plan(shape(**batch))
    assert p["path"] == pad.PAD_PATH_DOT and p["persistent"] == 0 and p["grid_y"] == 200
    assert plan(shape(num_seqs=200, query_len=1))["persistent"] == 1  # the key-split family does go persistent
    with pytest.raises(pad.PadError) as e:
        plan(shape(schedule=pad.PAD_SCHED_PERSISTENT, **batch))
    assert e.value.status == pad.PAD_EUNSUPPORTED


def test_noalloc_validates_before_launch():
    """The allocation-free entry point runs the decode's host checks, and
    rejects a call whose workspace exceeds its fixed array, before it
    touches the device (fake addresses: nothing here reaches a GPU)."""
    L = pad.lib
    P = ctypes.c_void_p

    def call(sh, q=0x1000, kv=0x2000, bt=0x3000, sl=0x4000, scale=0.1, window=0, out=0x5000):
        return L.pad_decode_attn_noalloc(ctypes.byref(sh) if sh is not None else None, P(q), P(kv), P(bt), P(sl),
                                         ctypes.c_float(scale), window, P(out), None)

    assert pad.PAD_NOALLOC_SCRATCH_BYTES == 64 << 20
    m = re.search(r"#define PAD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == pad.PAD_NOALLOC_SCRATCH_BYTES
    one_seg = shape(num_segments=1)
    assert plan(one_seg)["workspace_bytes"] == 0
    assert call(None) == pad.PAD_EINVAL
    assert call(one_seg, scale=float("nan")) == pad.PAD_EINVAL
    assert call(one_seg, q=0) == pad.PAD_EINVAL
    assert call(one_seg, q=0x1008) == pad.PAD_EINVAL
    assert call(one_seg, bt=0x3002) == pad.PAD_EINVAL
    assert call(one_seg, window=-1) == pad.PAD_EINVAL
    assert call(shape(query_len=4097)) == pad.PAD_EUNSUPPORTED
    # a split call with bad pointers fails on the pointers, not the device
    assert plan(shape(num_segments=4))["workspace_bytes"] > 0
    assert call(shape(num_segments=4), out=0) == pad.PAD_EINVAL
    big = shape(num_seqs=64, num_q_heads=64, num_kv_heads=8, head_size=512, query_len=8, page_size=16,
                max_blocks_per_seq=2048, num_segments=64, schedule=pad.PAD_SCHED_GRID)
    assert plan(big)["workspace_bytes"] > pad.PAD_NOALLOC_SCRATCH_BYTES
    assert call(big) == pad.PAD_ESCRATCH
    assert call(big, q=0) == pad.PAD_ESCRATCH  # the size bound is checked first
    assert call(shape(num_seqs=0), q=0, kv=0, bt=0, sl=0, out=0) == pad.PAD_OK


def test_octave_validation():
    """Host checks of the packed-cache entry points (no GPU: every call
    fails or returns before a launch)."""
    L = pad.lib
    P = ctypes.c_void_p
    for fmt, want in ((pad.PAD_KV_OCTAVE_K3V4, 240), (pad.PAD_KV_OCTAVE_K3V3, 208),
                      (pad.PAD_KV_OCTAVE_K3V3_COMPACT, 208)):
        assert pad.pad_octave_slot_bytes(fmt) == want
    n = ctypes.c_int32(0)
    assert L.pad_octave_slot_bytes(0, 256, ctypes.byref(n)) == pad.PAD_EINVAL
    assert L.pad_octave_slot_bytes(4, 256, ctypes.byref(n)) == pad.PAD_EINVAL
    assert L.pad_octave_slot_bytes(1, 128, ctypes.byref(n)) == pad.PAD_EUNSUPPORTED
    assert L.pad_octave_slot_bytes(1, 256, None) == pad.PAD_EINVAL

    def dec(sh, fmt=1, q=0x1000, cache=0x2000, bt=0x3000, sl=0x4000, ks=0x5000, vs=0x6000, out=0x7000):
        return L.pad_decode_attn_octave(ctypes.byref(sh), fmt, P(q), P(cache), P(bt), P(sl), P(ks), P(vs),
                                        ctypes.c_float(0.1), P(out), P(0), ctypes.c_size_t(0), None)

    base = dict(num_q_heads=16, num_kv_heads=2, head_size=256, num_segments=1)
    assert dec(shape(**base), fmt=0) == pad.PAD_EINVAL
    assert dec(shape(**base), fmt=4) == pad.PAD_EINVAL
    assert dec(shape(num_q_heads=16, num_kv_heads=2, head_size=128)) == pad.PAD_EUNSUPPORTED
    assert dec(shape(path=pad.PAD_PATH_DOT, **base)) == pad.PAD_EUNSUPPORTED
    assert dec(shape(**base), ks=0) == pad.PAD_EINVAL
    assert dec(shape(**base), vs=0x6002) == pad.PAD_EINVAL
    assert dec(shape(**base), q=0) == pad.PAD_EINVAL
    assert dec(shape(num_seqs=0, **base), q=0, cache=0, bt=0, sl=0, ks=0, vs=0, out=0) == pad.PAD_OK
    # a split plan needs a workspace
    split = shape(num_q_heads=16, num_kv_heads=2, head_size=256, num_segments=4)
    assert dec(split) == pad.PAD_EWORKSPACE
    # the packed format's bytes per key shrink the planned workspace's K/V
    # span, never below the control prefix
    assert pad.pad_decode_attn_octave_workspace_size(split, 1) >= 1 << 20

    def dec_v(sh, fmt=1, q=0x1000, qs=0x1800, cache=0x2000, bt=0x3000, sl=0x4000, ks=0x5000, vs=0x6000, out=0x7000):
        return L.pad_decode_attn_octave_varlen(ctypes.byref(sh), fmt, P(q), P(qs), P(cache), P(bt), P(sl), P(ks),
                                               P(vs), ctypes.c_float(0.1), P(out), P(0), ctypes.c_size_t(0), None)

    # the per-sequence-count entry: q_start required and 4-byte aligned,
    # the format and the rest checked as above
    assert dec_v(shape(**base), qs=0) == pad.PAD_EINVAL
    assert dec_v(shape(**base), qs=0x1802) == pad.PAD_EINVAL
    assert dec_v(shape(**base), fmt=0) == pad.PAD_EINVAL
    assert dec_v(shape(**base), ks=0) == pad.PAD_EINVAL
    assert dec_v(shape(num_q_heads=16, num_kv_heads=2, head_size=128)) == pad.PAD_EUNSUPPORTED
    assert dec_v(shape(num_seqs=0, **base), q=0, qs=0, cache=0, bt=0, sl=0, ks=0, vs=0, out=0) == pad.PAD_OK
    assert dec_v(split) == pad.PAD_EWORKSPACE
    assert L.pad_decode_attn_octave_varlen(None, 1, P(0x1000), P(0x1800), P(0x2000), P(0x3000), P(0x4000),
                                           P(0x5000), P(0x6000), ctypes.c_float(0.1), P(0x7000), P(0),
                                           ctypes.c_size_t(0), None) == pad.PAD_EINVAL

    def wr(fmt=1, head_size=256, tokens=4, key=0x1000, ks=0x2000, cache=0x3000):
        sh = pad.pad_octave_cache_shape(num_tokens=tokens, num_kv_heads=2, head_size=head_size, page_size=16,
                                        num_blocks=4, dtype=pad.PAD_BF16, layout=pad.PAD_HND, format=fmt)
        return L.pad_octave_cache_write(ctypes.byref(sh), P(key), P(key), P(0x4000), P(ks), P(ks), P(cache), None)

    assert wr(tokens=0, key=0) == pad.PAD_OK
    assert wr(fmt=0) == pad.PAD_EINVAL
    assert wr(head_size=128) == pad.PAD_EUNSUPPORTED
    assert wr(key=0) == pad.PAD_EINVAL
    assert wr(ks=0x2002) == pad.PAD_EINVAL
    assert wr(cache=0x3008) == pad.PAD_EINVAL


@pytest.mark.parametrize("window", [0, 1, 512, 65535, 65536, 100000])
@pytest.mark.parametrize("nseg", [0, 1, 3])
def test_workspace_covers_every_window(window, nseg):
    """The window-independent workspace size covers the plan of any window,
    also where the table holds exactly as many tiles as one segment may
    stage (a windowed plan once counted one tile more than the table and
    split such a unit, needing a workspace the size query never reported)."""
    sh = shape(num_seqs=65, query_len=256, num_q_heads=4, num_kv_heads=4, head_size=256, page_size=32,
               max_blocks_per_seq=2048, num_segments=nseg, schedule=pad.PAD_SCHED_GRID)
    ws = pad.pad_decode_attn_workspace_size(sh)
    p = pad.pad_decode_attn_plan(sh, window, 256)
    assert p["workspace_bytes"] <= ws, (window, nseg, p)
    if nseg:
        assert p["num_segments"] == nseg


@pytest.mark.parametrize("M", [1, 8, 31, 32, 33, 256, 2048])
@pytest.mark.parametrize("head_size", [64, 128, 256])
def test_plan_prefill_family(M, head_size):
    """AUTO takes the prefill family (head sizes 64 and 128) for at least
    128 GQA-packed rows per kv head when its 128-row blocks fill a quarter
    of the device, with at least 2^20 rows x keys per kv head: 128-row
    blocks of one workgroup each, segments of a multiple of 8 16-key tiles
    (one 128-key LDS tile) within the LDS id area, about
    one workgroup per CU; batches keep it on the grid schedule."""
    sh = shape(num_q_heads=32, num_kv_heads=8, head_size=head_size, query_len=M, max_blocks_per_seq=512)
    p = plan(sh)
    rows = 4 * M
    units = 8 * -(-rows // 128)
    if rows >= 128 and head_size in (64, 128) and 4 * units >= 256:
        assert p["path"] == pad.PAD_PATH_PREFILL
        assert p["row_tiles"] == 8 and p["row_groups"] == -(-rows // 128) and p["waves"] == 8
        assert p["persistent"] == 0
        assert p["segment_tiles"] <= 1024
        assert p["num_segments"] == 1 or p["segment_tiles"] % 8 == 0
        assert p["grid_x"] == p["num_segments"] * 8 * p["row_groups"]
        assert p["workspace_bytes"] >= 0
    else:
        assert p["path"] == pad.PAD_PATH_MFMA
    # the window-free workspace covers every window
    ws = pad.pad_decode_attn_workspace_size(sh)
    for w in (1, 100, 4096):
        assert plan(sh, w)["workspace_bytes"] <= ws
    # a batch of prompts stays on the grid with the prefill family
    if rows >= 128 and head_size in (64, 128):
        b = plan(shape(num_seqs=16, num_q_heads=32, num_kv_heads=8, head_size=head_size, query_len=M,
                       max_blocks_per_seq=512))
        assert b["path"] == pad.PAD_PATH_PREFILL and b["persistent"] == 0


def _plan_log(env_value):
    """stderr of a child process that plans the same shape twice and a second shape once."""
    import os
    import subprocess
    import sys

    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import paged_kv_decode_block_amd as pad\n"
        "a = pad.pad_shape(num_seqs=1, query_len=4, num_q_heads=32, num_kv_heads=8, head_size=128, page_size=16,\n"
        "                  max_blocks_per_seq=2048, max_seq_len=32768, dtype=pad.PAD_BF16, layout=pad.PAD_HND)\n"
        "b = pad.pad_shape(num_seqs=1, query_len=1, num_q_heads=32, num_kv_heads=8, head_size=128, page_size=16,\n"
        "                  max_blocks_per_seq=2048, max_seq_len=32768, dtype=pad.PAD_BF16, layout=pad.PAD_HND)\n"
        "pad.pad_decode_attn_plan(a, 0, num_cus=256)\n"
        "pad.pad_decode_attn_plan(a, 0, num_cus=256)\n"
        "pad.pad_decode_attn_plan(b, 0, num_cus=256)\n"
    ) % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ)
    env.pop("PAD_LOG", None)
    if env_value is not None:
        env["PAD_LOG"] = env_value
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return [l for l in r.stderr.splitlines() if l.startswith("pad plan:")]


def test_plan_logging():
    """PAD_LOG prints each new plan once (repeats of the previous line are
    dropped); unset or "0" prints nothing."""
    lines = _plan_log("1")
    assert len(lines) == 2, lines
    assert "M=4" in lines[0] and "M=1" in lines[1]
    assert all("path=mfma" in l and "segments=" in l and "workspace=" in l for l in lines)
    assert _plan_log(None) == []
    assert _plan_log("0") == []


@pytest.mark.parametrize(
    "M,keys,expect",
    [
        (256, 1023, pad.PAD_PATH_MFMA),  # 1024 rows x 1023 keys: just below 2^20
        (256, 1024, pad.PAD_PATH_PREFILL),  # exactly 2^20
        (256, 768, pad.PAD_PATH_MFMA),  # 256 tokens over 512 keys of context
        (384, 384, pad.PAD_PATH_MFMA),  # a 384-token prompt
        (512, 512, pad.PAD_PATH_PREFILL),  # a 512-token prompt
        (96, 8192, pad.PAD_PATH_MFMA),  # enough work, but 24 row blocks leave the device idle
        (1024, 4096, pad.PAD_PATH_PREFILL),
    ],
)
def test_plan_prefill_work_rule(M, keys, expect):
    """AUTO's prefill threshold: at least 2^20 query rows x keys per kv
    head (32/8 heads: 4 rows per token), besides 128 rows and row blocks
    for a quarter of the device; the key count is the shape's largest
    sequence length."""
    p = plan(shape(query_len=M, max_seq_len=keys, max_blocks_per_seq=1024))
    assert p["path"] == expect, p


def test_window_plan_strided_rows():
    """A 512-key window over an NHD cache with two kv heads (strided key
    rows): one query row per kv head's workgroup takes two-tile segments
    (17 of them); four rows make the partial too large for that and keep
    the longer segments, as does the head-major layout or one kv head."""
    kw = dict(num_q_heads=8, num_kv_heads=2, head_size=256, dtype=pad.PAD_F16, max_seq_len=8192,
              max_blocks_per_seq=512)
    nhd1 = plan(shape(layout=pad.PAD_NHD, query_len=1, **kw), window=512)
    assert (nhd1["num_segments"], nhd1["segment_tiles"]) == (17, 2)
    nhd4 = plan(shape(layout=pad.PAD_NHD, query_len=4, **kw), window=512)
    hnd1 = plan(shape(layout=pad.PAD_HND, query_len=1, **kw), window=512)
    one = plan(shape(layout=pad.PAD_NHD, query_len=1, **dict(kw, num_q_heads=4, num_kv_heads=1)), window=512)
    for p in (nhd4, hnd1, one):
        assert p["segment_tiles"] > 2 and p["num_segments"] < 17, p
        assert p["num_segments"] * p["segment_tiles"] * 16 >= 512 + 15
    # without a window the span is long and keeps the usual segments
    full = plan(shape(layout=pad.PAD_NHD, query_len=1, **kw))
    assert full["segment_tiles"] >= 4


def _octave_plan_log(shapes):
    """PAD_LOG lines of a child process that sizes the packed-cache (k3v4)
    workspace of each shape (keyword dicts for pad_shape) and then the
    plain one of the first, with 256 CUs (no device here)."""
    import os
    import subprocess
    import sys

    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import paged_kv_decode_block_amd as pad\n"
        "for kw in %r:\n"
        "    pad.pad_decode_attn_octave_workspace_size(pad.pad_shape(**kw), pad.OCTAVE_FORMATS['octave_k3v4'])\n"
        "pad.pad_decode_attn_workspace_size(pad.pad_shape(**%r[0]))\n"
    ) % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))), shapes, shapes)
    env = dict(os.environ, PAD_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("pad plan:")]
    return [dict(kv.split("=", 1) for kv in l.split("->", 1)[1].split() if "=" in kv) for l in lines]


def test_packed_cache_plans():
    """A packed cache runs one 16-row tile per wave, so two workgroups share
    a CU: the balanced grid has two workgroups per CU and 64 lead tiles per
    unit (12 for the plain cache of the same batch); a single sequence on
    the grid schedule fills the device counting one workgroup per CU."""
    base = dict(num_q_heads=16, num_kv_heads=2, head_size=256, dtype=pad.PAD_BF16, layout=pad.PAD_HND,
                num_segments=0, path=0, schedule=0)
    batch = dict(base, num_seqs=65, query_len=4, page_size=1056, max_blocks_per_seq=16, max_seq_len=16384)
    single = dict(base, num_seqs=1, query_len=4, page_size=32, max_blocks_per_seq=1024, max_seq_len=32768)
    one_row = dict(single, query_len=1)
    pb, ps, p1, plain = _octave_plan_log([batch, single, one_row])
    assert pb["persistent"] == "1" and pb["grid"] == "512x1" and pb["lead"] == "64", pb
    assert pb["row_tiles"] == "1" and pb["row_groups"] == "2", pb
    assert plain["persistent"] == "1" and plain["grid"] == "256x1" and plain["lead"] == "12", plain
    assert plain["row_tiles"] == "2" and plain["row_groups"] == "1", plain
    for p, rg in ((ps, 2), (p1, 1)):
        assert p["persistent"] == "0" and p["row_tiles"] == "1" and p["row_groups"] == str(rg), p
        nseg = int(p["segments"].split("x")[0])
        gx, gy = (int(v) for v in p["grid"].split("x"))
        assert gx * gy == nseg * 2 * rg <= 256, p
