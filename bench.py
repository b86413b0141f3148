#!/usr/bin/env python3
"""Benchmark of paged-KV decode attention on one MI355X.

A step is one pad_decode_attn call (the whole hot path: plan, page gather,
QK^T, mask, online softmax, PV, split partials and in-kernel merge) over one
batch of seeded synthetic inputs.  The default workload is benchmark
configuration 5, the largest: a batch of 64 bf16 sequences with lengths
uniform in [512, 16384] plus one padded sequence, head size 256, 16 q heads
/ 2 kv heads, page size 1056, HND, random block table, M = 4 -- about
1.15 GB of K/V per call, so no call is served from the 256 MiB last-level
cache.

The metric is effective HBM bandwidth: bytes of the distinct K/V rows the
call must read, plus Q and O, per second; and its fraction of the 8 TB/s
HBM peak.  Beside it, ``read_ceiling`` reports what plain reads reach on
the same device (a gather of exactly the call's pages with the same table
walk and no arithmetic, contiguous streams over a 512 MiB buffer with
several workgroup sizes and loads in flight, and a device-to-device copy),
and ``sweep`` times every (context, M) point of the other benchmark
configurations, graph-timed.  One JSON line is printed.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of one MI355X
POOL_BYTES = 512 << 20
COPY_BYTES = 256 << 20  # --copy-calibration: bytes read (and written) per copy
# Committed HBM-traffic counter runs, by (config, context, M) of the
# workload they were taken on (MFMA family, automatic plan; a packed
# cache's runs by its format name in place of the config).
TRAFFIC_FILES = {
    (2, 32768, 4): "traffic_decode_mfma_bf16_D128_Hq32_Hkv8_L32768_M4.json",
    (3, 16384, 4): "traffic_decode_mfma_fp16_D256_Hq8_Hkv2_NHD_W512_L16384_M4.json",
    (4, 32768, 1): "traffic_decode_mfma_bf16_D512_Hq16_Hkv2_L32768_M1.json",
    (4, 32768, 8): "traffic_decode_mfma_bf16_D512_Hq16_Hkv2_L32768_M8.json",
    (5, 16384, 4): "traffic_decode_mfma_persistent_bf16_D256_Hq16_Hkv2_P1056_batch64_M4.json",
    ("octave_k3v4", 16384, 4): "traffic_decode_octave_k3v4_D256_Hq16_Hkv2_P1056_batch64_M4.json",
}
CSRC = os.path.join(ROOT, "paged_kv_decode_block_amd", "csrc")


def effective_bytes(case) -> int:
    """Distinct K/V bytes the call must read plus Q and O bytes.

    A sequence of length L reads L keys, or min(L, W + M - 1) keys when a
    window W limits the M query tokens; each key costs 2 * D elements per kv
    head.  Padded sequences (L = 0) move nothing.
    """
    spec = case.spec
    eb = case.q.element_size()
    M = case.query_len
    W = case.window
    total = 0
    for L in case.seq_lens.tolist():
        if L <= 0:
            continue
        keys = min(L, W + M - 1) if W > 0 else L
        total += keys * spec.num_kv_heads * 2 * spec.head_size * eb
        total += 2 * M * spec.num_q_heads * spec.head_size * eb  # Q in, O out
    return total


def tile_bytes(case) -> int:
    """K/V bytes the gather-ceiling kernel reads: the same key ranges as the
    call, rounded out to whole 16-key tiles."""
    spec = case.spec
    eb = case.q.element_size()
    total = 0
    for L in case.seq_lens.tolist():
        if L <= 0:
            continue
        lo = max(0, L - case.query_len - case.window + 1) if case.window > 0 else 0
        tiles = -(-L // 16) - lo // 16
        total += tiles * 16 * spec.num_kv_heads * 2 * spec.head_size * eb
    return total


def _event_time(call, n_warm: int, n_timed: int) -> float:
    """Average ms per call(i), timed with HIP events on the current stream."""
    import torch

    for i in range(n_warm):
        call(i)
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(n_timed):
        call(n_warm + i)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / n_timed


def read_ceiling(case, nseg_hint: int) -> dict:
    """Practical read ceilings beside the result: the best rate of a kernel
    that gathers exactly this call's pages (same table walk, 16-byte loads,
    no arithmetic) over a small sweep of launch shapes, and a contiguous
    16-byte stream over the whole pool."""
    import torch

    import paged_kv_decode_block_amd as pad

    sink = torch.zeros(1, dtype=torch.int32, device=case.q.device)
    n_inst = len(case.block_tables)
    M, Hq, D = case.query_len, case.q.shape[2], case.q.shape[3]
    nbytes = tile_bytes(case)
    best = None
    segs = sorted({max(1, min(256, s)) for s in (nseg_hint, 2 * nseg_hint, 4 * nseg_hint, 64, 128, 256)})
    for waves in (4, 8):
        for tif in (1, 2):
            if tif == 2 and D == 512:
                continue
            for sg in segs:
                def call(i, waves=waves, tif=tif, sg=sg):
                    pad.pad_calib_gather_read(case.kv_cache, case.block_tables[i % n_inst], case.seq_lens, M, Hq,
                                              case.window, sink, layout=case.layout, waves=waves,
                                              tiles_in_flight=tif, segments=sg)

                ms = _event_time(call, 10, 100)
                gbs = nbytes / (ms * 1e-3) / 1e9
                if best is None or gbs > best["GB/s"]:
                    best = {"GB/s": round(gbs, 1), "us": round(ms * 1e3, 3), "waves": waves,
                            "tiles_in_flight": tif, "segments": sg}
    buf = torch.empty(POOL_BYTES // 2, dtype=torch.bfloat16, device=case.q.device)
    buf_bytes = buf.numel() * buf.element_size()
    stream_best, stream_all = None, []
    for threads in (256, 512, 1024):
        for loads in (4, 8, 16):
            for blocks in (1024, 2048, 4096, 8192):
                ms = _event_time(lambda i, b=blocks, t=threads, u=loads: pad.pad_calib_stream_read(
                    buf, sink, blocks=b, threads=t, loads_in_flight=u), 3, 10)
                gbs = buf_bytes / (ms * 1e-3) / 1e9
                stream_all.append(round(gbs, 1))
                if stream_best is None or gbs > stream_best["GB/s"]:
                    stream_best = {"GB/s": round(gbs, 1), "blocks": blocks, "threads": threads,
                                   "loads_in_flight": loads}
    # torch's device-to-device copy of half the buffer into the other half:
    # bytes read plus bytes written per second
    half = buf.numel() // 2
    src, dst = buf[:half], buf[half:]
    ms = _event_time(lambda i: dst.copy_(src), 3, 10)
    copy = {"GB/s": round(2 * half * buf.element_size() / (ms * 1e-3) / 1e9, 1),
            "bytes_read": half * buf.element_size()}
    del buf, src, dst
    return {
        "gather_read": best,
        "gather_bytes_per_launch": nbytes,
        "stream_read": stream_best,
        "stream_read_variants": len(stream_all),
        "stream_read_median_GB/s": sorted(stream_all)[len(stream_all) // 2],
        "stream_bytes": buf_bytes,
        "device_copy": copy,
    }


# Sources the decode kernel (both schedules) is built from or planned by,
# with the headers they include; the prefill, cache-write, packed-store,
# calibration and allocation-free sources are not among them.
DECODE_SOURCES = ("decode_mfma.hip", "decode_common.h", "octave_dev.h", "kernels.h", "plan.h", "plan.cpp",
                  "api.cpp", "entry.h", "launch.hip")


def kernel_hash() -> str:
    """Hash of the decode kernel's sources (DECODE_SOURCES), the public
    headers they include and the build script (its compiler flags): a
    change to any of them makes the committed traffic counters stale."""
    h = hashlib.sha256()
    paths = [os.path.join(CSRC, n) for n in DECODE_SOURCES]
    paths += [os.path.join(ROOT, "include", n) for n in ("pad_attn.h", "pad_octave.h")]
    paths.append(os.path.join(ROOT, "paged_kv_decode_block_amd", "build.py"))
    for path in paths:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def time_calls(case, n_warm: int, n_timed: int, graph: bool = False, **kw):
    """Average ms per call over n_timed calls rotating through the instances,
    timed with HIP events on the stream the kernel is launched on.  With
    ``graph`` the n_timed calls are captured once into a HIP graph and the
    replay is timed, which removes host launch overhead between kernels."""
    import torch

    import paged_kv_decode_block_amd as pad

    out = torch.empty_like(case.q)
    shape = pad.make_shape(case.q, case.kv_cache, case.block_tables[0], case.layout, **kw)
    ws = pad.Workspace(case.q.device).get(shape)
    n_inst = len(case.block_tables)

    def call(i):
        pad.pad_decode_attn(case.q, case.kv_cache, case.block_tables[i % n_inst], case.seq_lens, case.scale,
                            case.window, out, layout=case.layout, workspace=ws, **kw)

    for i in range(n_warm):
        call(i)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_timed):
                call(n_warm + i)
        g.replay()  # warm replay
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    if g is not None:
        g.replay()
    else:
        for i in range(n_timed):
            call(n_warm + i)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / n_timed, pad.pad_decode_attn_plan(shape, case.window)


def _blas_threads() -> int:
    """Threads the oracle's BLAS calls may use (as the thread pools report)."""
    try:
        from threadpoolctl import threadpool_info

        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(cfg: int, context: int, M: int, budget_s: float = 12.0) -> dict:
    """The fp64 oracle on the host, on a bounded sample of the workload."""
    import numpy as np

    import oracle
    import workloads as wl

    case = wl.config_case(cfg, context, M, device="cpu")
    kv64, table, lens = wl.compact(case)
    q64 = wl.as_f64(case.q)
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_attention(q64, kv64, table, lens, case.scale, case.window, case.layout)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 1000:
            break
    cores = _blas_threads()
    gbs = effective_bytes(case) * calls / el / 1e9
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": int(cores),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{calls} full call(s) of the config {cfg} workload at context {context}, M={M} "
                  f"({case.num_seqs} sequence(s), all kv heads), {el:.1f} s of host time; cores = the BLAS "
                  f"threads the oracle's products use, host_cpus = os.cpu_count()",
    }


def copy_calibration() -> None:
    """Ten device copies of COPY_BYTES: a counter run's reference for
    scaling the HBM byte counters of the kernels around it."""
    import torch

    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def traffic_entry(cfg, context: int, M: int):
    """Measured HBM bytes per launch from the committed counter runs of
    this workload, if there are any and they were taken on the current
    kernel source."""
    name = TRAFFIC_FILES.get((cfg, context, M))
    if name is None:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash():
        return None
    return t.get("bytes_per_launch")


def varlen_main(args) -> int:
    """Mixed decode / speculative-verify batch through pad_decode_attn_varlen:
    the batched workload's 64 sequences (plus one padded) with a seeded
    query count of 1..4 each, queries packed, counts read on the device."""
    import numpy as np
    import torch

    import workloads as wl

    import paged_kv_decode_block_amd as pad

    cfg, ctx, mmax = 5, 16384, 4
    spec = wl.CONFIGS[cfg]
    case = wl.config_case(cfg, ctx, mmax, device="cuda")
    S = case.num_seqs
    counts = torch.randint(1, mmax + 1, (S,), generator=torch.Generator().manual_seed(20261202)).tolist()
    q = torch.cat([case.q[s, :n] for s, n in enumerate(counts)], dim=0).contiguous()
    starts = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    q_start = torch.from_numpy(starts).to("cuda")
    out = torch.empty_like(q)
    eb = q.element_size()
    lens = case.seq_lens.tolist()
    nbytes = sum(L * spec.num_kv_heads * 2 * spec.head_size * eb + 2 * n * spec.num_q_heads * spec.head_size * eb
                 for L, n in zip(lens, counts) if L > 0)
    q_like = torch.empty((S, mmax, spec.num_q_heads, spec.head_size), dtype=q.dtype, device="meta")
    shape = pad.make_shape(q_like, case.kv_cache, case.block_tables[0], case.layout)
    ws = pad.Workspace(q.device).get(shape)

    def call(i):
        pad.pad_decode_attn_varlen(q, q_start, case.kv_cache, case.block_tables[0], case.seq_lens, case.scale,
                                   case.window, out, max_query_len=mmax, layout=case.layout, workspace=ws)

    ms = _event_time(call, args.warmup, args.steps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu:
        import oracle

        kv64, table, lens64 = wl.compact(case)
        q64 = wl.as_f64(q)
        t0, done, moved = time.perf_counter(), 0, 0
        while done < S and time.perf_counter() - t0 < 12.0:
            a, b = int(starts[done]), int(starts[done + 1])
            oracle.decode_attention_varlen(q64[a:b], [0, b - a], kv64, table[done:done + 1], lens64[done:done + 1],
                                           case.scale, case.window, case.layout)
            L = int(lens64[done])
            if L > 0:
                moved += L * spec.num_kv_heads * 2 * spec.head_size * eb + 2 * (b - a) * spec.num_q_heads * spec.head_size * eb
            done += 1
        el = time.perf_counter() - t0
        cpu = {"value": round(moved / el / 1e9, 4), "unit": "GB/s", "cores": _blas_threads(), "host_cpus": os.cpu_count(), "kind": "oracle",
               "sample": f"{done} of {S} sequences of the mixed batch, one varlen oracle call each, {el:.1f} s"}
    line = {
        "metric": "decode-attention effective HBM GB/s (K+V rows read + Q + O) and fraction of 8 TB/s",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": f"mixed decode/verify batch: {S} sequences (one padded), bf16, D={spec.head_size}, "
                               f"{spec.num_q_heads}/{spec.num_kv_heads} heads, page {spec.page_size}, lengths "
                               f"512..{ctx}, per-sequence M in 1..{mmax} packed ({int(starts[-1])} query tokens)",
                   "bytes_per_step": nbytes, "plan": pad.pad_decode_attn_plan(shape, case.window)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def cache_write_main(args) -> int:
    """The KV-cache write with a full-width rotation (the step before decode)
    on one prefill-sized chunk of tokens of the default workload's shapes:
    new keys and values land in shuffled slots of a 512 MiB pool and the
    query rows are rotated in place."""
    import numpy as np
    import torch

    import workloads as wl

    import paged_kv_decode_block_amd as pad

    spec = wl.CONFIGS[2]
    T, Hq, Hkv, D = 16384, spec.num_q_heads, spec.num_kv_heads, spec.head_size
    rd, max_pos = D, 32768
    eb = 2
    g = torch.Generator(device="cuda").manual_seed(20261202)
    nb = POOL_BYTES // spec.block_bytes
    kv = torch.empty((nb, Hkv, spec.page_size, 2, D), dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    key = torch.randn((T, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    val = torch.randn((T, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((T, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    slots = torch.randperm(nb * spec.page_size, generator=g, device="cuda")[:T].to(torch.int64)
    pos = torch.randint(0, max_pos, (T,), generator=g, device="cuda", dtype=torch.int64)
    inv = 10000.0 ** (-np.arange(rd // 2) * 2.0 / rd)
    ang = np.arange(max_pos)[:, None] * inv[None, :]
    tab = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)).to("cuda")
    # bytes the step must move: key and value in, the K+V slots out, the
    # rotated query rows in and out, and one cos/sin row per token
    nbytes = 2 * T * Hkv * D * eb * 2 + 2 * T * Hq * rd * eb + T * rd * 4

    def call(i):
        pad.pad_rope_cache_write(key, val, kv, slots, q=q, positions=pos, cos_sin_cache=tab)

    ms = _event_time(call, args.warmup, args.steps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu:
        from oracle import rope as orope

        n = 256
        f64 = lambda t: t[:n].to(torch.float64).cpu().numpy()  # noqa: E731
        kv_small = np.zeros((n, Hkv, 1, 2, D))
        t0, calls = time.perf_counter(), 0
        while time.perf_counter() - t0 < 10.0 and calls < 20:
            orope.cache_write(kv_small, wl.HND, f64(key), f64(val), np.arange(n), pos[:n].cpu().numpy(),
                              tab.cpu().numpy(), rd, f64(q))
            calls += 1
        el = time.perf_counter() - t0
        per_tok = nbytes / T
        cpu = {"value": round(per_tok * n * calls / el / 1e9, 4), "unit": "GB/s", "cores": _blas_threads(),
               "host_cpus": os.cpu_count(),
               "kind": "oracle", "sample": f"{calls} oracle call(s) on the first {n} tokens, {el:.1f} s"}
    line = {
        "metric": "KV-cache write effective HBM GB/s (key, value, query rows, cos/sin in; cache slots, query rows out) "
                  "and fraction of 8 TB/s",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"cache write: {T} tokens, bf16, D={D}, {Hq}/{Hkv} heads, page {spec.page_size}, HND, "
                               f"rotation over all {rd} dims, shuffled slots in a {POOL_BYTES >> 20} MiB pool",
                   "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def octave_main(args) -> int:
    """Decode over a quantized (octave) packed cache on the batch workload's
    shapes: 64 sequences of 512..16384 keys plus one padded, 16/2 heads of
    256, page 1056, M = 4, q/out bf16.  The cache is written from seeded
    N(0,1) rows by the library's store kernel before timing.  Effective
    bytes: the packed slots of the attended keys, plus Q and O."""
    import numpy as np
    import torch

    import workloads as wl

    import paged_kv_decode_block_amd as pad

    fmt = pad.OCTAVE_FORMATS[args.octave]
    cfg, ctx, M = 5, 16384, 4
    spec = wl.CONFIGS[cfg]
    case = wl.config_case(cfg, ctx, M, device="cuda")
    nb, Hkv, P = case.kv_cache.shape[0], spec.num_kv_heads, spec.page_size
    sb = pad.pad_octave_slot_bytes(fmt)
    cache = torch.zeros((nb, Hkv, P, sb), dtype=torch.uint8, device="cuda")
    ks, vs = wl.sign_words(20261203).to("cuda"), wl.sign_words(20261204).to("cuda")
    # write the pool token by token (a block's slots are block * P + offset)
    rows = case.kv_cache.permute(0, 2, 1, 3, 4).reshape(nb * P, Hkv, 2, spec.head_size)
    chunk = 1 << 16
    for t0 in range(0, nb * P, chunk):
        part = rows[t0:t0 + chunk]
        slots = torch.arange(t0, t0 + part.shape[0], dtype=torch.int64, device="cuda")
        pad.pad_octave_cache_write(part[:, :, 0].contiguous(), part[:, :, 1].contiguous(), cache, slots, ks, vs, fmt)
    torch.cuda.synchronize()
    del rows
    lens = case.seq_lens.tolist()
    eb = case.q.element_size()
    nbytes = sum(L * Hkv * sb + 2 * M * spec.num_q_heads * spec.head_size * eb for L in lens if L > 0)
    out = torch.empty_like(case.q)
    bt = case.block_tables[0]

    def call(i):
        pad.pad_decode_attn_octave(case.q, cache, bt, case.seq_lens, ks, vs, case.scale, out, fmt)

    ms = _event_time(call, args.warmup, args.steps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    if getattr(args, "copy_calibration", False):
        copy_calibration()
    cpu = None
    if not args.no_cpu:
        from oracle import octave as oc

        name = args.octave
        s_k = oc.signs_from_bits(ks.cpu().numpy().view(np.uint32), spec.head_size)
        s_v = oc.signs_from_bits(vs.cpu().numpy().view(np.uint32), spec.head_size)
        bt_np = bt.cpu().numpy()
        t0, done, moved = time.perf_counter(), 0, 0
        while done < len(lens) and time.perf_counter() - t0 < 12.0:
            L = lens[done]
            if L > 0:
                used = np.unique(bt_np[done, : -(-L // P)])
                packed = cache[torch.as_tensor(used, device="cuda")].cpu().numpy()
                table = np.arange(len(used))[None, :]
                q64 = case.q[done:done + 1].to(torch.float64).cpu().numpy()
                oc.decode_attention_quant(q64, packed, table, [L], case.scale, wl.HND, name, s_k, s_v)
                moved += L * Hkv * sb + 2 * M * spec.num_q_heads * spec.head_size * eb
            done += 1
        el = time.perf_counter() - t0
        cpu = {"value": round(moved / el / 1e9, 4), "unit": "GB/s", "cores": _blas_threads(), "host_cpus": os.cpu_count(),
               "kind": "oracle", "sample": f"{done} of {len(lens)} sequences, one oracle call each, {el:.1f} s"}
    line = {
        "metric": "packed-cache decode effective HBM GB/s (packed K+V slots read + Q + O) and fraction of 8 TB/s",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 q/out, fp16 products over " + args.octave + " codes", "data": "synthetic",
        "config": {"workload": f"{args.octave} cache, batch {case.num_seqs} ({case.num_seqs - 1} sequences of "
                               f"512..{ctx} keys + 1 padded), D={spec.head_size}, {spec.num_q_heads}/{Hkv} heads, "
                               f"page {P}, HND, M={M}, {sb}-byte slots",
                   "bytes_per_step": nbytes,
                   "bf16_cache_bytes_per_step": int(sum(L * Hkv * 2 * spec.head_size * 2 for L in lens if L > 0))},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_entry(args.octave, ctx, M)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def prefill_main(args) -> int:
    """A prefill chunk through the same entry point: 256 new tokens over a
    4096-key context, the default workload's shapes (1024 GQA-packed rows
    per kv head; the planner takes the prefill family: eight 128-row
    blocks, each reading only the keys its tokens reach).  Arithmetic
    intensity ~1000 flop/byte: bound by the matrix cores, reported against
    the dense bf16 MFMA peak."""
    import torch

    import workloads as wl

    import paged_kv_decode_block_amd as pad

    cfg, context, M = 2, 4096, 256
    spec = wl.CONFIGS[cfg]
    L = context + M
    case = wl.make_case(spec, [L], M, seed=20261202 + 7, device="cuda")
    G, D = spec.num_q_heads // spec.num_kv_heads, spec.head_size
    # QK^T and PV: 2 flops per multiply-add, two products per visible key and head dim
    visible = sum(context + m + 1 for m in range(M))
    flops = 4 * visible * spec.num_q_heads * D
    ms, plan = time_calls(case, args.warmup, args.steps, num_segments=args.segments)
    tflops = flops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu:
        import oracle

        kv64, table, lens = wl.compact(case)
        q64 = wl.as_f64(case.q)
        t0 = time.perf_counter()
        oracle.decode_attention(q64, kv64, table, lens, case.scale, case.window, case.layout)
        el = time.perf_counter() - t0
        cpu = {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": _blas_threads(), "host_cpus": os.cpu_count(), "kind": "oracle",
               "sample": f"one full call, {el:.1f} s"}
    line = {
        "metric": "prefill-chunk attention TFLOP/s (QK^T + PV over visible keys) and fraction of the bf16 MFMA peak",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": f"prefill chunk: {M} tokens over a {context}-key context, bf16, D={D}, "
                               f"{spec.num_q_heads}/{spec.num_kv_heads} heads, page {spec.page_size}, HND",
                   "flops_per_step": flops, "plan": plan},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--context", type=int, default=None)
    ap.add_argument("--queries", type=int, default=None)
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the per-(context, M) sweep of every benchmark configuration")
    ap.add_argument("--sweep-configs", default="1,2,3,4,5",
                    help="configurations whose points the sweep times (comma-separated)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-ceiling calibration kernels")
    ap.add_argument("--segments", type=int, default=0,
                    help="force the split-KV segment count of the timed call (0 = the planner's choice)")
    ap.add_argument("--path", choices=["auto", "mfma", "dot"], default="auto",
                    help="kernel family (auto = the planner's choice)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run device copies of COPY_BYTES (reference for HBM byte counters)")
    ap.add_argument("--prefill", action="store_true",
                    help="time a 256-token prefill chunk over a 4096-key context instead (matrix-core bound)")
    ap.add_argument("--cache-write", action="store_true",
                    help="time the KV-cache write with rotation (the step before decode) instead")
    ap.add_argument("--varlen", action="store_true",
                    help="time a mixed decode/verify batch through the per-sequence-count entry point instead")
    ap.add_argument("--octave", choices=["octave_k3v4", "octave_k3v3", "octave_k3v3_compact"], default=None,
                    help="time decode over a quantized packed cache of this format instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode-attention path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        return 2

    if args.varlen:
        return varlen_main(args)
    if args.octave:
        return octave_main(args)
    if args.cache_write:
        return cache_write_main(args)
    if args.prefill:
        return prefill_main(args)

    import torch

    import workloads as wl

    import paged_kv_decode_block_amd as pad

    path = {"auto": pad.PAD_PATH_AUTO, "mfma": pad.PAD_PATH_MFMA, "dot": pad.PAD_PATH_DOT}[args.path]
    cfg = args.config
    pts = wl.CONFIG_POINTS[cfg]
    context = args.context or max(pts["contexts"])
    M = args.queries or max(pts["queries"])
    spec = wl.CONFIGS[cfg]

    def build_case(c, ctx, m):
        sp = wl.CONFIGS[c]
        per_inst = sp.block_bytes * (-(-ctx // sp.page_size))
        inst = max(1, POOL_BYTES // per_inst) if c != 5 else 1
        return wl.config_case(c, ctx, m, device="cuda", instances=inst, pool_bytes=POOL_BYTES)

    print(f"[bench] config {cfg}: context {context}, M={M}: building inputs", file=sys.stderr, flush=True)
    case = build_case(cfg, context, M)
    nbytes = effective_bytes(case)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms, plan = time_calls(case, args.warmup, args.steps, path=path, num_segments=args.segments)
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps: {ms * 1e3:.2f} us/step", file=sys.stderr, flush=True)
    gbs = nbytes / (ms * 1e-3) / 1e9
    if args.copy_calibration:
        copy_calibration()

    ceiling = None
    if not args.no_ceiling:
        ceiling = read_ceiling(case, plan["num_segments"])
        ceiling["frac_of_gather_read"] = round(gbs / ceiling["gather_read"]["GB/s"], 4)
        print(f"[bench] read ceiling: gather {ceiling['gather_read']['GB/s']} GB/s, "
              f"stream {ceiling['stream_read']['GB/s']} GB/s, copy {ceiling['device_copy']['GB/s']} GB/s",
              file=sys.stderr, flush=True)

    sweep = []
    if not args.no_sweep:
        for c in [int(x) for x in args.sweep_configs.split(",") if x]:
            pts_c, spec_c = wl.CONFIG_POINTS[c], wl.CONFIGS[c]
            for ctx in pts_c["contexts"]:
                for m in pts_c["queries"]:
                    if (c, ctx, m) == (cfg, context, M):
                        continue  # the headline itself
                    if path == pad.PAD_PATH_DOT and m * spec_c.num_q_heads // spec_c.num_kv_heads > 4:
                        continue  # the dot family serves at most 4 query rows per kv head
                    cs = build_case(c, ctx, m)
                    try:
                        t, p = time_calls(cs, 20, 100, graph=True, path=path)
                    except pad.PadError as e:
                        if e.status != pad.PAD_EUNSUPPORTED:
                            raise
                        del cs
                        continue  # a forced family that does not serve this shape
                    b = effective_bytes(cs)
                    sweep.append({"config": c, "context": ctx, "M": m, "us": round(t * 1e3, 3),
                                  "GB/s": round(b / (t * 1e-3) / 1e9, 1),
                                  "frac": round(b / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "segments": p["num_segments"]})
                    del cs
            print(f"[bench] sweep of config {c} done ({len(sweep)} points so far)", file=sys.stderr, flush=True)

    cpu = None if args.no_cpu else cpu_baseline(cfg, context, M)
    line = {
        "metric": "decode-attention effective HBM GB/s (K+V rows read + Q + O) and fraction of 8 TB/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"config {cfg}: batch {case.num_seqs}"
                        + (f" ({case.num_seqs - 1} sequences of 512..{context} keys + 1 padded)" if cfg == 5 else "")
                        + f", {spec.dtype}, D={spec.head_size}, {spec.num_q_heads}/{spec.num_kv_heads} heads, "
                        f"page {spec.page_size}, {'HND' if spec.layout == wl.HND else 'NHD'}, window {case.window}, M={M}",
            "context": context,
            "query_len": M,
            "pool_bytes": max(POOL_BYTES, case.kv_cache.numel() * case.kv_cache.element_size()),
            "instances": len(case.block_tables),
            "bytes_per_step": nbytes,
            "plan": plan,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            # HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE
            # runs of this workload, while the kernel source is unchanged
            "traffic": traffic_entry(cfg, context, M) if path != pad.PAD_PATH_DOT and args.segments == 0 else None,
        },
        "read_ceiling": ceiling,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
