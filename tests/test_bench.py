"""Host-side checks of the benchmark: the effective-byte formula against the
closed forms of each workload, and the one-GPU contract.  No GPU needed."""

from __future__ import annotations

import os
import subprocess
import sys
import types

import torch

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _case(cfg: int, lens, M: int):
    spec = wl.CONFIGS[cfg]
    dtype = torch.bfloat16 if spec.dtype == "bf16" else torch.float16
    return types.SimpleNamespace(
        spec=spec,
        q=torch.empty(len(lens), M, spec.num_q_heads, spec.head_size, dtype=dtype),
        query_len=M,
        window=spec.window,
        seq_lens=torch.tensor(lens, dtype=torch.int32),
    )


def test_effective_bytes_closed_forms():
    # One sequence without a window: 2 * D * eb bytes per key per kv head
    # (4096 B per key over 8 kv heads of 128 in bf16), plus Q in and O out.
    for L in (128, 4096, 32768):
        for M in (1, 2, 4):
            assert bench.effective_bytes(_case(2, [L], M)) == 4096 * L + 16384 * M
    # Head size 512 over 2 kv heads: 4096 B per key, 32768 B of Q + O per token.
    for M in (1, 8):
        assert bench.effective_bytes(_case(4, [32768], M)) == 4096 * 32768 + 32768 * M
    # A 512-key window read by M query tokens reaches W + M - 1 distinct keys.
    assert bench.effective_bytes(_case(3, [16384], 1)) == 1_056_768
    assert bench.effective_bytes(_case(3, [16384], 4)) == 1_087_488
    # A window longer than the sequence reads the whole sequence.
    assert bench.effective_bytes(_case(3, [100], 4)) == 100 * 2 * 2 * 256 * 2 + 2 * 4 * 8 * 256 * 2


def test_effective_bytes_skip_padded_sequences():
    # Padded sequences (length 0) move nothing, not even Q and O.
    per_key = 2 * 2 * 256 * 2
    qo = 2 * 4 * 16 * 256 * 2
    lens = [512, 0, 1000]
    assert bench.effective_bytes(_case(5, lens, 4)) == (512 + 1000) * per_key + 2 * qo


def test_tile_bytes_round_to_whole_tiles():
    # The gather ceiling reads whole 16-key tiles: 1000 keys -> 63 tiles.
    c = _case(2, [1000], 4)
    assert bench.tile_bytes(c) == 63 * 16 * 8 * 2 * 128 * 2
    # With a window the first tile is the one holding the window's first key.
    c3 = _case(3, [16384], 4)
    lo = 16384 - 4 - 512 + 1
    tiles = 16384 // 16 - lo // 16
    assert bench.tile_bytes(c3) == tiles * 16 * 2 * 2 * 256 * 2


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_traffic_hash_covers_decode_includes():
    """The sources the traffic counters' staleness hash covers include every
    local file the decode kernel's translation units include, transitively."""
    import os
    import re

    import bench

    csrc = bench.CSRC
    seen, todo = set(), ["decode_mfma.hip", "api.cpp", "plan.cpp", "launch.hip"]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.add(name)
        with open(os.path.join(csrc, name)) as f:
            for inc in re.findall(r'#include\s+"([^"]+)"', f.read()):
                if "/" not in inc:
                    todo.append(inc)
    assert seen <= set(bench.DECODE_SOURCES), seen - set(bench.DECODE_SOURCES)
    assert all(os.path.exists(os.path.join(csrc, n)) for n in bench.DECODE_SOURCES)
