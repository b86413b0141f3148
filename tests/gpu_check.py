"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the fp64 oracle on the same seeded inputs."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_decode_block_amd as pad
import workloads as wl

# Gate of the benchmark spec: max |error| on unit-scale outputs.
ABS_TOL = {torch.float16: 2e-3, torch.bfloat16: 1.5e-2}
# Scale-aware bound, max |error| / max |reference|: long contexts give
# outputs far below unit scale, where the absolute gate alone is too loose.
REL_TOL = {torch.float16: 2e-3, torch.bfloat16: 1e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(case: wl.Case, instance: int = 0, *, num_segments=0, path=0, max_seq_len=0, workspace=None,
            out=None, window=None, scale=None, schedule=0):
    """One pad_decode_attn call on the case's device tensors."""
    if out is None:
        out = torch.full_like(case.q, float("nan"))
    pad.pad_decode_attn(
        case.q, case.kv_cache, case.block_tables[instance], case.seq_lens,
        case.scale if scale is None else scale, case.window if window is None else window, out,
        layout=case.layout, workspace=workspace, num_segments=num_segments, path=path, max_seq_len=max_seq_len,
        schedule=schedule,
    )
    return out


def oracle_out(case: wl.Case, instance: int = 0, seqs=None, window=None, scale=None, seq_lens=None):
    """fp64 oracle output of the selected sequences (all by default)."""
    kv64, table, lens = wl.compact(case, instance, seqs)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int64)
    idx = list(range(case.num_seqs)) if seqs is None else list(seqs)
    q64 = wl.as_f64(case.q[idx])
    return oracle.decode_attention(
        q64, kv64, table, lens, case.scale if scale is None else scale,
        case.window if window is None else window, case.layout,
    )


def errors(got: torch.Tensor, ref: np.ndarray) -> tuple[float, float]:
    g = wl.as_f64(got)
    if not np.all(np.isfinite(g)):
        return float("inf"), float("inf")
    err = float(np.abs(g - ref).max()) if ref.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    return err, (err / scale if scale > 0 else err)


def check(got: torch.Tensor, ref: np.ndarray, dtype, what: str = "") -> None:
    err, rel = errors(got, ref)
    say(f"  {what}: max|err|={err:.3e} rel={rel:.3e}")
    assert err <= ABS_TOL[dtype], f"{what}: max abs error {err} > {ABS_TOL[dtype]}"
    assert rel <= REL_TOL[dtype], f"{what}: scale-aware error {rel} > {REL_TOL[dtype]}"


def passes(got: torch.Tensor, ref: np.ndarray, dtype) -> bool:
    err, rel = errors(got, ref)
    return err <= ABS_TOL[dtype] and rel <= REL_TOL[dtype]
