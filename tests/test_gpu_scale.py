"""Softmax scales other than 1/sqrt(D) on every kernel family, against the
fp64 oracle.  The boundary takes any finite scale (the header's formula
multiplies each q.k by it): a negative scale reverses which keys dominate
(the prefill family folds its sign into the query rows), zero gives the
plain average of the visible V rows (masked keys, NaN-filled page tails
included, must still get no weight), a tiny one nearly so, a large one an
almost one-hot softmax."""

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_decode_block_amd as pad
import workloads as wl
from gpu_check import ABS_TOL, REL_TOL, errors, oracle_out, run_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALES = [-0.5, 0.0, 1e-3, 3.0]


def check(got, ref, dtype, what):
    """The absolute gate holds for unit-scale outputs; a sharp softmax
    reproduces single V rows, whose entries reach about 4 here, and bf16's
    own rounding of such an output is up to 2^-6 -- so above unit scale the
    absolute bound grows with the largest reference value.  The
    scale-aware bound is the usual one."""
    err, rel = errors(got, ref)
    top = float(np.abs(ref).max()) if ref.size else 0.0
    say(f"  {what}: max|err|={err:.3e} rel={rel:.3e} max|ref|={top:.3f}")
    assert err <= ABS_TOL[dtype] * max(1.0, top), f"{what}: max abs error {err}"
    assert rel <= REL_TOL[dtype], f"{what}: scale-aware error {rel} > {REL_TOL[dtype]}"


# name, spec, lens, M, window, run kwargs
CASES = [
    ("mfma grid", wl.CONFIGS[2], [1000, 37], 4, 0, {"path": pad.PAD_PATH_MFMA, "schedule": pad.PAD_SCHED_GRID}),
    ("mfma window NHD", wl.Spec("fp16", 256, 8, 2, 32, wl.NHD, window=96), [700], 3, 96, {}),
    ("mfma d512", wl.CONFIGS[4], [600], 8, 0, {}),
    ("balanced grid", wl.CONFIGS[2], [900, 0, 2000, 45], 3, 0, {"schedule": pad.PAD_SCHED_PERSISTENT}),
    ("prefill family", wl.Spec("bf16", 128, 32, 8, 16, wl.HND, window=50), [700], 64, 50,
     {"path": pad.PAD_PATH_PREFILL, "schedule": pad.PAD_SCHED_GRID}),
    ("prefill family d64", wl.Spec("fp16", 64, 8, 2, 32, wl.NHD), [40, 1, 0, 77], 33, 0,
     {"path": pad.PAD_PATH_PREFILL, "schedule": pad.PAD_SCHED_GRID}),
    ("dot family", wl.CONFIGS[1], [256, 13], 1, 0, {"path": pad.PAD_PATH_DOT}),
]


@pytest.mark.parametrize("scale", SCALES, ids=[f"s{s:g}" for s in SCALES])
@pytest.mark.parametrize("case", CASES, ids=[c[0].replace(" ", "_") for c in CASES])
def test_scales(case, scale):
    name, spec, lens, M, window, kw = case
    say(f"scale {scale}: {name} D={spec.head_size} {spec.num_q_heads}/{spec.num_kv_heads} lens={lens} M={M} "
        f"window={window} {kw}")
    c = wl.make_case(spec, lens, M, seed=8700 + M + len(lens), device=DEV, window=window)
    out = run_gpu(c, scale=scale, **kw)
    for s, L in enumerate(lens):
        if L == 0:
            assert torch.all(out[s] == 0), "padded sequence must be zero"
    check(out, oracle_out(c, scale=scale), c.q.dtype, f"{name}, scale {scale}")


@pytest.mark.parametrize("scale", [-0.5, 0.0], ids=["s-0.5", "s0"])
def test_scales_packed_cache(scale):
    """The packed (octave k3v4) cache on the balanced grid."""
    from test_gpu_octave import _oracle, _packed_case, _run

    say(f"scale {scale}: packed cache k3v4, lens [1500, 0, 700], M=4, 16/2 heads, page 32")
    c, packed, kw_, vw_, sk, sv = _packed_case(1, "bf16", wl.HND, [1500, 0, 700], 4, 16, 2, 32, 8800)
    c = dataclasses.replace(c, scale=scale)
    out = _run(c, packed, 1, kw_, vw_, schedule=pad.PAD_SCHED_PERSISTENT)
    assert torch.all(out[1] == 0), "padded sequence must be zero"
    check(out, _oracle(c, packed, 1, sk, sv), c.q.dtype, f"packed cache, scale {scale}")
