"""Build libpad_attn.so (HIP kernels for gfx950 plus the C ABI) in-tree.

Run as ``python paged_kv_decode_block_amd/build.py`` or through
``__graft_entry__.build()``; it imports nothing of the package, so it works
when the library is missing or out of date.  hipcc cross-compiles for gfx950 without a GPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpad_attn.so")
# The decode kernels keep MFMA accumulators in the VGPR form (results and
# accumulator operands in ordinary vector registers): in the default form
# the compiler parked the accumulators in the accumulation registers and
# moved them back and forth around the softmax rescale on every pass of
# the tile loop (thousands of v_accvgpr moves per kernel), and at head
# size 512 it spilled.
MFMA_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form=1",
              # The decode kernel's first 11 arguments -- three pointers and
              # eight int32 scalars, 14 dwords: what its first loads depend
              # on -- are preloaded into scalar registers (the count is in
              # arguments, not dwords).
              "-mllvm", "-amdgpu-kernarg-preload-count=11"]

# (source, object name, extra flags): the decode kernels build once per
# head size, in parallel.
SOURCES = [("decode_mfma.hip", f"decode_mfma_d{d}", [f"-DPAD_HEAD_SIZE={d}", *MFMA_FLAGS]) for d in (64, 128, 256, 512)] + [
    # the packed (quantized) cache's kernels: a further build at head size 256
    # (a missed two-waves-per-SIMD register target is an error: two of its
    # workgroups must fit one CU)
    ("decode_mfma.hip", "decode_octave_d256", ["-DPAD_HEAD_SIZE=256", "-DPAD_OCTAVE=1", "-Werror=pass-failed",
                                               *MFMA_FLAGS]),
    # the prefill kernels (head sizes 64 and 128)
    ("prefill_mfma.hip", "prefill_mfma", [*MFMA_FLAGS]),
] + [
    (src, src.rsplit(".", 1)[0], [])
    for src in ("launch.hip", "cache_write.hip", "octave_store.hip", "calib.hip", "noalloc.hip", "plan.cpp", "api.cpp")
]

# Packed fp32 VALU ops are turned off for every HIP source (the host pass
# reports the feature as unknown; that warning is harmless).
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpad_attn.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}) on {cmd[-1]}:\n{errs}")
    if errs.strip() and verbose:
        print(errs, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the
    shared library; the result replaces LIB atomically."""
    from concurrent.futures import ThreadPoolExecutor

    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, jobs = [], []
    for src, name, extra in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, name + ".o")
        objs.append(obj)
        # .cpp files hold host code only; compile them as HIP too so the
        # link step sees one toolchain.
        jobs.append([cc, *HIP_FLAGS, *extra, "-c", "-o", obj] + (["-x", "hip"] if src.endswith(".cpp") else []) +
                    [path])
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([cc, *HIP_FLAGS, "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
