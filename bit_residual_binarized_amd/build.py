"""Build librabit.so (all HIP sources, gfx950) in-tree with hipcc.

Usage: python -m bit_residual_binarized_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librabit.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    # packed fp32 ALU ops are not used on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
]
# MFMA accumulators in VGPRs: with AGPRs the allocator rotated the GEMV's 64
# loop-carried accumulators through copies on every iteration. train.hip keeps
# the default form: its dW kernel holds 256 accumulators per lane, which fit
# only as AGPRs.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
NO_VGPR_FORM = {"train.hip"}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature name and says so: harmless
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every .hip source (one object each, in parallel) and link
    bit_residual_binarized_amd/librabit.so."""
    from concurrent.futures import ThreadPoolExecutor
    import tempfile
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="rabit_build_") as d:
        jobs = []
        for src in sources():
            name = os.path.basename(src)
            extra = [] if name in NO_VGPR_FORM else VGPR_FORM
            obj = os.path.join(d, name + ".o")
            jobs.append((obj, [HIPCC, *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]))
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
        with ThreadPoolExecutor(workers) as ex:
            errs = list(ex.map(lambda j: _run(j[1]), jobs))
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]
        errs.append(_run(link))
    if verbose:
        for _, cmd in jobs:
            print(" ".join(cmd), flush=True)
        print(" ".join(link), flush=True)
        for e in errs:
            if e.strip():
                print(e, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
