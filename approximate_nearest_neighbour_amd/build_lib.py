"""Build the HIP library ``libivfpq.so`` in-tree for gfx950 with hipcc.

Every translation unit under ``csrc/`` is compiled to an object in
``_build/`` (in parallel) and linked into ``libivfpq.so`` next to this file.
Packed-FP32 instructions are switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libivfpq.so")
ARCH = os.environ.get("IVFPQ_ARCH", "gfx950")

HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-file flags.  The exact search kernels take each matrix product's result
# straight into a minimum (minima pass) or a test (collect): with the results
# in VGPRs instead of accumulator registers no copy-out instruction is needed
# per element (same occupancy), and as their arithmetic never makes a NaN
# from finite inputs (padding rows are +inf, never inf - inf) they are built
# NaN-free, so that a float minimum is one instruction (IEEE mode would
# otherwise quiet both inputs first).  NaN in the database or the queries is
# outside their contract.
FILE_FLAGS = {
    "kernels_flat.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if err:
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
