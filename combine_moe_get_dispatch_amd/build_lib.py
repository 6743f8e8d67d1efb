"""Build the HIP library in-tree: combine_moe_get_dispatch_amd/libmoe_dispatch_combine.so.

hipcc for gfx950 only.  Floating point flags matter for bit-exact parity:
  -ffp-contract=off                          no implicit fused multiply-add
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE fp32 division (int8 scale)
  -fno-gpu-flush-denormals-to-zero           keep fp32 subnormals
  -fno-fast-math
Packed fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libmoe_dispatch_combine.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# Test build of the same sources with a grid cap of 2^6 workgroups, so that the
# grid-stride iterations of the kernels run at test sizes.
SMALL_GRID_LIB_PATH = os.path.join(HERE, "libmoe_dispatch_combine_smallgrid.so")
SMALL_GRID_FLAGS = ["-DMOE_MAX_GRID_LOG2=6"]
SOURCES = ["moe_api.hip", "layout.hip", "dispatch.hip", "combine.hip", "small_batch.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def headers():
    """Every header the sources include: all of csrc/*.h and the public header."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")) + [
        os.path.join(ROOT, "include", "moe_dispatch_combine.h")]


def _command(out_path, extra_flags):
    return [HIPCC, *FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
            *sources(), "-o", out_path]


def build(verbose: bool = True, extra_flags=None, with_test_build: bool = False) -> str:
    """Compile the library (and, with with_test_build, the small-grid test
    build alongside it, in parallel)."""
    jobs = [(LIB_PATH, extra_flags)]
    if with_test_build:
        jobs.append((SMALL_GRID_LIB_PATH, SMALL_GRID_FLAGS + list(extra_flags or [])))
    procs = []
    for path, flags in jobs:
        cmd = _command(path + ".tmp", flags)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((path, subprocess.Popen(cmd)))
    failed = [path for path, p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, f"hipcc ({', '.join(failed)})")
    for path, _ in procs:
        os.replace(path + ".tmp", path)
    return LIB_PATH


def is_stale(path: str = LIB_PATH) -> bool:
    """True when the library at `path` is missing or older than a source or
    header it is built from."""
    if not os.path.exists(path):
        return True
    t = os.path.getmtime(path)
    return any(os.path.getmtime(d) > t for d in sources() + headers())


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
