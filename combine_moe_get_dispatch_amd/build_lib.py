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
SOURCES = ["moe_api.hip", "layout.hip", "dispatch.hip", "combine.hip"]
HEADERS = ["device_common.h", "launch.h"]

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


def build(verbose: bool = True, extra_flags=None) -> str:
    out_tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
           *sources(), "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out_tmp, LIB_PATH)
    return LIB_PATH


def is_stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    deps = sources() + [os.path.join(CSRC, h) for h in HEADERS] + [
        os.path.join(ROOT, "include", "moe_dispatch_combine.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
