"""Build libmq.so (HIP, gfx950) in-tree with hipcc.

Flags: -O3, no fast-math (IEEE f32 divide and roundf keep the quantizer
bit-exact), correctly rounded f32 divide/sqrt, and packed-FP32 instructions
disabled.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIBRARY = os.path.join(HERE, "libmq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # matrix-core results in ordinary VGPRs (no copies out of AGPRs)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(output: str = LIBRARY, extra=()) -> str:
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), *sources(), "-o", output + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    print(build(*sys.argv[1:]))
