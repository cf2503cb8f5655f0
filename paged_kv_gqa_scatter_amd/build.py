"""Build libpkv.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 VALU instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no AGPR copies around the VALU rescale)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) + glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


def build(out: str = LIB, extra=()) -> str:
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), *sources(), "-o", out]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(*(sys.argv[1:2] or [LIB])))
