"""Build the gfx950 HIP library in-tree (``libattn_fwd.so`` next to this file)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "attn_fwd.hip")
SOURCES = [SRC, os.path.join(PKG, "csrc", "quantize.hip"), os.path.join(PKG, "csrc", "qknorm.hip")]
LIB = os.path.join(PKG, "libattn_fwd.so")
# the matrix-core rate calibration kernel (bench.py --mfma-ceiling), a library of its own
RATE_SRC = os.path.join(PKG, "csrc", "mfma_rate.hip")
RATE_LIB = os.path.join(PKG, "libmfma_rate.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs (no AGPR copies around the softmax rescale)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(out: str = LIB, extra: list[str] | None = None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *(extra or []), *SOURCES, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    if out == LIB:
        subprocess.run([hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), RATE_SRC, "-o", RATE_LIB + ".tmp"],
                       check=True)
        os.replace(RATE_LIB + ".tmp", RATE_LIB)
    return out


if __name__ == "__main__":
    print(build())
