"""Compile the HIP library (gfx950 only) into the package directory."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("na3d.cpp", "kernel_general.hip", "kernel_roll.hip", "kernel_rmsnorm.hip")]
LIB = os.path.join(HERE, "libna3d.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU forms are kept out of the generated code on purpose.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaN inputs are in contract: max needs no NaN-quieting; infinities
    # (the -inf window masks) are still honoured
    "-fno-honor-nans",
    # MFMA accumulators in VGPRs: the rare rescale path multiplies them with
    # VALU ops, which cannot read AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]
# .cpp sources go through the HIP compiler as well
LANG = ["-x", "hip"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + LANG + SOURCES + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        noise = "is not a recognized feature for this target"
        for line in (res.stdout + res.stderr).splitlines():
            if noise not in line:
                print(line)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
