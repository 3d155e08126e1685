"""Build the q4g64 HIP library in-tree for gfx950.

    python -m bit_weight_only_q4g64_amd.build

compiles ``csrc/api.hip`` (which includes every kernel) into
``bit_weight_only_q4g64_amd/libq4g64.so``. Strict IEEE float32: no fast-math and
no floating-point contraction (every fused multiply-add in the kernels is an
explicit fma), no packed-fp32 instructions, and matrix-core results kept in
ordinary vector registers.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "api.hip")
OUT = os.path.join(HERE, "libq4g64.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    # matrix-core results in ordinary vector registers rather than the
    # accumulation registers: the same instructions (so the same bits), minus
    # the copies between the two files before each fold; measured 1.2x on
    # the short-window GEMM, no change on the others
    "-mllvm",
    "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the q4g64 library)")


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path."""
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
