"""Build libconvrot.so (gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBRARY = os.path.join(PKG, "libconvrot.so")
SOURCES = ["convrot_api.cpp", "quantize.hip", "gemm_i8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # binary32 results must match the oracle bit for bit: no contraction, no
    # fast-math, IEEE denormals kept (the HIP default for gfx950)
    "-ffp-contract=off",
    # no packed-FP32 VALU instructions in the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def build(output: str = LIBRARY, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source into one shared library (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = output + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if verbose and res.stderr:
        sys.stderr.write(res.stderr)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
