"""Build libconvrot.so (gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import re
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


# the compiler's per-kernel resource report, checked below
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def register_spills(remarks: str) -> list[str]:
    """Kernels whose resource report shows VGPRs or SGPRs spilled to scratch.

    A spill in these kernels is a performance fault (the GEMM's accumulators
    and the quantizer's row data are sized to stay in registers), so the build
    refuses it rather than ship a silently slower library."""
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+([VS])GPRs Spill: (\d+)", line)
        if m and int(m.group(2)) > 0:
            bad.append(f"{name}: {m.group(1)}GPRs spill {m.group(2)}")
    return bad


def build(output: str = LIBRARY, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source into one shared library (always recompiles) and
    refuse a build in which any kernel spills registers."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = output + ".tmp"
    cmd = [HIPCC, *FLAGS, *RESOURCE_REMARKS, *(extra or []), *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    spills = register_spills(res.stderr)
    if spills:
        os.remove(tmp)
        raise RuntimeError("kernels spill registers:\n  " + "\n  ".join(spills))
    if verbose:
        warnings = [l for l in res.stderr.splitlines() if "warning" in l]
        if warnings:
            sys.stderr.write("\n".join(warnings) + "\n")
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
