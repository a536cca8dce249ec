"""Build libconvrot.so (gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBRARY = os.path.join(PKG, "libconvrot.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["convrot_api.cpp", "quantize.hip", "gemm_i8.hip", "static_workspace.hip"]
# the measurement probes of the roofline report (MFMA rate, plain copy), a
# library of their own
PROBE_SOURCE = "probes.hip"
PROBE_LIBRARY = os.path.join(PKG, "libconvrot_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
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


def _compile(src: str, extra: list[str]) -> tuple[str, subprocess.CompletedProcess]:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *RESOURCE_REMARKS, *extra, "-c", src, "-o", obj]
    return obj, subprocess.run(cmd, capture_output=True, text=True)


def build(output: str = LIBRARY, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source (in parallel, always recompiling) and link one
    shared library; refuse a build in which any kernel spills registers."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    probe_src = os.path.join(CSRC, PROBE_SOURCE)
    with ThreadPoolExecutor(max_workers=len(srcs) + 1) as pool:
        results = list(pool.map(lambda s: _compile(s, list(extra or [])), srcs + [probe_src]))
    probe_obj, probe_res = results.pop()
    if probe_res.returncode != 0:
        sys.stderr.write(probe_res.stdout + probe_res.stderr)
        raise RuntimeError(f"hipcc failed ({probe_res.returncode}) on {probe_src}")
    remarks = ""
    for src, (obj, res) in zip(srcs, results):
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed ({res.returncode}) on {src}")
        remarks += res.stderr
    spills = register_spills(remarks)
    if spills:
        raise RuntimeError("kernels spill registers:\n  " + "\n  ".join(spills))
    if verbose:
        warnings = [l for l in remarks.splitlines() if "warning" in l]
        if warnings:
            sys.stderr.write("\n".join(warnings) + "\n")
    tmp = output + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in results], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"link failed ({res.returncode}): {' '.join(cmd)}")
    os.replace(tmp, output)
    if output == LIBRARY:
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", probe_obj, "-o", PROBE_LIBRARY + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"link failed ({res.returncode}): {' '.join(cmd)}")
        os.replace(PROBE_LIBRARY + ".tmp", PROBE_LIBRARY)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
