"""Build the in-tree HIP library libgns.so for gfx950 with hipcc.

Usage: python -m gram_newton_schulz_amd.build  (or __graft_entry__.build()).
The library lands next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libgns.so")
# measurement build: every GEMM workgroup records timestamps (GNS_TIMELINE in
# gns_kernels.hip); read by gram_newton_schulz_amd.timeline
TIMELINE_LIB = os.path.join(HERE, "libgns_timeline.so")
SOURCES = ["gns_kernels.hip", "gns_host.cpp", "gns_noalloc.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm required to build the HIP library)")


def build(verbose: bool = False, timeline: bool = False) -> str:
    target = TIMELINE_LIB if timeline else LIB
    tmp = target + ".tmp"
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 instructions are kept out of all generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the epilogues index the accumulator tiles with unrolled loop
        # counters; a larger budget keeps them fully unrolled (in registers)
        "-mllvm", "-pragma-unroll-threshold=200000",
        "-I", INCLUDE, "-I", CSRC,
        *(["-DGNS_TIMELINE"] if timeline else []),
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", tmp,
    ]
    # the compiler's resource report of every kernel (checked below)
    cmd.insert(-2, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    spills = scratch_users(res.stderr)
    if spills:
        raise RuntimeError("GEMM kernels that use scratch memory: " + ", ".join(spills))
    os.replace(tmp, target)
    return target


def scratch_users(report: str) -> list:
    """Names of GEMM kernels whose resource report shows scratch memory.

    The GEMM main loop waits on explicit counts of its own outstanding
    LDS-DMA loads and sets m0 inside inline assembly; both assume that the
    compiler adds no memory traffic and keeps nothing of its own in m0,
    which spilling to scratch would break.  A build in which any GEMM kernel
    spills is therefore refused."""
    out, name = [], None
    for line in report.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
        elif name and "gemm_nt" in name and ("ScratchSize [bytes/lane]:" in line or "VGPRs Spill:" in line
                                               or "SGPRs Spill:" in line):
            val = int(line.split(":")[-1].split("[")[0].strip())
            if val > 0 and name not in out:
                out.append(name)
    return out


if __name__ == "__main__":
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
