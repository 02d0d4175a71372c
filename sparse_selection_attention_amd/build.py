"""Build step for libqsa.so: hipcc, gfx950, in-tree.

Run as `python -m sparse_selection_attention_amd.build` or through
__graft_entry__.build(). The library is compiled every time this runs.
"""
from __future__ import annotations

import glob
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqsa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 VALU forms stay disabled; see the kernel sources' notes on fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    # MFMA accumulators in ordinary VGPRs: no accumulator read-backs, lower register count
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def kernel_resources(remarks: str) -> dict:
    """Per-kernel VGPRs, scratch bytes per lane, occupancy and scalar registers
    spilled into vector lanes, parsed from the compiler's kernel-resource-usage
    remarks."""
    out, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|SGPRs Spill): (\d+)", line)
        if m and name:
            key = "SGPRSpill" if m.group(1) == "SGPRs Spill" else m.group(1).split()[0]
            out[name][key] = int(m.group(2))
    return out


def build(verbose: bool = False) -> str:
    cmd = [HIPCC] + FLAGS + ["-Rpass-analysis=kernel-resource-usage",
                             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + sources() + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    remarks = r.stdout + r.stderr
    if r.returncode != 0:
        sys.stderr.write("\n".join(l for l in remarks.splitlines() if "remark:" not in l) + "\n")
        raise subprocess.CalledProcessError(r.returncode, cmd)
    res = kernel_resources(remarks)
    if not res:
        raise RuntimeError("no kernel-resource-usage remarks from %s" % HIPCC)
    # every kernel keeps its state in registers and LDS: a register spill to
    # scratch is a build error, not a silent slowdown, and so is a scalar
    # register spilled into vector lanes (each spill and reload is a VALU
    # instruction; 70 such spills once cost the selection kernel 18%)
    spills = {k: v for k, v in res.items() if v.get("ScratchSize", 0) != 0 or v.get("SGPRSpill", 0) != 0}
    if spills:
        os.remove(LIB + ".tmp")
        raise RuntimeError("kernels spill registers: %s" % spills)
    if verbose:
        for k, v in sorted(res.items()):
            print(k, v, flush=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
