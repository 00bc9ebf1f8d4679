"""Builds libw4a16.so (all HIP kernels + host code) for gfx950 with hipcc.

Run ``python -m int4_weight_only_dequant_amd.build`` (or call ``build()``).
The library is written next to this file, in-tree.  ``--trace`` builds
libw4a16_trace.so instead: the same library with the persistent decode
kernel's phase timestamps compiled in (loaded by ``bench.py --phase-trace``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libw4a16.so")
TRACE_LIB = os.path.join(HERE, "libw4a16_trace.so")
ARCH = os.environ.get("W4_OFFLOAD_ARCH", "gfx950")

SOURCES = ["w4a16.hip", "pack.cpp", "container.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libw4a16.so)")


def build(verbose: bool = False, trace: bool = False) -> str:
    target = TRACE_LIB if trace else LIB
    out_tmp = target + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           f"-I{INCLUDE}", f"-I{CSRC}", "-o", out_tmp] + (["-DW4_PK_TRACE"] if trace else [])
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "ignoring feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)
    os.replace(out_tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, trace="--trace" in sys.argv))
