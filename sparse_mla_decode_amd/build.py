"""Build libsmla.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m sparse_mla_decode_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsmla.so")
SOURCES = [os.path.join(CSRC, "smla_kernels.hip"), os.path.join(CSRC, "smla_topk.hip"),
           os.path.join(CSRC, "smla_noalloc.hip"), os.path.join(CSRC, "smla_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU ops stay disabled in every device compile.  Kernel-argument
# preloading: up to 14 leading scalar or pointer arguments of a kernel arrive
# in SGPRs when its waves start (the decode kernels put their first-needed
# fields there); struct arguments are never preloaded.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-kernarg-preload-count=14"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-Wall", "-I", os.path.join(ROOT, "include"),
           *DEVICE_FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag: that note is expected
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    errs = [ln for ln in r.stderr.splitlines() if noise not in ln and "--hip-link" not in ln]
    if r.returncode != 0:
        sys.stderr.write("\n".join(errs) + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
