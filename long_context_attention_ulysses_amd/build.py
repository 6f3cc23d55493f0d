"""Builds libulysses.so (all HIP sources, gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libulysses.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]

# The TiledMLP GEMMs go to hipBLASLt. In a process that has imported torch,
# the already-loaded copy with the same soname is the one used.
LINK_FLAGS = ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lhipblaslt"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra=None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + list(extra or []) + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                                          "-o", tmp] + sources() + LINK_FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "unknown target feature" not in l and "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, msgs))
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    print("built", LIB)
