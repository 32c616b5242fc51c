"""Build step for the HIP library: one hipcc invocation, output in-tree.

    python -m exact_io_aware_37_amd.build

runs csrc/gen_fwd_w64.py (which writes csrc/fa_fwd_w64.inc, the assembly
body of the 64-row forward kernel) and compiles csrc/fa_fwd.hip for gfx950
into exact_io_aware_37_amd/libfa.so.
Every HIP source is built with packed-fp32 instruction selection disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know that feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "fa_fwd.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG_DIR, "libfa.so")
ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return exe


def generate() -> str:
    """Write csrc/fa_fwd_w64.inc (the 64-row forward body) from its generator."""
    sys.path.insert(0, os.path.join(PKG_DIR, "csrc"))
    try:
        import gen_fwd_w64
    finally:
        sys.path.pop(0)
    return gen_fwd_w64.write_inc()


def build(verbose: bool = False, extra_flags=()) -> str:
    """Generate the asm body, compile the library; returns the built shared object's path."""
    generate()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-result", f"-I{INCLUDE}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *extra_flags, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
