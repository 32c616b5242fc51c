"""Build step for the HIP library: one hipcc invocation, output in-tree.

    python -m exact_io_aware_37_amd.build

runs csrc/gen_fwd_w64.py (which writes csrc/fa_fwd_w64.inc, the assembly
body of the 64-row forward kernel) and compiles csrc/fa_fwd.hip for gfx950
into exact_io_aware_37_amd/libfa.so.  The compiler's intermediate files go to
exact_io_aware_37_amd/_build/; the device assembly among them is checked by
mfma_latency.py (no vector instruction may touch an MFMA result register
before the matrix unit has written it), and a library that fails the check
is not installed.
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
BUILD_DIR = os.path.join(PKG_DIR, "_build")
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
    os.makedirs(BUILD_DIR, exist_ok=True)
    out = os.path.join(BUILD_DIR, "libfa.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-result", f"-I{INCLUDE}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-save-temps=obj", *extra_flags, SRC, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    asm = device_asm()
    sys.path.insert(0, PKG_DIR)
    try:
        import mfma_latency
    finally:
        sys.path.pop(0)
    bad = mfma_latency.check_file(asm)
    if bad:
        lines = [f"{name}: {x}  ({short} wait state(s) short of: {src})"
                 for name, items in bad.items() for x, src, short in items[:4]]
        raise RuntimeError("compiled code reads MFMA results before they are written; library not "
                           "installed:\n" + "\n".join(lines))
    tmp = LIB + ".tmp"
    shutil.copyfile(out, tmp)
    os.replace(tmp, LIB)
    return LIB


def device_asm() -> str:
    """Path of the gfx950 assembly that the last build assembled into the library."""
    for name in os.listdir(BUILD_DIR):
        if name.endswith("-hip-amdgcn-amd-amdhsa-gfx950.s"):
            return os.path.join(BUILD_DIR, name)
    raise RuntimeError(f"no gfx950 device assembly in {BUILD_DIR}")


if __name__ == "__main__":
    print(build(verbose=True))
