"""Measurement behind the wait-state table of mfma_latency.py (MI355X, gfx950).

    python exact_io_aware_37_amd/csrc/probe_mfma_latency.py OUTDIR [--run]

writes OUTDIR/mfma_latency_probe.hip, builds it with hipcc and, with --run
(needs the GPU), runs it and prints per MFMA instruction and result register
the first wait-state count at which a read of the register returns the
product.  Each probe kernel is one wave: it fills A and B with 1.0, sets the
destination registers to -1.0, issues one MFMA, waits exactly N issue slots
(s_nop), copies one result register and stores it.  A read that comes too
early returns -1.0.  Registers only, apart from one 4-byte store per lane.
"""

from __future__ import annotations

import os
import subprocess
import sys

# name: (A registers, B registers, result registers, the value 1.0 in a packed A/B register, product)
KINDS = {
    "v_mfma_f32_32x32x64_f8f6f4": (8, 8, 16, "0x38383838", 64.0),
    "v_mfma_f32_16x16x128_f8f6f4": (8, 8, 4, "0x38383838", 128.0),
    "v_mfma_f32_32x32x16_bf16": (4, 4, 16, "0x3f803f80", 16.0),
    "v_mfma_f32_32x32x16_f16": (4, 4, 16, "0x3c003c00", 16.0),
    "v_mfma_f32_16x16x32_bf16": (4, 4, 4, "0x3f803f80", 32.0),
    "v_mfma_f32_16x16x32_f16": (4, 4, 4, "0x3c003c00", 32.0),
    "v_mfma_f32_32x32x2_f32": (1, 1, 16, "1.0", 2.0),
    # block-scaled forms, both scales 1.0 (E8M0 127 in v80 and v81)
    "v_mfma_scale_f32_32x32x64_f8f6f4": (8, 8, 16, "0x38383838", 64.0),
    "v_mfma_scale_f32_16x16x128_f8f6f4": (8, 8, 4, "0x38383838", 128.0),
}
SCALED_OPERANDS = ", v80, v81 op_sel_hi:[0,0,0]"
WAITS = range(2, 26)
A0, B0, D0 = 40, 50, 60


def source():
    variants, src = [], ["#include <hip/hip_runtime.h>", "#include <cstdio>", ""]
    for mn, (na, nb, nd, one, val) in KINDS.items():
        for r in range(nd):
            for n in WAITS:
                vid = len(variants)
                variants.append((mn, r, n, val))
                body = [f"v_mov_b32 v{A0 + i}, {one}" for i in range(na)]
                body += [f"v_mov_b32 v{B0 + i}, {one}" for i in range(nb)]
                body += [f"v_mov_b32 v{D0 + i}, -1.0" for i in range(nd)]
                scaled = "_scale_" in mn
                if scaled:
                    body += ["v_mov_b32 v80, 127", "v_mov_b32 v81, 127"]
                body.append("s_nop 7")
                a = f"v[{A0}:{A0 + na - 1}]" if na > 1 else f"v{A0}"
                b = f"v[{B0}:{B0 + nb - 1}]" if nb > 1 else f"v{B0}"
                body.append(f"{mn} v[{D0}:{D0 + nd - 1}], {a}, {b}, 0" + (SCALED_OPERANDS if scaled else ""))
                left = n
                while left > 0:
                    k = min(left, 8)
                    body.append(f"s_nop {k - 1}")
                    left -= k
                body.append(f"v_mov_b32 %[o], v{D0 + r}")
                body += ["s_nop 7"] * 12
                clob = ", ".join(f'"v{x}"' for x in list(range(A0, A0 + 8)) + list(range(B0, B0 + 8))
                                 + list(range(D0, D0 + 16)) + [80, 81])
                src.append(f"__global__ void __launch_bounds__(64) p{vid}(float* out) {{")
                src.append("  float o;")
                text = "\\n".join(body)
                src.append(f'  asm volatile("{text}" : [o] "=&v"(o) : : {clob});')
                src.append("  out[threadIdx.x] = o;")
                src.append("}")
    src.append("typedef void (*kfn)(float*);")
    src.append("static kfn K[] = {" + ", ".join(f"p{i}" for i in range(len(variants))) + "};")
    src.append("static const char* NAME[] = {"
               + ", ".join(f'"{v[0]} {v[1]} {v[2]} {v[3]:g}"' for v in variants) + "};")
    src.append(r'''
int main() {
  const int n = sizeof(K) / sizeof(K[0]);
  float* dev;
  float host[64];
  if (hipMalloc(&dev, sizeof host) != hipSuccess) return 1;
  for (int v = 0; v < n; ++v) {
    float mn = 1e30f, mx = -1e30f;
    for (int rep = 0; rep < 5; ++rep) {
      if (hipMemset(dev, 0, sizeof host) != hipSuccess) return 1;
      hipLaunchKernelGGL(K[v], dim3(1), dim3(64), 0, 0, dev);
      if (hipDeviceSynchronize() != hipSuccess) return 1;
      if (hipMemcpy(host, dev, sizeof host, hipMemcpyDeviceToHost) != hipSuccess) return 1;
      for (int i = 0; i < 64; ++i) { mn = host[i] < mn ? host[i] : mn; mx = host[i] > mx ? host[i] : mx; }
    }
    printf("%s %g %g\n", NAME[v], mn, mx);
  }
  return 0;
}''')
    return "\n".join(src) + "\n"


def table(lines):
    """First wait-state count from which every later count read the product, per (MFMA, register)."""
    rows = {}
    for line in lines:
        mn, r, n, val, lo, hi = line.split()
        ok = float(lo) == float(val) and float(hi) == float(val)
        rows.setdefault((mn, int(r)), []).append((int(n), ok))
    out = {}
    for (mn, r), v in rows.items():
        v.sort()
        first = None
        for n, ok in v:
            if ok and first is None:
                first = n
            elif not ok:
                first = None
        out.setdefault(mn, {})[r] = first
    return out


def main(argv):
    outdir = argv[1]
    os.makedirs(outdir, exist_ok=True)
    src = os.path.join(outdir, "mfma_latency_probe.hip")
    exe = os.path.join(outdir, "mfma_latency_probe")
    with open(src, "w") as f:
        f.write(source())
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O2", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", src, "-o", exe], check=True, capture_output=True)
    if "--run" not in argv:
        print(exe)
        return 0
    res = subprocess.run([exe], check=True, capture_output=True, text=True)
    for mn, regs in table(res.stdout.splitlines()).items():
        print(mn, [regs[r] for r in sorted(regs)])
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
