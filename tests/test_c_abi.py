"""The C ABI from plain C: include/fa.h compiles as strict C99 (and as C++), and a
C program linked against libfa.so gets the documented results from the entry
points that make no HIP call (argument checks, status strings, launch shape,
workspace sizes).  Runs on the CPU; nothing here touches a device."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "exact_io_aware_37_amd")
LIB = os.path.join(LIBDIR, "libfa.so")

PROGRAM = r"""
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include "fa.h"

#define CHECK(cond) \
    do { \
        if (!(cond)) { printf("FAILED: %s (line %d)\n", #cond, __LINE__); return 1; } \
    } while (0)

int main(void) {
    /* fake, well-aligned, non-overlapping addresses: fa_check_args only inspects them */
    const uintptr_t gb = (uintptr_t)1 << 30, base = (uintptr_t)1 << 40;
    const void* q = (const void*)base;
    const void* k = (const void*)(base + gb);
    const void* v = (const void*)(base + 2 * gb);
    void* o = (void*)(base + 3 * gb);
    float* lse = (float*)(base + 4 * gb);
    int rows, keys, threads, lds;
    long long blocks;

    CHECK(fa_check_args(q, k, v, o, lse, 2, 32, 32, 8192, 8192, 128, 0.088f, 0, FA_BF16) == FA_OK);
    CHECK(fa_check_args(q, k, v, o, lse, 1, 28, 4, 4096, 4096, 128, 0.088f, 1, FA_F16) == FA_OK);
    CHECK(fa_check_args(NULL, k, v, o, lse, 1, 1, 1, 256, 256, 64, 0.125f, 0, FA_F32) == FA_ERR_NULL_PTR);
    CHECK(fa_check_args(q, k, v, o, lse, 1, 6, 4, 256, 256, 64, 0.125f, 0, FA_BF16) == FA_ERR_HEAD_GROUP);
    CHECK(fa_check_args(q, k, v, o, lse, 1, 1, 1, 256, 256, 96, 0.125f, 0, FA_BF16) == FA_ERR_HEAD_DIM);
    CHECK(fa_check_args(q, k, v, o, lse, 1, 1, 1, 0, 256, 64, 0.125f, 0, FA_BF16) == FA_ERR_BAD_DIM);
    CHECK(fa_check_args(q, k, v, o, lse, 1, 1, 1, 256, 256, 64, 0.125f, 0, 7) == FA_ERR_DTYPE);
    CHECK(fa_check_args(q, k, v, q, lse, 1, 1, 1, 256, 256, 64, 0.125f, 0, FA_BF16) == FA_ERR_ALIAS);
    CHECK(fa_check_args((const void*)(base + 2), k, v, o, lse, 1, 1, 1, 256, 256, 64, 0.125f, 0,
                        FA_BF16) == FA_ERR_ALIGN);

    CHECK(strlen(fa_status_string(FA_OK)) > 0);
    CHECK(strlen(fa_status_string(FA_ERR_HEAD_DIM)) > 0);

    CHECK(fa_launch_info(2, 32, 32, 8192, 8192, 128, 0, FA_BF16, &rows, &keys, &threads, &blocks,
                         &lds) == FA_OK);
    CHECK(rows == 256 && keys == 64 && threads == 256 && blocks == 2 * 32 * 32);
    CHECK(lds == 4 * 2 * 64 * 128 * 2);
    CHECK(fa_launch_info(1, 1, 1, 0, 256, 64, 0, FA_F32, &rows, &keys, &threads, &blocks, &lds)
          == FA_ERR_BAD_DIM);

    /* fp32 chunk outputs and chunk lse of every (split, row) */
    CHECK(fa_splitkv_workspace_bytes(8, 28, 1, 128, 64) >= (size_t)64 * 8 * 28 * (128 + 1) * 4);
    CHECK(fa_bwd_workspace_bytes(1, 4, 2, 600, 600, 128) >= (size_t)4 * 600 * 8);
    printf("ok\n");
    return 0;
}
"""


def _compile(tmp_path, compiler, std, src_name, extra=()):
    src = tmp_path / src_name
    src.write_text(PROGRAM)
    exe = tmp_path / (src_name + ".out")
    cmd = [compiler, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{INC}",
           str(src), "-o", str(exe), f"-L{LIBDIR}", "-lfa", f"-Wl,-rpath,{LIBDIR}",
           "-Wl,--allow-shlib-undefined", *extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.skipif(not os.path.exists(LIB), reason="libfa.so not built")
@pytest.mark.parametrize("compiler,std,name", [("gcc", "c99", "abi.c"), ("g++", "c++17", "abi.cpp")])
def test_c_program_calls_the_host_entry_points(tmp_path, compiler, std, name):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    exe = _compile(tmp_path, compiler, std, name)
    env = dict(os.environ)
    rocm_lib = "/opt/rocm/lib"
    env["LD_LIBRARY_PATH"] = rocm_lib + (":" + env["LD_LIBRARY_PATH"] if env.get("LD_LIBRARY_PATH") else "")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
