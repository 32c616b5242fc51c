"""C-ABI checks that need no GPU: the library loads, exports what include/fa.h
declares, and rejects every invalid call on the host before any HIP call."""

import ctypes
import math

import pytest

import exact_io_aware_37_amd as fa

# Fake, 16-byte aligned, non-overlapping addresses: only fa_check_args and the
# argument-check path of fa_fwd see them; no call here reaches a launch.
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
GOOD = dict(B=2, Hq=8, Hkv=2, N_q=100, N_kv=77, d=128, scale=0.125, causal=1, dtype=fa.FA_BF16)


def args(**kw):
    a = dict(GOOD)
    a.update(kw)
    return a


def check(q=Q, k=K, v=V, o=O, lse=L, **kw):
    a = args(**kw)
    return fa.fa_check_args(q, k, v, o, lse, a["B"], a["Hq"], a["Hkv"], a["N_q"], a["N_kv"],
                            a["d"], a["scale"], a["causal"], a["dtype"])


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = fa.header_functions()
    assert set(names) == {"fa_fwd", "fa_fwd_stream", "fa_check_args", "fa_status_string",
                          "fa_launch_info", "fa_splitkv_workspace_bytes",
                          "fa_splitkv_default_splits", "fa_fwd_splitkv",
                          "fa_bwd_workspace_bytes", "fa_bwd", "fa_fwd_fp8",
                          "fa_fwd_paged", "fa_fwd_splitkv_noalloc"}
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_valid_arguments_pass(lib):
    assert check() == fa.FA_OK
    for dt in (fa.FA_F32, fa.FA_F16, fa.FA_BF16):
        for d in (64, 128):
            assert check(dtype=dt, d=d) == fa.FA_OK
    assert check(scale=0.0) == fa.FA_OK and check(scale=-2.0) == fa.FA_OK


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_null_pointers(lib, which):
    assert check(**{which: 0}) == fa.FA_ERR_NULL_PTR


@pytest.mark.parametrize("field", ["B", "Hq", "Hkv", "N_q", "N_kv"])
@pytest.mark.parametrize("value", [0, -1])
def test_non_positive_dims(lib, field, value):
    kw = {field: value}
    if field == "Hkv" and value == 0:
        kw["Hq"] = 8
    assert check(**kw) == fa.FA_ERR_BAD_DIM


def test_head_group(lib):
    assert check(Hq=7, Hkv=2) == fa.FA_ERR_HEAD_GROUP
    assert check(Hq=28, Hkv=4) == fa.FA_OK


@pytest.mark.parametrize("d", [1, 32, 63, 96, 127, 256])
def test_head_dim(lib, d):
    assert check(d=d) == fa.FA_ERR_HEAD_DIM


@pytest.mark.parametrize("dtype", [-1, 3, 99])
def test_dtype(lib, dtype):
    assert check(dtype=dtype) == fa.FA_ERR_DTYPE


@pytest.mark.parametrize("scale", [math.nan, math.inf, -math.inf])
def test_scale(lib, scale):
    assert check(scale=scale) == fa.FA_ERR_SCALE


def test_alignment(lib):
    assert check(q=Q + 8) == fa.FA_ERR_ALIGN
    assert check(o=O + 2) == fa.FA_ERR_ALIGN
    assert check(lse=L + 2) == fa.FA_ERR_ALIGN
    assert check(lse=L + 4) == fa.FA_OK


def test_aliasing(lib):
    assert check(o=Q) == fa.FA_ERR_ALIAS
    assert check(lse=V + 64) == fa.FA_ERR_ALIAS
    assert check(lse=O + 16) == fa.FA_ERR_ALIAS
    # o = [B,Hq,N_q,d] bf16 = 409600 bytes: a buffer right after it is fine
    assert check(lse=O + 2 * 8 * 100 * 128 * 2) == fa.FA_OK


def test_grid_too_large(lib):
    assert check(B=65536, Hq=65536, Hkv=1, N_q=128) == fa.FA_ERR_BAD_DIM


def test_fwd_rejects_on_host_without_touching_hip(lib):
    # Invalid calls return their code from fa_fwd and fa_fwd_stream too; with
    # no GPU in this process a call that reached HIP would report FA_ERR_HIP.
    a = args(d=96)
    st = fa.fa_fwd(Q, K, V, O, L, a["B"], a["Hq"], a["Hkv"], a["N_q"], a["N_kv"], a["d"],
                   a["scale"], a["causal"], a["dtype"])
    assert st == fa.FA_ERR_HEAD_DIM
    st = fa.fa_fwd_stream(0, K, V, O, L, 1, 1, 1, 1, 1, 64, 1.0, 0, fa.FA_BF16, None)
    assert st == fa.FA_ERR_NULL_PTR
    st = fa.fa_fwd_stream(Q, K, V, O, L, 1, 3, 2, 1, 1, 64, 1.0, 0, fa.FA_BF16, None)
    assert st == fa.FA_ERR_HEAD_GROUP


def test_status_strings(lib):
    for st in range(0, 11):
        s = fa.fa_status_string(st)
        assert isinstance(s, str) and s
    assert fa.fa_status_string(123) == "unknown status"


def test_launch_info(lib):
    st, info = fa.fa_launch_info(2, 32, 32, 8192, 8192, 128, 0, fa.FA_BF16)
    assert st == fa.FA_OK
    # d = 128 in 16 bits: four waves of 64 query rows each
    assert info["threads"] == 256 and info["rows_per_block"] == 256 and info["keys_per_tile"] == 64
    assert info["blocks"] == 2 * 32 * math.ceil(8192 / info["rows_per_block"])
    assert info["lds_bytes"] == 4 * 2 * 64 * 128 * 2   # 4 stages of a K and a V tile
    # d = 64 in 16 bits: the same kernel and shape, half the LDS
    st, info = fa.fa_launch_info(4, 16, 16, 1024, 1024, 64, 0, fa.FA_BF16)
    assert st == fa.FA_OK
    assert info["threads"] == 256 and info["rows_per_block"] == 256 and info["keys_per_tile"] == 64
    assert info["blocks"] == 4 * 16 * 4 and info["lds_bytes"] == 4 * 2 * 64 * 64 * 2
    st, info = fa.fa_launch_info(1, 1, 1, 256, 256, 64, 0, fa.FA_F32)
    assert st == fa.FA_OK and info["blocks"] == math.ceil(256 / info["rows_per_block"])
    assert fa.fa_launch_info(1, 1, 1, 0, 1, 64, 0, fa.FA_F32)[0] == fa.FA_ERR_BAD_DIM


def test_python_wrapper_rejects_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(fa.FAError):
        fa.attention(q, q, q)


def test_sequence_length_limit(lib):
    # one head of k/v (+256 rows) must stay below 2 GiB
    n_ok = (1 << 31) // (128 * 2) - 257
    far = dict(q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40, lse=5 << 40)
    assert check(N_q=16, N_kv=n_ok, B=1, Hq=1, Hkv=1, **far) == fa.FA_OK
    assert check(N_q=16, N_kv=n_ok + 2, B=1, Hq=1, Hkv=1, **far) == fa.FA_ERR_BAD_DIM


# ---- split-KV entry points ------------------------------------------------

W = 0x60000000   # fake workspace, clear of Q, K, V, O, L above


def split(q=Q, k=K, v=V, o=O, lse=L, ws=W, ws_bytes=None, S=2, **kw):
    a = args(**kw)
    if ws_bytes is None:
        ws_bytes = fa.fa_splitkv_workspace_bytes(a["B"], a["Hq"], a["N_q"], a["d"], S)
    # Every case below fails its host checks, so no call reaches HIP.
    return fa.fa_fwd_splitkv(q, k, v, o, lse, a["B"], a["Hq"], a["Hkv"], a["N_q"], a["N_kv"],
                             a["d"], a["scale"], a["causal"], a["dtype"], S, ws, ws_bytes, None)


def test_splitkv_workspace_bytes(lib):
    # O_s in fp32 for every (split, row, dim) plus one fp32 lse per (split, row)
    assert fa.fa_splitkv_workspace_bytes(8, 28, 1, 128, 64) == 64 * 8 * 28 * (128 + 1) * 4
    assert fa.fa_splitkv_workspace_bytes(2, 3, 5, 64, 1) == 2 * 3 * 5 * 65 * 4
    for bad in [(0, 1, 1, 64, 1), (1, 0, 1, 64, 1), (1, 1, 0, 64, 1), (1, 1, 1, 96, 1),
                (1, 1, 1, 64, 0), (1, 1, 1, 64, fa.FA_SPLITKV_MAX_SPLITS + 1)]:
        assert fa.fa_splitkv_workspace_bytes(*bad) == 0


def test_splitkv_default_splits(lib):
    # decode, 8 x 4 kv heads x 1 row block: 2048 waves / 32 items = 64 splits
    assert fa.fa_splitkv_default_splits(8, 28, 4, 1, 32768, 128, fa.FA_BF16) == 64
    # short keys: at least 4 tiles of 32 keys per split
    assert fa.fa_splitkv_default_splits(1, 8, 1, 1, 256, 64, fa.FA_F16) == 2
    # plenty of row blocks already: no split
    assert fa.fa_splitkv_default_splits(4, 32, 32, 2048, 2048, 128, fa.FA_BF16) == 1
    # never above the cap, invalid sizes give 0
    assert fa.fa_splitkv_default_splits(1, 1, 1, 1, 1 << 20, 64, fa.FA_BF16) == \
        fa.FA_SPLITKV_MAX_SPLITS
    assert fa.fa_splitkv_default_splits(1, 1, 1, 1, 64, 64, fa.FA_F32) == 0
    assert fa.fa_splitkv_default_splits(1, 3, 2, 1, 64, 64, fa.FA_BF16) == 0


def test_splitkv_rejects_on_host(lib):
    good = dict(N_q=1, N_kv=1000)
    assert split(ws=0, **good) == fa.FA_ERR_NULL_PTR
    assert split(dtype=fa.FA_F32, **good) == fa.FA_ERR_DTYPE
    assert split(S=0, **good) == fa.FA_ERR_BAD_DIM
    assert split(S=33, **good) == fa.FA_ERR_BAD_DIM          # 1000 keys = 32 tiles: S <= 32
    assert split(ws_bytes=16, **good) == fa.FA_ERR_WORKSPACE
    assert split(ws=W + 4, **good) == fa.FA_ERR_ALIGN
    assert split(ws=O, **good) == fa.FA_ERR_ALIAS
    assert split(ws=Q - 64, **good) == fa.FA_ERR_ALIAS
    assert split(d=96, **good) == fa.FA_ERR_HEAD_DIM
    assert split(Hq=7, **good) == fa.FA_ERR_HEAD_GROUP
    assert split(q=0, **good) == fa.FA_ERR_NULL_PTR


# ---- backward entry points ---------------------------------------------------

DO, DQ, DK, DV = 0x70000000, 0x80000000, 0x90000000, 0xA0000000


def bwd(q=Q, k=K, v=V, o=O, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, ws=W, ws_bytes=None, **kw):
    a = args(**kw)
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_bytes(a["B"], a["Hq"], a["Hkv"], a["N_q"], a["N_kv"], a["d"])
    # Every case below fails its host checks, so no call reaches HIP.
    return fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, a["B"], a["Hq"], a["Hkv"], a["N_q"],
                     a["N_kv"], a["d"], a["scale"], a["causal"], a["dtype"], ws, ws_bytes, None)


def test_bwd_workspace_bytes(lib):
    # row statistics (8 B per query row, rounded up to 256 B) ...
    assert fa.fa_bwd_workspace_bytes(2, 32, 32, 8192, 8192, 128) == 2 * 32 * 8192 * 8
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 10, 10, 64) == 256
    # ... plus fp32 partial dK, dV per head share when few key/value heads:
    # 1 x 4 kv heads x 16 key tiles = 64 workgroups -> 7 shares (all 7 heads)
    assert fa.fa_bwd_workspace_bytes(1, 28, 4, 4096, 4096, 128) == \
        28 * 4096 * 8 + 7 * 2 * 4 * 4096 * 128 * 4
    for bad in [(0, 8, 8, 100, 100, 64), (1, 7, 2, 10, 10, 64), (1, 1, 1, 0, 1, 64),
                (1, 1, 1, 1, 1, 96)]:
        assert fa.fa_bwd_workspace_bytes(*bad) == 0


def test_bwd_rejects_on_host(lib):
    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "ws"):
        assert bwd(**{name: 0}) == fa.FA_ERR_NULL_PTR, name
    assert bwd(dtype=fa.FA_F32) == fa.FA_ERR_DTYPE
    assert bwd(d=96) == fa.FA_ERR_HEAD_DIM
    assert bwd(Hq=7) == fa.FA_ERR_HEAD_GROUP
    assert bwd(N_kv=0) == fa.FA_ERR_BAD_DIM
    assert bwd(scale=math.nan) == fa.FA_ERR_SCALE
    assert bwd(dq=DQ + 8) == fa.FA_ERR_ALIGN
    assert bwd(lse=L + 2) == fa.FA_ERR_ALIGN
    assert bwd(ws_bytes=8) == fa.FA_ERR_WORKSPACE
    assert bwd(dq=Q) == fa.FA_ERR_ALIAS          # output over an input
    assert bwd(dk=DO + 64) == fa.FA_ERR_ALIAS
    assert bwd(dv=DK) == fa.FA_ERR_ALIAS         # outputs over each other
    assert bwd(ws=DQ + 16) == fa.FA_ERR_ALIAS


def fp8(q=Q, k=K, v=V, o=O, lse=L, dq_=0.01, dk_=0.02, dv_=0.03, **kw):
    a = args(**kw)
    return fa.fa_fwd_fp8(q, k, v, o, lse, a["B"], a["Hq"], a["Hkv"], a["N_q"], a["N_kv"], a["d"],
                         a["scale"], a["causal"], dq_, dk_, dv_, None)


def test_fp8_rejects_on_host(lib):
    for name in ("q", "k", "v", "o", "lse"):
        assert fp8(**{name: 0}) == fa.FA_ERR_NULL_PTR, name
    assert fp8(d=96) == fa.FA_ERR_HEAD_DIM
    assert fp8(Hq=7) == fa.FA_ERR_HEAD_GROUP
    assert fp8(N_q=0) == fa.FA_ERR_BAD_DIM
    assert fp8(B=-1) == fa.FA_ERR_BAD_DIM
    assert fp8(N_kv=1 << 30) == fa.FA_ERR_BAD_DIM
    assert fp8(scale=math.inf) == fa.FA_ERR_SCALE
    for bad in (0.0, -0.5, math.nan, math.inf):
        assert fp8(dq_=bad) == fa.FA_ERR_SCALE
        assert fp8(dk_=bad) == fa.FA_ERR_SCALE
        assert fp8(dv_=bad) == fa.FA_ERR_SCALE
    assert fp8(q=Q + 8) == fa.FA_ERR_ALIGN
    assert fp8(o=O + 4) == fa.FA_ERR_ALIGN
    assert fp8(lse=L + 2) == fa.FA_ERR_ALIGN
    # o holds 2-byte elements over 1-byte inputs: its extent is twice q's
    nq = 2 * 8 * 100 * 128
    assert fp8(o=Q + nq - 16) == fa.FA_ERR_ALIAS
    assert fp8(lse=O + 2 * nq - 16) == fa.FA_ERR_ALIAS


KC, VC, TB, SL, WS = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000
PG = dict(B=2, Hq=8, Hkv=2, N_q=1, d=128, num_blocks=64, block_size=16, mbps=32, scale=0.125,
          causal=0, dtype=fa.FA_BF16, splits=4)


def paged(q=Q, kc=KC, vc=VC, tb=TB, sl=SL, o=O, lse=L, ws=WS, ws_bytes=1 << 20, **kw):
    a = dict(PG)
    a.update(kw)
    return fa.fa_fwd_paged(q, kc, vc, tb, sl, o, lse, a["B"], a["Hq"], a["Hkv"], a["N_q"], a["d"],
                           a["num_blocks"], a["block_size"], a["mbps"], a["scale"], a["causal"],
                           a["dtype"], a["splits"], ws, ws_bytes, None)


def test_paged_rejects_on_host(lib):
    for name in ("q", "kc", "vc", "tb", "sl", "o", "lse", "ws"):
        assert paged(**{name: 0}) == fa.FA_ERR_NULL_PTR, name
    assert paged(dtype=fa.FA_F32) == fa.FA_ERR_DTYPE
    assert paged(d=96) == fa.FA_ERR_HEAD_DIM
    assert paged(Hq=7) == fa.FA_ERR_HEAD_GROUP
    for bs in (8, 24, 0, -16, 1 << 17):
        assert paged(block_size=bs) == fa.FA_ERR_BAD_DIM, bs
    assert paged(num_blocks=0) == fa.FA_ERR_BAD_DIM
    assert paged(mbps=0) == fa.FA_ERR_BAD_DIM
    assert paged(num_blocks=1 << 20, block_size=256) == fa.FA_ERR_BAD_DIM   # cache >= 4 GiB
    assert paged(splits=0) == fa.FA_ERR_BAD_DIM
    assert paged(splits=17) == fa.FA_ERR_BAD_DIM       # 32 blocks x 16 keys = 16 tiles
    assert paged(scale=math.nan) == fa.FA_ERR_SCALE
    assert paged(ws_bytes=64) == fa.FA_ERR_WORKSPACE
    assert paged(kc=KC + 8) == fa.FA_ERR_ALIGN
    assert paged(tb=TB + 2) == fa.FA_ERR_ALIGN
    assert paged(sl=SL + 1) == fa.FA_ERR_ALIGN
    assert paged(o=KC + 64) == fa.FA_ERR_ALIAS          # output inside a cache
    assert paged(ws=TB) == fa.FA_ERR_ALIAS              # workspace over the block table
    assert paged(lse=O + 16) == fa.FA_ERR_ALIAS         # outputs over each other


def test_noalloc_rejects_on_host(lib):
    """fa_fwd_splitkv_noalloc checks everything on the host first: invalid
    arguments and sizes whose chunk results exceed its scratch array return
    before any HIP call (no GPU in this process: reaching HIP would give
    FA_ERR_HIP)."""
    f = lib.fa_fwd_splitkv_noalloc
    # B=8 Hq=28 N_q=1 d=128: 115584 bytes per split; 145 splits fit in 16 MiB, 146 do not.
    per = fa.fa_splitkv_workspace_bytes(8, 28, 1, 128, 1)
    assert per == 8 * 28 * 129 * 4
    assert 145 * per <= fa.FA_NOALLOC_SCRATCH_BYTES < 146 * per
    st = f(Q, K, V, O, L, 8, 28, 4, 1, 32768, 128, 0.1, 0, fa.FA_BF16, 146, None)
    assert st == fa.FA_ERR_WORKSPACE
    assert f(Q, K, V, O, L, 8, 28, 4, 1, 1000, 128, 0.1, 0, fa.FA_F32, 8, None) == fa.FA_ERR_DTYPE
    assert f(0, K, V, O, L, 8, 28, 4, 1, 32768, 128, 0.1, 0, fa.FA_BF16, 8, None) == fa.FA_ERR_NULL_PTR
    assert f(Q, K, V, O, L, 8, 28, 4, 1, 100, 128, 0.1, 0, fa.FA_BF16, 5, None) == fa.FA_ERR_BAD_DIM
    assert f(Q, K, V, Q, L, 8, 28, 4, 1, 100, 128, 0.1, 0, fa.FA_BF16, 2, None) == fa.FA_ERR_ALIAS
