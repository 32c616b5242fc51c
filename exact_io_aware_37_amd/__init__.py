"""Python binding of the exact attention forward library (libfa.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/fa.h.  The functions named like
the C entry points take the same arguments (pointers may be given as ints or
as torch tensors) and return the C status code.  ``attention`` is the
convenience form: it checks the tensors, allocates O and lse with torch on
the inputs' device and launches on torch's current stream.

There is no fallback: if libfa.so is missing or fails to load, every call
raises.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "fa.h")

FA_OK = 0
FA_ERR_NULL_PTR = 1
FA_ERR_BAD_DIM = 2
FA_ERR_HEAD_GROUP = 3
FA_ERR_HEAD_DIM = 4
FA_ERR_DTYPE = 5
FA_ERR_SCALE = 6
FA_ERR_ALIGN = 7
FA_ERR_HIP = 8
FA_ERR_ALIAS = 9
FA_ERR_WORKSPACE = 10
FA_SPLITKV_MAX_SPLITS = 256
FA_NOALLOC_SCRATCH_BYTES = 16 << 20

FA_F32 = 0
FA_F16 = 1
FA_BF16 = 2


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fa status {status}: {message}")
        self.status = status


_lib = None

_VP = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_FWD_ARGS = [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _F, _I, _I]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FAError(-1, f"{path} is missing: build it with "
                          "`python -m exact_io_aware_37_amd.build`")
    lib = ctypes.CDLL(path)
    lib.fa_fwd.argtypes = list(_FWD_ARGS)
    lib.fa_fwd.restype = _I
    lib.fa_fwd_stream.argtypes = list(_FWD_ARGS) + [_VP]
    lib.fa_fwd_stream.restype = _I
    lib.fa_check_args.argtypes = list(_FWD_ARGS)
    lib.fa_check_args.restype = _I
    lib.fa_status_string.argtypes = [_I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_launch_info.argtypes = [_I] * 8 + [ctypes.POINTER(_I)] * 3 + \
        [ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(_I)]
    lib.fa_launch_info.restype = _I
    lib.fa_splitkv_workspace_bytes.argtypes = [_I] * 5
    lib.fa_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_splitkv_default_splits.argtypes = [_I] * 7
    lib.fa_splitkv_default_splits.restype = _I
    lib.fa_fwd_splitkv.argtypes = list(_FWD_ARGS) + [_I, _VP, ctypes.c_size_t, _VP]
    lib.fa_fwd_splitkv.restype = _I
    lib.fa_fwd_splitkv_noalloc.argtypes = list(_FWD_ARGS) + [_I, _VP]
    lib.fa_fwd_splitkv_noalloc.restype = _I
    lib.fa_bwd_workspace_bytes.argtypes = [_I] * 6
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [_VP] * 9 + [_I] * 6 + [_F, _I, _I, _VP, ctypes.c_size_t, _VP]
    lib.fa_bwd.restype = _I
    lib.fa_fwd_fp8.argtypes = list(_FWD_ARGS[:13]) + [_F, _F, _F, _VP]
    lib.fa_fwd_fp8.restype = _I
    lib.fa_fwd_paged.argtypes = [_VP] * 7 + [_I] * 8 + [_F, _I, _I, _I, _VP, ctypes.c_size_t, _VP]
    lib.fa_fwd_paged.restype = _I
    _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/fa.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype) -> int:
    return load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                 N_q, N_kv, d, scale, int(causal), dtype)


def fa_fwd_stream(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype,
                  stream) -> int:
    s = stream if (stream is None or isinstance(stream, int)) else stream.cuda_stream
    return load_library().fa_fwd_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq,
                                        Hkv, N_q, N_kv, d, scale, int(causal), dtype, s)


def fa_check_args(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype) -> int:
    return load_library().fa_check_args(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq,
                                        Hkv, N_q, N_kv, d, scale, int(causal), dtype)


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(status).decode()


def fa_launch_info(B, Hq, Hkv, N_q, N_kv, d, causal, dtype):
    """(status, dict) with rows_per_block, keys_per_tile, threads, blocks, lds_bytes."""
    r, kt, th, lds = _I(), _I(), _I(), _I()
    nb = ctypes.c_longlong()
    st = load_library().fa_launch_info(B, Hq, Hkv, N_q, N_kv, d, int(causal), dtype,
                                       ctypes.byref(r), ctypes.byref(kt), ctypes.byref(th),
                                       ctypes.byref(nb), ctypes.byref(lds))
    return st, dict(rows_per_block=r.value, keys_per_tile=kt.value, threads=th.value,
                    blocks=nb.value, lds_bytes=lds.value)


def fa_splitkv_workspace_bytes(B, Hq, N_q, d, num_splits) -> int:
    return load_library().fa_splitkv_workspace_bytes(B, Hq, N_q, d, num_splits)


def fa_splitkv_default_splits(B, Hq, Hkv, N_q, N_kv, d, dtype) -> int:
    return load_library().fa_splitkv_default_splits(B, Hq, Hkv, N_q, N_kv, d, dtype)


def fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype, num_splits,
                   workspace, workspace_bytes, stream) -> int:
    s = stream if (stream is None or isinstance(stream, int)) else stream.cuda_stream
    return load_library().fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq,
                                         Hkv, N_q, N_kv, d, scale, int(causal), dtype,
                                         num_splits, _ptr(workspace), workspace_bytes, s)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype,
                           num_splits, stream) -> int:
    s = stream if (stream is None or isinstance(stream, int)) else stream.cuda_stream
    return load_library().fa_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                 B, Hq, Hkv, N_q, N_kv, d, scale, int(causal),
                                                 dtype, num_splits, s)


def fa_bwd_workspace_bytes(B, Hq, Hkv, N_q, N_kv, d) -> int:
    return load_library().fa_bwd_workspace_bytes(B, Hq, Hkv, N_q, N_kv, d)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype,
           workspace, workspace_bytes, stream) -> int:
    s = stream if (stream is None or isinstance(stream, int)) else stream.cuda_stream
    return load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                 _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, N_q, N_kv, d, scale,
                                 int(causal), dtype, _ptr(workspace), workspace_bytes, s)


def fa_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, descale_q, descale_k,
               descale_v, stream) -> int:
    s = stream if (stream is None or isinstance(stream, int)) else stream.cuda_stream
    return load_library().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                     N_q, N_kv, d, scale, int(causal), descale_q, descale_k,
                                     descale_v, s)


def fa_fwd_paged(q, k_cache, v_cache, block_table, seqlens_k, o, lse, B, Hq, Hkv, N_q, d,
                 num_blocks, block_size, max_blocks_per_seq, scale, causal, dtype, num_splits,
                 workspace, workspace_bytes, stream) -> int:
    s = stream if (stream is None or isinstance(stream, int)) else stream.cuda_stream
    return load_library().fa_fwd_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                       _ptr(seqlens_k), _ptr(o), _ptr(lse), B, Hq, Hkv, N_q, d,
                                       num_blocks, block_size, max_blocks_per_seq, scale,
                                       int(causal), dtype, num_splits, _ptr(workspace),
                                       workspace_bytes, s)


def dtype_code(torch_dtype) -> int:
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if torch_dtype not in codes:
        raise FAError(FA_ERR_DTYPE, f"unsupported dtype {torch_dtype}")
    return codes[torch_dtype]


def attention(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
              stream=None):
    """O, lse = softmax(scale * q k^T) v on the GPU; q [B,Hq,Nq,d], k/v [B,Hkv,Nkv,d].

    ``scale`` defaults to 1/sqrt(d).  ``out``/``lse`` may be given to reuse
    buffers.  Launches on ``stream`` (default: torch's current stream of q's
    device) and returns without synchronising.
    """
    import torch
    B, Hq, Hkv, Nq, Nkv, d = _check_tensors(q, k, v)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    out = torch.empty_like(q) if out is None else \
        _check_out(out, "out", q.shape, q.dtype, q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else \
        _check_out(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd_stream(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, d, float(scale), causal,
                       dtype_code(q.dtype), stream)
    if st != FA_OK:
        raise FAError(st, fa_status_string(st))
    return out, lse


def fwd(q, k, v, *, causal: bool = False, scale: float | None = None):
    """(o, lse) = the exact attention forward of q [B,Hq,N_q,d] over k, v [B,Hkv,N_kv,d].

    o has q's dtype and shape; lse [B,Hq,N_q] is fp32, the natural-log
    logsumexp of each row's scaled scores.  ``scale`` defaults to 1/sqrt(d).
    Both are allocated by torch on q's device; the call launches fa_fwd_stream
    on torch's current stream and returns without synchronising.
    """
    return attention(q, k, v, causal=causal, scale=scale)


def _check_tensors(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise FAError(FA_ERR_NULL_PTR, f"{name} must be a GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise FAError(FA_ERR_BAD_DIM, f"{name} must be a contiguous 4-D tensor")
    if not (q.dtype == k.dtype == v.dtype):
        raise FAError(FA_ERR_DTYPE, "q, k and v must share one dtype")
    if not (q.device == k.device == v.device):
        raise FAError(FA_ERR_NULL_PTR, "q, k and v must be on one GPU")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nkv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise FAError(FA_ERR_BAD_DIM, f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} "
                                      f"v{tuple(v.shape)}")
    return B, Hq, Hkv, Nq, Nkv, d


def _check_out(t, name: str, shape, dtype, device):
    """Raise unless a caller-supplied output buffer is exactly what the kernels write.

    The C ABI sizes every store from the input dimensions, so a buffer on
    another device, of another dtype or shape, or not contiguous would be
    written out of bounds (or through a host address).  Checked before any
    launch."""
    if not getattr(t, "is_cuda", False) or t.device != device:
        raise FAError(FA_ERR_NULL_PTR, f"{name} must be a GPU tensor on {device}")
    if t.dtype != dtype:
        raise FAError(FA_ERR_DTYPE, f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise FAError(FA_ERR_BAD_DIM, f"{name} must have shape {tuple(shape)}, got "
                                      f"{tuple(t.shape)}")
    if not t.is_contiguous():
        raise FAError(FA_ERR_BAD_DIM, f"{name} must be contiguous")
    return t


def _check_workspace(t, device):
    """A caller-supplied workspace: a contiguous tensor on the inputs' GPU (its byte
    size is passed to the C ABI, which rejects one that is too small)."""
    if not getattr(t, "is_cuda", False) or t.device != device:
        raise FAError(FA_ERR_NULL_PTR, f"workspace must be a GPU tensor on {device}")
    if not t.is_contiguous():
        raise FAError(FA_ERR_BAD_DIM, "workspace must be contiguous")
    return t


def attention_splitkv(q, k, v, causal: bool = False, scale: float | None = None,
                      num_splits: int | None = None, workspace=None, out=None, lse=None,
                      stream=None):
    """Split-KV (FlashDecoding) form of ``attention``: same result, for few query rows.

    ``num_splits`` defaults to fa_splitkv_default_splits.  ``workspace`` (a
    CUDA tensor of at least fa_splitkv_workspace_bytes bytes) may be given to
    reuse memory; otherwise torch allocates one.  Returns (out, lse).
    """
    import torch
    B, Hq, Hkv, Nq, Nkv, d = _check_tensors(q, k, v)
    dt = dtype_code(q.dtype)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if num_splits is None:
        num_splits = fa_splitkv_default_splits(B, Hq, Hkv, Nq, Nkv, d, dt)
        if num_splits < 1:
            raise FAError(FA_ERR_BAD_DIM, "no valid split count for these sizes")
    need = fa_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    out = torch.empty_like(q) if out is None else \
        _check_out(out, "out", q.shape, q.dtype, q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else \
        _check_out(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd_splitkv(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, d, float(scale), causal, dt,
                        num_splits, workspace, ws_bytes, stream)
    if st != FA_OK:
        raise FAError(st, fa_status_string(st))
    return out, lse


def attention_splitkv_noalloc(q, k, v, out, lse, causal: bool = False,
                              scale: float | None = None, num_splits: int | None = None,
                              stream=None):
    """``attention_splitkv`` through the allocation-free entry point: the chunk
    results live in the library's per-GPU scratch array, and ``out``/``lse``
    are caller-owned (nothing is allocated here or in the library).  Calls
    that overlap on one GPU race on the scratch array; order them on one
    stream.  Returns (out, lse)."""
    import torch
    B, Hq, Hkv, Nq, Nkv, d = _check_tensors(q, k, v)
    dt = dtype_code(q.dtype)
    _check_out(out, "out", q.shape, q.dtype, q.device)
    _check_out(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if num_splits is None:
        num_splits = fa_splitkv_default_splits(B, Hq, Hkv, Nq, Nkv, d, dt)
        if num_splits < 1:
            raise FAError(FA_ERR_BAD_DIM, "no valid split count for these sizes")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd_splitkv_noalloc(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, d, float(scale), causal,
                                dt, num_splits, stream)
    if st != FA_OK:
        raise FAError(st, fa_status_string(st))
    return out, lse


def attention_fp8(q, k, v, descale_q: float, descale_k: float, descale_v: float,
                  causal: bool = False, scale: float | None = None, out=None, lse=None,
                  stream=None):
    """E4M3 form of ``attention``: q, k, v are torch.float8_e4m3fn (or uint8 code) GPU
    tensors whose values are code * descale; returns (out bf16, lse fp32)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise FAError(FA_ERR_DTYPE, f"{name} must hold E4M3 codes (float8_e4m3fn or uint8)")
    B, Hq, Hkv, Nq, Nkv, d = _check_tensors(q, k, v)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    out = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=q.device) if out is None \
        else _check_out(out, "out", (B, Hq, Nq, d), torch.bfloat16, q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else \
        _check_out(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd_fp8(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, d, float(scale), causal,
                    float(descale_q), float(descale_k), float(descale_v), stream)
    if st != FA_OK:
        raise FAError(st, fa_status_string(st))
    return out, lse


def attention_paged(q, k_cache, v_cache, block_table, seqlens_k, causal: bool = False,
                    scale: float | None = None, num_splits: int | None = None, workspace=None,
                    out=None, lse=None, stream=None):
    """Split-KV attention of q [B, Hq, N_q, d] over paged caches.

    k_cache, v_cache: [num_blocks, block_size, Hkv, d] GPU tensors of q's dtype;
    block_table: int32 [B, max_blocks]; seqlens_k: int32 [B] (GPU).  With
    ``causal`` the N_q queries are the last N_q positions of each sequence.
    Returns (out, lse).
    """
    import torch
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seqlens_k", seqlens_k)):
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise FAError(FA_ERR_NULL_PTR, f"{name} must be a contiguous tensor on q's GPU")
    if block_table.dtype != torch.int32 or seqlens_k.dtype != torch.int32:
        raise FAError(FA_ERR_DTYPE, "block_table and seqlens_k must be int32")
    if q.dtype != k_cache.dtype or q.dtype != v_cache.dtype or k_cache.shape != v_cache.shape:
        raise FAError(FA_ERR_DTYPE, "q, k_cache and v_cache must share dtype; caches one shape")
    B, Hq, Nq, d = q.shape
    nb, bs, Hkv, dk = k_cache.shape
    if dk != d or block_table.dim() != 2 or block_table.shape[0] != B or seqlens_k.shape != (B,):
        raise FAError(FA_ERR_BAD_DIM, "shape mismatch between q, caches, block_table and seqlens")
    mbps = block_table.shape[1]
    dt = dtype_code(q.dtype)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if num_splits is None:
        num_splits = fa_splitkv_default_splits(B, Hq, Hkv, Nq, mbps * bs, d, dt)
        if num_splits < 1:
            raise FAError(FA_ERR_BAD_DIM, "no valid split count for these sizes")
    need = fa_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
    out = torch.empty_like(q) if out is None else \
        _check_out(out, "out", q.shape, q.dtype, q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else \
        _check_out(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd_paged(q, k_cache, v_cache, block_table, seqlens_k, out, lse, B, Hq, Hkv, Nq, d,
                      nb, bs, mbps, float(scale), causal, dt, num_splits, workspace,
                      workspace.numel() * workspace.element_size(), stream)
    if st != FA_OK:
        raise FAError(st, fa_status_string(st))
    return out, lse


def attention_backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
                       workspace=None, dq=None, dk=None, dv=None, stream=None):
    """(dq, dk, dv): gradients of sum(o * dout) for o, lse = attention(q, k, v, causal, scale).

    ``o`` and ``lse`` are the forward's outputs.  ``workspace`` (at least
    fa_bwd_workspace_bytes bytes) may be given to reuse memory.
    """
    import torch
    B, Hq, Hkv, Nq, Nkv, d = _check_tensors(q, k, v)
    for name, t in (("o", o), ("dout", dout)):
        _check_out(t, name, q.shape, q.dtype, q.device)
    _check_out(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    need = fa_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device)
    dq = torch.empty_like(q) if dq is None else _check_out(dq, "dq", q.shape, q.dtype, q.device)
    dk = torch.empty_like(k) if dk is None else _check_out(dk, "dk", k.shape, k.dtype, q.device)
    dv = torch.empty_like(v) if dv is None else _check_out(dv, "dv", v.shape, v.dtype, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, d, float(scale), causal,
                dtype_code(q.dtype), workspace, workspace.numel() * workspace.element_size(), stream)
    if st != FA_OK:
        raise FAError(st, fa_status_string(st))
    return dq, dk, dv


__all__ = ["fa_fwd", "fa_fwd_stream", "fa_check_args", "fa_status_string", "fa_launch_info",
           "fa_splitkv_workspace_bytes", "fa_splitkv_default_splits", "fa_fwd_splitkv",
           "fa_fwd_splitkv_noalloc", "attention_splitkv_noalloc",
           "fa_bwd_workspace_bytes", "fa_bwd", "fa_fwd_fp8", "fa_fwd_paged",
           "fwd", "attention", "attention_splitkv", "attention_backward", "attention_fp8",
           "attention_paged", "load_library", "header_functions", "FAError", "dtype_code",
           "FA_F32", "FA_F16", "FA_BF16"]
