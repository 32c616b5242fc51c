"""Seeded synthetic inputs for the attention forward.

This module only draws random tensors; it holds none of the attention
arithmetic.  Both sides of every comparison take their inputs from here: the
HIP library (through its Python binding) and the fp64 oracle (which widens the
very same low-precision values exactly to float64).

The five named workloads have the shapes of the pages' setting: the course
lab of "FlashAttention: IO-aware attention kernel" (§5) uses random
[B, H, S, D] bf16 tensors in a 7B decoder's attention shape (28 heads of 128)
with a causal mask; the others are multi-head and long-sequence variants.
Workload 6 is one decoding step of that 7B shape (one new query row per
sequence against a 32768-key cache, batch 8), the case the same page (§3,
where the method helps and where it does not) sends to the split-KV
FlashDecoding variant.  Workload 7 is workload 3's shape with 8-bit E4M3
inputs (the FP8 direction the pages name for FlashAttention-3), quantised from
the same kind of draws by ``make_inputs_fp8``.  Workload 8 is workload 6
with its K/V cache scattered into 16-key blocks of a paged cache
(``paginate``), the form a serving engine keeps a cache in.  No public
dataset is involved; nothing is read from disk.

Recipe (all workloads): ``numpy.random.default_rng(seed)`` (PCG64), draw Q,
then K, then (for outlier workloads) the outlier rows of K, then V, each as
``standard_normal(shape, float32) * sigma``; outlier rows are
``round(frac * Nkv)`` row indices per (b, kv-head) chosen without
replacement and multiplied by a power of two (exact, commutes with the cast);
finally each tensor is cast to the workload dtype with torch's CPU
round-to-nearest-even conversion.  ``scale`` is float32(1/sqrt(D)).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, asdict

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    dtype: str
    causal: bool
    sigma: float = 1.0
    outlier_frac: float = 0.0
    outlier_mult: float = 8.0
    block_size: int = 0          # > 0: K/V held in a paged cache of blocks of this many keys

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def scale(self) -> float:
        return default_scale(self.D)

    def flops(self) -> float:
        """4*B*Hq*Nq*Nkv*D, halved for causal (the throughput metric's count)."""
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nkv * self.D
        return f / 2.0 if self.causal else f

    def io_bytes(self) -> float:
        """Compulsory HBM bytes of one forward: Q, K, V read once, O and lse written once
        (an e4m3 workload reads 1-byte Q, K, V and writes a bf16 O)."""
        es_in = {"f32": 4, "e4m3": 1}.get(self.dtype, 2)
        es_out = 4 if self.dtype == "f32" else 2
        q = self.B * self.Hq * self.Nq * self.D
        kv = self.B * self.Hkv * self.Nkv * self.D
        return float(es_in * (q + 2 * kv) + es_out * q + 4 * self.B * self.Hq * self.Nq)

    def as_dict(self) -> dict:
        d = asdict(self)
        d["seed"] = self.seed
        return d


WORKLOADS = {
    1: Workload(1, "tiny_exact_f32", 1, 1, 1, 256, 256, 64, "f32", False),
    2: Workload(2, "multihead_bf16_n1024_d64", 4, 16, 16, 1024, 1024, 64, "bf16", False),
    3: Workload(3, "long_noncausal_bf16_n8192_d128", 2, 32, 32, 8192, 8192, 128, "bf16", False),
    4: Workload(4, "causal_gqa_7b_prefill_n4096", 1, 28, 4, 4096, 4096, 128, "bf16", True),
    5: Workload(5, "long_causal_gqa_n32768_outlier_keys", 1, 28, 4, 32768, 32768, 128, "bf16",
                True, sigma=0.5, outlier_frac=0.01, outlier_mult=8.0),
    6: Workload(6, "decode_gqa_7b_b8_n32768", 8, 28, 4, 1, 32768, 128, "bf16", False),
    7: Workload(7, "long_noncausal_e4m3_n8192_d128", 2, 32, 32, 8192, 8192, 128, "e4m3", False),
    8: Workload(8, "decode_gqa_7b_b8_n32768_paged_bs16", 8, 28, 4, 1, 32768, 128, "bf16", False,
                block_size=16),
}


def default_scale(D: int) -> float:
    return float(np.float32(1.0 / math.sqrt(D)))


def make_inputs(B, Hq, Hkv, Nq, Nkv, D, dtype="bf16", seed=0, sigma=1.0,
                outlier_frac=0.0, outlier_mult=8.0):
    """Draw (q, k, v) as contiguous CPU torch tensors of ``dtype``."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Nkv, D), dtype=np.float32)
    if sigma != 1.0:
        q *= np.float32(sigma)
        k *= np.float32(sigma)
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * Nkv))
        for b in range(B):
            for g in range(Hkv):
                rows = rng.choice(Nkv, size=n_out, replace=False)
                k[b, g, rows, :] *= np.float32(outlier_mult)
    v = rng.standard_normal((B, Hkv, Nkv, D), dtype=np.float32)
    if sigma != 1.0:
        v *= np.float32(sigma)
    tdt = DTYPES[dtype]
    return tuple(torch.from_numpy(x).to(tdt).contiguous() for x in (q, k, v))


E4M3_MAX = 448.0


def make_inputs_fp8(B, Hq, Hkv, Nq, Nkv, D, seed=0, sigma=1.0, outlier_frac=0.0,
                    outlier_mult=8.0):
    """Draw (q8, k8, v8) as torch.float8_e4m3fn CPU tensors plus their fp32 descales.

    The float32 draws are those of ``make_inputs`` with the same arguments.
    Each tensor is quantised with one factor: descale = float32(max|x| / 448)
    (1 for an all-zero tensor), codes = x / descale rounded to nearest even by
    torch's CPU conversion (clamped to +-448 first against a last-bit overshoot
    of the division).  Value of a code: decode(code) * descale.
    """
    xs = make_inputs(B, Hq, Hkv, Nq, Nkv, D, "f32", seed, sigma, outlier_frac, outlier_mult)
    codes, descales = [], []
    for x in xs:
        amax = float(x.abs().max()) if x.numel() else 0.0
        ds = float(np.float32(amax / E4M3_MAX)) if amax > 0.0 else 1.0
        y = (x / torch.tensor(ds, dtype=torch.float32)).clamp(-E4M3_MAX, E4M3_MAX)
        codes.append(y.to(torch.float8_e4m3fn).contiguous())
        descales.append(ds)
    return tuple(codes), tuple(descales)


def workload_inputs_fp8(w: Workload):
    """((q8, k8, v8), (descale_q, descale_k, descale_v), scale) for an e4m3 workload."""
    codes, ds = make_inputs_fp8(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, w.seed, w.sigma,
                                w.outlier_frac, w.outlier_mult)
    return codes, ds, w.scale


def paginate(k: torch.Tensor, v: torch.Tensor, seqlens, block_size: int, seed: int = 0,
             spare_blocks: int = 2):
    """Scatter dense K/V [B, Hkv, N, D] into paged caches, as a serving engine would hold them.

    Returns (k_cache, v_cache, block_table, seqlens): caches
    [num_blocks, block_size, Hkv, D] (the layout vLLM's flash-attention backend
    passes to its kernel), int32 block_table [B, max_blocks] and int32
    seqlens [B].  Sequence b's keys 0..seqlens[b]-1 go to blocks drawn from a
    seeded permutation of the pool; table entries past a sequence's blocks are
    -1.  Every slot that holds no key (spare blocks, the tail of a sequence's
    last block) is NaN, so a read outside the table's keys shows in results.
    """
    B, Hkv, N, D = k.shape
    lens = [int(x) for x in seqlens]
    assert len(lens) == B and all(0 <= n <= N for n in lens)
    nblk = [(n + block_size - 1) // block_size for n in lens]
    total = sum(nblk) + spare_blocks
    perm = np.random.default_rng(seed).permutation(total)
    kc = torch.full((total, block_size, Hkv, D), float("nan"), dtype=k.dtype)
    vc = torch.full((total, block_size, Hkv, D), float("nan"), dtype=v.dtype)
    table = torch.full((B, max(1, max(nblk))), -1, dtype=torch.int32)
    nxt = 0
    for b in range(B):
        ids = torch.from_numpy(perm[nxt:nxt + nblk[b]].astype(np.int64))
        nxt += nblk[b]
        table[b, :nblk[b]] = ids.to(torch.int32)
        full = lens[b] // block_size
        if full:
            kc[ids[:full]] = k[b, :, :full * block_size].reshape(Hkv, full, block_size, D).permute(1, 2, 0, 3)
            vc[ids[:full]] = v[b, :, :full * block_size].reshape(Hkv, full, block_size, D).permute(1, 2, 0, 3)
        rest = lens[b] - full * block_size
        if rest:
            kc[ids[full], :rest] = k[b, :, full * block_size:lens[b]].permute(1, 0, 2)
            vc[ids[full], :rest] = v[b, :, full * block_size:lens[b]].permute(1, 0, 2)
    return kc.contiguous(), vc.contiguous(), table, torch.tensor(lens, dtype=torch.int32)


def codes_of(t: torch.Tensor) -> np.ndarray:
    """The raw byte codes of a float8 CPU tensor, as a uint8 array."""
    return t.detach().to("cpu").contiguous().view(torch.uint8).numpy()


def workload_inputs(w: Workload):
    """(q, k, v, scale) for a named workload."""
    q, k, v = make_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, w.dtype, w.seed,
                          w.sigma, w.outlier_frac, w.outlier_mult)
    return q, k, v, w.scale


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a CPU tensor (f32/f16/bf16) to a float64 array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
