"""fp64 reference for the FP8 (e4m3) variant of the attention forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* [P1] "FlashAttention: IO-aware attention kernel" (inference-learning-path
  course, part 2), §3.3 and [P2] the omica exam notes, §四.5 name the
  FlashAttention-3 line of work, whose new ingredient is FP8 inputs to the
  same exact tiled algorithm.  The pages fix neither the 8-bit format nor a
  scaling recipe.  The plainest reading, taken here:
    - Q, K and V arrive as 8-bit codes of the OCP "8-bit floating point"
      E4M3 format with one fp32 dequantisation factor per tensor
      (value = decode(code) * descale);
    - the attention itself is the exact one of ``attention_ref`` applied to
      the dequantised values: O = softmax(scale * Q K^T) V, lse per row.
* The OCP 8-bit floating point specification (E4M3 variant) defines the
  decoding written out in ``e4m3_decode``: 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals at exponent field 0, no infinities, and
  NaN only for exponent and mantissa fields all ones (largest finite 448).

``fp8_p_rounding_bound`` is the tolerance model of the GPU path, which
rounds the probabilities to E4M3 before the P*V product (the way the
FlashAttention-3 line feeds its second product) and divides by the sum of
the unrounded probabilities.
"""

from __future__ import annotations

import numpy as np

from .attention_ref import _check_shapes, _sigma, attention_fp64, kv_head_of


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each OCP E4M3 code (uint8 array-like).

    sign * 2^(e-7) * (1 + m/8) for exponent field e in 1..15, sign * 2^-6 *
    (m/8) for e = 0; the codes with e = 15 and m = 7 (0x7F, 0xFF) are NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def dequantize_e4m3(codes, descale: float) -> np.ndarray:
    """decode(codes) * descale, with descale taken as the float32 the GPU receives."""
    return e4m3_decode(codes) * float(np.float32(descale))


def attention_fp8_fp64(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float,
                       scale: float, causal: bool = False, rows=None):
    """Exact attention of the dequantised E4M3 inputs, in float64.

    q8 [B, Hq, Nq, D], k8 and v8 [B, Hkv, Nkv, D] are uint8 code arrays.
    Returns (o, lse) of ``attention_fp64`` on (decode(q8) * descale_q, ...).
    """
    q = dequantize_e4m3(q8, descale_q)
    k = dequantize_e4m3(k8, descale_k)
    v = dequantize_e4m3(v8, descale_v)
    return attention_fp64(q, k, v, scale, causal, rows=rows)


# Rounding of a probability p >= 0 to E4M3 (round to nearest):
#   normal range (p >= 2^-6): relative error at most half a unit in the last
#   place, 2^-4;
#   subnormal range (spacing 2^-9): absolute error at most 2^-10, and a value
#   below 2^-10 that becomes 0 loses at most itself.
REL_E4M3 = 2.0 ** -4
ABS_E4M3 = 2.0 ** -10


def fp8_p_rounding_bound(q, k, v, scale: float, causal: bool = False, rows=None,
                         row_chunk: int = 256) -> np.ndarray:
    """Per-element bound on |O_gpu - O| caused by rounding P to E4M3.

    The GPU forms p_j = 2^(s_j - r) against an exponent reference r that is
    never above the row maximum of the scores (it moves to a running maximum),
    rounds every p_j to E4M3 for the P*V product and divides by the fp32 sum
    of the unrounded p_j.  With weights w_j = p_j / sum p (the exact softmax
    row) and w_max their maximum, p_j = c * w_j / w_max for some c >= 1, so
    the rounding error of key j, divided by the sum, is at most

        max(2^-4 * w_j, min(w_j, 2^-10 * w_max))

    for every admissible c.  Summed against |V| this bounds the error of each
    output element (to first order; the fp32 arithmetic around it is far
    below).  q, k, v are the dequantised float64 inputs.  Returns an array
    shaped like the output ([B, Hq, R, D], R = Nq or len(rows)).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v)
    sigma = _sigma(scale)
    idx_all = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    R = idx_all.size
    out = np.empty((B, Hq, R, D), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            av = np.abs(v[b, g])
            for r0 in range(0, R, row_chunk):
                idx = idx_all[r0:r0 + row_chunk]
                s = sigma * (q[b, h, idx] @ k[b, g].T)
                if causal:
                    s = np.where(np.arange(Nkv)[None, :] <= idx[:, None], s, -np.inf)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                w = e / e.sum(axis=1, keepdims=True)
                wmax = w.max(axis=1, keepdims=True)
                per_key = np.maximum(REL_E4M3 * w, np.minimum(w, ABS_E4M3 * wmax))
                out[b, h, r0:r0 + idx.size] = per_key @ av
    return out
