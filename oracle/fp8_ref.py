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

``fp8_p_rounding_bound`` and ``fp8_tolerances`` are the tolerance model of
the GPU path, which rounds the probabilities to E4M3 before the P*V product
(the way the FlashAttention-3 line feeds its second product), divides by the
sum of the unrounded probabilities, and forms the scores on a matrix
instruction that does not sum its 64 products in IEEE fp32 (see
``SCORE_SUM_REL``).
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


# The 8-bit matrix instruction (v_mfma_f32_32x32x64_f8f6f4) forms each of
# its 64 products exactly but sums them with less than fp32 precision.
# Measured on MI355X over 2^16 outputs per input family (uniform codes over
# the whole E4M3 range, quantised normals, cancelling pairs, one dominant
# product): |error| <= 2^-12.3 * sum|products| and <= 2^-11.2 * max|product|.
# The tolerance model takes 2^-10 * sum|products| per score, a margin of
# about 4.6x over the worst case seen; the GPU tests check it on single-key
# rows, where lse is the score itself.
SCORE_SUM_REL = 2.0 ** -10


def fp8_tolerances(q, k, v, scale: float, causal: bool = False, rows=None):
    """(tol_o, tol_lse): per-element bounds on |O_gpu - O| and |lse_gpu - lse|.

    q, k, v are the dequantised float64 inputs.  Model:
      * each score is off by at most d_j = 2^-10 * |scale| * sum_k |q_k k_jk|
        (``SCORE_SUM_REL``); D = max of d_j over a row's allowed keys;
      * lse = ln sum exp(s_j) then moves by at most D;
      * the weights move by a factor within e^(+-2D), so O moves by at most
        (e^(2D) - 1) * sum_j w_j |v_j| = (e^(2D) - 1) * W, W being the exact
        attention of |V|, and the E4M3 rounding bound E of those weights grows
        to at most e^(2D) * E;
      * O is rounded to bf16 at the end (relative 2^-8), and the fp32 work
        around it (exp2, sums, the final division) stays below
        1e-4 * max|V| on O and 1e-5 * (1 + |lse|) on lse.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v)
    sigma = abs(_sigma(scale))
    idx_all = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    R = idx_all.size
    dmax = np.zeros((B, Hq, R), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            sabs = sigma * (np.abs(q[b, h, idx_all]) @ np.abs(k[b, g]).T)
            if causal:
                sabs = np.where(np.arange(Nkv)[None, :] <= idx_all[:, None], sabs, 0.0)
            dmax[b, h] = SCORE_SUM_REL * sabs.max(axis=1)
    o, lse = attention_fp64(q, k, v, scale, causal, rows=rows)
    w_abs, _ = attention_fp64(q, k, np.abs(v), scale, causal, rows=rows)
    e = fp8_p_rounding_bound(q, k, v, scale, causal, rows=rows)
    grow = np.exp(2.0 * dmax)[..., None]
    vmax = float(np.max(np.abs(v))) if v.size else 0.0
    tol_o = (grow * e + (grow - 1.0) * w_abs) * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(o) + 1e-4 * vmax
    tol_lse = dmax + 1e-5 * (1.0 + np.abs(lse))
    return tol_o, tol_lse
