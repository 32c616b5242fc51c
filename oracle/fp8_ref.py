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
sum of those rounded probabilities (the convention of the 16-bit path, so
that O is a convex combination of V rows), and forms its sums on a matrix
instruction that does not add its 64 products in IEEE fp32 (see
``MFMA8_SUM_REL``).  The probabilities of each block of keys are formed
against a power-of-two reference of that block (at least its largest
probability, less than twice it) and carried to the row's common reference
by an exact power-of-two factor; every block lies inside one tile of
``P_TILE`` consecutive keys (tiles start at key 0).
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
# keys per tile: every block of probabilities that shares one reference lies
# inside one tile
P_TILE = 64

# The 8-bit matrix instruction (v_mfma_f32_32x32x64_f8f6f4) forms each of
# its 64 products exactly but adds them with less than fp32 precision.
# Measured on MI355X over 2^16 outputs per input family (uniform codes over
# the whole E4M3 range, quantised normals, cancelling pairs, one dominant
# product): |error| <= 2^-12.3 * sum|products| and <= 2^-11.2 * max|product|.
# The tolerance model allows 2^-10 * sum|products| for every such sum (a
# margin of about 4.6x over the worst case seen): the scores, the P*V
# products and the row sums; the GPU tests check it on single-key rows,
# where lse is the score itself.
MFMA8_SUM_REL = 2.0 ** -10


# Fixed bars beside the per-element model: |O_gpu - O| <= 2^-3 max|V| and
# |lse_gpu - lse| <= 2^-3 for every row.  Where every rounded probability
# lies in E4M3's normal range relative to its block's reference, each weight
# carries a relative error of at most 2^-4, so the normalised weights of a
# row move by at most a factor (1 +- 2^-4) / (1 -+ 2^-4): O moves by at most
# about 2^-4 max_j |v_j - O| <= 2^-3 max|V|, and the row sum by a factor whose
# logarithm is below 0.065, leaving more than 0.06 of the lse bar for the
# scores' accumulation error (2^-10 |scale| sum|q k|, about 0.007 for the
# unit-variance inputs of the tests) and the subnormal tail.  A path that
# loses a large part of a row's mass (for example by flushing a long row of
# small probabilities to zero against one far larger key) fails them.
FIXED_BAR_O_REL = 2.0 ** -3
FIXED_BAR_LSE = 2.0 ** -3


def _rows(Nq, rows):
    return np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)


def _rounding_terms(q, k, v, scale, causal, rows, row_chunk=None):
    """Per-row softmax terms of the rounding model (exact fp64 weights w_j).

    eta_j = max(2^-4 w_j, min(w_j, 2^-9 t_j)), t_j the largest weight of the
    tile of key j, bounds the E4M3 rounding error of key j divided by the row
    sum, for every block of the tile and every position of the block's
    reference (see ``fp8_p_rounding_bound``).  Returns, per output
    element or row:
      A   = sum_j eta_j |v_j - O|        rho = sum_j eta_j
      Bw  = sum_j w_j |v_j - O|          W   = sum_j w_j |v_j|
      S   = max_j |scale| sum_d |q_d k_jd|   (allowed keys), and O.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nkv, D = _check_shapes(q, k, v)
    sigma = _sigma(scale)
    idx_all = _rows(Nq, rows)
    R = idx_all.size
    if row_chunk is None:   # |v_j - O| is materialised per chunk: keep it near 16 Mi elements
        row_chunk = max(1, min(256, (1 << 24) // max(1, Nkv * D)))
    A = np.empty((B, Hq, R, D))
    Bw = np.empty((B, Hq, R, D))
    W = np.empty((B, Hq, R, D))
    O = np.empty((B, Hq, R, D))
    rho = np.empty((B, Hq, R))
    S = np.empty((B, Hq, R))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            vb, kb = v[b, g], k[b, g]
            for r0 in range(0, R, row_chunk):
                idx = idx_all[r0:r0 + row_chunk]
                sl = slice(r0, r0 + idx.size)
                s = sigma * (q[b, h, idx] @ kb.T)
                sabs = abs(sigma) * (np.abs(q[b, h, idx]) @ np.abs(kb).T)
                if causal:
                    allowed = np.arange(Nkv)[None, :] <= idx[:, None]
                    s = np.where(allowed, s, -np.inf)
                    sabs = np.where(allowed, sabs, 0.0)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                w = e / e.sum(axis=1, keepdims=True)
                eta = np.maximum(REL_E4M3 * w, np.minimum(w, 2.0 * ABS_E4M3 * tile_max(w)))
                o = w @ vb
                dev = np.abs(vb[None, :, :] - o[:, None, :])          # |v_j - O| per row
                A[b, h, sl] = np.einsum("rj,rjd->rd", eta, dev)
                Bw[b, h, sl] = np.einsum("rj,rjd->rd", w, dev)
                W[b, h, sl] = w @ np.abs(vb)
                O[b, h, sl] = o
                rho[b, h, sl] = eta.sum(axis=1)
                S[b, h, sl] = sabs.max(axis=1)
    return A, rho, Bw, W, S, O


def tile_max(w: np.ndarray) -> np.ndarray:
    """Per key, the largest value of its tile of P_TILE keys along the last axis (same shape)."""
    n = w.shape[-1]
    t = -(-n // P_TILE)
    pad = np.zeros(w.shape[:-1] + (t * P_TILE,), dtype=w.dtype)
    pad[..., :n] = w
    m = pad.reshape(w.shape[:-1] + (t, P_TILE)).max(axis=-1)
    return np.repeat(m, P_TILE, axis=-1)[..., :n]


def fp8_p_rounding_bound(q, k, v, scale: float, causal: bool = False, rows=None) -> np.ndarray:
    """Per-element bound on |O_gpu - O| caused by rounding P to E4M3 alone.

    The GPU forms the probabilities of each block of keys (a subset of one
    tile of P_TILE keys) as p_j = 2^(s_j - r_b) against a reference r_b of
    the block whose power of two 2^r_b lies in [m_b, 2 m_b), m_b the block's
    largest 2^(s_j); it rounds every p_j to E4M3 (p~_j), carries the block to
    the row's common reference by an exact power of two, and returns
    sum_j p~_j v_j / sum_j p~_j.  In units of the exact weights w_j (which sum
    to 1), key j is rounded with a relative error of at most 2^-4 in E4M3's
    normal range and an absolute one of at most 2^-10 times the block's
    reference, itself below 2 t_j (t_j the largest weight of the tile), in
    the subnormal range; a value flushed to zero loses at most itself.  So
    the rounding error e_j of key j, divided by the exact sum L, is at most
    eta_j = max(2^-4 w_j, min(w_j, 2^-9 t_j)) for every admissible block and
    reference.  The rounded weights p~_j / sum p~ then differ from w_j by
    at most (eta_j + w_j rho) / (1 - rho), rho = sum eta, and since both sets
    of weights sum to 1,
        |O_gpu - O| <= (sum_j eta_j |v_j - O| + rho sum_j w_j |v_j - O|) / (1 - rho).
    q, k, v are the dequantised float64 inputs.  Returns an array shaped like
    the output ([B, Hq, R, D], R = Nq or len(rows)).
    """
    A, rho, Bw, _, _, _ = _rounding_terms(q, k, v, scale, causal, rows)
    r = rho[..., None]
    return (A + r * Bw) / (1.0 - r)


def fp8_tolerances(q, k, v, scale: float, causal: bool = False, rows=None):
    """(tol_o, tol_lse): per-element bounds on |O_gpu - O| and |lse_gpu - lse|.

    q, k, v are the dequantised float64 inputs.  Model:
      * every score is off by at most 2^-10 |scale| sum_k |q_k k_jk|
        (``MFMA8_SUM_REL``); D = its maximum over the row's allowed keys.  The
        unrounded weights then move by a factor within e^(+-2D): with
        g = e^(2D), the rounding terms of ``fp8_p_rounding_bound`` grow to at
        most g eta_j and g rho, and
          |O_gpu - O| <= (g A + g^2 rho Bw) / (1 - g rho) + (g - 1) Bw
        with A = sum eta_j |v_j - O|, Bw = sum w_j |v_j - O|;
      * the P*V sums add at most 2^-10 g W (1 + 2^-4) / (1 - g rho), W the
        exact attention of |V|;
      * O is rounded to bf16 at the end (relative 2^-8), and the fp32 work
        around it stays below 1e-4 * max|V|;
      * lse = r + ln(sum p~): it moves by at most D from the scores, by
        -ln(1 - g rho) from the rounding of the summed probabilities, by
        2^-10 from the sum's own accumulation, and 1e-5 (1 + |lse|) of fp32.
    """
    A, rho, Bw, W, S, O = _rounding_terms(q, k, v, scale, causal, rows)
    _, lse = attention_fp64(q, k, v, scale, causal, rows=rows)
    dmax = MFMA8_SUM_REL * S
    g = np.exp(2.0 * dmax)
    gr = (g * rho)[..., None]
    gg = g[..., None]
    if np.any(gr >= 1.0):
        raise ValueError("rounding model not applicable (g * rho >= 1)")
    e = (gg * A + gg * gr * Bw) / (1.0 - gr) + (gg - 1.0) * Bw
    e += MFMA8_SUM_REL * gg * W * (1.0 + REL_E4M3) / (1.0 - gr)
    v = np.asarray(v, dtype=np.float64)
    vmax = float(np.max(np.abs(v))) if v.size else 0.0
    tol_o = e * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(O) + 1e-4 * vmax
    tol_lse = dmax - np.log1p(-(g * rho)) + MFMA8_SUM_REL + 1e-5 * (1.0 + np.abs(lse))
    return tol_o, tol_lse
