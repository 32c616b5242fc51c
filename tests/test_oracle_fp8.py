"""Pins of the FP8 (E4M3) part of the oracle (oracle/fp8_ref.py), CPU only.

* ``e4m3_decode`` against the closed forms of the OCP E4M3 format and against
  torch's own float8_e4m3fn conversion, code by code.
* ``attention_fp8_fp64`` against ``attention_fp64`` on inputs dequantised by
  torch, and against scaling laws of the dequantisation factors.
* ``fp8_p_rounding_bound`` against a simulation of the GPU's rounding of P
  (torch's float8_e4m3fn conversion, an independent round-to-nearest-even)
  with a power-of-two reference per block of keys, for tiles and half-tiles
  and every admissible reference offset; and shown not to be vacuous: the
  slip of dividing by the unrounded sum breaks it, and so does a single
  reference for a whole long row with one dominant key (the flush to zero
  the per-block references avoid), which also breaks the fixed bars.
* ``fp8_tolerances`` against a simulation of both error sources of the GPU
  path at once (scores moved by the modelled accumulation error, randomly and
  adversarially, then P rounded), and against its own special case without
  score error.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import (attention_fp64, attention_fp8_fp64, dequantize_e4m3, e4m3_decode,
                    fp8_p_rounding_bound, probabilities_fp64)
from oracle.fp8_ref import FIXED_BAR_LSE, FIXED_BAR_O_REL


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = e4m3_decode(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_closed_forms():
    d = lambda c: float(e4m3_decode(np.array([c]))[0])   # noqa: E731
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x30) == 0.5
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0          # largest finite
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9   # subnormals
    assert d(0x08) == 2.0 ** -6                             # smallest normal
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)                         # monotone, no gaps or repeats
    assert np.array_equal(e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8)), -pos)


def test_dequantize_widens_the_float32_descale():
    codes = np.arange(0x7F, dtype=np.uint8)
    got = dequantize_e4m3(codes, 0.1)
    assert np.array_equal(got, e4m3_decode(codes) * float(np.float32(0.1)))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_equals_attention_of_torch_dequantised_inputs(causal):
    (q8, k8, v8), (dq, dk, dv) = workloads.make_inputs_fp8(1, 4, 2, 37, 53, 64, seed=5)
    o, lse = attention_fp8_fp64(workloads.codes_of(q8), workloads.codes_of(k8),
                                workloads.codes_of(v8), dq, dk, dv, 0.125, causal)
    deq = [x.to(torch.float64).numpy() * float(np.float32(s)) for x, s in ((q8, dq), (k8, dk), (v8, dv))]
    ro, rl = attention_fp64(*deq, 0.125, causal)
    assert np.array_equal(o, ro) and np.array_equal(lse, rl)


def _codes(seed, shape):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38          # no NaN codes
    return c


def test_descale_laws():
    q8, k8, v8 = _codes(1, (1, 2, 9, 16)), _codes(2, (1, 1, 11, 16)), _codes(3, (1, 1, 11, 16))
    o, lse = attention_fp8_fp64(q8, k8, v8, 0.01, 0.02, 0.03, 0.25)
    # V's factor scales O only (a power of two: exactly)
    o2, lse2 = attention_fp8_fp64(q8, k8, v8, 0.01, 0.02, 0.06, 0.25)
    assert np.array_equal(o2, 2 * o) and np.array_equal(lse2, lse)
    # Q's and K's factors enter through their product with scale
    o3, lse3 = attention_fp8_fp64(q8, k8, v8, 0.02, 0.01, 0.03, 0.25)
    assert np.allclose(o3, o, rtol=0, atol=1e-13) and np.allclose(lse3, lse, rtol=0, atol=1e-13)
    o4, lse4 = attention_fp8_fp64(q8, k8, v8, 0.02, 0.02, 0.03, 0.125)
    assert np.allclose(o4, o, rtol=0, atol=1e-13) and np.allclose(lse4, lse, rtol=0, atol=1e-13)


def test_all_one_value_codes_give_descale():
    q8, k8 = _codes(4, (2, 2, 7, 64)), _codes(5, (2, 1, 13, 64))
    v8 = np.full((2, 1, 13, 64), 0x38, dtype=np.uint8)
    o, _ = attention_fp8_fp64(q8, k8, v8, 0.05, 0.05, 0.75, 0.125, True)
    assert np.allclose(o, 0.75, rtol=0, atol=1e-15)


def test_quantisation_recipe():
    (q8, k8, v8), ds = workloads.make_inputs_fp8(2, 3, 1, 40, 50, 64, seed=9, sigma=0.5)
    xs = workloads.make_inputs(2, 3, 1, 40, 50, 64, "f32", 9, 0.5)
    for c, s, x in zip((q8, k8, v8), ds, xs):
        assert c.dtype == torch.float8_e4m3fn
        assert s == float(np.float32(s)) and s > 0
        val = e4m3_decode(workloads.codes_of(c))
        assert np.max(np.abs(val)) == 448.0               # the largest |x| maps to the top code
        xd = x.double().numpy() / s
        normal = np.abs(xd) >= 2.0 ** -6
        rel = np.abs(val[normal] - xd[normal]) / np.abs(xd[normal])
        assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)        # round to nearest, 3 mantissa bits
        assert np.max(np.abs(val[~normal] - xd[~normal]), initial=0.0) <= 2.0 ** -10 * (1 + 1e-6)


# ---- the tolerance model of the GPU path ----

def _round_blocks(w, rng=None, split=False, offsets=None, fmt=torch.float8_e4m3fn):
    """Rounded weights of the GPU path: each block of keys (a tile of P_TILE keys, or with
    ``split`` its two halves of keys j with (j // 4) % 2 = 0 / 1) is taken against a
    power-of-two reference T in [m, 2m), m its largest weight, rounded to ``fmt`` (torch's
    round-to-nearest-even) and scaled back by T exactly.  The reference offset log2(T/m) is
    drawn from ``rng`` per block, or taken from ``offsets``."""
    from oracle.fp8_ref import P_TILE
    n = w.shape[-1]
    out = np.zeros_like(w)
    key = np.arange(n)
    groups = []
    for t0 in range(0, n, P_TILE):
        tile = key[t0:t0 + P_TILE]
        if split:
            groups += [tile[(tile // 4) % 2 == 0], tile[(tile // 4) % 2 == 1]]
        else:
            groups.append(tile)
    for gi, g in enumerate(groups):
        if g.size == 0:
            continue
        m = w[..., g].max(axis=-1, keepdims=True)
        if offsets is not None:
            f = offsets[gi % len(offsets)]
        else:
            f = rng.uniform(0.0, 1.0, size=m.shape)
        T = np.where(m > 0, m * 2.0 ** f, 1.0)
        p = w[..., g] / T
        pr = torch.from_numpy(np.ascontiguousarray(p)).to(fmt).to(torch.float64).numpy()
        out[..., g] = pr * T
    return out


def _round_rowwide(w, log2_c, fmt=torch.float8_e4m3fn):
    """Rounded weights with one reference for the whole row, log2_c above its largest weight:
    the scheme the per-block references replace."""
    wmax = w.max(axis=-1, keepdims=True)
    p = (2.0 ** log2_c) * w / wmax
    return torch.from_numpy(p).to(fmt).to(torch.float64).numpy() * wmax / 2.0 ** log2_c


def _output(wr, v, Hkv):
    B, Hq = wr.shape[:2]
    o = np.empty(wr.shape[:3] + (v.shape[-1],))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            o[b, h] = (wr[b, h] @ v[b, g]) / wr[b, h].sum(axis=-1, keepdims=True)
    return o


def _simulate(q, k, v, scale, causal, rng=None, split=False, offsets=None):
    """O of the GPU path's rounding of P alone (exact scores, per-block references)."""
    w = probabilities_fp64(q, k, scale, causal)
    return _output(_round_blocks(w, rng, split, offsets), v, k.shape[1])


REGIMES = [("diffuse", 0.05), ("typical", 0.125), ("sharp", 0.6), ("very sharp", 2.5)]


@pytest.mark.parametrize("name,scale", REGIMES)
@pytest.mark.parametrize("causal", [False, True])
def test_bound_holds_for_every_reference_offset(name, scale, causal):
    rng = np.random.default_rng(int(scale * 1000) + causal)
    q = rng.standard_normal((1, 2, 24, 32))
    k = rng.standard_normal((1, 1, 300, 32))
    v = rng.standard_normal((1, 1, 300, 32))
    o_ref, _ = attention_fp64(q, k, v, scale, causal)
    bound = fp8_p_rounding_bound(q, k, v, scale, causal)
    cases = [dict(offsets=[0.0]), dict(offsets=[0.999]), dict(offsets=[0.37, 0.0, 0.9]),
             dict(rng=rng), dict(rng=rng, split=True), dict(offsets=[0.5, 0.01], split=True)]
    for c in cases:
        err = np.abs(_simulate(q, k, v, scale, causal, **c) - o_ref)
        assert np.all(err <= bound * (1 + 1e-9) + 1e-15), (name, c.keys(), float((err - bound).max()))


def test_bound_is_not_vacuous():
    """A plausible slip, dividing by the sum of the unrounded P, breaks the bound (a V with
    equal rows makes the rounded-sum error exactly 0); and on random data the true
    rounding error uses a fair share of the bound."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 64, 32))
    k = rng.standard_normal((1, 1, 64, 32))
    v = np.broadcast_to(rng.standard_normal((1, 1, 1, 32)), (1, 1, 64, 32)).copy()
    o_ref, _ = attention_fp64(q, k, v, 0.6, False)
    bound = fp8_p_rounding_bound(q, k, v, 0.6, False)
    w = probabilities_fp64(q, k, 0.6, False)
    wr = _round_blocks(w, offsets=[0.37])
    o_slip = (wr[0, 0] @ v[0, 0]) / w[0, 0].sum(axis=-1, keepdims=True)
    assert np.any(np.abs(o_slip - o_ref[0, 0]) > bound[0, 0])
    v = rng.standard_normal((1, 1, 64, 32))
    o_ref, _ = attention_fp64(q, k, v, 0.6, False)
    bound = fp8_p_rounding_bound(q, k, v, 0.6, False)
    err = np.abs(_simulate(q, k, v, 0.6, False, offsets=[0.37]) - o_ref)
    assert err.max() > 0.05 * bound.max()


def test_one_reference_per_row_breaks_the_bound_and_the_fixed_bar():
    """One key far above a long row of keys: with one reference for the whole row every other
    probability falls below E4M3's subnormal range and is flushed, losing most of the mass;
    the model (per-block references) and the fixed bar both reject that, and accept the
    per-block rounding of the same row."""
    rng = np.random.default_rng(11)
    n = 1 << 18
    q = np.zeros((1, 1, 1, 16))
    q[0, 0, 0, 0] = 1.0
    k = 0.05 * rng.standard_normal((1, 1, n, 16))
    k[0, 0, 4321, 0] = 8.0                # e^-8 < 2^-10: the rest flush against its reference
    v = rng.standard_normal((1, 1, n, 16))
    o_ref, lse_ref = attention_fp64(q, k, v, 1.0)
    w = probabilities_fp64(q, k, 1.0)
    assert w[0, 0, 0, 4321] < 0.02 and w[0, 0, 0, 4321] > 1e-4   # the planted key holds little mass
    bound = fp8_p_rounding_bound(q, k, v, 1.0)
    bar_o = FIXED_BAR_O_REL * np.abs(v).max()
    wr = _round_rowwide(w, 0.0)
    o_row = _output(wr, v, 1)
    assert np.any(np.abs(o_row - o_ref) > bound) and np.max(np.abs(o_row - o_ref)) > bar_o
    lse_row = np.log(wr.sum(axis=-1)) + lse_ref
    assert np.max(np.abs(lse_row - lse_ref)) > FIXED_BAR_LSE
    for split in (False, True):
        wb = _round_blocks(w, rng, split)
        err = np.abs(_output(wb, v, 1) - o_ref)
        assert np.all(err <= bound * (1 + 1e-9)) and err.max() <= bar_o
        assert np.max(np.abs(np.log(wb.sum(axis=-1)))) <= FIXED_BAR_LSE


@pytest.mark.parametrize("name,scale", [("diffuse", 0.05), ("typical", 0.125), ("sharp", 0.6)])
def test_fixed_bar_holds_for_per_block_rounding(name, scale):
    """The fixed bars (|dO| <= 2^-3 max|V|, |dlse| <= 2^-3) hold for the per-block rounding on
    random rows, reference offsets drawn at random."""
    rng = np.random.default_rng(21 + int(100 * scale))
    q = rng.standard_normal((1, 2, 16, 64))
    k = rng.standard_normal((1, 1, 2000, 64))
    v = rng.standard_normal((1, 1, 2000, 64))
    o_ref, lse_ref = attention_fp64(q, k, v, scale)
    w = probabilities_fp64(q, k, scale)
    for split in (False, True):
        wb = _round_blocks(w, rng, split)
        err = np.abs(_output(wb, v, 1) - o_ref)
        assert err.max() <= FIXED_BAR_O_REL * np.abs(v).max()
        assert np.max(np.abs(np.log(wb.sum(axis=-1)))) <= FIXED_BAR_LSE


def test_bound_special_cases():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 8, 16))
    k = rng.standard_normal((1, 1, 20, 16))
    v = rng.standard_normal((1, 1, 20, 16))
    assert np.all(fp8_p_rounding_bound(q, k, np.zeros_like(v), 0.3) == 0)
    # the rounded weights still sum to 1: a V whose rows are all equal comes back exactly
    vc = np.broadcast_to(v[:, :, :1], v.shape).copy()
    assert np.all(fp8_p_rounding_bound(q, k, vc, 0.3) <= 1e-15)   # |v_j - O| is fp64 rounding only
    # one key: weight 1, output = that value row, nothing to round away
    assert np.all(fp8_p_rounding_bound(q, k[:, :, :1], v[:, :, :1], 0.3) == 0)
    b = fp8_p_rounding_bound(q, k, v, 0.3)
    w = probabilities_fp64(q, k, 0.3)
    o = w[0, 0] @ v[0, 0]
    dev = np.abs(v[0, 0][None] - o[:, None])
    assert np.all(b[0, 0] >= 2.0 ** -4 * np.einsum("rj,rjd->rd", w[0, 0], dev) - 1e-15)
    # rows restricted
    br = fp8_p_rounding_bound(q, k, v, 0.3, rows=[5, 2])
    assert np.array_equal(br[:, :, 0], b[:, :, 5]) and np.array_equal(br[:, :, 1], b[:, :, 2])


@pytest.mark.parametrize("name,scale", REGIMES)
@pytest.mark.parametrize("causal", [False, True])
def test_tolerances_cover_perturbed_scores_and_rounded_p(name, scale, causal):
    """Simulate the GPU path's two error sources together: every score moved by up to the
    modelled accumulation error (random, and adversarially signed against V), P formed
    against per-block references, rounded to E4M3, divided by the rounded sum."""
    from oracle import fp8_tolerances
    from oracle.fp8_ref import MFMA8_SUM_REL
    rng = np.random.default_rng(int(scale * 100) + 7 * causal)
    q = rng.standard_normal((1, 1, 20, 32)) * 2
    k = rng.standard_normal((1, 1, 200, 32)) * 2
    v = rng.standard_normal((1, 1, 200, 32))
    o_ref, l_ref = attention_fp64(q, k, v, scale, causal)
    tol_o, tol_l = fp8_tolerances(q, k, v, scale, causal)
    s = scale * (q[0, 0] @ k[0, 0].T)
    d = MFMA8_SUM_REL * abs(scale) * (np.abs(q[0, 0]) @ np.abs(k[0, 0]).T)
    mask = np.arange(200)[None, :] <= np.arange(20)[:, None] if causal else np.ones((20, 200), bool)
    for trial in range(4):
        if trial < 2:
            eps = d * rng.uniform(-1, 1, size=d.shape)
        else:                                   # push weight towards large (or small) v[:, 0]
            sign = np.sign(v[0, 0, :, 0])[None, :] * (1 if trial == 2 else -1)
            eps = d * sign
        st = np.where(mask, s + eps, -np.inf)
        mx = st.max(axis=1, keepdims=True)
        p = np.exp(st - mx)                       # unnormalised, largest 1
        pr = _round_blocks(p, rng, split=trial % 2 == 1)
        o = (pr @ v[0, 0]) / pr.sum(axis=1, keepdims=True)
        lse = mx[:, 0] + np.log(pr.sum(axis=1))
        assert np.all(np.abs(o - o_ref[0, 0]) <= tol_o[0, 0]), (name, trial)
        assert np.all(np.abs(lse - l_ref[0, 0]) <= tol_l[0, 0]), (name, trial)


def test_tolerances_reduce_to_the_rounding_bound_without_score_error():
    from oracle import fp8_tolerances
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 2, 9, 16))
    k = rng.standard_normal((1, 1, 30, 16))
    v = rng.standard_normal((1, 1, 30, 16))
    t0, l0 = fp8_tolerances(q, k, v, 0.0)            # scale 0: no score error at all
    o, lse = attention_fp64(q, k, v, 0.0)
    w_abs, _ = attention_fp64(q, k, np.abs(v), 0.0)
    e = fp8_p_rounding_bound(q, k, v, 0.0)
    rho = 2.0 ** -4                                    # uniform weights, all in the normal range
    pv = 2.0 ** -10 * w_abs * (1 + 2.0 ** -4) / (1 - rho)
    assert np.allclose(t0, (e + pv) * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(o) + 1e-4 * np.abs(v).max(),
                       rtol=1e-14, atol=0)
    assert np.allclose(l0, -np.log1p(-rho) + 2.0 ** -10 + 1e-5 * (1 + np.abs(lse)), rtol=1e-14, atol=0)
