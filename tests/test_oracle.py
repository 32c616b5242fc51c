"""Pins for the fp64 oracle, independent of the oracle's own code paths.

Each test checks the oracle against something fixed outside it: the values
the course page "FlashAttention: IO-aware attention kernel" prints for its
worked example (section 4), closed forms, the induction invariant of the
"online softmax" section of the kyonqi FlashAttention walkthrough,
probability-row normalisation, a pure-Python compensated brute force and
torch's float64 CPU scaled_dot_product_attention.  A dropped term, a wrong
sign, a wrong index or a transposed operand in the oracle fails at least one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

from oracle import (attention_bruteforce, attention_bwd_fp64, attention_bwd_fp64_rows,
                    attention_fp64,
                    attention_fp64_key_range, attention_fp64_keys, attention_online_blocked,
                    probabilities_fp64, kv_head_of)
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _worked():
    with open(GOLDEN) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[None, None, None, :]
    K = np.array(g["K"], dtype=np.float64)[None, None]
    V = np.array(g["V"], dtype=np.float64)[None, None]
    return g, q, K, V


def _rand(B, Hq, Hkv, Nq, Nkv, D, seed, scale_q=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, D)) * scale_q
    k = rng.standard_normal((B, Hkv, Nkv, D))
    v = rng.standard_normal((B, Hkv, Nkv, D))
    return q, k, v


def _scores(q, k, sigma, causal):
    """Independent score tensor [B,Hq,Nq,Nkv] via einsum over repeated K heads."""
    Hq, Hkv = q.shape[1], k.shape[1]
    kr = np.repeat(k, Hq // Hkv, axis=1)
    s = sigma * np.einsum("bhid,bhjd->bhij", q, kr)
    if causal:
        Nq, Nkv = q.shape[2], k.shape[2]
        s = np.where(np.arange(Nkv)[None, :] <= np.arange(Nq)[:, None], s, -np.inf)
    return s


# ---- T1: the page's worked example -----------------------------------------

def test_worked_example_printed_output():
    g, q, K, V = _worked()
    printed = np.array(g["printed_output_6dp"])
    for fn in (attention_fp64, attention_bruteforce):
        o, _ = fn(q, K, V, g["scale"])
        assert np.max(np.abs(o[0, 0, 0] - printed)) <= 5e-7 + 1e-12
    for block in range(1, 7):
        o_b, _ = attention_online_blocked(q, K, V, g["scale"], block=block)
        assert np.max(np.abs(o_b[0, 0, 0] - printed)) <= 5e-7 + 1e-12


def test_worked_example_online_matches_full_to_machine_precision():
    g, q, K, V = _worked()
    o_full, l_full = attention_fp64(q, K, V, g["scale"])
    for block in range(1, 7):
        o_b, l_b = attention_online_blocked(q, K, V, g["scale"], block=block)
        # The page prints 1.11e-16 for its block size; allow a few ulps.
        assert np.max(np.abs(o_b - o_full)) <= 4.5e-16
        assert abs(l_b[0, 0, 0] - l_full[0, 0, 0]) <= 4.5e-16


def test_worked_example_lse_and_probabilities_from_hand_scores():
    g, q, K, V = _worked()
    hand = np.array(g["hand_scores"]["values"])
    o, lse = attention_fp64(q, K, V, g["scale"])
    assert abs(lse[0, 0, 0] - logsumexp(hand)) <= 1e-13
    # V's first four rows are the identity, row 5 is all 0.5, row 6 all ones:
    # O_t = p_t + 0.5 p_5 + p_6 with p the softmax of the hand scores.
    p = softmax(hand)
    expect = p[:4] + 0.5 * p[4] + p[5]
    assert np.max(np.abs(o[0, 0, 0] - expect)) <= 1e-15
    P = probabilities_fp64(q, K, g["scale"])
    assert np.max(np.abs(P[0, 0, 0] - p)) <= 1e-15


# ---- T2/T3: block-size independence and the induction invariant ------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 37, 300, 16), (2, 4, 2, 64, 129, 8),
                                   (1, 3, 1, 100, 77, 12)])
def test_blocked_equals_full_for_every_block(causal, shape):
    B, Hq, Hkv, Nq, Nkv, D = shape
    q, k, v = _rand(B, Hq, Hkv, Nq, Nkv, D, seed=11)
    o_f, l_f = attention_fp64(q, k, v, 0.3, causal)
    for block in (1, 2, 3, 5, 7, 64, Nkv):
        o_b, l_b = attention_online_blocked(q, k, v, 0.3, causal, block=block)
        assert np.max(np.abs(o_b - o_f)) <= 1e-14
        assert np.max(np.abs(l_b - l_f)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_running_sum_invariant_after_every_block(causal):
    q, k, v = _rand(1, 2, 1, 40, 90, 8, seed=5, scale_q=3.0)
    sigma = float(np.float32(0.4))
    s = _scores(q, k, sigma, causal)
    checked = []

    def on_step(b, h, j1, m, l):
        seen = s[b, h, :, :j1]
        m_ref = seen.max(axis=1)
        fin = np.isfinite(m_ref)
        assert np.array_equal(np.isfinite(m), fin)
        assert np.allclose(m[fin], m_ref[fin], rtol=1e-14, atol=1e-14)
        l_ref = np.where(fin[:, None], np.exp(seen - np.where(fin, m_ref, 0)[:, None]),
                         0).sum(axis=1)
        assert np.max(np.abs(l - l_ref) / np.maximum(l_ref, 1)) <= 1e-14
        checked.append(j1)

    attention_online_blocked(q, k, v, 0.4, causal, block=7, on_step=on_step)
    assert len(checked) == 2 * math.ceil(90 / 7)


# ---- T4/T5: normalisation, V = ones, V = identity --------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one_via_lse(causal):
    q, k, v = _rand(2, 4, 2, 50, 70, 16, seed=3, scale_q=2.0)
    _, lse = attention_fp64(q, k, v, 0.25, causal)
    s = _scores(q, k, float(np.float32(0.25)), causal)
    P = np.exp(s - lse[..., None])
    assert np.max(np.abs(P.sum(axis=-1) - 1.0)) <= 1e-13
    if causal:
        assert np.all(P[..., np.triu_indices(50, 1, 70)[0], np.triu_indices(50, 1, 70)[1]] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_v_all_ones_gives_all_ones(causal):
    q, k, _ = _rand(1, 3, 3, 33, 45, 8, seed=4, scale_q=4.0)
    v = np.ones_like(k)
    o, _ = attention_fp64(q, k, v, 0.7, causal)
    assert np.max(np.abs(o - 1.0)) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_v_identity_recovers_probabilities(causal):
    D = 24
    q, k, _ = _rand(1, 2, 1, 30, D, D, seed=8, scale_q=2.0)
    v = np.broadcast_to(np.eye(D), (1, 1, D, D)).copy()
    o, lse = attention_fp64(q, k, v, 0.3, causal)
    s = _scores(q, k, float(np.float32(0.3)), causal)
    P = softmax(s, axis=-1)
    assert np.max(np.abs(o - P)) <= 1e-15
    assert np.max(np.abs(lse - logsumexp(s, axis=-1))) <= 1e-13


# ---- T6: pure-Python brute force on tiny inputs ----------------------------

@pytest.mark.parametrize("shape,causal", [
    ((1, 1, 1, 6, 6, 4), False), ((2, 2, 2, 9, 13, 5), False),
    ((1, 7, 1, 11, 11, 3), True), ((1, 4, 2, 16, 5, 6), True),
    ((2, 2, 1, 5, 16, 7), True), ((1, 1, 1, 1, 1, 1), False)])
def test_matches_pure_python_bruteforce(shape, causal):
    B, Hq, Hkv, Nq, Nkv, D = shape
    q, k, v = _rand(B, Hq, Hkv, Nq, Nkv, D, seed=sum(shape), scale_q=1.5)
    o_r, l_r = attention_bruteforce(q, k, v, 0.45, causal)
    o, l = attention_fp64(q, k, v, 0.45, causal, row_chunk=4)
    assert np.max(np.abs(o - o_r)) <= 1e-14
    assert np.max(np.abs(l - l_r)) <= 1e-14


# ---- T7: closed forms ------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_means_of_allowed_values(causal):
    _, k, v = _rand(1, 2, 2, 1, 40, 8, seed=9)
    q = np.zeros((1, 2, 40, 8))
    o, lse = attention_fp64(q, k, v, 0.35, causal)
    for i in range(40):
        n = i + 1 if causal else 40
        assert np.allclose(o[:, :, i], v[:, :, :n].mean(axis=2), rtol=0, atol=1e-14)
        assert np.allclose(lse[:, :, i], math.log(n), rtol=0, atol=1e-14)


def test_single_key_returns_its_value_and_score():
    q, k, v = _rand(2, 3, 1, 17, 1, 8, seed=10)
    o, lse = attention_fp64(q, k, v, 0.5, False)
    assert np.max(np.abs(o - v[:, [0, 0, 0]].repeat(17, axis=2))) <= 1e-15
    s00 = 0.5 * np.einsum("bhid,bd->bhi", q, k[:, 0, 0])
    assert np.max(np.abs(lse - s00)) <= 1e-14


def test_causal_first_row_is_first_value():
    q, k, v = _rand(1, 4, 2, 20, 20, 8, seed=12, scale_q=5.0)
    o, lse = attention_fp64(q, k, v, 0.5, True)
    for h in range(4):
        g = kv_head_of(h, 4, 2)
        assert np.array_equal(o[0, h, 0], v[0, g, 0])


def test_dominant_key_without_overflow():
    """Scores of +/-1e4 would overflow exp without the max subtraction."""
    D = 8
    k = np.zeros((1, 1, 5, D))
    k[0, 0, :, 0] = [-1.0, 0.5, 1.0, 0.25, -0.5]
    q = np.zeros((1, 1, 3, D))
    q[0, 0, :, 0] = [2e4, -2e4, 1e4]
    v = np.arange(5 * D, dtype=np.float64).reshape(1, 1, 5, D)
    o, lse = attention_fp64(q, k, v, 1.0, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.array_equal(o[0, 0, 0], v[0, 0, 2])      # q*k largest at key 2
    assert np.array_equal(o[0, 0, 1], v[0, 0, 0])      # sign flips -> key 0
    assert lse[0, 0, 0] == pytest.approx(2e4, abs=1e-9)
    assert lse[0, 0, 1] == pytest.approx(2e4, abs=1e-9)


# ---- T8: structural identities ---------------------------------------------

def test_causal_row_equals_noncausal_prefix():
    q, k, v = _rand(1, 2, 2, 30, 30, 8, seed=13)
    o_c, l_c = attention_fp64(q, k, v, 0.3, True)
    for i in (0, 1, 7, 29):
        o_p, l_p = attention_fp64(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.3)
        assert np.max(np.abs(o_c[:, :, i] - o_p[:, :, 0])) <= 1e-15
        assert np.max(np.abs(l_c[:, :, i] - l_p[:, :, 0])) <= 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha_with_repeated_kv(causal):
    q, k, v = _rand(2, 7, 1, 21, 25, 8, seed=14)
    o_g, l_g = attention_fp64(q, k, v, 0.3, causal)
    o_m, l_m = attention_fp64(q, np.repeat(k, 7, axis=1), np.repeat(v, 7, axis=1), 0.3, causal)
    assert np.array_equal(o_g, o_m) and np.array_equal(l_g, l_m)
    q, k, v = _rand(1, 6, 3, 9, 12, 4, seed=15)
    o_g, _ = attention_fp64(q, k, v, 0.3, causal)
    # head h reads kv head h // 2: heads (0,1)->0, (2,3)->1, (4,5)->2
    o_m, _ = attention_fp64(q, k[:, [0, 0, 1, 1, 2, 2]], v[:, [0, 0, 1, 1, 2, 2]], 0.3, causal)
    assert np.array_equal(o_g, o_m)


def test_key_permutation_invariance_noncausal():
    q, k, v = _rand(1, 2, 2, 15, 40, 8, seed=16)
    perm = np.random.default_rng(0).permutation(40)
    o1, l1 = attention_fp64(q, k, v, 0.3)
    o2, l2 = attention_fp64(q, k[:, :, perm], v[:, :, perm], 0.3)
    assert np.max(np.abs(o1 - o2)) <= 1e-14 and np.max(np.abs(l1 - l2)) <= 1e-14


# ---- T9: library routine ---------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    q, k, v = _rand(2, 4, 4, 70, 70, 16, seed=17, scale_q=2.0)
    o, _ = attention_fp64(q, k, v, 0.25, causal, row_chunk=32)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=0.25)
    assert np.max(np.abs(o - ref.numpy())) <= 1e-12


def test_threaded_equals_serial():
    q, k, v = _rand(2, 3, 1, 300, 260, 16, seed=18)
    a = attention_fp64(q, k, v, 0.3, True, row_chunk=64, threads=1)
    b = attention_fp64(q, k, v, 0.3, True, row_chunk=64, threads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---- input generators ------------------------------------------------------

def test_generator_is_deterministic_and_outliers_exact():
    a = workloads.make_inputs(1, 2, 2, 40, 300, 8, "bf16", seed=3, sigma=0.5,
                              outlier_frac=0.01, outlier_mult=8.0)
    b = workloads.make_inputs(1, 2, 2, 40, 300, 8, "bf16", seed=3, sigma=0.5,
                              outlier_frac=0.01, outlier_mult=8.0)
    for x, y in zip(a, b):
        assert torch.equal(x, y) and x.dtype == torch.bfloat16 and x.is_contiguous()
    plain = workloads.make_inputs(1, 2, 2, 40, 300, 8, "bf16", seed=3, sigma=0.5)
    assert torch.equal(a[0], plain[0])
    ratio = a[1].double() / plain[1].double()
    scaled = (ratio == 8.0).all(dim=-1)
    same = (ratio == 1.0).all(dim=-1)
    assert torch.all(scaled | same)
    assert scaled.sum(dim=-1).tolist() == [[3, 3]]


def test_named_workloads_match_their_descriptions():
    w = workloads.WORKLOADS
    assert (w[3].B, w[3].Hq, w[3].Nq, w[3].D, w[3].causal) == (2, 32, 8192, 128, False)
    assert w[3].flops() == pytest.approx(2.199023e12, rel=1e-6)
    assert (w[5].Hq, w[5].Hkv, w[5].Nkv, w[5].causal) == (28, 4, 32768, True)
    assert w[1].dtype == "f32" and w[1].scale == np.float32(0.125)


@pytest.mark.parametrize("causal", [False, True])
def test_row_subset_matches_whole(causal):
    q, k, v = _rand(1, 4, 2, 300, 280, 16, seed=19)
    o, l = attention_fp64(q, k, v, 0.3, causal)
    rows = np.array([299, 0, 5, 137, 256, 255, 1])
    o_r, l_r = attention_fp64(q, k, v, 0.3, causal, rows=rows, row_chunk=3)
    assert np.array_equal(o_r, o[:, :, rows]) or np.max(np.abs(o_r - o[:, :, rows])) <= 1e-15
    assert np.max(np.abs(l_r - l[:, :, rows])) <= 1e-15


# ---- key-range partials (the chunk results of the split-KV form) ----------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [(0, 100), (0, 1, 100), (0, 37, 64, 65, 100), (0, 50, 50, 100)])
def test_key_range_chunks_merge_to_full(causal, cuts):
    """Chunk results over a partition of the keys, merged by the [P2] §二.3 rule
    (new max, every part rescaled to it, sums added), give the full result."""
    q, k, v = _rand(2, 6, 2, 40, 100, 16, seed=23)
    full_o, full_l = attention_fp64(q, k, v, 0.4, causal)
    parts = [attention_fp64_key_range(q, k, v, 0.4, causal, a, b)
             for a, b in zip(cuts[:-1], cuts[1:])]
    m = np.max(np.stack([pl for _, pl in parts]), axis=0)
    w = [np.exp(pl - m) for _, pl in parts]            # exp(-inf) = 0 for empty parts
    l_sum = sum(w)
    o = sum(wi[..., None] * po for wi, (po, _) in zip(w, parts)) / l_sum[..., None]
    assert np.max(np.abs(o - full_o)) <= 1e-13
    assert np.max(np.abs(m + np.log(l_sum) - full_l)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 3, 4])
def test_interleaved_tile_chunks_merge_to_full(causal, S):
    """Chunks dealt tile by tile (chunk s: tiles s, s+S, ... of 8 keys) merge to the full result."""
    q, k, v = _rand(1, 4, 2, 30, 75, 8, seed=37)
    full_o, full_l = attention_fp64(q, k, v, 0.6, causal)
    tiles = np.arange(75) // 8
    parts = [attention_fp64_keys(q, k, v, 0.6, causal, np.nonzero(tiles % S == s)[0])
             for s in range(S)]
    m = np.max(np.stack([pl for _, pl in parts]), axis=0)
    w = [np.exp(pl - m) for _, pl in parts]
    l_sum = sum(w)
    o = sum(wi[..., None] * po for wi, (po, _) in zip(w, parts)) / l_sum[..., None]
    assert np.max(np.abs(o - full_o)) <= 1e-13
    assert np.max(np.abs(m + np.log(l_sum) - full_l)) <= 1e-13


def test_key_set_order_and_duplicates_do_not_matter():
    q, k, v = _rand(1, 2, 1, 6, 20, 4, seed=41)
    a = attention_fp64_keys(q, k, v, 0.9, True, [3, 1, 7, 7, 12])
    b = attention_fp64_keys(q, k, v, 0.9, True, [1, 3, 7, 12])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_key_range_whole_range_equals_full():
    q, k, v = _rand(1, 3, 3, 20, 33, 8, seed=29)
    for causal in (False, True):
        o, l = attention_fp64_key_range(q, k, v, 0.7, causal, 0, 33)
        fo, fl = attention_fp64(q, k, v, 0.7, causal)
        assert np.max(np.abs(o - fo)) <= 1e-14 and np.max(np.abs(l - fl)) <= 1e-14


def test_key_range_empty_rows_and_single_key():
    q, k, v = _rand(1, 1, 1, 10, 10, 4, seed=31)
    # causal rows i < 6 have no key in [6, 10): O = 0, lse = -inf
    o, l = attention_fp64_key_range(q, k, v, 1.0, True, 6, 10)
    assert np.all(o[0, 0, :6] == 0) and np.all(np.isneginf(l[0, 0, :6]))
    assert np.all(np.isfinite(l[0, 0, 6:]))
    # one key: O is that value row, lse its score
    o, l = attention_fp64_key_range(q, k, v, 0.5, False, 3, 4)
    assert np.allclose(o[0, 0], np.broadcast_to(v[0, 0, 3], (10, 4)), rtol=0, atol=1e-15)
    assert np.allclose(l[0, 0], 0.5 * q[0, 0] @ k[0, 0, 3], rtol=0, atol=1e-14)


# ---- backward (gradients of L = sum(O * dO)) --------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(causal):
    """Every entry of dQ, dK, dV against a central difference of L = sum(O * dO)."""
    q, k, v = _rand(1, 2, 1, 5, 7, 3, seed=43)
    do = np.random.default_rng(44).standard_normal(q.shape)
    scale = 0.7
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        return float(np.sum(attention_fp64(q_, k_, v_, scale, causal)[0] * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{a + "_": b for a, b in args_p.items()}) -
                        loss(**{a + "_": b for a, b in args_m.items()})) / (2 * h)
        assert np.max(np.abs(num - g)) <= 1e-7 * max(1.0, np.max(np.abs(g))), name


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_float64(causal):
    """dQ, dK, dV against torch's float64 autograd of its own attention routine
    (K/V repeated over the query heads of a group, gradients summed back)."""
    B, Hq, Hkv, N, D = 2, 6, 2, 17, 8
    q, k, v = _rand(B, Hq, Hkv, N, N, D, seed=47)
    do = np.random.default_rng(48).standard_normal(q.shape)
    scale = float(np.float32(0.35))          # the fp32 value both sides use
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, scale, causal)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    g = Hq // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1),
        is_causal=causal, scale=scale)
    o.backward(torch.tensor(do))
    assert np.max(np.abs(tq.grad.numpy() - dq)) <= 1e-12
    assert np.max(np.abs(tk.grad.numpy() - dk)) <= 1e-12
    assert np.max(np.abs(tv.grad.numpy() - dv)) <= 1e-12


def test_backward_closed_forms():
    """One key: O = v0 for every row, so dV0 = sum of dO rows and dQ = dK = 0."""
    q, k, v = _rand(1, 1, 1, 4, 1, 5, seed=53)
    do = np.random.default_rng(54).standard_normal(q.shape)
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, 0.9, False)
    assert np.allclose(dv[0, 0, 0], do[0, 0].sum(axis=0), rtol=0, atol=1e-14)
    assert np.max(np.abs(dq)) <= 1e-15 and np.max(np.abs(dk)) <= 1e-15
    # scale 0: P uniform, dV = (1/N) * column sums of dO for every key, dQ = dK = 0
    q, k, v = _rand(1, 1, 1, 3, 4, 2, seed=55)
    do = np.random.default_rng(56).standard_normal(q.shape)
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, 0.0, False)
    assert np.allclose(dv[0, 0], np.broadcast_to(do[0, 0].sum(axis=0) / 4, (4, 2)), atol=1e-14)
    assert np.max(np.abs(dq)) == 0 and np.max(np.abs(dk)) == 0


@pytest.mark.parametrize("causal", [False, True])
def test_backward_rows_match_whole_backward(causal):
    """Selected gradient rows (lse and O taken from the forward oracle) equal the
    whole-matrix backward, which the tests above pin to central differences."""
    q, k, v = _rand(2, 6, 2, 37, 41, 8, seed=59)
    do = np.random.default_rng(60).standard_normal(q.shape)
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, 0.45, causal)
    qr, kr = np.array([0, 5, 36, 17]), np.array([40, 0, 3, 22])
    rq, rk, rv = attention_bwd_fp64_rows(q, k, v, do, 0.45, causal, qr, kr)
    assert np.max(np.abs(rq - dq[:, :, qr])) <= 1e-12
    assert np.max(np.abs(rk - dk[:, :, kr])) <= 1e-12
    assert np.max(np.abs(rv - dv[:, :, kr])) <= 1e-12
