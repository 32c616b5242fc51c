"""GPU parity of the FP8 (E4M3) forward (fa_fwd_fp8) against the fp64 oracle.

Inputs are E4M3 codes with per-tensor factors (workloads.make_inputs_fp8); the
oracle is exact attention of the dequantised values (attention_fp8_fp64).

Bar, per output element: the oracle's fp8_tolerances, derived from the
arithmetic of the path.  Its two sources of error:
  * the E4M3 rounding of every probability before P*V (relative 2^-4, or
    2^-10 absolute in the subnormal range), with the normaliser summing the
    rounded values (fp8_p_rounding_bound);
  * the 8-bit matrix instruction forms its 64 products exactly but adds them
    with less than fp32 precision.  The model allows 2^-10 of the sum of
    |products| for every such sum (scores, P*V, row sums);
    test_score_accumulation_model checks it on single-key rows, where lse is
    the score itself.
plus the final bf16 rounding of O (2^-8 relative) and the fp32 arithmetic.
Beside that model every case also meets two fixed bars, |dO| <= 2^-3 max|V|
and |dlse| <= 2^-3 (oracle.fp8_ref.FIXED_BAR_O_REL / FIXED_BAR_LSE), which a
path that loses a sizeable part of a row's mass fails whatever the model
admits.  Outputs are poisoned with NaN first, so an unwritten element fails.
"""

import numpy as np
import pytest
import torch

import exact_io_aware_37_amd as fa
import workloads
from oracle import attention_fp8_fp64, dequantize_e4m3, fp8_tolerances
from oracle.fp8_ref import FIXED_BAR_LSE, FIXED_BAR_O_REL, MFMA8_SUM_REL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def run_gpu(codes, ds, causal, scale):
    q8, k8, v8 = (x.to(DEV) for x in codes)
    B, Hq, Nq, d = q8.shape
    o = torch.full((B, Hq, Nq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=DEV)
    fa.attention_fp8(q8, k8, v8, *ds, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def compare(name, o_gpu, l_gpu, codes, ds, causal, scale, rows=None):
    c = [workloads.codes_of(x) for x in codes]
    ref_o, ref_l = attention_fp8_fp64(*c, *ds, scale, causal, rows=rows)
    deq = [dequantize_e4m3(x, s) for x, s in zip(c, ds)]
    tol_o, tol_l = fp8_tolerances(*deq, scale, causal, rows=rows)
    og = workloads.to_f64(o_gpu)
    lg = l_gpu.double().numpy()
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), "unwritten or non-finite output"
    err_o = np.abs(og - ref_o)
    err_l = np.abs(lg - ref_l)
    say(f"    {name}: max|dO|={err_o.max():.3e} (worst err/tol {np.max(err_o / tol_o):.3f}) "
        f"max|dlse|={err_l.max():.3e} (worst err/tol {np.max(err_l / tol_l):.3f})")
    bar_o = FIXED_BAR_O_REL * float(np.max(np.abs(deq[2])))
    say(f"    {name}: fixed bars: max|dO| / (2^-3 max|V|) = {err_o.max() / bar_o:.3f}, "
        f"max|dlse| / 2^-3 = {err_l.max() / FIXED_BAR_LSE:.3f}")
    assert np.all(err_o <= tol_o), float(np.max(err_o / tol_o))
    assert np.all(err_l <= tol_l), float(np.max(err_l / tol_l))
    assert err_o.max() <= bar_o and err_l.max() <= FIXED_BAR_LSE


def run_case(name, B, Hq, Hkv, Nq, Nkv, D, causal, seed=0, sigma=1.0, scale=None,
             outlier_frac=0.0):
    if scale is None:
        scale = workloads.default_scale(D)
    say(f"[case] {name}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} d={D} causal={causal} "
        f"scale={scale} sigma={sigma}")
    codes, ds = workloads.make_inputs_fp8(B, Hq, Hkv, Nq, Nkv, D, seed, sigma, outlier_frac)
    o, l = run_gpu(codes, ds, causal, scale)
    compare(name, o, l, codes, ds, causal, scale)
    return codes, ds, o, l


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_mha_multi_tile_ragged(D, causal):
    run_case("mha", 1, 4, 4, 300, 300, D, causal, seed=D + causal)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_ragged(causal):
    run_case("gqa", 2, 8, 2, 257, 513, 128, causal, seed=3)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq_nkv", [(1, 333), (100, 257), (257, 100), (40, 40), (256, 64),
                                    (600, 1)])
def test_unequal_lengths(causal, nq_nkv):
    run_case("lengths", 1, 4, 2, nq_nkv[0], nq_nkv[1], 64, causal, seed=11)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_scale_values(scale):
    run_case("scale", 1, 4, 2, 96, 160, 128, False, scale=scale, seed=13)


@pytest.mark.parametrize("causal", [False, True])
def test_sharp_scores_and_outlier_keys(causal):
    """Scores spread over tens of units and 1% keys x8: reference moves, rescales, tiny p."""
    run_case("sharp", 1, 4, 1, 512, 1024, 128, causal, seed=17, sigma=3.0, outlier_frac=0.01)


@pytest.mark.parametrize("family", ["uniform codes", "quantised normals"])
def test_score_accumulation_model(family):
    """One key per row: lse is the score q.k * scale exactly, so its error is the score's.
    Checks |error| <= 2^-10 * |scale| * sum_k |q_k k_k| (+ fp32 rounding of the result)
    over 8 x 4096 rows, and reports how much of the allowance the worst row uses."""
    B, Hq, Nq, D = 1, 8, 4096, 128
    rng = np.random.default_rng(31)
    if family == "uniform codes":
        def draw(shape):
            c = rng.integers(0, 256, size=shape).astype(np.uint8)
            c[(c & 0x7F) == 0x7F] = 0x38
            return torch.from_numpy(c).view(torch.float8_e4m3fn)
        codes, ds, scale = (draw((B, Hq, Nq, D)), draw((B, 1, 1, D)), draw((B, 1, 1, D))), \
            (1.0, 1.0, 1.0), 1e-4
    else:
        codes, ds = workloads.make_inputs_fp8(B, Hq, 1, Nq, 1, D, seed=37)
        scale = workloads.default_scale(D)
    say(f"[case] score accumulation, {family}")
    _, l = run_gpu(codes, ds, False, scale)
    c = [workloads.codes_of(x) for x in codes]
    q, k = dequantize_e4m3(c[0], ds[0]), dequantize_e4m3(c[1], ds[1])
    s = float(np.float32(scale)) * np.einsum("bhnd,bd->bhn", q, k[:, 0, 0])
    sabs = abs(float(np.float32(scale))) * np.einsum("bhnd,bd->bhn", np.abs(q), np.abs(k[:, 0, 0]))
    err = np.abs(l.double().numpy() - s)
    allow = MFMA8_SUM_REL * sabs + 1e-6 * (1 + np.abs(s))
    say(f"    max|dS|={err.max():.3e} worst err/allowance {np.max(err / allow):.3f} "
        f"(log2 of worst err/sum|terms|: {np.log2(np.max(err / np.maximum(sabs, 1e-300))):.2f})")
    assert np.all(err <= allow)


def test_descale_laws_bitwise():
    codes, ds = workloads.make_inputs_fp8(1, 4, 2, 200, 300, 128, seed=19)
    o1, l1 = run_gpu(codes, ds, False, 0.1)
    o2, l2 = run_gpu(codes, (ds[0], ds[1], 2 * ds[2]), False, 0.1)
    assert torch.equal(o2.float(), 2 * o1.float()) and torch.equal(l1, l2)
    o3, l3 = run_gpu(codes, (ds[1], ds[0], ds[2]), False, 0.1)
    assert torch.equal(o3, o1) and torch.equal(l3, l1)


def test_deterministic():
    codes, ds = workloads.make_inputs_fp8(1, 8, 2, 300, 700, 128, seed=23)
    a = run_gpu(codes, ds, True, 0.09)
    b = run_gpu(codes, ds, True, 0.09)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_uint8_codes_accepted():
    codes, ds = workloads.make_inputs_fp8(1, 2, 1, 70, 90, 64, seed=29)
    a = run_gpu(codes, ds, False, 0.125)
    b = run_gpu(tuple(x.view(torch.uint8) for x in codes), ds, False, 0.125)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_full_workload7_sampled_rows():
    """B=2 H=32 N=8192 d=128 (E4M3): every (batch, head), sampled rows including both
    ends and workgroup boundaries, in the launch configuration the benchmark times."""
    w = workloads.WORKLOADS[7]
    say(f"[case] {w.name}")
    codes, ds, scale = workloads.workload_inputs_fp8(w)
    o, l = run_gpu(codes, ds, w.causal, scale)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(3), np.arange(w.Nq - 3, w.Nq), [255, 256, 4095, 4096],
                                     rng.choice(w.Nq, 20, replace=False)]))
    compare(w.name, o, l, codes, ds, w.causal, scale, rows=rows)



def test_longest_key_sequence_the_host_accepts():
    """Maximum size for fa_fwd_fp8: the longest key sequence the host accepts at d = 128,
    N_kv = 2^31 / (2 * 128) - 257 (the limit is shared with the 16-bit path; here K and V
    are 1 GiB of E4M3 codes each), one query head of 300 rows (one full and one ragged
    256-row tile), non-causal.  For each of 3 checked rows one key row is replaced by the
    E4M3 codes of 32 times that row's unit vector, in the last key, at key 2^22 and at the
    start of the ragged last tile: its score (about 30) exceeds the log of the other keys'
    summed weight (about 16.4) by so much that the exact output is that key's V row to ~1e-6,
    and a wrong offset changes it at order one.  (The regime of a dominant key holding only
    part of a long row's mass is test_long_rows_flat_and_dominant_key.)"""
    n_kv = (1 << 31) // (128 * 2) - 257
    codes, ds = workloads.make_inputs_fp8(1, 1, 1, 300, n_kv, 128, seed=4444)
    q8, k8, v8 = codes
    rows = np.array([0, 256, 299])
    hot = [n_kv - 1, 1 << 22, 8388288]
    for j, i in zip(hot, rows):
        x = q8[0, 0, i].to(torch.float64) * ds[0]
        y = (32.0 * x / x.norm() / ds[1]).clamp(-448.0, 448.0)
        k8[0, 0, j] = y.to(torch.float32).to(torch.float8_e4m3fn)
    scale = workloads.default_scale(128)
    say(f"[case] longest accepted N_kv (E4M3): q{tuple(q8.shape)} k{tuple(k8.shape)}")
    o, l = run_gpu((q8, k8, v8), ds, False, scale)
    say(f"    max|O| over the checked rows {float(o[0, 0, rows].float().abs().max()):.3f}")
    compare("longest accepted N_kv (E4M3)", o, l, (q8, k8, v8), ds, False, scale, rows=rows)


def test_long_rows_flat_and_dominant_key():
    """N_kv = 2^20 + 37 keys, d = 128, two query heads on one K/V head, 64 query rows, not
    causal; 8 rows per head go to the oracle.  Head 0 has flat scores (its Q scaled down by
    1/16: every key carries a comparable share of the mass).  In head 1 each checked row has
    one planted key whose score is about 12.5 above the others' typical one (e^-12 < 2^-10):
    against a single exponent reference for the whole row every other probability would round
    to zero, although together they hold most of the row's mass.  Against per-block
    references they keep E4M3's precision; both heads must meet the per-element model and
    the fixed bars."""
    n_kv, nq, d = (1 << 20) + 37, 64, 128
    rows = np.array([0, 5, 17, 31, 32, 50, 62, 63])
    codes, ds = workloads.make_inputs_fp8(1, 2, 1, nq, n_kv, d, seed=4321)
    q8, k8, v8 = codes
    q8[0, 0] = (q8[0, 0].to(torch.float32) / 16.0).to(torch.float8_e4m3fn)
    rng = np.random.default_rng(5)
    planted = rng.choice(n_kv - 1000, rows.size, replace=False)
    scale = workloads.default_scale(d)
    for i, j in zip(rows, planted):
        x = q8[0, 1, i].to(torch.float64) * ds[0]
        y = (12.5 / scale) * x / (x.norm() ** 2) / ds[1]
        k8[0, 0, j] = y.clamp(-448.0, 448.0).to(torch.float32).to(torch.float8_e4m3fn)
    kd = k8[0, 0].to(torch.float64) * ds[1]
    for i, j in zip(rows, planted):
        sc = scale * (kd @ (q8[0, 1, i].to(torch.float64) * ds[0])).numpy()
        w = np.exp(sc - sc.max())
        share = w[j] / w.sum()
        assert sc.argmax() == j and 0.01 < share < 0.5, (i, share)
        assert np.median(w) < 2.0 ** -10                # flushed against a row-wide reference
    say(f"[case] long rows: N_kv={n_kv}")
    o, l = run_gpu((q8, k8, v8), ds, False, scale)
    compare("long rows", o, l, (q8, k8, v8), ds, False, scale, rows=rows)
