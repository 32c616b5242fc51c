"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle.

Each case runs the library's forward for o and lse, draws dO, calls fa_bwd
and compares dQ, dK, dV element by element with ``attention_bwd_fp64`` on the
same inputs.  Outputs are poisoned with NaN first.

Bar: max|error| <= 2e-2 * max(1, max|reference|) per tensor.  The gradients
are sums of products of bf16/f16-rounded P and dS (relative rounding 2^-9
for bf16) with rounded inputs, accumulated in fp32 and rounded once; the
forward's O (rounded) enters through D = rowsum(dO * O).  The resulting
error is a small multiple of 2^-9 of the tensor's magnitude, which the bar
bounds with margin; it is scaled because gradient magnitudes grow with the
sequence length and the spread of the scores.
"""

import numpy as np
import pytest
import torch

import exact_io_aware_37_amd as fa
import workloads
from oracle import attention_bwd_fp64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def run_case(name, B, Hq, Hkv, Nq, Nkv, D, causal, dtype="bf16", scale=None, seed=0,
             sigma=1.0):
    say(f"[case] {name}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} d={D} {dtype} "
        f"causal={causal} scale={scale}")
    q, k, v = workloads.make_inputs(B, Hq, Hkv, Nq, Nkv, D, dtype, seed, sigma)
    do = workloads.make_inputs(B, Hq, Hq, Nq, 1, D, dtype, seed + 1)[0]
    if scale is None:
        scale = workloads.default_scale(D)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    fa.attention_backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, dq=dq, dk=dk,
                          dv=dv)
    torch.cuda.synchronize()
    ref = attention_bwd_fp64(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                             workloads.to_f64(do), scale, causal)
    out = []
    for nm, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        gg = workloads.to_f64(g.cpu())
        assert np.all(np.isfinite(gg)), f"{nm}: unwritten or non-finite"
        err = float(np.max(np.abs(gg - r)))
        mag = float(np.max(np.abs(r)))
        say(f"    {nm}: max|err|={err:.3e} max|ref|={mag:.3e} rel={err / max(mag, 1e-30):.3e}")
        assert err <= 2e-2 * max(1.0, mag), (nm, err, mag)
        out.append(g.cpu())
    return out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_mha_square(D, causal):
    run_case("mha", 1, 4, 4, 128, 128, D, causal, seed=D + causal)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_ragged(dtype, causal):
    run_case("gqa ragged", 1, 8, 2, 300, 300, 128, causal, dtype=dtype, seed=7)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq_nkv", [(100, 257), (257, 100), (1, 333), (40, 40)])
def test_unequal_lengths(causal, nq_nkv):
    run_case("lengths", 2, 4, 2, nq_nkv[0], nq_nkv[1], 64, causal, seed=11)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_scale_values(scale):
    run_case("scale", 1, 4, 2, 96, 160, 128, False, scale=scale, seed=13)


def test_multi_tile_gqa_causal():
    """Several 256-key tiles and 256-row query tiles, 7 query heads per key/value head."""
    run_case("7:1 multi-tile", 1, 14, 2, 700, 700, 128, True, seed=17)


def test_deterministic():
    a = run_case("det", 1, 8, 2, 200, 300, 128, True, seed=19)
    b = run_case("det", 1, 8, 2, 200, 300, 128, True, seed=19)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---- full-size workloads, in the launch configuration bench.py --backward times ----

def full_size(widx):
    w = workloads.WORKLOADS[widx]
    q, k, v, scale = workloads.workload_inputs(w)
    do = workloads.make_inputs(w.B, w.Hq, w.Hq, w.Nq, 1, w.D, w.dtype, w.seed + 100)[0]
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa.attention(qd, kd, vd, causal=w.causal, scale=scale)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    fa.attention_backward(qd, kd, vd, o, lse, dod, causal=w.causal, scale=scale, dq=dq, dk=dk,
                          dv=dv)
    torch.cuda.synchronize()
    return w, (q, k, v, do, scale), (dq.cpu(), dk.cpu(), dv.cpu())


def compare_slice(name, got, ref):
    for nm, g, r in zip(("dq", "dk", "dv"), got, ref):
        gg = workloads.to_f64(g)
        assert np.all(np.isfinite(gg)), f"{nm}: unwritten or non-finite"
        err = float(np.max(np.abs(gg - r)))
        mag = float(np.max(np.abs(r)))
        say(f"    {name} {nm}: max|err|={err:.3e} max|ref|={mag:.3e}")
        assert err <= 2e-2 * max(1.0, mag), (nm, err, mag)


def test_full_workload3_one_head():
    """B=2 H=32 N=8192 d=128: the last (batch, head), every gradient element."""
    say("[case] workload 3 backward, head (1, 31)")
    w, (q, k, v, do, scale), (dq, dk, dv) = full_size(3)
    sl = (slice(1, 2), slice(31, 32))
    ref = attention_bwd_fp64(*(workloads.to_f64(x[sl]) for x in (q, k, v, do)), scale, w.causal)
    compare_slice("w3", (dq[sl], dk[sl], dv[sl]), ref)


def test_full_workload4_one_group():
    """B=1 Hq=28 Hkv=4 N=4096 causal: the last key/value group (7 query heads), every element."""
    say("[case] workload 4 backward, kv group 3")
    w, (q, k, v, do, scale), (dq, dk, dv) = full_size(4)
    hq, hk = slice(21, 28), slice(3, 4)
    ref = attention_bwd_fp64(workloads.to_f64(q[:, hq]), workloads.to_f64(k[:, hk]),
                             workloads.to_f64(v[:, hk]), workloads.to_f64(do[:, hq]), scale,
                             w.causal)
    compare_slice("w4", (dq[:, hq], dk[:, hk], dv[:, hk]), ref)


def test_full_workload5_sampled_rows():
    """B=1 Hq=28 Hkv=4 N=32768 causal, outlier keys: group 0, sampled dQ rows and dK/dV rows
    (first and last 64, both sides of 4096-row boundaries, 128 at random)."""
    from oracle import attention_bwd_fp64_rows
    say("[case] workload 5 backward, kv group 0, sampled rows")
    w, (q, k, v, do, scale), (dq, dk, dv) = full_size(5)
    N = w.Nq
    rng = np.random.default_rng(91)
    picks = [np.arange(64), np.arange(N - 64, N), rng.choice(N, 128, replace=False)]
    for b in range(4096, N, 4096):
        picks.append(np.arange(b - 2, b + 2))
    rows = np.unique(np.concatenate(picks))
    hq, hk = slice(0, 7), slice(0, 1)
    ref = attention_bwd_fp64_rows(workloads.to_f64(q[:, hq]), workloads.to_f64(k[:, hk]),
                                  workloads.to_f64(v[:, hk]), workloads.to_f64(do[:, hq]), scale,
                                  w.causal, rows, rows)
    compare_slice("w5", (dq[:, hq][:, :, rows], dk[:, hk][:, :, rows], dv[:, hk][:, :, rows]), ref)


def test_longest_key_sequence_the_host_accepts():
    """Maximum size for fa_bwd: one key/value head of N_kv = 2^31 / (2 * 128) - 257 keys at
    d = 128 in bf16 (2 GiB of K and of V, the most the 32-bit offsets inside a head allow),
    two query heads of 16 rows each, non-causal.  Like the forward's maximum-size case, one key
    row per query row of head 0 is replaced by 16 times that row's unit vector (≈ 20% of the
    row's softmax mass), at the first and last keys, tile and 256-key boundaries, the middle and
    the ragged last tile, so that the checked gradients are of order one.  Checked: every dQ
    row, and dK/dV at the planted keys plus 16 random keys."""
    from oracle import attention_bwd_fp64_rows

    n_kv = (1 << 31) // (128 * 2) - 257
    rng = np.random.default_rng(4343)
    to_bf16 = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    q = to_bf16(rng.standard_normal((1, 2, 16, 128), dtype=np.float32))
    k = to_bf16(rng.standard_normal((1, 1, n_kv, 128), dtype=np.float32))
    v = to_bf16(rng.standard_normal((1, 1, n_kv, 128), dtype=np.float32))
    do = to_bf16(rng.standard_normal((1, 2, 16, 128), dtype=np.float32))
    hot = [n_kv - 1, 0, n_kv - 64, n_kv - 65, 1 << 22, (1 << 22) - 1, n_kv // 2, 4096,
           n_kv - 200, 8388095, 8388096, 12345, n_kv - 2, 255, 256, 8388288]
    for j, i in zip(hot, range(16)):
        x = q[0, 0, i].double()
        k[0, 0, j] = (16.0 * x / x.norm()).to(torch.bfloat16)
    scale = workloads.default_scale(128)
    say(f"[case] longest accepted N_kv backward: q{tuple(q.shape)} k{tuple(k.shape)}")
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa.attention(qd, kd, vd, causal=False, scale=scale)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    fa.attention_backward(qd, kd, vd, o, lse, dod, causal=False, scale=scale, dq=dq, dk=dk,
                          dv=dv)
    torch.cuda.synchronize()
    keys = np.unique(np.concatenate([np.array(hot), rng.choice(n_kv, 16, replace=False)]))
    rows = np.arange(16)
    dq_g = dq.cpu()
    dk_g = dk[:, :, torch.from_numpy(keys).to(DEV)].cpu()
    dv_g = dv[:, :, torch.from_numpy(keys).to(DEV)].cpu()
    del qd, kd, vd, dod, o, lse, dq, dk, dv
    ref = attention_bwd_fp64_rows(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                  workloads.to_f64(do), scale, False, rows, keys)
    compare_slice("max N_kv", (dq_g, dk_g, dv_g), ref)
