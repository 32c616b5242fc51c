"""GPU parity of the split-KV (FlashDecoding) entry point against the fp64 oracle.

Same bars as the main path: max-abs error <= 2e-2 on O and lse for bf16/f16.
Outputs and the workspace are poisoned with NaN before every call, so an
element the kernels fail to write fails the comparison.  Besides the merged
result, the chunk results left in the workspace are checked one by one
against the oracle restricted to each chunk's keys.
"""

import numpy as np
import pytest
import torch

import exact_io_aware_37_amd as fa
import workloads
from oracle import attention_fp64, attention_fp64_keys

pytestmark = pytest.mark.gpu

TOL = 2e-2
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def run_split(q, k, v, causal, scale, num_splits=None, stream=None):
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    B, Hq, Nq, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    dt = fa.dtype_code(q.dtype)
    if num_splits is None:
        num_splits = fa.fa_splitkv_default_splits(B, Hq, Hkv, Nq, Nkv, d, dt)
    nbytes = fa.fa_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    if stream is not None:
        stream.wait_stream(torch.cuda.current_stream())   # the fills above come first
    fa.attention_splitkv(qd, kd, vd, causal=causal, scale=scale, num_splits=num_splits,
                         workspace=ws, out=o, lse=lse, stream=stream)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), ws.cpu(), num_splits


def check(name, q, k, v, causal, scale, num_splits=None):
    B, Hq, Nq, d = q.shape
    say(f"[case] {name}: q{tuple(q.shape)} k{tuple(k.shape)} {q.dtype} causal={causal} "
        f"scale={scale} splits={num_splits}")
    o_g, l_g, ws, S = run_split(q, k, v, causal, scale, num_splits)
    ref_o, ref_l = attention_fp64(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                  scale, causal)
    og, lg = workloads.to_f64(o_g), l_g.double().numpy()
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), "unwritten or non-finite output"
    err_o = float(np.max(np.abs(og - ref_o)))
    err_l = float(np.max(np.abs(lg - ref_l)))
    say(f"    splits={S} max|dO|={err_o:.3e} max|dlse|={err_l:.3e}")
    assert err_o <= TOL and err_l <= TOL, (err_o, err_l)
    return o_g, l_g, ws, S


def inputs(B, Hq, Hkv, Nq, Nkv, D, dtype="bf16", seed=0, sigma=1.0):
    q, k, v = workloads.make_inputs(B, Hq, Hkv, Nq, Nkv, D, dtype, seed, sigma)
    return q, k, v, workloads.default_scale(D)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Nkv", [1, 31, 33, 1000, 4097])
def test_decode_gqa(D, Nkv):
    q, k, v, scale = inputs(2, 28, 4, 1, Nkv, D, seed=Nkv + D)
    n_tiles = (Nkv + 31) // 32
    for S in sorted({1, min(3, n_tiles), min(n_tiles, fa.FA_SPLITKV_MAX_SPLITS), None} - {0},
                    key=lambda x: -1 if x is None else x):
        check(f"decode d{D} n{Nkv}", q, k, v, False, scale, S)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 8, 2, 37, 300, 128), (2, 4, 4, 100, 257, 64),
                                   (1, 7, 1, 5, 2000, 128)])
def test_prefill_like(shape, causal, dtype):
    q, k, v, scale = inputs(*shape, dtype=dtype, seed=sum(shape))
    for S in (1, 3, 9):
        check(f"rows {shape}", q, k, v, causal, scale, S)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_scale_values(scale):
    q, k, v, _ = inputs(1, 8, 2, 3, 700, 128, seed=5)
    check("scale", q, k, v, False, scale, 4)


def test_large_scores():
    q, k, v, scale = inputs(1, 8, 1, 2, 3000, 128, seed=6, sigma=4.0)
    v = workloads.make_inputs(1, 8, 1, 2, 3000, 128, "bf16", 7)[2]
    check("large scores", q, k, v, False, scale, 5)


def test_decode_workload_full_tensor():
    w = workloads.WORKLOADS[6]
    q, k, v, scale = workloads.workload_inputs(w)
    check(w.name, q, k, v, w.causal, scale, None)


@pytest.mark.parametrize("causal", [False, True])
def test_chunk_results_in_workspace(causal):
    """Every chunk's (O_s, lse_s) equals the oracle over that chunk's keys alone."""
    q, k, v, scale = inputs(1, 6, 2, 20, 500, 64, seed=11)
    B, Hq, Nq, d = q.shape
    Nkv = k.shape[2]
    S = 5
    _, _, ws, _ = check("chunks", q, k, v, causal, scale, S)
    rows = B * Hq * Nq
    o_s = ws[: S * rows * d].double().numpy().reshape(S, B, Hq, Nq, d)
    l_s = ws[S * rows * d: S * rows * (d + 1)].double().numpy().reshape(S, B, Hq, Nq)
    tile = np.arange(Nkv) // 32
    for s in range(S):
        keys = np.nonzero(tile % S == s)[0]          # chunk s: tiles s, s+S, s+2S, ...
        ref_o, ref_l = attention_fp64_keys(workloads.to_f64(q), workloads.to_f64(k),
                                           workloads.to_f64(v), scale, causal, keys)
        empty = np.isneginf(ref_l)
        assert np.array_equal(np.isneginf(l_s[s]), empty), f"chunk {s}: empty rows differ"
        assert np.all(o_s[s][empty] == 0)
        full = ~empty
        if full.any():
            eo = float(np.max(np.abs(o_s[s][full] - ref_o[full])))
            el = float(np.max(np.abs(l_s[s][full] - ref_l[full])))
            say(f"    chunk {s} ({keys.size} keys) max|dO_s|={eo:.3e} max|dlse_s|={el:.3e} "
                f"empty rows={int(empty.sum())}")
            assert eo <= TOL and el <= TOL


def test_agrees_with_main_path():
    q, k, v, scale = inputs(1, 8, 2, 64, 1500, 128, seed=13)
    o_s, l_s, _, _ = check("vs main", q, k, v, True, scale, 6)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o_m, l_m = fa.attention(qd, kd, vd, causal=True, scale=scale)
    torch.cuda.synchronize()
    d_o = float((o_s.float() - o_m.cpu().float()).abs().max())
    d_l = float((l_s - l_m.cpu()).abs().max())
    say(f"    split vs main: max|dO|={d_o:.3e} max|dlse|={d_l:.3e}")
    assert d_o <= TOL and d_l <= TOL


def test_deterministic_and_workspace_reuse():
    q, k, v, scale = inputs(2, 28, 4, 1, 5000, 128, seed=17)
    a = run_split(q, k, v, False, scale, 16)
    b = run_split(q, k, v, False, scale, 16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # one workspace, a large call then a smaller one: the second result is exact too
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    nbytes = fa.fa_splitkv_workspace_bytes(2, 28, 1, 128, 16)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    fa.attention_splitkv(qd, kd, vd, scale=scale, num_splits=16, workspace=ws)
    q2, k2, v2, _ = inputs(1, 28, 4, 1, 900, 128, seed=19)
    o2, l2 = fa.attention_splitkv(q2.to(DEV), k2.to(DEV), v2.to(DEV), scale=scale, num_splits=7,
                                  workspace=ws)
    torch.cuda.synchronize()
    ro, rl = attention_fp64(workloads.to_f64(q2), workloads.to_f64(k2), workloads.to_f64(v2),
                            scale, False)
    assert float(np.max(np.abs(workloads.to_f64(o2.cpu()) - ro))) <= TOL
    assert float(np.max(np.abs(l2.cpu().double().numpy() - rl))) <= TOL


def test_side_stream():
    q, k, v, scale = inputs(1, 28, 4, 1, 2048, 128, seed=21)
    s = torch.cuda.Stream()
    o, l, _, _ = run_split(q, k, v, False, scale, 8, stream=s)
    ro, rl = attention_fp64(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                            scale, False)
    assert float(np.max(np.abs(workloads.to_f64(o) - ro))) <= TOL


def test_invalid_split_count_raises():
    q, k, v, scale = inputs(1, 4, 4, 1, 100, 64, seed=23)
    with pytest.raises(fa.FAError):
        fa.attention_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), num_splits=5)   # 4 tiles only
