"""The library's launches inside a captured HIP graph (torch.cuda.CUDAGraph).

No entry point allocates device memory, sets memory with a memset or
synchronises, so a caller can capture a call once and replay it.  Each test
captures one call on caller-owned buffers, then three times: writes new
inputs in place with eager torch work, replays, and checks the replay
bitwise against an eager call on the same inputs and, within the 16-bit bar,
against the fp64 oracle."""

import numpy as np
import pytest
import torch

import exact_io_aware_37_amd as fa
import workloads
from oracle import attention_fp64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2


def say(msg):
    print(msg, flush=True)


def new_inputs(B, Hq, Hkv, Nq, Nkv, d, dt, seed):
    q, k, v = workloads.make_inputs(B, Hq, Hkv, Nq, Nkv, d, dt, seed, 1.0)
    return q, k, v


def oracle_err(q, k, v, causal, scale, o, lse):
    ref_o, ref_l = attention_fp64(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                  scale, causal)
    err_o = float(np.max(np.abs(o.double().cpu().numpy() - ref_o)))
    err_l = float(np.max(np.abs(lse.double().cpu().numpy() - ref_l)))
    return err_o, err_l


@pytest.mark.parametrize("d,causal,dt", [(128, False, "bf16"), (64, True, "f16")])
def test_forward_replays(d, causal, dt):
    B, Hq, Hkv, N = 1, 4, 2, 700
    say(f"[case] graph forward d={d} causal={causal} {dt} N={N}")
    q, k, v = (x.to(DEV) for x in new_inputs(B, Hq, Hkv, N, N, d, dt, 1))
    scale = workloads.default_scale(d)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, dtype=torch.float32, device=DEV)
    fa.attention(q, k, v, causal=causal, scale=scale, out=o, lse=lse)   # one-time set-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.attention(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    for rep in range(3):
        qn, kn, vn = new_inputs(B, Hq, Hkv, N, N, d, dt, 10 + rep)
        q.copy_(qn.to(DEV)); k.copy_(kn.to(DEV)); v.copy_(vn.to(DEV))
        o.fill_(float("nan")); lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = fa.fwd(q, k, v, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, lse_e), rep
        err_o, err_l = oracle_err(qn, kn, vn, causal, scale, o, lse)
        say(f"    replay {rep}: max|dO|={err_o:.3e} max|dlse|={err_l:.3e}")
        assert err_o <= TOL and err_l <= TOL


def test_splitkv_noalloc_replays():
    B, Hq, Hkv, Nq, Nkv, d = 2, 8, 2, 1, 5000, 128
    say(f"[case] graph split-KV (no-alloc) B={B} Hq={Hq} Hkv={Hkv} N_kv={Nkv}")
    q, k, v = (x.to(DEV) for x in new_inputs(B, Hq, Hkv, Nq, Nkv, d, "bf16", 2))
    scale = workloads.default_scale(d)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=DEV)
    fa.attention_splitkv_noalloc(q, k, v, o, lse, scale=scale)           # one-time set-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.attention_splitkv_noalloc(q, k, v, o, lse, scale=scale)
    for rep in range(3):
        qn, kn, vn = new_inputs(B, Hq, Hkv, Nq, Nkv, d, "bf16", 20 + rep)
        q.copy_(qn.to(DEV)); k.copy_(kn.to(DEV)); v.copy_(vn.to(DEV))
        o.fill_(float("nan")); lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e = torch.empty_like(q)
        lse_e = torch.empty_like(lse)
        fa.attention_splitkv_noalloc(q, k, v, o_e, lse_e, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, lse_e), rep
        err_o, err_l = oracle_err(qn, kn, vn, False, scale, o, lse)
        say(f"    replay {rep}: max|dO|={err_o:.3e} max|dlse|={err_l:.3e}")
        assert err_o <= TOL and err_l <= TOL


def test_backward_replays():
    B, Hq, Hkv, N, d = 1, 4, 2, 600, 128
    say(f"[case] graph backward B={B} Hq={Hq} Hkv={Hkv} N={N} causal")
    q, k, v = (x.to(DEV) for x in new_inputs(B, Hq, Hkv, N, N, d, "bf16", 3))
    scale = workloads.default_scale(d)
    gen = torch.Generator().manual_seed(4)
    dout = torch.randn(q.shape, generator=gen).to(q.dtype).to(DEV)
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    ws = torch.empty(max(fa.fa_bwd_workspace_bytes(B, Hq, Hkv, N, N, d), 16), dtype=torch.uint8,
                     device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa.attention_backward(q, k, v, o, lse, dout, causal=True, scale=scale, workspace=ws,
                          dq=dq, dk=dk, dv=dv)                           # one-time set-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.attention_backward(q, k, v, o, lse, dout, causal=True, scale=scale, workspace=ws,
                              dq=dq, dk=dk, dv=dv)
    for rep in range(3):
        qn, kn, vn = new_inputs(B, Hq, Hkv, N, N, d, "bf16", 30 + rep)
        q.copy_(qn.to(DEV)); k.copy_(kn.to(DEV)); v.copy_(vn.to(DEV))
        o_n, lse_n = fa.fwd(q, k, v, causal=True, scale=scale)
        o.copy_(o_n); lse.copy_(lse_n)
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = fa.attention_backward(q, k, v, o, lse, dout, causal=True, scale=scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), eager):
            assert torch.isfinite(a.float()).all(), (rep, name)
            assert torch.equal(a, b), (rep, name)
        say(f"    replay {rep}: dq, dk, dv bitwise equal to the eager call")
