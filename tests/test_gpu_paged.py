"""GPU parity of the paged-cache split-KV forward (fa_fwd_paged) against the fp64 oracle.

Caches come from ``workloads.paginate``: sequences scattered over a seeded
permutation of pool blocks, every slot that holds no key set to NaN (spare
blocks, the tail of each sequence's last block), table entries past a
sequence set to -1.  A kernel that reads anything but the sequence's keys
shows NaN.  Outputs and the workspace are poisoned with NaN first.

Bar: the split-KV path's, max-abs error <= 2e-2 on O and on lse (bf16/f16);
rows that see no key must come back as exactly O = 0, lse = -inf.
"""

import numpy as np
import pytest
import torch

import exact_io_aware_37_amd as fa
import workloads
from oracle import attention_fp64_paged

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2


def say(msg):
    print(msg, flush=True)


def run_paged(q, kc, vc, tab, sl, causal, scale, splits=None):
    B, Hq, Nq, d = q.shape
    qd, kcd, vcd, tbd, sld = (x.to(DEV) for x in (q, kc, vc, tab, sl))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=DEV)
    if splits is None:
        splits = fa.fa_splitkv_default_splits(B, Hq, kc.shape[2], Nq, tab.shape[1] * kc.shape[1], d,
                                              fa.dtype_code(q.dtype))
    nbytes = fa.fa_splitkv_workspace_bytes(B, Hq, Nq, d, splits)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    fa.attention_paged(qd, kcd, vcd, tbd, sld, causal=causal, scale=scale, num_splits=splits,
                       workspace=ws, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), splits


def check(name, B, Hq, Hkv, Nq, lens, D, bs, causal, dtype="bf16", seed=0, splits=None, scale=None):
    scale = workloads.default_scale(D) if scale is None else scale
    nmax = max(max(lens), 1)
    q, k, v = workloads.make_inputs(B, Hq, Hkv, Nq, nmax, D, dtype, seed)
    kc, vc, tab, sl = workloads.paginate(k, v, lens, bs, seed=seed + 1)
    say(f"[case] {name}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} lens={lens} d={D} block={bs} "
        f"causal={causal} {dtype} splits={splits}")
    o, lse, S = run_paged(q, kc, vc, tab, sl, causal, scale, splits)
    ro, rl = attention_fp64_paged(workloads.to_f64(q), workloads.to_f64(kc), workloads.to_f64(vc),
                                  tab.numpy(), sl.numpy(), scale, causal)
    og, lg = workloads.to_f64(o), lse.double().numpy()
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lg), empty), "rows without keys differ"
    assert np.all(og[empty] == 0), "a row without keys has a nonzero output"
    full = ~empty
    assert np.all(np.isfinite(og[full])) and np.all(np.isfinite(lg[full])), "unwritten or NaN output"
    eo = float(np.max(np.abs(og[full] - ro[full]), initial=0.0))
    el = float(np.max(np.abs(lg[full] - rl[full]), initial=0.0))
    say(f"    splits={S} max|dO|={eo:.3e} max|dlse|={el:.3e} empty rows={int(empty.sum())}")
    assert eo <= TOL and el <= TOL, (eo, el)
    return o, lse


@pytest.mark.parametrize("bs", [16, 32, 64, 256])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_variable_lengths(bs, D):
    check("decode", 3, 28, 4, 1, [1, 700, 5000], D, bs, False, seed=bs + D)


@pytest.mark.parametrize("splits", [1, 3, 16, None])
def test_split_counts(splits):
    check("splits", 2, 8, 2, 1, [2000, 333], 128, 16, False, seed=3, splits=splits)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq", [4, 37])
def test_several_new_queries(causal, Nq):
    """Chunked prefill / speculative decoding: N_q queries at the end of each sequence."""
    check("queries", 3, 8, 2, Nq, [Nq, 300, 1025], 128, 16, causal, seed=Nq + causal)


@pytest.mark.parametrize("causal", [False, True])
def test_odd_kv_head_count(causal):
    """Hkv = 3 with 37 new queries per sequence (4 row blocks of the 3 query heads of a group):
    work items are numbered with the key/value head fastest, so here the 8 waves of a workgroup
    straddle chunks and row blocks."""
    check("odd kv heads", 2, 9, 3, 37, [500, 2100], 128, 16, causal, seed=11 + causal)
    check("odd kv heads, 3 splits", 3, 9, 3, 37, [37, 500, 2100], 64, 32, causal, seed=13 + causal,
          splits=3)


def test_rows_without_keys():
    """Causal with N_q above a sequence's length, and an empty sequence: O = 0, lse = -inf."""
    check("empty rows", 3, 4, 2, 8, [3, 0, 40], 64, 16, True, seed=5)


def test_f16_and_scale_values():
    check("f16", 2, 8, 4, 2, [129, 64], 128, 32, False, dtype="f16", seed=6)
    for scale in (0.0, -0.09):
        check("scale", 2, 8, 4, 1, [129, 64], 128, 32, False, seed=7, scale=scale)


def test_bad_table_entries_stay_inside_the_pool():
    """Out-of-range block numbers are clamped into the pool: finite output, no fault."""
    q, k, v = workloads.make_inputs(2, 4, 2, 1, 100, 64, "bf16", 8)
    kc, vc, tab, sl = workloads.paginate(k, v, [100, 100], 16, seed=9, spare_blocks=0)
    tab = tab.clone()
    tab[0, 1] = 10 ** 6
    tab[1, 2] = -5
    kc = torch.nan_to_num(kc)   # every slot a finite value, so any clamped read is finite
    vc = torch.nan_to_num(vc)
    o, lse, _ = run_paged(q, kc, vc, tab, sl, False, 0.125)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_matches_dense_split_bitwise():
    """Full-length sequences, one sequence and one key/value head (there the dense kernel takes
    its tiles in the plain order too): the paged kernel does the dense split-KV kernel's
    arithmetic on the same keys in the same order, so the outputs agree bit for bit."""
    B, Hq, Hkv, Nq, N, D = 1, 7, 1, 1, 8192, 128
    q, k, v = workloads.make_inputs(B, Hq, Hkv, Nq, N, D, "bf16", 10)
    kc, vc, tab, sl = workloads.paginate(k, v, [N] * B, 16, seed=11)
    o_p, l_p, S = run_paged(q, kc, vc, tab, sl, False, 0.088388, 12)
    o_d, l_d = fa.attention_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), scale=0.088388, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_d.cpu()) and torch.equal(l_p, l_d.cpu())


def test_full_workload8_against_oracle():
    """Decode B=8 Hq=28 Hkv=4 N=32768 in 16-key blocks, the launch the benchmark times, every row."""
    w = workloads.WORKLOADS[8]
    q, k, v, scale = workloads.workload_inputs(w)
    kc, vc, tab, sl = workloads.paginate(k, v, [w.Nkv] * w.B, w.block_size, seed=w.seed)
    say(f"[case] {w.name}")
    o, lse, S = run_paged(q, kc, vc, tab, sl, w.causal, scale)
    ro, rl = attention_fp64_paged(workloads.to_f64(q), workloads.to_f64(kc), workloads.to_f64(vc),
                                  tab.numpy(), sl.numpy(), scale, w.causal)
    eo = float(np.max(np.abs(workloads.to_f64(o) - ro)))
    el = float(np.max(np.abs(lse.double().numpy() - rl)))
    say(f"    splits={S} max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL and el <= TOL


@pytest.mark.parametrize("causal, Nq", [(False, 1), (True, 4)])
def test_largest_pool_the_host_accepts(causal, Nq):
    """Maximum size for fa_fwd_paged: block offsets inside a pool are 32-bit, so the host
    accepts pools of at most 2^32 - 4097 bytes.  With 16-key blocks, Hkv = 2 and d = 128 in
    bf16 (8 KiB per block) that is 524287 blocks (4 GiB per pool); one block more is rejected.
    Two sequences (5000 and 3001 keys, GQA 4:1) live in that pool: the first in the last 313
    blocks, the second in block 0, blocks from the middle and the pool's last-but-313 region,
    with a ragged last block.  Every other slot of both pools is NaN, so a read outside the
    sequences shows.  In each sequence one key per key/value head (the last key, key 0, or one
    in the middle) is replaced by 16 times a query row's unit vector: it outweighs the other
    keys (score about 16 against a log-sum of about 9.5), so the output is of order one and
    tracks that key's V row.  The oracle sees the referenced blocks only, with the table
    renumbered accordingly (the same keys in the same order)."""
    bs, Hkv, Hq, d = 16, 2, 8, 128
    nb = (2 ** 32 - 4097) // (bs * Hkv * d * 2)
    assert nb == 524287
    lens = [5000, 3001]
    mb = max((n + bs - 1) // bs for n in lens)
    scale = workloads.default_scale(d)
    st = fa.fa_fwd_paged(1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40, 6 << 40, 7 << 40, 2, Hq, Hkv,
                         Nq, d, nb + 1, bs, mb, scale, int(causal), fa.FA_BF16, 4, 8 << 40,
                         1 << 30, None)
    assert st == fa.FA_ERR_BAD_DIM   # rejected before any memory is touched
    rng = np.random.default_rng(4545 + Nq)
    n0 = (lens[0] + bs - 1) // bs
    n1 = (lens[1] + bs - 1) // bs
    tab = np.full((2, mb), -1, dtype=np.int32)
    tab[0, :n0] = np.arange(nb - n0, nb)                                   # the pool's last blocks
    mid = rng.choice(np.arange(1, nb - n0 - 200), n1 - 2, replace=False)
    tab[1, :n1] = np.concatenate([[0], mid, [nb - n0 - 1]])               # first, middle, high
    q = torch.from_numpy(rng.standard_normal((2, Hq, Nq, d), dtype=np.float32)).to(torch.bfloat16)
    kc = torch.full((nb, bs, Hkv, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full((nb, bs, Hkv, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    plant = {0: [(lens[0] - 1, 0, 0), (0, 1, 4)], 1: [(lens[1] - 1, 0, 1), (1600, 1, 7)]}
    for b, n in enumerate(lens):
        kb = torch.from_numpy(rng.standard_normal((n, Hkv, d), dtype=np.float32)).to(torch.bfloat16)
        vb = torch.from_numpy(rng.standard_normal((n, Hkv, d), dtype=np.float32)).to(torch.bfloat16)
        for key, g, h in plant[b]:   # key row of kv head g aligned with query head h, last row
            x = q[b, h, Nq - 1].double()
            kb[key, g] = (16.0 * x / x.norm()).to(torch.bfloat16)
        t = np.arange(n)
        slots = torch.from_numpy(tab[b, t // bs].astype(np.int64) * bs + t % bs).to(DEV)
        kc.view(nb * bs, Hkv, d)[slots] = kb.to(DEV)
        vc.view(nb * bs, Hkv, d)[slots] = vb.to(DEV)
    tabd = torch.from_numpy(tab)
    sl = torch.tensor(lens, dtype=torch.int32)
    say(f"[case] largest accepted pool: {nb} blocks of {bs} keys, Hkv={Hkv}, d={d}, lens={lens}, "
        f"Nq={Nq}, causal={causal}")
    o, lse, S = run_paged(q, kc, vc, tabd, sl, causal, scale)
    used = np.unique(tab[tab >= 0])
    remap = np.full(nb, -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    tab_c = np.where(tab >= 0, remap[np.maximum(tab, 0)], -1).astype(np.int32)
    idx = torch.from_numpy(used).to(DEV)
    kcc, vcc = kc[idx].cpu(), vc[idx].cpu()
    del kc, vc
    ro, rl = attention_fp64_paged(workloads.to_f64(q), workloads.to_f64(kcc), workloads.to_f64(vcc),
                                  tab_c, np.array(lens), scale, causal)
    og, lg = workloads.to_f64(o), lse.double().numpy()
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), "unwritten or NaN output"
    eo, el = float(np.max(np.abs(og - ro))), float(np.max(np.abs(lg - rl)))
    say(f"    splits={S} max|dO|={eo:.3e} max|dlse|={el:.3e} max|O|={float(np.abs(og).max()):.3f}")
    assert eo <= TOL and el <= TOL, (eo, el)
