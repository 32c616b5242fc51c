"""CPU checks of the generated 64-row forward body (gen_fwd_w64.py).

The generated gfx950 assembly runs in a functional emulator (asm_emu.py), one
workgroup at a time, with the operands the kernel in fa_fwd.hip computes for
it (the same address formulas, restated below), on seeded inputs; its O and
lse are compared with the fp64 oracle at the 16-bit bar (max-abs 2e-2).  The
emulator also fails on a missing s_waitcnt, an LDS read of a transfer not yet
waited for and out-of-range LDS accesses, and every case runs with the four
waves in two orders between barriers, which must give identical bytes.  The
generator's own checks (wait states between dependent instructions) run as it
emits the code."""

import math
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "exact_io_aware_37_amd", "csrc"))

import gen_fwd_w64 as gen  # noqa: E402
import workloads  # noqa: E402
from asm_emu import Emu  # noqa: E402
from oracle import attention_fp64  # noqa: E402

TOL = 2e-2
KBUF, VBUF, QBUF, OBUF, LBUF = 1, 2, 3, 4, 5


def operands(wave, q0, Nq, Nkv, causal, scale, dt="bf16", qhead_bytes=0, kvhead_bytes=0, d=128):
    """Inline-asm operands of one wave: register name -> value (per lane or scalar)."""
    lane = np.arange(64)
    l32, half = lane & 31, lane >> 5
    lds = 0
    rowb = 2 * d
    vring = 4 * 64 * rowb
    nch = rowb // 16           # 16-byte chunks per row
    rpp = 1024 // rowb         # rows per 1 KiB DMA piece

    def sw_k(row):             # K rows: 16-byte chunk index XOR
        return row & 15 if d == 128 else (row >> 1) & 7

    def sw_v(row):             # V rows
        return (row & 3) << 2 if d == 128 else ((row >> 1) & 1) << 2
    # K fragment addresses: row l32, logical chunk 2cd + half, physical chunk ^ sw_k(row)
    swz = sw_k(l32)
    kbase = l32 * rowb + ((half ^ (swz & 1)) * 16) + ((swz >> 1) * 32)
    # V^T fragment addresses (ds_read_b64_tr_b16)
    g16, s16 = lane >> 4, lane & 15
    vrow = (g16 >> 1) * 4 + (s16 >> 2)
    vbase = vrow * rowb + sw_v(vrow) * 16 + (g16 & 1) * 32 + ((s16 & 3) >> 1) * 16 + (s16 & 1) * 8
    isv = wave >= 2
    npiece = 64 * rowb // 2048
    ci0 = (npiece * wave) & (2 * npiece - 1)
    dmaoff = []
    for u in range(4):
        row = (ci0 + u) * rpp + lane // nch
        sw = sw_v(row) if isv else sw_k(row)
        dmaoff.append(row * rowb + ((lane % nch) ^ sw) * 16)
    q0w = q0 + 64 * wave
    big = 0x3FFFFFFF
    lim = [np.minimum(Nkv - 1, (q0w + 32 * h + l32) if causal else big) for h in range(2)]
    kv_end = min(Nkv, q0 + 256) if causal else Nkv
    ntiles = (kv_end + 63) // 64
    nmain = min((q0 + 1) // 64, Nkv // 64) if causal else Nkv // 64
    if scale > 0:
        sl2, qxor, qand = scale * 1.4426950408889634, 0, 0xFFFFFFFF
    elif scale < 0:
        sl2, qxor, qand = -scale * 1.4426950408889634, 0x80008000, 0xFFFFFFFF
    else:
        sl2, qxor, qand = 1.0, 0, 0
    sv = {
        "rq": [QBUF, qhead_bytes, Nq * rowb, 0],
        "rdma": [VBUF if isv else KBUF, kvhead_bytes, Nkv * rowb, 0],
        "ro": [OBUF, qhead_bytes, Nq * rowb, 0],
        "rl": [LBUF, qhead_bytes // (rowb // 4), Nq * 4, 0],
        "dmabase": lds + (vring if isv else 0) + ci0 * 1024,
        "sl2": int(np.float32(sl2).view(np.uint32)),
        "qxor": qxor, "qand": qand, "ntiles": ntiles, "nmain": nmain,
        "obase": lds + wave * 64 * rowb,
    }
    vv = {f"kaddr{cd}": lds + (kbase ^ (cd * 32)) for cd in range(d // 16)}
    vv.update({f"vaddr{db}": lds + vring + (vbase ^ (db * 64)) for db in range(d // 32)})
    vv.update({f"dmaoff{u}": dmaoff[u] for u in range(4)})
    vv["qoff"] = (q0w + l32) * rowb + half * 16
    vv["lim0"], vv["lim1"] = lim
    vv["ooff"] = (q0w + lane // nch) * rowb + (lane % nch) * 16
    vv["lseoff"] = (q0w + l32) * 4
    one = 0x3F803F80 if dt == "bf16" else 0x3C003C00
    vv["selv"] = np.where((lane & 7) == ((lane >> 2) & 4), one, 0)
    return sv, vv


def assign_registers(text):
    names = sorted(set(__import__("re").findall(r"\{(\w+)\}", text)))
    sreg, vreg, s_at, v_at = {}, {}, 0, 230
    for n in names:
        if gen.OPERANDS[n] == "s":
            width = 4 if n in ("rq", "rdma", "ro", "rl") else 1
            s_at = (s_at + width - 1) // width * width
            sreg[n] = f"s[{s_at}:{s_at + 3}]" if width == 4 else f"s{s_at}"
            s_at += width
        else:
            vreg[n] = f"v{v_at}"
            v_at += 1
    assert s_at <= 72 and v_at <= 256
    return sreg, vreg


def run_workgroup(text, q, k, v, q0, causal, scale, dt, order):
    B, H, Nq, D = q.shape
    rowb = 2 * D
    Nkv = k.shape[2]
    sreg, vreg = assign_registers(text)
    body = text
    for n, r in {**sreg, **vreg}.items():
        body = body.replace("{" + n + "}", r)
    bits = (lambda t: t.view(torch.int16).numpy().view(np.uint8).copy())
    bufs = {QBUF: bits(q.contiguous()).reshape(-1), KBUF: bits(k.contiguous()).reshape(-1),
            VBUF: bits(v.contiguous()).reshape(-1),
            OBUF: np.full(Nq * rowb, 0xFF, np.uint8), LBUF: np.full(Nq * 4, 0xFF, np.uint8)}
    emu = Emu(body, bufs, order=order)
    for w in range(4):
        sv, vv = operands(w, q0, Nq, Nkv, causal, scale, dt, d=D)
        wave = emu.waves[w]
        for n, val in sv.items():
            r = gen.regs(sreg[n])
            vals = val if isinstance(val, list) else [val]
            for reg, x in zip(r, vals):
                wave.s[int(reg[1:])] = int(x) & 0xFFFFFFFF
        for n, val in vv.items():
            wave.v[int(vreg[n][1:])] = np.asarray(val, np.int64).astype(np.uint32)
    emu.run()
    run_workgroup.rescales = emu.executed.get(emu.labels[".Lrescale"], 0)
    return bufs[OBUF], bufs[LBUF]


def check(dt, causal, Nq, Nkv, q0, scale=None, sigma=1.0, seed=0, outliers=0.0, d=128,
          rescales=None):
    torch_dt = workloads.DTYPES[dt]
    q, k, v = workloads.make_inputs(1, 1, 1, Nq, Nkv, d, dt, seed, sigma)
    if outliers:
        rng = np.random.default_rng(seed + 99)
        idx = rng.choice(Nkv, max(1, int(outliers * Nkv)), replace=False)
        k[0, 0, idx] = (k[0, 0, idx].float() * 8).to(torch_dt)
    scale = workloads.default_scale(d) if scale is None else scale
    text = gen.body(dt, causal, d)
    outs = []
    for order in ([0, 1, 2, 3], [3, 2, 1, 0]):
        outs.append(run_workgroup(text, q, k, v, q0, causal, scale, dt, order))
    if rescales is not None:
        # executions of the rescale block, summed over the 4 waves
        assert rescales(run_workgroup.rescales), run_workgroup.rescales
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    o_bytes, l_bytes = outs[0]
    rows = np.arange(q0, min(q0 + 256, Nq))
    o = torch.from_numpy(o_bytes.view(np.int16).copy()).view(torch_dt).reshape(Nq, d)[rows]
    lse = l_bytes.view(np.float32).reshape(Nq)[rows]
    ref_o, ref_l = attention_fp64(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                  scale, causal, rows=rows)
    err_o = float(np.max(np.abs(o.double().numpy() - ref_o[0, 0])))
    err_l = float(np.max(np.abs(lse.astype(np.float64) - ref_l[0, 0])))
    print(f"max|dO|={err_o:.3e} max|dlse|={err_l:.3e}", flush=True)
    assert np.isfinite(err_o) and np.isfinite(err_l)
    assert err_o <= TOL and err_l <= TOL, (err_o, err_l)
    # untouched rows outside the workgroup
    others = np.setdiff1d(np.arange(Nq), rows)
    if others.size:
        assert np.all(l_bytes.view(np.uint32).reshape(Nq)[others] == 0xFFFFFFFF)
    return err_o, err_l


CASES = [
    # dt, causal, Nq, Nkv, q0
    ("bf16", False, 256, 256, 0),      # 4 unmasked tiles: every parity once
    ("bf16", False, 256, 640, 0),      # 10 tiles: parities twice, steady state
    ("bf16", False, 256, 200, 0),      # ragged tail: last step masked
    ("bf16", False, 256, 64, 0),       # one tile: prologue then drain
    ("bf16", False, 100, 300, 0),      # ragged query rows
    ("bf16", True, 512, 512, 256),     # causal second query tile: 4 unmasked, 4 masked
    ("bf16", True, 256, 256, 0),       # causal first tile: masked prologue
    ("f16", False, 256, 330, 0),
    ("f16", True, 300, 300, 256),
    ("bf16", True, 512, 700, 256),     # causal, more keys than query rows
    ("f16", False, 40, 1000, 0),       # 16 tiles, rows only in part of one wave
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_generated_body_matches_oracle(case):
    dt, causal, Nq, Nkv, q0 = case
    check(dt, causal, Nq, Nkv, q0, seed=Nq + Nkv + q0)


CASES_D64 = [
    ("bf16", False, 256, 256, 0),      # every parity once
    ("bf16", False, 256, 650, 0),      # parities twice, ragged tail
    ("bf16", True, 512, 512, 256),     # causal second query tile
    ("bf16", True, 256, 256, 0),       # causal first tile: masked prologue
    ("f16", False, 100, 64, 0),        # one tile, ragged rows
    ("f16", True, 300, 700, 256),
]


@pytest.mark.parametrize("case", CASES_D64, ids=lambda c: "-".join(map(str, c)))
def test_generated_body_d64_matches_oracle(case):
    """The same body generated for head dimension 64."""
    dt, causal, Nq, Nkv, q0 = case
    check(dt, causal, Nq, Nkv, q0, seed=Nq + Nkv + q0 + 64, d=64)


@pytest.mark.parametrize("d", [128, 64])
def test_reference_moves_and_rescales(d):
    """Scores spread over tens of units: the lazy reference moves and O is rescaled."""
    check("bf16", False, 256, 512, 0, scale=1.0, sigma=2.0, seed=5, outliers=0.02, d=d,
          rescales=lambda n: n > 0)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_reference_moves_only_past_its_threshold(dt):
    """Keys in three blocks whose scores sit 14, then 16, log2 units above the first
    block's: the first step stays on the old reference (probabilities up to 2^14,
    finite in f16 too), the second moves it, once per wave."""
    d, nkv = 128, 192
    q, k, v = workloads.make_inputs(1, 1, 1, 256, nkv, d, dt, 11, 1.0)
    torch_dt = workloads.DTYPES[dt]
    qq = torch.zeros(1, 1, 256, d)
    qq[..., 0] = 1.0
    kk = torch.zeros(1, 1, nkv, d)
    kk[0, 0, 64:128, 0] = 14.0
    kk[0, 0, 128:, 0] = 30.0
    scale = math.log(2)            # score * scale * log2(e) = key[0] in log2 units
    got = []
    for order in ([0, 1, 2, 3], [3, 2, 1, 0]):
        o, lse = run_workgroup(gen.body(dt, False, d), qq.to(torch_dt), kk.to(torch_dt), v,
                               0, False, scale, dt, order)
        got.append(run_workgroup.rescales)
    assert got == [4, 4], got
    o = torch.from_numpy(o.view(np.int16).copy()).view(torch_dt).reshape(256, d)
    lse = lse.view(np.float32)
    ref_o, ref_l = attention_fp64(workloads.to_f64(qq.to(torch_dt)), workloads.to_f64(kk.to(torch_dt)),
                                  workloads.to_f64(v), scale, False)
    assert float(np.max(np.abs(o.double().numpy() - ref_o[0, 0]))) <= TOL
    assert float(np.max(np.abs(lse.astype(np.float64) - ref_l[0, 0]))) <= TOL


@pytest.mark.parametrize("scale", [0.0, -0.09])
def test_scale_zero_and_negative(scale):
    check("bf16", True, 256, 192, 0, scale=scale, seed=6)
