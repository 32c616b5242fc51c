"""The 64-row-per-wave forward body for OCP E4M3 inputs (head dimension 128), gfx950 assembly.

Built on the 16-bit generator (gen_fwd_w64.py: instruction records, the hazard-aware block,
the issue-cost list scheduler, the K/V DMA ring, masking and the epilogue) and run the same
way: the kernel in fa_fwd.hip computes the operands and runs the body as one inline-asm
statement.  What the body computes is the FP8 forward of the same file: S = K Q^T on the
8-bit matrix instruction, probabilities rounded to E4M3 against a power-of-two reference of
their own 64-key tile, the tile-to-row factor 2^-k carried as the E8M0 block scale of the
P operand, row sums of the rounded P on the matrix instruction (an all-ones operand), O in
fp32 and written in bf16 as O * (V's descale) / l, lse = (m + log2 l) ln 2 (the recurrence
of "FlashAttention: IO-aware attention kernel", section 3.2, with the FP8 direction of its
section 3.3).

Tile geometry in bytes is that of the 16-bit body at d = 64: K and V rows of 128 bytes, 8 KiB
per tile, a 4-stage ring of 64 KiB, each wave moving 4 KiB of each tile it carries.

Register map (per wave; O and the row-sum blocks in AGPRs):
  a[0:127]    O^T accumulators, block (h, db): a[16*(4h+db) : +16]
  a[128:159]  Q operand, (h, cd): a[128 + 8*(2h+cd) : +8], bytes 64cd + 32*(l/32) + j
  a[160:191]  row-sum accumulators, half h: a[160 + 16h : +16] (register 0 is read)
  v[0:127]    two score buffers, block (h, kt) as in the 16-bit body; P of half h (32
              E4M3 bytes per lane) packed over the first 8 registers of its block kt = 0
  v[128:151]  K fragment ring (3 slots of 8), v[152:175] V fragment ring (3 slots of 8)
  v[176:193]  row statistics of the 16-bit body (reference, maxima, alpha, masks)
  v194-v199   per-tile reference and block scale of the tile being multiplied, 127
  v[200:207]  E4M3 ones (the row-sum operand), v[208:223] rescale temporaries
  v224-v227   per-tile reference and block scale of the next tile
"""

from __future__ import annotations

import re

import gen_fwd_w64 as g
from gen_fwd_w64 import Block, Ins, Stream, mfma, raw, regs, schedule, valu

ROWB8 = 128                  # bytes of one E4M3 K or V row (d = 128)
KST8 = 64 * ROWB8            # one K (or V) tile in LDS
VRING8 = 4 * KST8
NPIECE8 = KST8 // 2048       # 1 KiB DMA pieces per wave and stage
KSL8 = 3                     # K fragment ring slots (8 registers each)
VSL8 = 3
VLEAD8 = 6
MFMA8_CYCLES = 64            # v_mfma_*_32x32x64_f8f6f4: 16 passes
LAZY8 = "0x41000000"         # 8.0: the row reference moves when the maximum passes it by 2^8
MF8 = "v_mfma_f32_32x32x64_f8f6f4"
MF8S = "v_mfma_scale_f32_32x32x64_f8f6f4"

MTILE = ["v194", "v195"]     # reference of the tile being exponentiated (per half)
SBYTE = ["v196", "v197"]     # its E8M0 block scale (127 - k)
SC127 = "v198"
MTN = ["v224", "v225"]       # the same for the next tile, committed at the end of a step
SBN = ["v226", "v227"]
ONES = "v[200:207]"


def Q8(h, cd):
    b = 128 + 8 * (2 * h + cd)
    return f"a[{b}:{b + 7}]"


def RS(h):
    b = 160 + 16 * h
    return f"a[{b}:{b + 15}]"


def P8(buf, h):
    b = 64 * buf + 32 * h
    return f"v[{b}:{b + 7}]"


def p8(buf, h, w):
    return f"v{64 * buf + 32 * h + w}"


def KF8(slot):
    b = 128 + 8 * slot
    return f"v[{b}:{b + 7}]"


def VF8(slot):
    b = 152 + 8 * slot
    return f"v[{b}:{b + 7}]"


def _half_regs(spec, part):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", spec)
    b = int(m.group(1)) + 4 * part
    return f"v[{b}:{b + 3}]"


def _pair(spec, i):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", spec)
    b = int(m.group(1)) + 2 * i
    return f"v[{b}:{b + 1}]"


def k_reads8(f, kstage):
    """Fragment f = 2cd + kt of K: key row 32kt + l%32, head-dimension bytes 64cd + 32*(l/32)
    .. +31, as two 16-byte chunks (address operands kaddr(2cd) and kaddr(2cd+1))."""
    cd, kt = f // 2, f % 2
    off = kstage * KST8 + kt * 32 * ROWB8
    dst = KF8(f % KSL8)
    return [Ins(f"ds_read_b128 {_half_regs(dst, part)}, {{kaddr{2 * cd + part}}} offset:{off}",
                "lds", writes=regs(_half_regs(dst, part))) for part in range(2)]


def s_mfmas8(buf, kstage, skip=0):
    ms, reads = [], []
    for cd in range(2):
        for kt in range(2):
            f = 2 * cd + kt
            if f >= skip:
                reads.append((2 * f, 2 * (f - KSL8) + 2 if f >= KSL8 else 0, k_reads8(f, kstage)))
            for h in range(2):
                c = "0" if cd == 0 else g.S(buf, h, kt)
                ms.append(mfma(MF8, g.S(buf, h, kt), KF8(f % KSL8), Q8(h, cd), c,
                               cycles=MFMA8_CYCLES))
    return ms, reads


def pv_mfmas8(vstage, base_index, buf):
    """O^T += V^T P^T per (db, h) with P's block scales, then the row sums of P.

    V fragment db: four ds_read_b64_tr_b8 (keys 16i .. of the tile in the order of the
    P bytes), ring slot db % VSL8, feeding h = 0, 1."""
    ms, uses = [], {}
    for db in range(4):
        for h in range(2):
            uses.setdefault(db, []).append(base_index + len(ms))
            ms.append(Ins(f"{MF8S} {g.O(h, db)}, {VF8(db % VSL8)}, {P8(buf, h)}, {g.O(h, db)}, "
                          f"{SC127}, {SBYTE[h]} op_sel_hi:[0,0,0]", "mfma",
                          regs(VF8(db % VSL8)) + regs(P8(buf, h)) + regs(g.O(h, db)) + [SC127, SBYTE[h]],
                          regs(g.O(h, db)), cost=MFMA8_CYCLES,
                          srcab=regs(VF8(db % VSL8)) + regs(P8(buf, h)) + [SC127, SBYTE[h]]))
    reads = []
    for db in range(4):
        off = vstage * KST8
        rd = [Ins(f"ds_read_b64_tr_b8 {_pair(VF8(db % VSL8), i)}, {{vaddr{db}}} offset:{off + 16 * i * ROWB8}",
                  "lds", writes=regs(_pair(VF8(db % VSL8), i))) for i in range(4)]
        free = max(uses[db - VSL8]) + 1 if db >= VSL8 else 0
        reads.append((min(uses[db]), free, rd))
    for h in range(2):
        ms.append(Ins(f"{MF8S} {RS(h)}, {ONES}, {P8(buf, h)}, {RS(h)}, {SC127}, {SBYTE[h]} "
                      f"op_sel_hi:[0,0,0]", "mfma",
                      regs(ONES) + regs(P8(buf, h)) + regs(RS(h)) + [SC127, SBYTE[h]], regs(RS(h)),
                      cost=MFMA8_CYCLES, srcab=regs(ONES) + regs(P8(buf, h)) + [SC127, SBYTE[h]]))
    return ms, reads


def exp_stream8(buf):
    """P(buf) = exp2(s * sl2 - m_tile) rounded to E4M3, four bytes per dword, dword w of half
    h = scores 4(w%4) .. +3 of block kt = w/4, packed in place over block (h, 0).  Dwords in
    the order the P*V instructions read them (h = 0 first); a dword's conversions come after
    the next dword's multiply-adds."""
    units = []
    for h in range(2):
        for w in range(8):
            kt, r0 = w // 4, 4 * (w % 4)
            sc = [g.s1(buf, h, kt, r0 + i) for i in range(4)]
            f = [valu(f"v_fma_f32 {x}, {x}, {{sl2}}, -{MTILE[h]}", [x, MTILE[h]], [x]) for x in sc]
            e = [valu(f"v_exp_f32 {x}, {x}", [x], [x], kind="trans", cost=8) for x in sc]
            p = p8(buf, h, w)
            c = [valu(f"v_cvt_pk_fp8_f32 {p}, {sc[0]}, {sc[1]}", [sc[0], sc[1], p], [p]),
                 valu(f"v_cvt_pk_fp8_f32 {p}, {sc[2]}, {sc[3]} op_sel:[0,0,1]", [sc[2], sc[3], p], [p])]
            units.append((f, e, c))
    ins = units[0][0] + units[0][1]
    for k in range(1, len(units)):
        ins += units[k][0] + units[k - 1][2] + units[k][1]
    return ins + units[-1][2]


def max_stream8(buf, h, first=False):
    """Row maximum of the tile (raw scores) -> its reference; the tile's own reference
    m_tile = m - k, k = min(floor(m - tile max), 200), and block scale 127 - k (>= 0)."""
    vals = [g.s1(buf, h, kt, r) for kt in range(2) for r in range(16)]
    MX, MXS, MRUN, MNEW, TMP, ALPHA = g.MX[h], g.MXS[h], g.MRUN[h], g.MNEW[h], g.TMP[h], g.ALPHA[h]
    ins = [valu(f"v_max3_f32 {MX}, {vals[0]}, {vals[1]}, {vals[2]}", vals[:3], [MX])]
    rest = vals[3:]
    while rest:
        if len(rest) >= 2:
            ins.append(valu(f"v_max3_f32 {MX}, {MX}, {rest[0]}, {rest[1]}", [MX, rest[0], rest[1]], [MX]))
            rest = rest[2:]
        else:
            ins.append(valu(f"v_max_f32 {MX}, {MX}, {rest[0]}", [MX, rest[0]], [MX]))
            rest = rest[1:]
    ins.append(valu(f"v_mov_b32 {MXS}, {MX}", [MX], [MXS]))
    ins.append(Ins(f"v_permlane32_swap_b32 {MX}, {MXS}", "perm", regs([MX, MXS]), regs([MX, MXS])))
    ins.append(valu(f"v_max_f32 {MX}, {MX}, {MXS}", [MX, MXS], [MX]))
    ins.append(valu(f"v_mul_f32 {MX}, {{sl2}}, {MX}", [MX], [MX]))
    mt, sb = (MTILE[h], SBYTE[h]) if first else (MTN[h], SBN[h])
    if first:
        # the first tile's maximum is the reference; k = 0
        ins.append(valu(f"v_mov_b32 {MRUN}, {MX}", [MX], [MRUN]))
        ins.append(valu(f"v_mov_b32 {mt}, {MX}", [MX], [mt]))
        ins.append(valu(f"v_mov_b32 {sb}, 0x7f", [], [sb]))
        return ins
    ins.append(valu(f"v_add_f32 {TMP}, {LAZY8}, {MRUN}", [MRUN], [TMP]))
    m = g.MASKS[h]
    ins.append(valu(f"v_cmp_gt_f32 {m}, {MX}, {TMP}", [MX, TMP], [m], kind="cmp"))
    ins.append(valu(f"v_cndmask_b32 {MNEW}, {MRUN}, {MX}, {m}", [MRUN, MX, m], [MNEW]))
    ins.append(valu(f"v_sub_f32 {TMP}, {MRUN}, {MNEW}", [MRUN, MNEW], [TMP]))
    ins.append(valu(f"v_exp_f32 {ALPHA}, {TMP}", [TMP], [ALPHA], kind="trans", cost=8))
    ins.append(valu(f"v_sub_f32 {TMP}, {MNEW}, {MX}", [MNEW, MX], [TMP]))
    ins.append(valu(f"v_floor_f32 {TMP}, {TMP}", [TMP], [TMP]))
    ins.append(valu(f"v_min_f32 {TMP}, 0x43480000, {TMP}", [TMP], [TMP]))        # 200.0
    ins.append(valu(f"v_sub_f32 {mt}, {MNEW}, {TMP}", [MNEW, TMP], [mt]))
    ins.append(valu(f"v_sub_f32 {TMP}, 0x42fe0000, {TMP}", [TMP], [TMP]))        # 127.0 - k
    ins.append(valu(f"v_max_f32 {TMP}, 0, {TMP}", [TMP], [TMP]))
    ins.append(valu(f"v_cvt_i32_f32 {sb}, {TMP}", [TMP], [sb]))
    return ins


def dma_issue8(stage):
    ins = []
    for u in range(NPIECE8):
        ins.append(raw(f"s_add_u32 m0, {{dmabase}}, {stage * KST8 + u * 1024}", "salu", writes=["m0"]))
        ins.append(Ins(f"buffer_load_dwordx4 {{dmaoff{u}}}, {{rdma}}, {g.S_TOFF} offen lds", "lds_dma", cost=4))
    ins.append(raw(f"s_add_u32 {g.S_TOFF}, {g.S_TOFF}, {KST8}"))
    return ins


def rescale_block8():
    """O and the row sums move to the new reference (rare: lazy reference)."""
    b = Block()
    b.pad(48)
    t = g.RTMP
    k = 0
    for h in range(2):
        for db in range(4):
            for r in range(16):
                a = 16 * (4 * h + db) + r
                x = t[k % 16]
                b.out.append(Ins(f"v_accvgpr_read_b32 {x}, a{a}", "accr"))
                b.out.append(Ins(f"v_mul_f32 {x}, {x}, {g.ALPHA[h]}", "valu"))
                b.out.append(Ins(f"v_accvgpr_write_b32 a{a}, {x}", "accw"))
                k += 1
        a = 160 + 16 * h
        x = t[k % 16]
        b.out.append(Ins(f"v_accvgpr_read_b32 {x}, a{a}", "accr"))
        b.out.append(Ins(f"v_mul_f32 {x}, {x}, {g.ALPHA[h]}", "valu"))
        b.out.append(Ins(f"v_accvgpr_write_b32 a{a}, {x}", "accw"))
        k += 1
    b.pad(8)
    return b


def commit8():
    """The next tile's reference and block scale become current (after this step's P*V)."""
    ins = []
    for h in range(2):
        ins.append(valu(f"v_mov_b32 {g.MRUN[h]}, {g.MNEW[h]}", [g.MNEW[h]], [g.MRUN[h]]))
        ins.append(valu(f"v_mov_b32 {MTILE[h]}, {MTN[h]}", [MTN[h]], [MTILE[h]]))
        ins.append(valu(f"v_mov_b32 {SBYTE[h]}, {SBN[h]}", [SBN[h]], [SBYTE[h]]))
    return ins


def tile_step8(j_parity, masked):
    """Step j: S(j+1) || exp S(j) -> P(j); then P(j) V(j) and the row sums || the reference
    of S(j+1); the K/V transfers of tile j+3 in the S phase, the barrier inside P*V."""
    kst = (j_parity + 1) % 4
    vst = j_parity % 4
    cur, nxt = j_parity % 2, (j_parity + 1) % 2
    b = Block()
    b.lgkm = [set(regs(KF8(f))) for f in range(KSL8)]
    ms_s, rd_s = s_mfmas8(nxt, kst, skip=KSL8)
    ms_pv, rd_pv = pv_mfmas8(vst, len(ms_s), cur)
    lds_plan = list(rd_s)
    for (use, free, ins) in rd_pv:
        lds_plan.append((use, max(free, use - VLEAD8), ins))
    sync_at = rd_pv[-1][0]
    sync = [Ins(f"s_waitcnt vmcnt({NPIECE8}) lgkmcnt(0)", "wait"), Ins("s_barrier", "barrier")]
    nextk = [r for f in range(KSL8) for r in k_reads8(f, (j_parity + 2) % 4)]
    dma = Stream(dma_issue8((j_parity + 3) % 4), 2, "dma", deadline=sync_at)
    dma.pace = g.DMA_PACE
    streams = [Stream(nextk, sync_at, "nextk"), dma, Stream(exp_stream8(cur), 0, "exp")]
    tail = []
    if masked:
        tail += [raw(f"s_add_u32 {g.S_KV0}, {g.S_KV0}, {g.BC}")]
        tail += g.mask_stream(nxt)
    tail += max_stream8(nxt, 0) + max_stream8(nxt, 1)
    tail.append(valu(f"v_cmp_neq_f32 vcc, 1.0, {g.ALPHA[0]}", [g.ALPHA[0]], ["vcc"], kind="cmp"))
    tail.append(valu(f"v_cmp_neq_f32 {g.S_ANY}, 1.0, {g.ALPHA[1]}", [g.ALPHA[1]], [g.S_ANY], kind="cmp"))
    streams.append(Stream(tail, len(ms_s), "max"))
    schedule(b, ms_s + ms_pv, streams, lds_plan, inserts=[(sync_at, sync)])
    if not masked:
        b.put(raw(f"s_add_u32 {g.S_KV0}, {g.S_KV0}, {g.BC}"))
    for ins in commit8():
        b.put(ins)
    b.put(raw(f"s_or_b64 vcc, vcc, {g.S_ANY}", reads=["vcc", g.S_ANY], writes=["vcc"]))
    b.put(raw("s_cbranch_vccnz .Lrescale", "branch"))
    b.put(raw(f"s_add_u32 {g.S_T}, {g.S_T}, 1"))
    if masked:
        b.put(raw("s_branch .Ldisp", "branch"))
    else:
        b.put(raw(f"s_add_u32 {g.S_TMP}, {g.S_T}, 1"))
        b.put(raw(f"s_cmp_lt_u32 {g.S_TMP}, {{nmain}}"))
        b.put(raw("s_cbranch_scc0 .Ldisp", "branch"))
        if j_parity == 3:
            b.put(raw("s_branch .Lu_0", "branch"))
    return b


def first_tile8(masked_first):
    """Prologue: Q to AGPRs, O and the row sums zeroed, constants, DMA of tiles 0-2, S(0) and
    its reference."""
    b = Block()
    b.put(raw(f"s_mov_b32 {g.S_M0}, m0"))
    b.put(raw(f"s_movk_i32 {g.S_H8K}, {hex(32 * ROWB8)}"))
    b.put(raw(f"s_mov_b32 {g.S_TOFF}, 0"))
    b.put(raw(f"s_mov_b32 {g.S_KV0}, 0"))
    # Q rows: per (h, cd) two 16-byte loads into v[0:31]
    for h in range(2):
        for cd in range(2):
            for part in range(2):
                i = 4 * (4 * h + 2 * cd + part)
                dst = f"v[{i}:{i + 3}]"
                soff = "0" if h == 0 else g.S_H8K
                b.put(Ins(f"buffer_load_dwordx4 {dst}, {{qoff}}, {{rq}}, {soff} offen offset:{cd * 64 + part * 16}",
                          "vmem", writes=regs(dst)))
    for stage in range(3):
        for ins in dma_issue8(stage):
            b.put(ins)
    for i in range(160):         # O: a[0:127]; row sums: a[160:191]
        b.put(Ins(f"v_accvgpr_write_b32 a{i if i < 128 else i + 32}, 0", "accw"))
    b.put(valu(f"v_mov_b32 {g.NEGINF}, 0xff800000", [], [g.NEGINF]))
    b.put(valu(f"v_mov_b32 {SC127}, 0x7f", [], [SC127]))
    for r in regs(ONES):
        b.put(valu(f"v_mov_b32 {r}, 0x38383838", [], [r]))
    b.put(valu(f"v_mbcnt_lo_u32_b32 {g.HALF4}, -1, 0", [], [g.HALF4]))
    b.put(valu(f"v_mbcnt_hi_u32_b32 {g.HALF4}, -1, {g.HALF4}", [g.HALF4], [g.HALF4]))
    b.put(valu(f"v_lshrrev_b32 {g.HALF4}, 5, {g.HALF4}", [g.HALF4], [g.HALF4]))
    b.put(valu(f"v_lshlrev_b32 {g.HALF4}, 2, {g.HALF4}", [g.HALF4], [g.HALF4]))
    for h in range(2):
        b.put(valu(f"v_sub_u32 {g.LIMH[h]}, {{lim{h}}}, {g.HALF4}", [g.HALF4], [g.LIMH[h]]))
        b.put(valu(f"v_mov_b32 {g.ALPHA[h]}, 1.0", [], [g.ALPHA[h]]))
    b.put(Ins(f"s_waitcnt vmcnt({3 * NPIECE8})", "wait"))   # Q, then tiles 0-2
    for i in range(32):
        b.put(valu(f"v_xor_b32 v{i}, {{qxor}}, v{i}", [f"v{i}"], [f"v{i}"]))
        b.put(valu(f"v_and_b32 v{i}, {{qand}}, v{i}", [f"v{i}"], [f"v{i}"]))
    for i in range(32):
        b.put(Ins(f"v_accvgpr_write_b32 a{128 + i}, v{i}", "accw", reads=[f"v{i}"]))
    b.pad(4)
    b.put(Ins(f"s_waitcnt vmcnt({2 * NPIECE8})", "wait"))   # tile 0
    b.put(Ins("s_barrier", "barrier"))
    ms, rd = s_mfmas8(0, 0)
    tail = []
    if masked_first:
        tail += g.mask_stream(0)
    tail += max_stream8(0, 0, first=True) + max_stream8(0, 1, first=True)
    schedule(b, ms, [Stream(tail, len(ms), "max")], rd)
    b.put(Ins(f"s_waitcnt vmcnt({NPIECE8}) lgkmcnt(0)", "wait"))
    b.put(Ins("s_barrier", "barrier"))
    b.lgkm = []
    for f in range(KSL8):
        for r in k_reads8(f, 1):
            b.put(r)
    return b


def drain8(parity):
    b = Block()
    b.lgkm = [set(regs(KF8(f))) for f in range(KSL8)]
    cur = parity % 2
    ms_pv, rd_pv = pv_mfmas8(parity % 4, 0, cur)
    schedule(b, ms_pv, [Stream(exp_stream8(cur), 0, "exp")], rd_pv)
    b.put(Ins("s_branch .Lepi", "branch"))
    return b


def epilogue8():
    """l of each row from its row-sum block (register 0) into the 16-bit epilogue's sum
    registers, then that epilogue with O scaled by V's descale (bf16 rows of 256 bytes)."""
    b = Block()
    b.put(Ins("s_waitcnt vmcnt(0) lgkmcnt(0)", "wait"))
    b.pad(24)                    # the last row-sum instructions have written their AGPRs
    for h in range(2):
        b.put(Ins(f"v_accvgpr_read_b32 {g.LRUN[h]}, a{160 + 16 * h}", "accr", writes=[g.LRUN[h]]))
        b.put(valu(f"v_mov_b32 {g.LACC0[h]}, 0", [], [g.LACC0[h]]))
    g.configure(128)             # bf16 output rows
    return b.text() + "\n" + g.epilogue("bf16", oscale="oscale").text()


def body8(causal):
    g.configure(128)
    parts = ["s_nop 7"]
    pm, pu = first_tile8(True), first_tile8(False)
    parts += ["s_cmp_eq_u32 {nmain}, 0", "s_cbranch_scc1 .Lpro_m", pu.text(),
              "s_branch .Lpro_done", ".Lpro_m:", pm.text(), ".Lpro_done:",
              f"s_mov_b32 {g.S_T}, 0", "s_branch .Ldisp"]
    parts += [".Lrescale:", rescale_block8().text(),
              ".Lnext:", f"s_add_u32 {g.S_T}, {g.S_T}, 1",
              ".Ldisp:",
              f"s_add_u32 {g.S_TMP}, {g.S_T}, 1",
              f"s_and_b32 {g.S_T2}, {g.S_T}, 3",
              "s_cmp_ge_u32 " + g.S_TMP + ", {ntiles}",
              "s_cbranch_scc1 .Ldd",
              "s_cmp_ge_u32 " + g.S_TMP + ", {nmain}",
              "s_cbranch_scc1 .Ldm"]
    for kind in ("u", "m", "d"):
        if kind != "u":
            parts.append(f".Ld{kind}:")
        for p in range(3):
            parts += [f"s_cmp_eq_u32 {g.S_T2}, {p}", f"s_cbranch_scc1 .L{kind}_{p}"]
        parts.append(f"s_branch .L{kind}_3")
    for p in range(4):
        parts += [f".Lu_{p}:", tile_step8(p, False).text()]
    for p in range(4):
        parts += [f".Lm_{p}:", tile_step8(p, True).text()]
        parts += [f".Ld_{p}:", drain8(p).text()]
    parts += [".Lepi:", epilogue8()]
    g.configure(128)
    return "\n".join(parts) + "\n"


OPERANDS8 = dict(g.OPERANDS, oscale="s")


def asm_text8(causal):
    t = body8(causal)
    t = re.sub(r"\{(\w+)\}", lambda m: "%[" + m.group(1) + "]", t)
    return t.replace(".L", ".Lf8%=_")
