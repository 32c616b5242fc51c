"""Generator of the 64-row-per-wave attention forward body for gfx950.

    python -m exact_io_aware_37_amd.csrc.gen_fwd_w64      (run by the build)

writes ``fa_fwd_w64.inc`` beside this file: one string constant per kernel
variant (bf16 / f16 inputs, causal or not, head dimension 64 or 128; and the
E4M3 variants of gen_fwd_w64_fp8.py) holding the
whole per-workgroup computation as gfx950 assembly, which the kernel in
``fa_fwd.hip`` runs in one inline-asm statement after computing addresses and
buffer descriptors in C++.

What the body computes is the recurrence of the course page "FlashAttention:
IO-aware attention kernel" (section 3.2: new row maximum, rescale the old sum
and accumulator by exp(m_old - m_new), add the tile's exponentials; divide by
the sum once at the end) inside the query-tile-outer, key-tile-inner loop of
its sections 2 and 3.3, for the 64 query rows of one wave, with the lazy
exponent reference of the 16-bit kernel (the reference moves only when the
row maximum passes it by more than 2^15; O / l and lse do not depend on where
it sits).

Why assembly.  A wave that owns 64 query rows reads every K and V fragment
from LDS once for two matrix instructions, half the LDS bytes per FLOP of the
32-row layout.  Its live state is O (128 registers), Q (64), two score tiles
(128): more than the 256 vector registers of a wave, so O and Q sit
in accumulation registers (AGPRs), which only the matrix instructions and
moves touch, while scores and probabilities stay in VGPRs for the vector
units.  The compiler picks one register form per function for every matrix
instruction and cannot express that split; here every register is assigned
by hand, and the matrix instructions, LDS reads, DMA transfers and vector
instructions of a tile are interleaved by the list scheduler below, which
also inserts the wait states gfx950 needs between dependent instructions
(the hardware does not check them for matrix results).  With one wave per
SIMD the wave's in-order issue is the bottleneck besides the matrix pipe:
the scheduler fills each matrix instruction's shadow by measured issue
costs and puts waits and LDS reads where they issue cheapest, right after
a matrix instruction.

Register map (per wave; one wave per SIMD, 512 registers):
  a[0:127]    O^T accumulators, block (h, db): a[16*(4h+db) : +16]
  a[128:191]  Q^T operand, (h, cd): a[128 + 4*(8h+cd) : +4]
  v[0:127]    two score buffers; buffer b, block (h, kt): v[64b + 16*(2h+kt) : +16];
              P of (h, kt, cc) is packed (two 16-bit values per register) in
              place over the first 4 of the 8 scores it is made from
  v[128:151]  K fragment ring (6 slots), v[152:175] V fragment ring (6 slots)
  v[176:229]  row statistics, row-sum selector and accumulators, temporaries
  v230..v255  left to the compiler for the statement's operands
h: which 32-row half of the wave's rows; kt: which 32 keys of a 64-key tile;
cd: which 16 head dimensions; db: which 32 output dimensions; cc: which 16
keys of a 32-key block.  Lane layouts are those of v_mfma_f32_32x32x16:
lane l of a 16-register accumulator holds column l % 32 and rows
8*(r/4) + 4*(l/32) + r%4 in register r.
"""

from __future__ import annotations

import os
import re
import sys

BC = 64
NSTAGE = 4
# The exponent reference of a row moves only when the row maximum passes it by more than
# 2^LAZY (log2 units), so probabilities stay <= 2^15: finite in f16 (largest 65504) and
# far from fp32 range in O and l.  Every move costs a pass over O (the rescale block);
# the larger headroom leaves it to rows whose maximum really jumps.
LAZY = 15
LAZY_HEX = "0x41700000"     # 15.0f
MFMA_CYCLES = 32            # v_mfma_f32_32x32x16: 8 passes of 4 cycles


def configure(d):
    """Head dimension d (128 or 64) and what follows from it; body() sets it."""
    global D, ROWB, KSTAGE, VRING, NCD, NDB, NPIECE
    assert d in (64, 128)
    D = d
    ROWB = 2 * D            # bytes of one K, V, Q or O row
    KSTAGE = BC * ROWB      # bytes of one K (or V) tile in LDS
    VRING = 4 * KSTAGE      # the V ring starts after the 4-stage K ring
    NCD = D // 16           # 16-dimension blocks of Q and K (the score contraction)
    NDB = D // 32           # 32-dimension blocks of O per 32-row half
    NPIECE = KSTAGE // 2048  # 1 KiB DMA pieces per wave and stage (two waves per tile)


configure(128)

# ----------------------------------------------------------------- registers


def O(h, db):
    b = 16 * (NDB * h + db)
    return f"a[{b}:{b + 15}]"


def Q(h, cd):
    b = 128 + 4 * (NCD * h + cd)
    return f"a[{b}:{b + 3}]"


def S(buf, h, kt):
    b = 64 * buf + 16 * (2 * h + kt)
    return f"v[{b}:{b + 15}]"


def s1(buf, h, kt, r):
    return f"v{64 * buf + 16 * (2 * h + kt) + r}"


def P(buf, h, kt, cc):
    """P of group (h, kt, cc), packed in place over the first 4 of its 8 scores."""
    b = 64 * buf + 16 * (2 * h + kt) + 8 * cc
    return f"v[{b}:{b + 3}]"


def p1(buf, h, kt, cc, w):
    return s1(buf, h, kt, 8 * cc + w)


KSLOTS = 6    # K fragment ring depth
VLEAD = 12    # V reads may start this many matrix instructions before their use
VSLOTS = 6    # V fragment ring depth


def KF(slot):
    b = 128 + 4 * slot
    return f"v[{b}:{b + 3}]"


def VF(slot):
    b = 128 + 4 * KSLOTS + 4 * slot
    return f"v[{b}:{b + 3}]"


def VFlo(slot):
    b = 128 + 4 * KSLOTS + 4 * slot
    return f"v[{b}:{b + 1}]"


def VFhi(slot):
    b = 130 + 4 * KSLOTS + 4 * slot
    return f"v[{b}:{b + 1}]"


MRUN = ["v176", "v177"]      # exponent reference per half (log2 units)
MX = ["v178", "v179"]        # tile row maximum
MXS = ["v180", "v181"]       # its partner-half copy
MNEW = ["v182", "v183"]
ALPHA = ["v184", "v185"]
TMP = ["v186", "v187"]
LIMR = ["v188", "v189"]      # mask limit relative to the tile's first key (+4*half)
LIMH = ["v190", "v191"]      # mask limit minus 4*half (per lane, per half)
NEGINF = "v192"
HALF4 = "v193"
LRUN = ["v194", "v195"]      # running row sum per half (both half-waves hold all of it)
SEL = "v[196:199]"           # 0/1 selector of the row-sum instruction
LACC = ["v[200:203]", "v[204:207]"]   # a tile's row sums per half (register 0; the others stay 0)
LACC0 = ["v200", "v204"]
RTMP = [f"v{208 + i}" for i in range(16)]   # rescale temporaries
ETMP = [f"v{i}" for i in range(64)]    # epilogue temporaries: score buffer 0, dead by then
EPI_DEPTH = 12               # epilogue: LDS reads of O rows in flight ahead of their stores

# SGPR temporaries (clobbered by the statement)
S_TOFF = "s72"       # byte offset of the tile being transferred (tile index * 16 KiB)
S_TOFF2 = "s73"      # S_TOFF + 4 KiB
S_T = "s74"          # index of the tile whose scores are being formed
S_KV0 = "s75"        # its first key
S_TMP = "s76"
S_M0 = "s77"         # saved M0
S_H8K = "s78"        # 8192 (row offset of the second query half)
S_T2 = "s79"         # tile index mod 4
MASKS = ["s[80:81]", "s[82:83]", "s[84:85]", "s[86:87]", "s[88:89]"]
S_ANY = "s[90:91]"
SGPR_CLOBBERS = [f"s{i}" for i in range(72, 92)]

# ---------------------------------------------------------------- instructions


class Ins:
    """One instruction with what the scheduler and the checker need to know.

    kind: 'mfma', 'valu', 'trans' (v_exp/v_log/v_rcp), 'lds', 'vmem', 'salu',
    'nop', 'wait', 'barrier', 'label', 'branch', 'cmp' (VALU writing an SGPR
    mask).  reads / writes: register names (single 32-bit registers)."""

    __slots__ = ("text", "kind", "reads", "writes", "cost", "srcab")

    def __init__(self, text, kind, reads=(), writes=(), cost=4, srcab=()):
        self.text = text
        self.kind = kind
        self.reads = tuple(reads)
        self.writes = tuple(writes)
        self.cost = cost
        self.srcab = tuple(srcab)


def regs(spec):
    """Expand 'v[4:7]' / 'a[0:15]' / 'v12' / 's[80:81]' into single registers."""
    out = []
    for part in spec if isinstance(spec, (list, tuple)) else [spec]:
        m = re.fullmatch(r"([vas])\[(\d+):(\d+)\]", part)
        if m:
            out += [f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)]
        elif re.fullmatch(r"[vas]\d+", part):
            out.append(part)
        elif part in ("vcc", "m0"):
            out.append(part)
    return out


def mfma(op, dst, a, b, c, cycles=MFMA_CYCLES):
    """A matrix instruction; `cost` holds the cycles it keeps the matrix pipe busy."""
    reads = regs(a) + regs(b) + (regs(c) if c != "0" else [])
    return Ins(f"{op} {dst}, {a}, {b}, {c}", "mfma", reads, regs(dst), cost=cycles,
               srcab=regs(a) + regs(b))


def valu(text, reads, writes, kind="valu", cost=4):
    return Ins(text, kind, regs(list(reads)), regs(list(writes)), cost)


def raw(text, kind="salu", cost=4, reads=(), writes=()):
    return Ins(text, kind, regs(list(reads)), regs(list(writes)), cost)


# --------------------------------------------------------------- the scheduler
#
# Wait states (instruction slots; s_nop N counts N + 1) required between a
# producer and a consumer, the rules the compiler applies on gfx950 (read
# off its own output for these instruction pairs):
#   matrix result (VGPR or AGPR)  -> vector read or accvgpr read : 12 (18 used)
#   vector write                  -> matrix operand read         : 2
#   transcendental result         -> vector read                 : 1
#   vector write of an SGPR mask  -> vector or scalar read        : 2 (4 used)
#   vector write                  -> v_permlane32_swap operand   : 2
#   SALU write of M0              -> LDS DMA                     : 1
# A matrix instruction's A/B operands are not rewritten within 8 slots of it.

WS_MFMA_VALU = 18
WS_MFMA8_VALU = 24   # the 64-cycle 8-bit 32x32x64 instruction writes its last results later
WS_VALU_MFMA = 2
WS_TRANS = 1
WS_MASK = 4
WS_PERM = 2
WS_WAR = 8
WS_WAR8 = 16


class Stream:
    def __init__(self, ins, start=0, name="", deadline=None):
        self.ins = list(ins)
        self.pos = 0
        self.start = start      # earliest matrix-instruction index after which it may run
        self.name = name
        self.deadline = deadline   # matrix-instruction index before which all of it has issued
        self.pace = 0              # > 0: instruction i not before matrix index start + pace * (i // 2)

    def ready_at(self, m):
        return self.start + self.pace * (self.pos // 2) <= m if self.pace else self.start <= m

    def done(self):
        return self.pos >= len(self.ins)

    def peek(self):
        return self.ins[self.pos]


class Block:
    """Linear instruction list with hazard-aware emission.

    Tracks, per register, the wait-state counter value from which a matrix
    consumer, a vector consumer or v_permlane32_swap may read it, and from
    which a vector instruction may overwrite a matrix A/B operand; pads with
    s_nop where needed and inserts s_waitcnt lgkmcnt for LDS results."""

    def __init__(self):
        self.out = []          # list of Ins
        self.slot = 0          # running wait-state counter
        self.rdy_m = {}        # reg -> first slot a matrix instruction may read it
        self.rdy_v = {}        # reg -> first slot a vector/scalar instruction may read it
        self.rdy_p = {}        # reg -> first slot v_permlane32_swap may read it
        self.war = {}          # reg -> first slot a vector write to it may issue
        self.m0 = 0            # first slot an LDS DMA may issue after an M0 write
        self.lgkm = []         # outstanding LDS reads: list of register sets, oldest first

    def need(self, ins):
        """Wait states still needed before `ins` may issue."""
        t = 0
        k = ins.kind
        for r in ins.reads:
            if k == "mfma":
                t = max(t, self.rdy_m.get(r, 0))
            elif k == "perm":
                t = max(t, self.rdy_v.get(r, 0), self.rdy_p.get(r, 0))
            else:
                t = max(t, self.rdy_v.get(r, 0))
        if k in ("valu", "trans", "cmp", "perm", "accw", "accr"):
            for r in ins.writes:
                t = max(t, self.war.get(r, 0))
        if k == "lds_dma":
            t = max(t, self.m0)
        return max(0, t - self.slot)

    def lds_pending(self, ins):
        rw = set(ins.reads) | set(ins.writes)
        return any(group & rw for group in self.lgkm)

    def waitcnt_for(self, ins):
        """Emit s_waitcnt lgkmcnt(n) so that every LDS read `ins` depends on has returned."""
        rw = set(ins.reads) | set(ins.writes)
        idx = -1
        for i, group in enumerate(self.lgkm):
            if group & rw:
                idx = i
        if idx >= 0:
            keep = len(self.lgkm) - idx - 1
            assert keep <= 15
            self._append(Ins(f"s_waitcnt lgkmcnt({keep})", "wait"))
            self.lgkm = self.lgkm[idx + 1:]

    def pad(self, n):
        while n > 0:
            k = min(n, 16)
            self._append(Ins(f"s_nop {k - 1}", "nop", cost=k))
            n -= k

    def _append(self, ins):
        self.out.append(ins)
        start = self.slot
        self.slot += int(ins.text.split()[1]) + 1 if ins.kind == "nop" else 1
        return start

    def put(self, ins):
        if ins.kind not in ("label", "branch", "wait", "barrier", "nop"):
            self.waitcnt_for(ins)
            self.pad(self.need(ins))
        start = self._append(ins)
        k = ins.kind
        if k == "wait" and "lgkmcnt(0)" in ins.text:
            self.lgkm = []
        for r in ins.writes:
            if k == "mfma":
                self.rdy_m[r] = start + 1                     # accumulation chains forward
                self.rdy_v[r] = start + 1 + (WS_MFMA_VALU if ins.cost <= 32 else WS_MFMA8_VALU)
            elif k == "trans":
                self.rdy_v[r] = start + 1 + WS_TRANS
                self.rdy_m[r] = start + 1 + WS_VALU_MFMA
                self.rdy_p[r] = start + 1 + WS_PERM
            elif k == "cmp":
                self.rdy_v[r] = start + 1 + WS_MASK
            elif k in ("valu", "perm", "accr"):
                self.rdy_v[r] = start + 1
                self.rdy_m[r] = start + 1 + WS_VALU_MFMA
                self.rdy_p[r] = start + 1 + WS_PERM
            elif k == "accw":
                self.rdy_m[r] = start + 1 + 4
                self.rdy_v[r] = start + 1 + 4
            elif k == "salu":
                self.rdy_v[r] = start + 1
            elif k in ("lds", "vmem"):
                pass
        if k == "salu" and "m0" in ins.writes:
            self.m0 = start + 2
        if k == "mfma":
            war = WS_WAR if ins.cost <= 32 else WS_WAR8
            for r in ins.srcab:
                self.war[r] = max(self.war.get(r, 0), start + 1 + war)
        if k == "lds":
            self.lgkm.append(set(ins.writes))
        return ins

    def text(self):
        return "\n".join(i.text for i in self.out)


# Issue costs of one wave's instruction stream (one wave per SIMD), measured on MI355X with
# register-only loops of v_mfma_f32_32x32x16_bf16 followed by the instructions in question:
# the wave issues in order, so the matrix pipe idles whenever the instructions between two
# matrix instructions take longer to issue than the first one takes to run.
ISSUE_MFMA = 8       # a matrix instruction; one scalar instruction right after it is free
COST_VALU = 4
COST_TRANS = 8       # v_exp_f32 and the other transcendentals
COST_SALU = 4        # s_waitcnt, s_add, s_nop 0 anywhere but right after a matrix instruction
COST_MEM = 7         # an LDS read or buffer load right after a matrix, scalar or memory instruction
COST_MEM_LATE = 16   # ... right after a vector instruction
DMA_PACE = 5         # the K/V transfers of a step: one piece per 5 matrix instructions at most
VECTOR_KINDS = ("valu", "trans", "cmp", "perm", "accr", "accw")


def issue_cost(ins, prev_kind, free_slot):
    k = ins.kind
    if k in ("salu", "wait"):
        return 0 if free_slot else COST_SALU
    if k in ("lds", "lds_dma", "vmem", "lds_w"):
        return COST_MEM_LATE if prev_kind in VECTOR_KINDS else COST_MEM
    if k == "trans":
        return COST_TRANS
    return COST_VALU


def issue_time(instructions):
    """Modelled cycles of a straight-line instruction list under the issue costs above:
    in-order issue, one matrix instruction at a time in the matrix pipe (its `cost`
    cycles); waits on memory and barriers are not modelled.  Returns (cycles, busy)."""
    t = mfree = busy = 0.0
    prev_kind, free_slot = "mfma", False
    for ins in instructions:
        k = ins.kind
        if k == "mfma":
            start = max(t, mfree)
            mfree = start + ins.cost
            busy += ins.cost
            t = start + ISSUE_MFMA
            prev_kind, free_slot = k, True
            continue
        if k == "nop":
            t += COST_SALU * (int(ins.text.split()[1]) + 1) - (COST_SALU if free_slot else 0)
        elif k in ("barrier", "label"):
            continue
        elif k == "branch":
            t += 0 if free_slot else COST_SALU
        else:
            t += issue_cost(ins, prev_kind, free_slot)
        prev_kind, free_slot = k, False
    return max(t, mfree), busy


def schedule(block, mfmas, streams, lds_plan, inserts=()):
    """Interleave `mfmas` (in order) with vector streams and LDS reads.

    lds_plan: list of (first consuming matrix index, matrix index from which
    the ring slot is free, [Ins ...]); `inserts`: (matrix index, [Ins])
    emitted right before that matrix instruction.  Right after each matrix
    instruction come, in this order: the s_waitcnt for the next matrix
    instruction's LDS operands (in the scalar slot that costs nothing there),
    the LDS reads that become due, and then ready stream instructions
    (streams in priority order, each in program order) until the issue
    cycles spent reach the matrix instruction's run time minus its own issue
    cycles.  A matrix instruction whose operands a stream still has to
    produce first pulls those producers in; a stream with a deadline is
    flushed before the matrix instruction of that index."""
    li = 0
    plan = sorted(lds_plan, key=lambda x: (x[1], x[0]))
    at = {}
    for idx, ins in inserts:
        at.setdefault(idx, []).extend(ins)
    for m, mi in enumerate(mfmas):
        while li < len(plan) and plan[li][1] <= m:
            for ins in plan[li][2]:
                block.put(ins)
            li += 1
        for st in streams:
            if st.deadline is not None and m >= st.deadline:
                while not st.done():
                    block.put(st.peek())
                    st.pos += 1
        for ins in at.get(m, []):
            block.put(ins)
        need = set(mi.reads)
        for st in streams:
            if st.start > m:
                continue          # not yet allowed to run: it produces nothing this one reads
            last = -1
            for i in range(st.pos, len(st.ins)):
                if set(st.ins[i].writes) & need:
                    last = i
            while st.pos <= last:
                block.put(st.peek())
                st.pos += 1
        block.put(mi)
        window = mi.cost - ISSUE_MFMA
        spent = 0
        prev_kind, free_slot = "mfma", True
        nxt = mfmas[m + 1] if m + 1 < len(mfmas) else None
        if nxt is not None and (m + 1) not in at and block.lds_pending(nxt):
            n0 = len(block.out)
            block.waitcnt_for(nxt)
            if len(block.out) > n0:
                prev_kind, free_slot = "wait", False
        while li < len(plan) and plan[li][1] <= m + 1 and (m + 1) not in at:
            for ins in plan[li][2]:
                spent += issue_cost(ins, prev_kind, free_slot)
                block.put(ins)
                prev_kind, free_slot = ins.kind, False
            li += 1
        progress = True
        while spent < window and progress:
            progress = False
            for st in streams:
                if st.done() or not st.ready_at(m):
                    continue
                ins = st.peek()
                if block.lds_pending(ins) or block.need(ins) > 0:
                    continue
                c = issue_cost(ins, prev_kind, free_slot)
                if spent + c > window and spent > 0:
                    continue
                block.put(ins)
                st.pos += 1
                spent += c
                prev_kind, free_slot = ins.kind, False
                progress = True
                break
    while li < len(plan):
        for ins in plan[li][2]:
            block.put(ins)
        li += 1
    for st in streams:
        while not st.done():
            block.put(st.peek())
            st.pos += 1


# --------------------------------------------------------------- tile pieces


def mfma_op(dt):
    return "v_mfma_f32_32x32x16_bf16" if dt == "bf16" else "v_mfma_f32_32x32x16_f16"


def cvt_op(dt):
    return "v_cvt_pk_bf16_f32" if dt == "bf16" else "v_cvt_pk_f16_f32"


def dot_op(dt):
    return ("v_dot2c_f32_bf16", "0x3f803f80") if dt == "bf16" else ("v_dot2c_f32_f16", "0x3c003c00")


def k_read(f, kstage):
    cd, kt = f // 2, f % 2
    off = kstage * KSTAGE + kt * (32 * ROWB)
    return Ins(f"ds_read_b128 {KF(f % KSLOTS)}, {{kaddr{cd}}} offset:{off}", "lds",
               reads=(), writes=regs(KF(f % KSLOTS)))


def s_mfmas_and_reads(dt, buf, kstage, skip=0):
    """Matrix instructions of S(buf) = K Q^T for the 64 rows, and the K reads.

    Fragment f = 2*cd + kt goes to ring slot f % KSLOTS; it feeds two matrix
    instructions (h = 0, 1)."""
    ms = []
    reads = []
    for cd in range(NCD):
        for kt in range(2):
            f = 2 * cd + kt
            off = kstage * KSTAGE + kt * (32 * ROWB)
            rd = k_read(f, kstage)
            # the ring slot is free once fragment f-KSLOTS's second matrix instruction has issued
            if f >= skip:
                reads.append((2 * f, 2 * (f - KSLOTS) + 2 if f >= KSLOTS else 0, [rd]))
            for h in range(2):
                c = "0" if cd == 0 else S(buf, h, kt)
                ms.append(mfma(mfma_op(dt), S(buf, h, kt), KF(f % KSLOTS), Q(h, cd), c))
    return ms, reads


def pv_mfmas_and_reads(dt, vstage, base_index, buf):
    """Matrix instructions of O += V^T P^T, then the row sums of P, and the V reads.

    Fragment g = NDB*(2*kt + cc) + db (two ds_read_b64_tr_b16 each) goes to ring
    slot g % VSLOTS and feeds h = 0, 1, one after the other."""
    ms = []
    uses = {}
    for kt in range(2):
        for cc in range(2):
            for (h, db) in [(h, db) for db in range(NDB) for h in range(2)]:
                g = NDB * (2 * kt + cc) + db
                uses.setdefault(g, []).append(base_index + len(ms))
                ms.append(mfma(mfma_op(dt), O(h, db), VF(g % VSLOTS), P(buf, h, kt, cc), O(h, db)))
    reads = []
    for g in range(4 * NDB):
        kt, cc, db = g // (2 * NDB), (g // NDB) % 2, g % NDB
        off = vstage * KSTAGE + (kt * 32 + cc * 16) * ROWB
        lo = Ins(f"ds_read_b64_tr_b16 {VFlo(g % VSLOTS)}, {{vaddr{db}}} offset:{off}", "lds",
                 writes=regs(VFlo(g % VSLOTS)))
        hi = Ins(f"ds_read_b64_tr_b16 {VFhi(g % VSLOTS)}, {{vaddr{db}}} offset:{off + 8 * ROWB}",
                 "lds", writes=regs(VFhi(g % VSLOTS)))
        free = max(uses[g - VSLOTS]) + 1 if g >= VSLOTS else 0
        reads.append((min(uses[g]), free, [lo, hi]))
    reads.sort(key=lambda r: r[0])
    # the row sums need P only: they run last, under the tile's barrier and transfers
    for kt in range(2):
        for cc in range(2):
            for h in range(2):
                ms.append(sum_mfma(dt, buf, h, kt, cc))
    return ms, reads


def exp_stream(dt, buf):
    """P(buf) = exp2(s * sl2 - m), rounded to the input type and packed as the P*V operand.

    Groups (h, kt, cc) in the order the P*V instructions consume them; within the
    stream the conversion of a pair of scores comes after the FMAs of the next
    pair, so that no instruction waits on the one issued right before it (a
    conversion reads two exponentials)."""
    units = []
    for kt in range(2):
        for cc in range(2):
            for h in range(2):
                for w in range(4):
                    a, b = s1(buf, h, kt, cc * 8 + 2 * w), s1(buf, h, kt, cc * 8 + 2 * w + 1)
                    f = [valu(f"v_fma_f32 {a}, {a}, {{sl2}}, -{MRUN[h]}", [a, MRUN[h]], [a]),
                         valu(f"v_fma_f32 {b}, {b}, {{sl2}}, -{MRUN[h]}", [b, MRUN[h]], [b])]
                    e = [valu(f"v_exp_f32 {a}, {a}", [a], [a], kind="trans", cost=8),
                         valu(f"v_exp_f32 {b}, {b}", [b], [b], kind="trans", cost=8)]
                    # packed in place over scores of the same group that earlier
                    # conversions (or this one) have consumed
                    p = p1(buf, h, kt, cc, w)
                    units.append((f, e, [valu(f"{cvt_op(dt)} {p}, {a}, {b}", [a, b], [p])]))
    ins = units[0][0] + units[0][1]
    for k in range(1, len(units)):
        ins += units[k][0] + units[k - 1][2] + units[k][1]
    return ins + units[-1][2]


def sum_mfma(dt, buf, h, kt, cc):
    """Row sums of the rounded P of group (h, kt, cc), added to LACC[h] on the matrix pipe.

    v_mfma_f32_16x16x32 reads the P operand with lane 16g + c as column c and
    k = 8g .. 8g+7: column c holds query c (g = 0, 2: the two half-waves) and
    query c + 16 (g = 1, 3).  The selector A is 1 at (row 0 or 8, g = 0 or 2)
    and (row 4 or 12, g = 1 or 3), so row 0 and 8 sum query c, rows 4 and 12
    query c + 16; register 0 of lane l is row 4 (l/16) (mod 16), column
    l % 16: the sum of query l % 32 in both half-waves.  Summing the rounded
    values makes O a convex combination of V rows with the weights used."""
    op = "v_mfma_f32_16x16x32_bf16" if dt == "bf16" else "v_mfma_f32_16x16x32_f16"
    c = "0" if (kt, cc) == (0, 0) else LACC[h]
    return mfma(op, LACC[h], SEL, P(buf, h, kt, cc), c, cycles=16)


def mask_stream(buf):
    """Scores of keys past the row's limit (tail, causal) -> -inf, both halves.

    One compare into a mask pair and one select per score; the compares run
    len(MASKS) - 1 ahead of their selects (rotating over the mask pairs), so
    that no select waits for the mask its compare wrote."""
    ins = [valu(f"v_sub_u32_e64 {LIMR[h]}, {LIMH[h]}, {S_KV0}", [LIMH[h]], [LIMR[h]]) for h in range(2)]
    pairs = []
    for h in range(2):
        for kt in range(2):
            for r in range(16):
                k = len(pairs)
                off = kt * 32 + (r >> 2) * 8 + (r & 3)
                m = MASKS[k % len(MASKS)]
                a = s1(buf, h, kt, r)
                pairs.append((valu(f"v_cmp_gt_i32 {m}, {off}, {LIMR[h]}", [LIMR[h]], [m], kind="cmp"),
                              valu(f"v_cndmask_b32 {a}, {a}, {NEGINF}, {m}", [a, NEGINF, m], [a])))
    lead = len(MASKS)
    for k in range(len(pairs) + lead):
        if k >= lead:
            ins.append(pairs[k - lead][1])
        if k < len(pairs):
            ins.append(pairs[k][0])
    return ins


def max_stream(buf, h, first=False):
    """New exponent reference of half h from S(buf); alpha moves the old sums to it."""
    vals = [s1(buf, h, kt, r) for kt in range(2) for r in range(16)]
    ins = [valu(f"v_max3_f32 {MX[h]}, {vals[0]}, {vals[1]}, {vals[2]}", vals[:3], [MX[h]])]
    rest = vals[3:]
    while rest:
        if len(rest) >= 2:
            ins.append(valu(f"v_max3_f32 {MX[h]}, {MX[h]}, {rest[0]}, {rest[1]}",
                            [MX[h], rest[0], rest[1]], [MX[h]]))
            rest = rest[2:]
        else:
            ins.append(valu(f"v_max_f32 {MX[h]}, {MX[h]}, {rest[0]}", [MX[h], rest[0]], [MX[h]]))
            rest = rest[1:]
    # combine the two half-waves (lanes l and l^32 hold the same query)
    ins.append(valu(f"v_mov_b32 {MXS[h]}, {MX[h]}", [MX[h]], [MXS[h]]))
    ins.append(Ins(f"v_permlane32_swap_b32 {MX[h]}, {MXS[h]}", "perm", regs([MX[h], MXS[h]]),
                   regs([MX[h], MXS[h]])))
    ins.append(valu(f"v_max_f32 {MX[h]}, {MX[h]}, {MXS[h]}", [MX[h], MXS[h]], [MX[h]]))
    ins.append(valu(f"v_mul_f32 {MX[h]}, {{sl2}}, {MX[h]}", [MX[h]], [MX[h]]))
    if first:
        # first tile: the reference is the tile maximum itself; nothing to rescale
        ins.append(valu(f"v_mov_b32 {MRUN[h]}, {MX[h]}", [MX[h]], [MRUN[h]]))
        return ins
    ins.append(valu(f"v_add_f32 {TMP[h]}, {LAZY_HEX}, {MRUN[h]}", [MRUN[h]], [TMP[h]]))
    m = MASKS[h]
    ins.append(valu(f"v_cmp_gt_f32 {m}, {MX[h]}, {TMP[h]}", [MX[h], TMP[h]], [m], kind="cmp"))
    ins.append(valu(f"v_cndmask_b32 {MNEW[h]}, {MRUN[h]}, {MX[h]}, {m}", [MRUN[h], MX[h], m],
                    [MNEW[h]]))
    ins.append(valu(f"v_sub_f32 {TMP[h]}, {MRUN[h]}, {MNEW[h]}", [MRUN[h], MNEW[h]], [TMP[h]]))
    ins.append(valu(f"v_exp_f32 {ALPHA[h]}, {TMP[h]}", [TMP[h]], [ALPHA[h]], kind="trans", cost=8))
    return ins


def dma_issue(stage):
    """The wave's share of a K/V tile (half of it) into ring stage `stage`: NPIECE x 1 KiB
    LDS DMA (8 at d = 128, 4 at d = 64).

    The tile's byte offset is S_TOFF (S_TOFF2 = S_TOFF + 4 KiB for the second
    four pieces); both advance by one tile after the issue."""
    ins = []
    for u in range(NPIECE):
        m0 = stage * KSTAGE + u * 1024
        ins.append(raw(f"s_add_u32 m0, {{dmabase}}, {m0}", "salu", writes=["m0"]))
        soff = S_TOFF if u < 4 else S_TOFF2
        ins.append(Ins(f"buffer_load_dwordx4 {{dmaoff{u % 4}}}, {{rdma}}, {soff} offen lds",
                       "lds_dma", cost=4))
    ins.append(raw(f"s_add_u32 {S_TOFF}, {S_TOFF}, {KSTAGE}"))
    ins.append(raw(f"s_add_u32 {S_TOFF2}, {S_TOFF2}, {KSTAGE}"))
    return ins


# ------------------------------------------------------------------ the body


def rescale_block():
    """O moves to the new reference (rare: lazy reference); then on to the next tile."""
    b = Block()
    b.pad(48)   # the last P*V products have written their AGPRs
    t = RTMP
    k = 0   # (RTMP)
    for h in range(2):
        for db in range(NDB):
            for r in range(16):
                a = 16 * (NDB * h + db) + r
                x = t[k % 16]
                b.out.append(Ins(f"v_accvgpr_read_b32 {x}, a{a}", "accr"))
                b.out.append(Ins(f"v_mul_f32 {x}, {x}, {ALPHA[h]}", "valu"))
                b.out.append(Ins(f"v_accvgpr_write_b32 a{a}, {x}", "accw"))
                k += 1
    b.pad(8)
    return b


def prefetch_k(b, kstage):
    """The first KSLOTS K fragment reads of the next tile's scores."""
    for f in range(KSLOTS):
        b.put(k_read(f, kstage))


def fold_stream():
    """l = (l + the previous tile's sums) * alpha, both against the reference of this tile.

    Runs early in a step, long after the previous tile's row-sum
    instructions, and before this step's new alpha is formed."""
    ins = []
    for h in range(2):
        ins.append(valu(f"v_add_f32 {LRUN[h]}, {LRUN[h]}, {LACC0[h]}", [LRUN[h], LACC0[h]], [LRUN[h]]))
        ins.append(valu(f"v_mul_f32 {LRUN[h]}, {LRUN[h]}, {ALPHA[h]}", [LRUN[h], ALPHA[h]], [LRUN[h]]))
    return ins


def tile_step(dt, j_parity, masked, causal, uid):
    """Steady step j: S(j+1) || exp S(j), then P(j)V(j) || max S(j+1), then row sums of P(j).

    During the S phase this wave sends its share of tile j+3 into ring stage
    (j+3) % 4 = (j-1) % 4, which every wave finished reading before the
    previous step's barrier.  The first 4 K reads of S(j+1) were issued at the
    end of the previous step.  Inside the P*V phase, once this wave's last V(j)
    read has returned: wait for this wave's share of tile j+2, barrier (every
    wave's share has landed and every wave is done with V(j)), then the first
    K reads of S(j+2); the last matrix instructions of the tile (the row
    sums) run while other waves reach the barrier.
    j_parity = j % 4 selects the ring stages and score buffers."""
    kst = (j_parity + 1) % 4
    vst = j_parity % 4
    cur, nxt = j_parity % 2, (j_parity + 1) % 2
    b = Block()
    b.lgkm = [set(regs(KF(f))) for f in range(KSLOTS)]
    ms_s, rd_s = s_mfmas_and_reads(dt, nxt, kst, skip=KSLOTS)
    ms_pv, rd_pv = pv_mfmas_and_reads(dt, vst, len(ms_s), cur)
    lds_plan = list(rd_s)
    for (use, free, ins) in rd_pv:
        lds_plan.append((use, max(free, use - VLEAD), ins))
    # the sync point: the matrix instruction that first uses the last V fragment
    # (so every V(j) read of this wave has been issued; the wait returns them)
    sync_at = rd_pv[-1][0]
    sync = [Ins(f"s_waitcnt vmcnt({NPIECE}) lgkmcnt(0)", "wait"), Ins("s_barrier", "barrier")]
    nextk = [k_read(f, (j_parity + 2) % 4) for f in range(KSLOTS)]
    # priority order: the next tile's first K reads, the K/V transfers (paced, all issued
    # before the sync), the exponentials, the running sum, the row maximum of S(j+1)
    dma = Stream(dma_issue((j_parity + 3) % 4), 2, "dma", deadline=sync_at)
    dma.pace = DMA_PACE
    streams = [
        Stream(nextk, sync_at, "nextk"),
        dma,
        Stream(exp_stream(dt, cur), 0, "exp"),
        Stream(fold_stream(), 8, "fold"),
    ]
    tail = []
    if masked:
        tail += [raw(f"s_add_u32 {S_KV0}, {S_KV0}, {BC}")]
        tail += mask_stream(nxt)
    tail += max_stream(nxt, 0) + max_stream(nxt, 1)
    # does any lane's reference move (O must then be rescaled before the next P*V)?
    tail.append(valu(f"v_cmp_neq_f32 vcc, 1.0, {ALPHA[0]}", [ALPHA[0]], ["vcc"], kind="cmp"))
    tail.append(valu(f"v_cmp_neq_f32 {S_ANY}, 1.0, {ALPHA[1]}", [ALPHA[1]], [S_ANY], kind="cmp"))
    streams.append(Stream(tail, len(ms_s), "max"))
    schedule(b, ms_s + ms_pv, streams, lds_plan, inserts=[(sync_at, sync)])
    if not masked:
        b.put(raw(f"s_add_u32 {S_KV0}, {S_KV0}, {BC}"))
    # the new reference (only now: the exponentials of S(j) above read the old one)
    for h in range(2):
        b.put(valu(f"v_mov_b32 {MRUN[h]}, {MNEW[h]}", [MNEW[h]], [MRUN[h]]))
    b.put(raw(f"s_or_b64 vcc, vcc, {S_ANY}", reads=["vcc", S_ANY], writes=["vcc"]))
    b.put(raw("s_cbranch_vccnz .Lrescale", "branch"))
    b.put(raw(f"s_add_u32 {S_T}, {S_T}, 1"))
    if masked:
        b.put(raw("s_branch .Ldisp", "branch"))
    else:
        # fast path: the next step is unmasked too -> straight on (blocks u_0..u_3 are laid out in order)
        b.put(raw(f"s_add_u32 {S_TMP}, {S_T}, 1"))
        b.put(raw(f"s_cmp_lt_u32 {S_TMP}, {{nmain}}"))
        b.put(raw("s_cbranch_scc0 .Ldisp", "branch"))
        if j_parity == 3:
            b.put(raw("s_branch .Lu_0", "branch"))
    return b


def first_tile(dt, masked_first):
    """Prologue: Q to AGPRs, zero O, DMA tiles 0-2, S(0) and its reference."""
    b = Block()
    b.put(raw(f"s_mov_b32 {S_M0}, m0"))
    b.put(raw(f"s_movk_i32 {S_H8K}, {hex(32 * ROWB)}"))
    b.put(raw(f"s_mov_b32 {S_TOFF}, 0"))
    b.put(raw(f"s_movk_i32 {S_TOFF2}, 0x1000"))
    b.put(raw(f"s_mov_b32 {S_KV0}, 0"))
    # Q rows: 2*NCD loads of 16 bytes per lane into v[0:8*NCD-1], then to AGPRs
    for h in range(2):
        for cd in range(NCD):
            dst = f"v[{4 * (NCD * h + cd)}:{4 * (NCD * h + cd) + 3}]"
            soff = "0" if h == 0 else S_H8K
            b.put(Ins(f"buffer_load_dwordx4 {dst}, {{qoff}}, {{rq}}, {soff} offen offset:{cd * 32}",
                      "vmem", writes=regs(dst)))
    for stage in range(3):
        for ins in dma_issue(stage):
            b.put(ins)
    # O = 0 while the loads are in flight
    for i in range(32 * NDB):
        b.put(Ins(f"v_accvgpr_write_b32 a{i}, 0", "accw"))
    b.put(valu(f"v_mov_b32 {NEGINF}, 0xff800000", [], [NEGINF]))
    for r in regs(SEL):
        b.put(valu(f"v_mov_b32 {r}, {{selv}}", [], [r]))
    b.put(valu(f"v_mbcnt_lo_u32_b32 {HALF4}, -1, 0", [], [HALF4]))
    b.put(valu(f"v_mbcnt_hi_u32_b32 {HALF4}, -1, {HALF4}", [HALF4], [HALF4]))
    b.put(valu(f"v_lshrrev_b32 {HALF4}, 5, {HALF4}", [HALF4], [HALF4]))
    b.put(valu(f"v_lshlrev_b32 {HALF4}, 2, {HALF4}", [HALF4], [HALF4]))
    for h in range(2):
        b.put(valu(f"v_sub_u32 {LIMH[h]}, {{lim{h}}}, {HALF4}", [HALF4], [LIMH[h]]))
        for r in regs(LACC[h]) + [LRUN[h]]:
            b.put(valu(f"v_mov_b32 {r}, 0", [], [r]))
        b.put(valu(f"v_mov_b32 {ALPHA[h]}, 1.0", [], [ALPHA[h]]))
    b.put(Ins(f"s_waitcnt vmcnt({3 * NPIECE})", "wait"))   # Q, then tiles 0-2
    for i in range(8 * NCD):
        b.put(valu(f"v_xor_b32 v{i}, {{qxor}}, v{i}", [f"v{i}"], [f"v{i}"]))
        b.put(valu(f"v_and_b32 v{i}, {{qand}}, v{i}", [f"v{i}"], [f"v{i}"]))
    for i in range(8 * NCD):
        b.put(Ins(f"v_accvgpr_write_b32 a{128 + i}, v{i}", "accw", reads=[f"v{i}"]))
    b.pad(4)
    b.put(Ins(f"s_waitcnt vmcnt({2 * NPIECE})", "wait"))   # tile 0
    b.put(Ins("s_barrier", "barrier"))
    ms, rd = s_mfmas_and_reads(dt, 0, 0)
    tail = []
    if masked_first:
        tail += mask_stream(0)
    tail += max_stream(0, 0, first=True) + max_stream(0, 1, first=True)
    schedule(b, ms, [Stream(tail, len(ms), "max")], rd)
    # tile 1 visible to every wave, then the first K reads of S(1)
    b.put(Ins(f"s_waitcnt vmcnt({NPIECE}) lgkmcnt(0)", "wait"))
    b.put(Ins("s_barrier", "barrier"))
    b.lgkm = []
    prefetch_k(b, 1)
    return b


def drain(dt, parity):
    """Last tile T-1 (T-1 % 4 == parity): exp S(T-1), then P V with nothing left to overlap."""
    b = Block()
    b.lgkm = [set(regs(KF(f))) for f in range(KSLOTS)]   # the K reads issued for a next tile
    cur = parity % 2
    ms_pv, rd_pv = pv_mfmas_and_reads(dt, parity % 4, 0, cur)
    schedule(b, ms_pv, [Stream(fold_stream(), 0, "fold"),
                        Stream(exp_stream(dt, cur), 0, "exp")],
             rd_pv)
    b.put(Ins("s_branch .Lepi", "branch"))
    return b


def epilogue(dt, oscale=None):
    """O / l through LDS to whole-row stores; lse = (m + log2 l) ln 2.  With `oscale` (an
    SGPR operand name) O is multiplied by it as well."""
    b = Block()
    b.put(Ins("s_waitcnt vmcnt(0) lgkmcnt(0)", "wait"))
    b.put(Ins("s_barrier", "barrier"))   # every wave is done with the ring
    t = ETMP
    for h in range(2):
        # l of the row (both half-waves hold the whole sum), the last tile's sums added
        lr = LRUN[h]
        if h == 0:
            b.pad(18)
        b.put(valu(f"v_add_f32 {lr}, {lr}, {LACC0[h]}", [lr, LACC0[h]], [lr]))
        b.put(valu(f"v_rcp_f32 {ALPHA[h]}, {lr}", [lr], [ALPHA[h]], kind="trans"))
        if oscale is not None:
            b.put(valu(f"v_mul_f32 {ALPHA[h]}, {{{oscale}}}, {ALPHA[h]}", [ALPHA[h]], [ALPHA[h]]))
        b.put(valu(f"v_log_f32 {TMP[h]}, {lr}", [lr], [TMP[h]], kind="trans"))
        b.put(valu(f"v_add_f32 {TMP[h]}, {MRUN[h]}, {TMP[h]}", [MRUN[h], TMP[h]], [TMP[h]]))
        b.put(valu(f"v_mul_f32 {TMP[h]}, 0x3f317218, {TMP[h]}", [TMP[h]], [TMP[h]]))
        b.put(Ins(f"buffer_store_dword {TMP[h]}, {{lseoff}}, {{rl}}, 0 offen offset:{h * 128}",
                  "vmem", reads=[TMP[h]]))
    # the wave's O tile (64 rows x ROWB bytes) into its own 64*ROWB bytes of LDS, row-swizzled
    # lane (l32, half) of block (h, db) holds row 32h + l32, columns db*32 + 8g + 4*half + (0..3)
    # byte address: row*ROWB + ((chunk ^ sw(row)) * 16) + half*8, chunk = 4*db + g, where
    # sw(row) = row & 15 with 16 chunks per row (d = 128), (row >> 1) & 7 with 8 (d = 64)
    lg_rowb = ROWB.bit_length() - 1
    nch = ROWB // 16

    def swizzle(dst, row):
        if nch == 16:
            b.put(valu(f"v_and_b32 {dst}, 15, {row}", [row], [dst]))
        else:
            b.put(valu(f"v_lshrrev_b32 {dst}, 1, {row}", [row], [dst]))
            b.put(valu(f"v_and_b32 {dst}, 7, {dst}", [dst], [dst]))
    b.put(valu(f"v_mbcnt_lo_u32_b32 {t[16]}, -1, 0", [], [t[16]]))
    b.put(valu(f"v_mbcnt_hi_u32_b32 {t[16]}, -1, {t[16]}", [t[16]], [t[16]]))
    b.put(valu(f"v_and_b32 {t[17]}, 31, {t[16]}", [t[16]], [t[17]]))           # l32
    b.pad(18)
    for h in range(2):
        # row = 32h + l32 -> sw(row) = sw(l32); base = lds + row*ROWB + half*8
        b.put(valu(f"v_lshlrev_b32 {t[14]}, {lg_rowb}, {t[17]}", [t[17]], [t[14]]))  # l32*ROWB
        b.put(valu(f"v_add_u32 {t[14]}, {{obase}}, {t[14]}", [t[14]], [t[14]]))
        b.put(valu(f"v_add_u32 {t[14]}, {h * 32 * ROWB}, {t[14]}", [t[14]], [t[14]]))
        b.put(valu(f"v_lshrrev_b32 {t[15]}, 2, {HALF4}", [HALF4], [t[15]]))      # half
        b.put(valu(f"v_lshlrev_b32 {t[15]}, 3, {t[15]}", [t[15]], [t[15]]))      # half*8
        b.put(valu(f"v_add_u32 {t[14]}, {t[14]}, {t[15]}", [t[14], t[15]], [t[14]]))
        swizzle(t[13], t[17])
        for db in range(NDB):
            for g in range(4):
                base = 16 * (NDB * h + db) + 4 * g
                x = [t[(4 * (db * 4 + g) + i) % 12] for i in range(4)]
                for i in range(4):
                    b.put(Ins(f"v_accvgpr_read_b32 {x[i]}, a{base + i}", "accr", writes=[x[i]]))
                for i in range(4):
                    b.put(valu(f"v_mul_f32 {x[i]}, {x[i]}, {ALPHA[h]}", [x[i], ALPHA[h]], [x[i]]))
                b.put(valu(f"{cvt_op(dt)} {x[0]}, {x[0]}, {x[1]}", [x[0], x[1]], [x[0]]))
                b.put(valu(f"{cvt_op(dt)} {x[1]}, {x[2]}, {x[3]}", [x[2], x[3]], [x[1]]))
                # address: base + ((4db+g) ^ sw(row)) * 16
                b.put(valu(f"v_xor_b32 {t[12]}, {4 * db + g}, {t[13]}", [t[13]], [t[12]]))
                b.put(valu(f"v_lshl_add_u32 {t[12]}, {t[12]}, 4, {t[14]}", [t[12], t[14]], [t[12]]))
                b.put(Ins(f"ds_write_b64 {t[12]}, v[{x[0][1:]}:{int(x[0][1:]) + 1}]", "lds_w",
                          reads=[t[12], x[0], x[1]]))
    b.put(Ins("s_waitcnt lgkmcnt(0)", "wait"))
    b.lgkm = []
    # read back whole rows: read i covers rows rpr*i .. rpr*i + rpr-1, lane -> row
    # rpr*i + lane / nch, logical chunk lane % nch at physical chunk (lane % nch) ^ sw(row).
    # sw(row) repeats every 16 rows, i.e. every `per` reads, so `per` base addresses serve
    # all reads (the rest is the instruction's offset).  The reads go to score buffer 1
    # (dead here), one register quad each, EPI_DEPTH in flight ahead of the stores.
    rpr = 64 // nch
    per = 16 // rpr
    nread = 64 // rpr
    b.put(valu(f"v_lshrrev_b32 {t[15]}, {nch.bit_length() - 1}, {t[16]}", [t[16]], [t[15]]))
    b.put(valu(f"v_and_b32 {t[13]}, {nch - 1}, {t[16]}", [t[16]], [t[13]]))
    bases = [t[18 + k] for k in range(per)]
    for k in range(per):
        b.put(valu(f"v_add_u32 {t[12]}, {rpr * k}, {t[15]}", [t[15]], [t[12]]))    # row
        swizzle(t[14], t[12])
        b.put(valu(f"v_xor_b32 {t[14]}, {t[14]}, {t[13]}", [t[14], t[13]], [t[14]]))
        b.put(valu(f"v_lshlrev_b32 {t[12]}, {lg_rowb}, {t[12]}", [t[12]], [t[12]]))
        b.put(valu(f"v_lshl_add_u32 {t[12]}, {t[14]}, 4, {t[12]}", [t[12], t[14]], [t[12]]))
        b.put(valu(f"v_add_u32 {bases[k]}, {{obase}}, {t[12]}", [t[12]], [bases[k]]))

    def y(i):
        return f"v[{64 + 4 * i}:{64 + 4 * i + 3}]"

    def store(i):
        if i > 0:
            b.put(raw(f"s_mov_b32 {S_TMP}, {(rpr * i) * ROWB}"))
        b.put(Ins(f"buffer_store_dwordx4 {y(i)}, {{ooff}}, {{ro}}, 0 offen offset:0" if i == 0 else
                  f"buffer_store_dwordx4 {y(i)}, {{ooff}}, {{ro}}, {S_TMP} offen", "vmem",
                  reads=regs(y(i))))
    for i in range(nread):
        b.put(Ins(f"ds_read_b128 {y(i)}, {bases[i % per]} offset:{(i // per) * 16 * ROWB}", "lds",
                  reads=[bases[i % per]], writes=regs(y(i))))
        if i >= EPI_DEPTH - 1:
            store(i - EPI_DEPTH + 1)
    for i in range(max(0, nread - EPI_DEPTH + 1), nread):
        store(i)
    b.put(raw(f"s_mov_b32 m0, {S_M0}"))
    return b


def body(dt, causal, d=128):
    """The whole per-workgroup asm body (head dimension d) as text with {operand} placeholders.

    Control flow: prologue (tile 0), then one block per tile j chosen by the
    dispatcher from j % 4 (ring stages, score buffer) and from whether tile
    j + 1 needs a mask or does not exist (then the drain of tile j), then the
    epilogue."""
    configure(d)
    try:
        return _body(dt, causal)
    finally:
        configure(128)


def _body(dt, causal):
    # s_nop: wait states for any vector write of an operand (SGPR or VGPR) made
    # by the compiled code just before the statement
    parts = ["s_nop 7"]
    pm = first_tile(dt, True)
    pu = first_tile(dt, False)
    parts += ["s_cmp_eq_u32 {nmain}, 0", "s_cbranch_scc1 .Lpro_m", pu.text(),
              "s_branch .Lpro_done", ".Lpro_m:", pm.text(), ".Lpro_done:",
              f"s_mov_b32 {S_T}, 0", "s_branch .Ldisp"]
    parts += [".Lrescale:", rescale_block().text(),
              ".Lnext:", f"s_add_u32 {S_T}, {S_T}, 1",
              ".Ldisp:",
              f"s_add_u32 {S_TMP}, {S_T}, 1",
              f"s_and_b32 {S_T2}, {S_T}, 3",
              f"s_cmp_ge_u32 {S_TMP}, {{ntiles}}",
              "s_cbranch_scc1 .Ldd",
              f"s_cmp_ge_u32 {S_TMP}, {{nmain}}",
              "s_cbranch_scc1 .Ldm"]
    for kind in ("u", "m", "d"):
        if kind != "u":
            parts.append(f".Ld{kind}:")
        for p in range(3):
            parts += [f"s_cmp_eq_u32 {S_T2}, {p}", f"s_cbranch_scc1 .L{kind}_{p}"]
        parts.append(f"s_branch .L{kind}_3")
    for p in range(4):
        parts += [f".Lu_{p}:", tile_step(dt, p, False, causal, f"u_{p}").text()]
    for p in range(4):
        parts += [f".Lm_{p}:", tile_step(dt, p, True, causal, f"m_{p}").text()]
        parts += [f".Ld_{p}:", drain(dt, p).text()]
    parts += [".Lepi:", epilogue(dt).text()]
    return "\n".join(parts) + "\n"


OPERANDS = {
    # name: (constraint, C++ expression supplied by the kernel)
    "rq": "s", "rdma": "s", "ro": "s", "rl": "s",
    "dmabase": "s", "sl2": "s", "qxor": "s", "qand": "s", "ntiles": "s", "nmain": "s",
    "obase": "s",
    "kaddr0": "v", "kaddr1": "v", "kaddr2": "v", "kaddr3": "v",
    "kaddr4": "v", "kaddr5": "v", "kaddr6": "v", "kaddr7": "v",
    "vaddr0": "v", "vaddr1": "v", "vaddr2": "v", "vaddr3": "v",
    "dmaoff0": "v", "dmaoff1": "v", "dmaoff2": "v", "dmaoff3": "v",
    "qoff": "v", "lim0": "v", "lim1": "v", "ooff": "v", "lseoff": "v", "selv": "v",
}


def asm_text(dt, causal, d=128):
    """Body with placeholders turned into named inline-asm operands, labels made unique."""
    t = body(dt, causal, d)
    t = re.sub(r"\{(\w+)\}", lambda m: "%[" + m.group(1) + "]", t)
    t = t.replace(".L", ".Lfw%=_")
    return t


def clobbers():
    c = [f"v{i}" for i in range(230)] + [f"a{i}" for i in range(256)]
    return c + SGPR_CLOBBERS + ["vcc", "scc", "memory"]


def c_macro(name, text):
    lines = [l for l in text.split("\n") if l]
    body = " \\\n".join('  "' + l.replace("\\", "\\\\").replace('"', '\\"') + '\\n"'
                          for l in lines)
    return f"#define {name} \\\n{body}\n"


def write_inc(path=None):
    """Write the asm bodies as string-literal macros (inline asm needs a literal)."""
    path = path or os.path.join(os.path.dirname(os.path.abspath(__file__)), "fa_fwd_w64.inc")
    out = ["// Generated by gen_fwd_w64.py (run by the library build): do not edit.", ""]
    for d in (128, 64):
        for dt in ("bf16", "f16"):
            for causal in (False, True):
                name = f"FA_W64{'' if d == 128 else 'D64'}_{dt.upper()}_{'CAUSAL' if causal else 'FULL'}"
                out.append(c_macro(name, asm_text(dt, causal, d)))
    here = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, here)
    try:
        import gen_fwd_w64_fp8
    finally:
        sys.path.remove(here)
    for causal in (False, True):
        name = f"FA_W64_E4M3_{'CAUSAL' if causal else 'FULL'}"
        out.append(c_macro(name, gen_fwd_w64_fp8.asm_text8(causal)))
    out.append("#define FA_W64_CLOBBERS " + ", ".join(f'"{c}"' for c in clobbers()))
    out.append("")
    text = "\n".join(out)
    old = open(path).read() if os.path.exists(path) else None
    if old != text:
        with open(path, "w") as f:
            f.write(text)
    return path


if __name__ == "__main__":
    print(write_inc(sys.argv[1] if len(sys.argv) > 1 else None))
