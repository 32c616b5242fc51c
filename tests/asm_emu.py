"""A functional emulator for the gfx950 instruction subset of the 64-row
forward body (exact_io_aware_37_amd/csrc/gen_fwd_w64.py), for CPU tests.

It runs the generated text for one workgroup: 4 waves of 64 lanes with their
VGPR, AGPR and SGPR files, the workgroup's LDS, raw buffers with bounds
checks, and s_barrier.  Beyond executing the instructions it checks what the
hardware would not report: a register read while an LDS or memory load into
it is still outstanding (a missing s_waitcnt), an LDS read of bytes a DMA
transfer has not been waited for, and LDS accesses outside the allocation.
Timing is not modelled (wait states are checked by the generator itself).

Matrix-instruction semantics (v_mfma_f32_32x32x16_{bf16,f16}, D = A B + C):
lane l holds A[l % 32][8*(l/32) + e] and B[8*(l/32) + e][l % 32] for e = 0..7
(two 16-bit values per register, low half first), and D[8*(r/4) + 4*(l/32) +
r % 4][l % 32] in accumulator register r.  ds_read_b64_tr_b16: within each
group of 16 lanes, result lane r gets element e (e = 0..3) from element
r % 4 of what lane 4e + r/4 addressed.  Both are the layouts the 16-bit
kernel of fa_fwd.hip relies on.
"""

from __future__ import annotations

import re

import numpy as np

L = 64


class EmuError(RuntimeError):
    pass


def bf16_bits(x):
    """float32 array -> bf16 bit patterns, round to nearest even."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    out = ((u + r) >> 16).astype(np.uint32)
    nan = np.isnan(np.asarray(x, np.float32))
    out[nan] = 0x7FC0
    return out & 0xFFFF


def bf16_val(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def f16_bits(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)


def f16_val(bits):
    return np.asarray(bits, np.uint16).astype(np.uint16).view(np.float16).astype(np.float32)


def e4m3_values():
    """The 256 OCP E4M3 codes as float64 (bias 7, subnormals below 2^-6, 0x7f / 0xff NaN)."""
    out = np.zeros(256, np.float64)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        out[c] = np.nan if (c & 0x7F) == 0x7F else (-v if s else v)
    return out


E4M3 = e4m3_values()
_E4M3_POS = E4M3[:0x7F]                      # codes 0 .. 126, increasing


def e4m3_bits(x):
    """float32 -> E4M3 codes, round to nearest, ties to the even code; |x| above 448
    saturates (the kernel never converts such values)."""
    x = np.asarray(x, np.float64)
    ax = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_E4M3_POS, ax, side="left").clip(0, 126)
    lo = (hi - 1).clip(0, 126)
    dlo, dhi = ax - _E4M3_POS[lo], _E4M3_POS[hi] - ax
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(ax == _E4M3_POS[hi], hi, pick)
    return (pick | np.where(x < 0, 0x80, 0)).astype(np.uint32)


def f32(u):
    return np.asarray(u, np.uint32).view(np.float32)


def u32(f):
    return np.asarray(f, np.float32).view(np.uint32)


class Wave:
    def __init__(self, wid):
        self.wid = wid
        self.v = np.zeros((256, L), np.uint32)
        self.a = np.zeros((256, L), np.uint32)
        self.s = np.zeros(108, np.uint64)
        self.vcc = 0
        self.m0 = 0
        self.scc = 0
        self.pc = 0
        self.done = False
        self.pend_lgkm = []     # list of sets of ('v', i)
        self.pend_vm = []       # list of ('regs', set) or ('lds', lo, hi)


def parse_reg(tok):
    m = re.fullmatch(r"([vas])\[(\d+):(\d+)\]", tok)
    if m:
        return m.group(1), int(m.group(2)), int(m.group(3)) - int(m.group(2)) + 1
    m = re.fullmatch(r"([vas])(\d+)", tok)
    if m:
        return m.group(1), int(m.group(2)), 1
    return None


class Emu:
    def __init__(self, text, buffers, lds_bytes=160 * 1024, order=None):
        self.lines = []
        self.labels = {}
        self.executed = {}     # line index -> times executed (all waves)
        for raw in text.split("\n"):
            line = raw.split(";")[0].strip()
            if not line:
                continue
            if line.endswith(":"):
                self.labels[line[:-1]] = len(self.lines)
                continue
            self.lines.append(line)
        self.buffers = buffers          # id -> np.uint8 array
        self.lds = np.zeros(lds_bytes, np.uint8)
        self.lds_pend = np.zeros(lds_bytes, np.int16) - 1   # wave id with an outstanding DMA
        self.waves = [Wave(i) for i in range(4)]
        self.order = order or [0, 1, 2, 3]
        self.count = 0

    # -------------------------------------------------------------- operands
    def _check_pending(self, w, f, i, n):
        if f != "v":
            return
        for grp in w.pend_lgkm:
            for k in range(i, i + n):
                if ("v", k) in grp:
                    raise EmuError(f"wave {w.wid}: v{k} read before its LDS load was waited for "
                                   f"(line {w.pc}: {self.lines[w.pc]})")
        for item in w.pend_vm:
            if item[0] == "regs":
                for k in range(i, i + n):
                    if ("v", k) in item[1]:
                        raise EmuError(f"wave {w.wid}: v{k} read before its memory load was waited "
                                       f"for (line {w.pc}: {self.lines[w.pc]})")

    def vread(self, w, tok, k=0):
        """32-bit per-lane value of operand token (register k of a range)."""
        neg = False
        if tok.startswith("-") and not re.fullmatch(r"-\d+", tok):
            neg, tok = True, tok[1:]
        r = parse_reg(tok)
        if r:
            f, i, n = r
            self._check_pending(w, f, i + k, 1)
            if f == "v":
                val = w.v[i + k].copy()
            elif f == "a":
                val = w.a[i + k].copy()
            else:
                val = np.full(L, w.s[i + k] & 0xFFFFFFFF, np.uint32)
        elif tok == "vcc":
            val = np.full(L, w.vcc & 0xFFFFFFFF, np.uint32)
        elif tok == "m0":
            val = np.full(L, w.m0, np.uint32)
        else:
            val = np.full(L, self.const(tok), np.uint32)
        if neg:
            val = u32(-f32(val))
        return val

    def const(self, tok):
        if tok.startswith("0x"):
            return int(tok, 16) & 0xFFFFFFFF
        if re.fullmatch(r"-?\d+", tok):
            return int(tok) & 0xFFFFFFFF
        if re.fullmatch(r"-?\d+\.\d+", tok):
            return int(np.float32(float(tok)).view(np.uint32))
        raise EmuError(f"bad operand {tok}")

    def sread(self, w, tok):
        r = parse_reg(tok)
        if r:
            return int(w.s[r[1]]) & 0xFFFFFFFF
        if tok == "m0":
            return w.m0
        return self.const(tok)

    def sread64(self, w, tok):
        if tok == "vcc":
            return w.vcc
        r = parse_reg(tok)
        if r and r[0] == "s":
            return (int(w.s[r[1]]) & 0xFFFFFFFF) | ((int(w.s[r[1] + 1]) & 0xFFFFFFFF) << 32)
        return self.const(tok) | (0xFFFFFFFF00000000 if tok.startswith("-") else 0)

    def swrite64(self, w, tok, val):
        val &= (1 << 64) - 1
        if tok == "vcc":
            w.vcc = val
            return
        r = parse_reg(tok)
        w.s[r[1]] = val & 0xFFFFFFFF
        w.s[r[1] + 1] = val >> 32

    def vwrite(self, w, tok, val, k=0):
        f, i, n = parse_reg(tok)
        (w.v if f == "v" else w.a)[i + k] = np.asarray(val, np.uint32)

    def mask_of(self, w, tok):
        m = self.sread64(w, tok)
        return np.array([(m >> l) & 1 for l in range(L)], bool)

    def desc(self, w, tok):
        f, i, n = parse_reg(tok)
        return [int(w.s[i + k]) & 0xFFFFFFFF for k in range(4)]

    # ------------------------------------------------------------ execution
    def run(self, max_steps=5_000_000):
        while True:
            progressed = False
            for wid in self.order:
                w = self.waves[wid]
                while not w.done:
                    line = self.lines[w.pc] if w.pc < len(self.lines) else None
                    if line is None:
                        w.done = True
                        break
                    if line == "s_barrier":
                        w.at_barrier = True
                        break
                    self.step(w, line)
                    progressed = True
                    self.count += 1
                    if self.count > max_steps:
                        raise EmuError("step limit")
            waiting = [w for w in self.waves if not w.done]
            if not waiting:
                return
            if all(getattr(w, "at_barrier", False) for w in waiting):
                if len(waiting) != 4:
                    raise EmuError("barrier with finished waves")
                for w in waiting:
                    w.at_barrier = False
                    w.pc += 1
                continue
            if not progressed:
                raise EmuError("deadlock")

    def retire_vm(self, w, keep):
        while len(w.pend_vm) > keep:
            item = w.pend_vm.pop(0)
            if item[0] == "lds":
                seg = self.lds_pend[item[1]:item[2]]
                seg[seg == w.wid] = -1

    def step(self, w, line):
        self.executed[w.pc] = self.executed.get(w.pc, 0) + 1
        op, _, rest = line.partition(" ")
        args = [a.strip() for a in rest.split(",")] if rest else []
        pc_next = w.pc + 1
        h = getattr(self, "op_" + op.replace(".", "_"), None)
        if h is None:
            raise EmuError(f"unsupported instruction: {line}")
        r = h(w, args, line)
        w.pc = r if r is not None else pc_next

    # -- scalar
    def op_s_nop(self, w, a, line):
        pass

    def op_s_waitcnt(self, w, a, line):
        vm = re.search(r"vmcnt\((\d+)\)", line)
        lg = re.search(r"lgkmcnt\((\d+)\)", line)
        if vm:
            self.retire_vm(w, int(vm.group(1)))
        if lg:
            keep = int(lg.group(1))
            while len(w.pend_lgkm) > keep:
                w.pend_lgkm.pop(0)

    def op_s_mov_b32(self, w, a, line):
        val = self.sread(w, a[1])
        if a[0] == "m0":
            w.m0 = val
        else:
            w.s[parse_reg(a[0])[1]] = val

    op_s_movk_i32 = op_s_mov_b32

    def op_s_add_u32(self, w, a, line):
        val = (self.sread(w, a[1]) + self.sread(w, a[2])) & 0xFFFFFFFF
        if a[0] == "m0":
            w.m0 = val
        else:
            w.s[parse_reg(a[0])[1]] = val

    def op_s_and_b32(self, w, a, line):
        w.s[parse_reg(a[0])[1]] = self.sread(w, a[1]) & self.sread(w, a[2])

    def op_s_or_b64(self, w, a, line):
        self.swrite64(w, a[0], self.sread64(w, a[1]) | self.sread64(w, a[2]))

    def op_s_cmp_eq_u32(self, w, a, line):
        w.scc = int(self.sread(w, a[0]) == self.sread(w, a[1]))

    def op_s_cmp_ge_u32(self, w, a, line):
        w.scc = int(self.sread(w, a[0]) >= self.sread(w, a[1]))

    def op_s_cmp_lt_u32(self, w, a, line):
        w.scc = int(self.sread(w, a[0]) < self.sread(w, a[1]))

    def op_s_cbranch_scc0(self, w, a, line):
        return self.labels[a[0]] if not w.scc else None

    def op_s_branch(self, w, a, line):
        return self.labels[a[0]]

    def op_s_cbranch_scc1(self, w, a, line):
        return self.labels[a[0]] if w.scc else None

    def op_s_cbranch_vccnz(self, w, a, line):
        return self.labels[a[0]] if w.vcc else None

    # -- memory
    def _buf(self, w, dtok):
        d = self.desc(w, dtok)
        return self.buffers[d[0]], d[1], d[2]

    def op_buffer_load_dwordx4(self, w, a, line):
        lds = line.endswith(" lds")
        off = re.search(r"offset:(\d+)", line)
        ioff = int(off.group(1)) if off else 0
        if lds:
            vo, dtok, so = a[0], a[1], a[2].split()[0]
        else:
            dst, vo, dtok, so = a[0], a[1], a[2], a[3].split()[0]
        buf, base, nrec = self._buf(w, dtok)
        voff = self.vread(w, vo).astype(np.int64)
        soff = self.sread(w, so)
        data = np.zeros((L, 4), np.uint32)
        for l in range(L):
            addr = int(voff[l]) + soff + ioff
            for k in range(4):
                if 0 <= addr + 4 * k and addr + 4 * k + 4 <= nrec:
                    p = base + addr + 4 * k
                    data[l, k] = int.from_bytes(buf[p:p + 4].tobytes(), "little")
        if lds:
            lo = w.m0
            hi = lo + 16 * L
            if hi > len(self.lds):
                raise EmuError(f"LDS DMA out of range: {lo}")
            self.lds[lo:hi] = data.reshape(-1).view(np.uint8)
            self.lds_pend[lo:hi] = w.wid
            w.pend_vm.append(("lds", lo, hi))
        else:
            f, i, n = parse_reg(dst)
            for k in range(4):
                w.v[i + k] = data[:, k]
            w.pend_vm.append(("regs", {("v", i + k) for k in range(4)}))

    def _store(self, w, a, line, nd):
        off = re.search(r"offset:(\d+)", line)
        ioff = int(off.group(1)) if off else 0
        src, vo, dtok, so = a[0], a[1], a[2], a[3].split()[0]
        buf, base, nrec = self._buf(w, dtok)
        voff = self.vread(w, vo).astype(np.int64)
        soff = self.sread(w, so)
        vals = [self.vread(w, src, k) for k in range(nd)]
        for l in range(L):
            addr = int(voff[l]) + soff + ioff
            for k in range(nd):
                if 0 <= addr + 4 * k and addr + 4 * k + 4 <= nrec:
                    p = base + addr + 4 * k
                    buf[p:p + 4] = np.frombuffer(int(vals[k][l]).to_bytes(4, "little"), np.uint8)

    def op_buffer_store_dword(self, w, a, line):
        self._store(w, a, line, 1)

    def op_buffer_store_dwordx4(self, w, a, line):
        self._store(w, a, line, 4)

    def _lds_addr(self, w, tok, line, nbytes):
        off = re.search(r"offset:(\d+)", line)
        base = self.vread(w, tok).astype(np.int64) + (int(off.group(1)) if off else 0)
        if base.min() < 0 or base.max() + nbytes > len(self.lds):
            raise EmuError(f"LDS access out of range: {line}")
        idx = base[:, None] + np.arange(nbytes)[None, :]
        pend = self.lds_pend[idx]
        if (pend >= 0).any():
            raise EmuError(f"wave {w.wid}: LDS read of bytes with a DMA not waited for by wave "
                           f"{int(pend[pend >= 0][0])}: {line}")
        return base

    def op_ds_read_b128(self, w, a, line):
        f, i, n = parse_reg(a[0])
        base = self._lds_addr(w, a[1].split()[0], line, 16)
        idx = base[:, None] + np.arange(16)[None, :]
        words = self.lds[idx].reshape(L, 16).copy().view(np.uint32)   # [L, 4]
        for k in range(4):
            w.v[i + k] = words[:, k]
        w.pend_lgkm.append({("v", i + k) for k in range(4)})

    def op_ds_read_b64_tr_b16(self, w, a, line):
        f, i, n = parse_reg(a[0])
        base = self._lds_addr(w, a[1].split()[0], line, 8)
        idx = base[:, None] + np.arange(8)[None, :]
        src = self.lds[idx].reshape(L, 8).copy().view(np.uint16).astype(np.uint32)   # [L, 4]
        res = np.zeros((L, 4), np.uint32)
        r = np.arange(16)
        for g in range(4):
            for e in range(4):
                res[16 * g + r, e] = src[16 * g + 4 * e + r // 4, r % 4]
        w.v[i] = res[:, 0] | (res[:, 1] << 16)
        w.v[i + 1] = res[:, 2] | (res[:, 3] << 16)
        w.pend_lgkm.append({("v", i), ("v", i + 1)})

    def op_ds_read_b64_tr_b8(self, w, a, line):
        """Within each group of 16 lanes, result lane r, byte t gets byte r % 8 of what
        source lane 2t + r / 8 addressed."""
        f, i, n = parse_reg(a[0])
        base = self._lds_addr(w, a[1].split()[0], line, 8)
        idx = base[:, None] + np.arange(8)[None, :]
        src = self.lds[idx].reshape(L, 8).copy()                      # [L, 8] bytes
        res = np.zeros((L, 8), np.uint8)
        r = np.arange(16)
        for g in range(4):
            for t in range(8):
                res[16 * g + r, t] = src[16 * g + 2 * t + r // 8, r % 8]
        words = res.view(np.uint32)                                   # [L, 2]
        w.v[i] = words[:, 0]
        w.v[i + 1] = words[:, 1]
        w.pend_lgkm.append({("v", i), ("v", i + 1)})

    def op_ds_write_b64(self, w, a, line):
        base = self.vread(w, a[0]).astype(np.int64)
        if base.min() < 0 or base.max() + 8 > len(self.lds):
            raise EmuError(f"LDS write out of range: {line}")
        x0, x1 = self.vread(w, a[1].split()[0], 0), self.vread(w, a[1].split()[0], 1)
        for l in range(L):
            self.lds[base[l]:base[l] + 8] = np.array([x0[l], x1[l]], np.uint32).view(np.uint8)
        w.pend_lgkm.append(set())

    # -- matrix
    def _mfma(self, w, a, conv):
        D, A, B, C = a
        lanes = np.arange(L)
        av = np.stack([self.vread(w, A, k) for k in range(4)])
        bv = np.stack([self.vread(w, B, k) for k in range(4)])
        ea = np.stack([(av[e // 2] >> (16 * (e % 2))) & 0xFFFF for e in range(8)])   # [8, L]
        eb = np.stack([(bv[e // 2] >> (16 * (e % 2))) & 0xFFFF for e in range(8)])
        A_m = np.zeros((32, 16), np.float64)
        B_m = np.zeros((16, 32), np.float64)
        for e in range(8):
            A_m[lanes % 32, 8 * (lanes // 32) + e] = conv(ea[e])
            B_m[8 * (lanes // 32) + e, lanes % 32] = conv(eb[e])
        prod = A_m @ B_m
        out = []
        for r in range(16):
            c = np.zeros(L, np.float64) if C == "0" else f32(self.vread(w, C, r)).astype(np.float64)
            rows = 8 * (r // 4) + 4 * (lanes // 32) + r % 4
            out.append(u32((c + prod[rows, lanes % 32]).astype(np.float32)))
        for r in range(16):
            self.vwrite(w, D, out[r], r)

    def _mfma16(self, w, a, conv):
        """v_mfma_f32_16x16x32: lane l holds A[l % 16][8*(l/16) + e], B[8*(l/16) + e][l % 16]
        and D[4*(l/16) + r][l % 16] in register r."""
        D, A, B, C = a
        lanes = np.arange(L)
        av = np.stack([self.vread(w, A, k) for k in range(4)])
        bv = np.stack([self.vread(w, B, k) for k in range(4)])
        A_m = np.zeros((16, 32), np.float64)
        B_m = np.zeros((32, 16), np.float64)
        for e in range(8):
            A_m[lanes % 16, 8 * (lanes // 16) + e] = conv((av[e // 2] >> (16 * (e % 2))) & 0xFFFF)
            B_m[8 * (lanes // 16) + e, lanes % 16] = conv((bv[e // 2] >> (16 * (e % 2))) & 0xFFFF)
        prod = A_m @ B_m
        out = []
        for r in range(4):
            c = np.zeros(L, np.float64) if C == "0" else f32(self.vread(w, C, r)).astype(np.float64)
            out.append(u32((c + prod[4 * (lanes // 16) + r, lanes % 16]).astype(np.float32)))
        for r in range(4):
            self.vwrite(w, D, out[r], r)

    def _mfma8(self, w, a, sa=None, sb=None):
        """v_mfma[_scale]_f32_32x32x64_f8f6f4 on E4M3 operands: 8 registers (32 bytes)
        per lane; byte j of lane-half h of A meets byte j of lane-half h of B, so
        D[i][c] = sum over (h, j) of A[lane i + 32h][j] B[lane c + 32h][j] (+ C).  With
        scales, lane x + 32b (low byte, E8M0, bias 127) scales bytes 16b .. 16b+15 of
        row (A) or column (B) x in both lane-halves."""
        D, A, B, C = a[:4]
        lanes = np.arange(L)
        ab = np.stack([self.vread(w, A, k) for k in range(8)]).T.copy().view(np.uint8)  # [L, 32]
        bb = np.stack([self.vread(w, B, k) for k in range(8)]).T.copy().view(np.uint8)
        av, bv = E4M3[ab], E4M3[bb]                                                      # [L, 32]
        if sa is not None:
            for blk in range(2):
                fa = 2.0 ** (sa[blk * 32 + lanes % 32].astype(np.float64) - 127)
                fb = 2.0 ** (sb[blk * 32 + lanes % 32].astype(np.float64) - 127)
                av[:, 16 * blk:16 * blk + 16] *= fa[:, None]
                bv[:, 16 * blk:16 * blk + 16] *= fb[:, None]
        A_m = np.concatenate([av[:32], av[32:]], axis=1)      # [32 rows, 64]
        B_m = np.concatenate([bv[:32], bv[32:]], axis=1)      # [32 cols, 64]
        prod = A_m @ B_m.T
        out = []
        for r in range(16):
            c = np.zeros(L, np.float64) if C == "0" else f32(self.vread(w, C, r)).astype(np.float64)
            rows = 8 * (r // 4) + 4 * (lanes // 32) + r % 4
            out.append(u32((c + prod[rows, lanes % 32]).astype(np.float32)))
        for r in range(16):
            self.vwrite(w, D, out[r], r)

    def op_v_mfma_f32_32x32x64_f8f6f4(self, w, a, line):
        self._mfma8(w, a)

    def op_v_mfma_scale_f32_32x32x64_f8f6f4(self, w, a, line):
        sa = self.vread(w, a[4]) & 0xFF
        sb = self.vread(w, a[5].split()[0]) & 0xFF
        self._mfma8(w, a, sa, sb)

    def op_v_mfma_f32_16x16x32_bf16(self, w, a, line):
        self._mfma16(w, a, lambda b: bf16_val(b).astype(np.float64))

    def op_v_mfma_f32_16x16x32_f16(self, w, a, line):
        self._mfma16(w, a, lambda b: f16_val(b).astype(np.float64))

    def op_v_mfma_f32_32x32x16_bf16(self, w, a, line):
        self._mfma(w, a, lambda b: bf16_val(b).astype(np.float64))

    def op_v_mfma_f32_32x32x16_f16(self, w, a, line):
        self._mfma(w, a, lambda b: f16_val(b).astype(np.float64))

    # -- vector
    def _w(self, w, tok, val):
        self.vwrite(w, tok, val)

    def op_v_mov_b32(self, w, a, line):
        self._w(w, a[0], self.vread(w, a[1]))

    def op_v_accvgpr_write_b32(self, w, a, line):
        self._w(w, a[0], self.vread(w, a[1]))

    op_v_accvgpr_read_b32 = op_v_accvgpr_write_b32

    def op_v_fma_f32(self, w, a, line):
        x, y, z = (f32(self.vread(w, t)) for t in a[1:4])
        self._w(w, a[0], u32((x.astype(np.float64) * y + z).astype(np.float32)))

    def op_v_mul_f32(self, w, a, line):
        self._w(w, a[0], u32(f32(self.vread(w, a[1])) * f32(self.vread(w, a[2]))))

    def op_v_add_f32(self, w, a, line):
        self._w(w, a[0], u32(f32(self.vread(w, a[1])) + f32(self.vread(w, a[2]))))

    def op_v_sub_f32(self, w, a, line):
        with np.errstate(invalid="ignore"):
            self._w(w, a[0], u32(f32(self.vread(w, a[1])) - f32(self.vread(w, a[2]))))

    def op_v_exp_f32(self, w, a, line):
        with np.errstate(over="ignore", invalid="ignore"):
            self._w(w, a[0], u32(np.exp2(f32(self.vread(w, a[1])))))

    def op_v_log_f32(self, w, a, line):
        with np.errstate(divide="ignore", invalid="ignore"):
            self._w(w, a[0], u32(np.log2(f32(self.vread(w, a[1])))))

    def op_v_rcp_f32(self, w, a, line):
        with np.errstate(divide="ignore"):
            self._w(w, a[0], u32(np.float32(1.0) / f32(self.vread(w, a[1]))))

    def op_v_max3_f32(self, w, a, line):
        x, y, z = (f32(self.vread(w, t)) for t in a[1:4])
        self._w(w, a[0], u32(np.maximum(np.maximum(x, y), z)))

    def op_v_max_f32(self, w, a, line):
        self._w(w, a[0], u32(np.maximum(f32(self.vread(w, a[1])), f32(self.vread(w, a[2])))))

    def op_v_cvt_pk_bf16_f32(self, w, a, line):
        lo = bf16_bits(f32(self.vread(w, a[1])))
        hi = bf16_bits(f32(self.vread(w, a[2])))
        self._w(w, a[0], lo | (hi << 16))

    def op_v_cvt_pk_fp8_f32(self, w, a, line):
        """Two E4M3 bytes into the low word of the destination, or its high word with
        op_sel:[0,0,1]; the other word keeps its value."""
        lo = e4m3_bits(f32(self.vread(w, a[1])))
        hi = e4m3_bits(f32(self.vread(w, a[2].split()[0])))
        pair = lo | (hi << 8)
        old = self.vread(w, a[0])
        if "op_sel:[0,0,1]" in line:
            val = (old & 0xFFFF) | (pair << 16)
        else:
            val = (old & 0xFFFF0000) | pair
        self._w(w, a[0], val.astype(np.uint32))

    def op_v_floor_f32(self, w, a, line):
        self._w(w, a[0], u32(np.floor(f32(self.vread(w, a[1])))))

    def op_v_min_f32(self, w, a, line):
        self._w(w, a[0], u32(np.minimum(f32(self.vread(w, a[1])), f32(self.vread(w, a[2])))))

    def op_v_cvt_i32_f32(self, w, a, line):
        x = f32(self.vread(w, a[1])).astype(np.float64)
        x = np.where(np.isnan(x), 0.0, np.clip(x, -2.0 ** 31, 2.0 ** 31 - 1))
        self._w(w, a[0], np.trunc(x).astype(np.int64).astype(np.uint32))

    def op_v_cvt_pk_f16_f32(self, w, a, line):
        lo = f16_bits(f32(self.vread(w, a[1])))
        hi = f16_bits(f32(self.vread(w, a[2])))
        self._w(w, a[0], lo | (hi << 16))

    def _dot2c(self, w, a, conv):
        c = f32(self.vread(w, a[0])).astype(np.float64)
        x, y = self.vread(w, a[1]), self.vread(w, a[2])
        s = conv(x & 0xFFFF) * conv(y & 0xFFFF) + conv(x >> 16) * conv(y >> 16)
        self._w(w, a[0], u32((c + s).astype(np.float32)))

    def op_v_dot2c_f32_bf16(self, w, a, line):
        self._dot2c(w, a, lambda b: bf16_val(b).astype(np.float64))

    def op_v_dot2c_f32_f16(self, w, a, line):
        self._dot2c(w, a, lambda b: f16_val(b).astype(np.float64))

    def op_v_permlane32_swap_b32(self, w, a, line):
        x, y = self.vread(w, a[0]), self.vread(w, a[1])
        nx, ny = x.copy(), y.copy()
        nx[32:] = y[:32]
        ny[:32] = x[32:]
        self._w(w, a[0], nx)
        self._w(w, a[1], ny)

    def _cmp(self, w, a, fn):
        res = fn(self.vread(w, a[1]), self.vread(w, a[2]))
        m = 0
        for l in range(L):
            if res[l]:
                m |= 1 << l
        self.swrite64(w, a[0], m)

    def op_v_cmp_gt_f32(self, w, a, line):
        self._cmp(w, a, lambda x, y: f32(x) > f32(y))

    def op_v_cmp_neq_f32(self, w, a, line):
        self._cmp(w, a, lambda x, y: ~(f32(x) == f32(y)))

    def op_v_cmp_gt_i32(self, w, a, line):
        self._cmp(w, a, lambda x, y: x.view(np.int32) > y.view(np.int32))

    def op_v_cndmask_b32(self, w, a, line):
        m = self.mask_of(w, a[3])
        self._w(w, a[0], np.where(m, self.vread(w, a[2]), self.vread(w, a[1])))

    def op_v_sub_u32(self, w, a, line):
        self._w(w, a[0], self.vread(w, a[1]) - self.vread(w, a[2]))

    op_v_sub_u32_e64 = op_v_sub_u32

    def op_v_add_u32(self, w, a, line):
        self._w(w, a[0], self.vread(w, a[1]) + self.vread(w, a[2]))

    def op_v_xor_b32(self, w, a, line):
        self._w(w, a[0], self.vread(w, a[1]) ^ self.vread(w, a[2]))

    def op_v_and_b32(self, w, a, line):
        self._w(w, a[0], self.vread(w, a[1]) & self.vread(w, a[2]))

    def op_v_lshrrev_b32(self, w, a, line):
        self._w(w, a[0], self.vread(w, a[2]) >> (self.vread(w, a[1]) & 31))

    def op_v_lshlrev_b32(self, w, a, line):
        self._w(w, a[0], self.vread(w, a[2]) << (self.vread(w, a[1]) & 31))

    def op_v_lshl_add_u32(self, w, a, line):
        self._w(w, a[0], (self.vread(w, a[1]) << (self.vread(w, a[2]) & 31)) + self.vread(w, a[3]))

    def op_v_mbcnt_lo_u32_b32(self, w, a, line):
        lane = np.arange(L, dtype=np.uint32)
        self._w(w, a[0], np.minimum(lane, 32) + self.vread(w, a[2]))

    def op_v_mbcnt_hi_u32_b32(self, w, a, line):
        lane = np.arange(L, dtype=np.int64)
        self._w(w, a[0], np.maximum(lane - 32, 0).astype(np.uint32) + self.vread(w, a[2]))
