"""Check of compiled gfx950 code: no vector instruction touches an MFMA result
register before the matrix unit has written it.

gfx950 does not interlock a vector instruction that reads (or overwrites) the
destination of an MFMA still in flight; the compiler pads such pairs with
independent instructions or s_nop.  The padding must cover the latency of
the register concerned: an MFMA writes its 4 or 16 result registers over
several passes, the last ones latest.  NEED below holds, per instruction and
result register, the number of wait states (issue slots after the MFMA) from
which a read returns the product, measured on MI355X with
csrc/probe_mfma_latency.py (one wave, the read placed exactly N slots after
the MFMA; every lane of several launches agreed).

For v_mfma_f32_32x32x64_f8f6f4 with 8-bit operands the last two result
registers need 20 wait states.  The compiler's padding for a read of that
instruction's VGPR result is 19, enough for every register but 14 and 15;
a schedule that reads those two at exactly 19 slots copies stale values.
That happened once in the FP8 forward kernel (a register copy of the P*V
accumulator right after the matrix instruction) and gave wrong outputs.  The
build runs this check on the device assembly of the library and refuses a
library with such a read, whatever register allocation and schedule the
compiler picks.

The check is a forward dataflow over the basic blocks of each function:
one wait state per instruction (a lower bound of the issue slots it takes),
s_nop N counting N + 1; at a merge the longest remaining wait of each
register is kept, and branches (loops included) propagate their state.
MFMAs reading an earlier MFMA's result are not checked here: the matrix unit
orders its own dependent operations.

    python -m exact_io_aware_37_amd.mfma_latency FILE.s
"""

from __future__ import annotations

import re
import sys

# wait states after the MFMA issue from which result register i holds the product
NEED = {
    "v_mfma_f32_32x32x64_f8f6f4": [7, 7, 8, 8, 11, 11, 12, 12, 15, 15, 16, 16, 19, 19, 20, 20],
    "v_mfma_f32_16x16x128_f8f6f4": [11, 11, 12, 12],
    "v_mfma_f32_32x32x16_bf16": [5, 5, 6, 6, 7, 7, 8, 8, 9, 9, 10, 10, 11, 11, 12, 12],
    "v_mfma_f32_32x32x16_f16": [5, 5, 6, 6, 7, 7, 8, 8, 9, 9, 10, 10, 11, 11, 12, 12],
    "v_mfma_f32_16x16x32_bf16": [7, 7, 8, 8],
    "v_mfma_f32_16x16x32_f16": [7, 7, 8, 8],
    # registers 0-13 read the product from 2 wait states on, 14-15 from 18;
    # the check takes 18 for every register
    "v_mfma_f32_32x32x2_f32": [18] * 16,
    "v_mfma_scale_f32_32x32x64_f8f6f4": [7, 7, 8, 8, 11, 11, 12, 12, 15, 15, 16, 16, 19, 19, 20, 20],
    "v_mfma_scale_f32_16x16x128_f8f6f4": [11, 11, 12, 12],
}

_VECTOR_PREFIXES = ("v_", "ds_", "buffer_", "global_", "flat_", "scratch_")
_END_BLOCK = ("s_branch", "s_cbranch", "s_endpgm", "s_setpc", "s_trap")


def _regs(tok: str):
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return [(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)]
    m = re.fullmatch(r"([va])(\d+)", tok)
    if m:
        return [(m.group(1), int(m.group(2)))]
    return []


def _operands(text: str):
    op = text.split()[0]
    return op, [t.strip().split()[0] for t in text[len(op):].split(",") if t.strip()]


def parse(path: str):
    """Function name -> list of ("label", name) / ("ins", text), from an assembly file."""
    funcs, cur = {}, None
    with open(path) as f:
        for line in f:
            m = re.match(r"^([A-Za-z_]\w*):", line)
            if m and not line.startswith(".") and not line.startswith("\t"):
                cur = m.group(1)
                funcs[cur] = []
                continue
            if cur is None:
                continue
            s = line.split(";")[0].strip()
            if not s:
                continue
            if s.endswith(":"):
                funcs[cur].append(("label", s[:-1]))
                continue
            if s.startswith("."):
                if s.startswith(".Lfunc_end"):
                    cur = None
                continue
            funcs[cur].append(("ins", s))
    return funcs


def check_function(items):
    """Early accesses in one function: list of (instruction, MFMA, wait states short)."""
    blocks, labels, cur = [], {}, []
    for kind, x in items:
        if kind == "label":
            if cur:
                blocks.append(cur)
                cur = []
            labels[x] = len(blocks)
            continue
        cur.append(x)
        if x.split()[0].startswith(_END_BLOCK):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    if not blocks:
        return []
    succ = []
    for bi, b in enumerate(blocks):
        op, ops = _operands(b[-1]) if b else ("", [])
        s = []
        if op.startswith("s_branch") or op.startswith("s_cbranch"):
            if ops and labels.get(ops[0], len(blocks)) < len(blocks):
                s.append(labels[ops[0]])
        if not op.startswith(("s_branch", "s_endpgm", "s_setpc", "s_trap")) and bi + 1 < len(blocks):
            s.append(bi + 1)
        succ.append(s)

    entry = [None] * len(blocks)
    entry[0] = {}
    work = [0]
    found = {}
    while work:
        bi = work.pop()
        state = dict(entry[bi])
        for x in blocks[bi]:
            op, ops = _operands(x)
            is_mfma = op.startswith("v_mfma")
            if not is_mfma and op.startswith(_VECTOR_PREFIXES):
                for t in ops:
                    for r in _regs(t):
                        if r in state:
                            key = (x, state[r][1])
                            found[key] = max(found.get(key, 0), state[r][0])
            ws = int(ops[0], 0) + 1 if op == "s_nop" else 1
            state = {r: (rem - ws, src) for r, (rem, src) in state.items() if rem - ws > 0}
            if is_mfma and op in NEED and ops:
                need = NEED[op]
                for i, r in enumerate(_regs(ops[0])):
                    state[r] = (need[min(i, len(need) - 1)], x)
        for sj in succ[bi]:
            if entry[sj] is None:
                entry[sj] = dict(state)
                work.append(sj)
                continue
            changed = False
            merged = entry[sj]
            for r, (rem, src) in state.items():
                if r not in merged or merged[r][0] < rem:
                    merged[r] = (rem, src)
                    changed = True
            if changed:
                work.append(sj)
    return [(x, src, short) for (x, src), short in found.items()]


def check_file(path: str):
    """Early accesses in every function of an assembly file: {function: [...]}."""
    out = {}
    for name, items in parse(path).items():
        bad = check_function(items)
        if bad:
            out[name] = bad
    return out


def main(argv) -> int:
    bad = check_file(argv[1])
    for name, items in bad.items():
        print(f"{name}: {len(items)} early access(es)")
        for x, src, short in items[:8]:
            print(f"    {x}    ({short} wait state(s) short of: {src})")
    print("ok" if not bad else "FAILED")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
