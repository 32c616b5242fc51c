"""CPU checks of the 64-row forward's instruction schedule (gen_fwd_w64.py).

The generator fills each matrix instruction's shadow by an issue-cost model
of one wave per SIMD.  Its constants were fitted to register-only loops on
MI355X (32 v_mfma_f32_32x32x16_bf16 per iteration on zero operands, full
clock, the listed instructions after each; cycles per matrix instruction,
the bare loop taking 32): the first test holds the model to those
measurements, the others hold the generated tile steps to the modelled
cycle counts this schedule reaches, so that a change that costs issue
cycles shows up on the CPU."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "exact_io_aware_37_amd", "csrc"))

import gen_fwd_w64 as gen  # noqa: E402

FMA = gen.valu("v_fma_f32 v100, v100, v98, v99", ["v100"], ["v100"])
EXP = gen.valu("v_exp_f32 v101, v101", ["v101"], ["v101"], kind="trans", cost=8)
CVT = gen.valu("v_cvt_pk_bf16_f32 v102, v150, v151", [], ["v102"])
NOP = gen.Ins("s_nop 0", "nop", cost=1)
SADD = gen.raw("s_add_u32 s91, s91, 1")
LDS = gen.Ins("ds_read_b128 v[200:203], v240", "lds")
MF = gen.mfma("v_mfma_f32_32x32x16_bf16", "a[0:15]", "v[0:3]", "v[4:7]", "a[0:15]")
FE = [FMA, EXP, FMA, EXP, CVT]

# (instructions after each matrix instruction, measured cycles per matrix instruction)
MEASURED = [
    ([], 32.0), (FE, 36.3), (FE + [NOP], 40.3), ([NOP] + FE, 36.4), ([SADD] + FE, 36.4),
    ([SADD, SADD] + FE, 40.3), (FE + [LDS], 52.0), ([LDS] + FE, 43.2), ([FMA] * 7, 36.5),
    ([LDS], 33.3), ([FMA, FMA, FMA, FMA], 32.0), ([EXP, EXP], 32.3),
]


@pytest.mark.parametrize("group,measured", MEASURED, ids=lambda x: str(x) if isinstance(x, float) else "")
def test_issue_model_matches_measurements(group, measured):
    n = 32
    seq = []
    for _ in range(n):
        seq += [MF] + group
    cycles, busy = gen.issue_time(seq + [MF])
    per = (cycles - 32) / n
    assert abs(per - measured) <= 2.0, (per, measured)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("parity", range(4))
def test_unmasked_step_stays_near_the_matrix_time(dt, parity):
    block = gen.tile_step(dt, parity, False, False, "t")
    cycles, busy = gen.issue_time(block.out)
    assert busy == 64 * 32 + 8 * 16
    assert cycles <= 2400, cycles          # 2368 for this schedule; 2729 for the earlier one


@pytest.mark.parametrize("parity", range(4))
def test_masked_step(parity):
    block = gen.tile_step("bf16", parity, True, True, "t")
    cycles, _ = gen.issue_time(block.out)
    assert cycles <= 2900, cycles          # 2848 for this schedule; 3904 with unpipelined masks


@pytest.mark.parametrize("parity", range(4))
def test_fp8_unmasked_step(parity):
    """The E4M3 body: 18 matrix instructions of 64 cycles per step; the softmax's vector
    work (the same per score as the 16-bit body, against half the matrix work) bounds it."""
    import gen_fwd_w64_fp8 as gen8
    block = gen8.tile_step8(parity, False)
    cycles, busy = gen.issue_time(block.out)
    assert busy == 16 * 64 + 2 * 64
    assert cycles <= 1850, cycles          # 1806-1810 for this schedule
