"""Static check of the generated gfx950 assembly (gated_delta_rule_45_amd/isa_check.py): no
instruction reads or overwrites a matrix-core (MFMA) result before the wait states it needs, on any
path of the control-flow graph.  The compiler has been seen to leave none where the read sits behind
a block join (the first read of an accumulator returned its stale value: wrong results, no fault),
so every kernel source is compiled to assembly and checked.  The checker itself is pinned on small
hand-written blocks first."""
import textwrap

import pytest

from gated_delta_rule_45_amd import isa_check


def _check(src):
    lines = textwrap.dedent(src).strip("\n").splitlines()
    return isa_check.check_function("f", isa_check.parse_function(lines, 0))


def test_flags_a_read_behind_a_join():
    # the shape of the case found in the prep kernel: the chain's last product ends its block,
    # one predecessor of the join has wait states, the other none
    viol = _check("""
        v_mfma_f32_16x16x4_f32 a[0:3], v5, v42, a[4:7]
        s_cbranch_execz .LBB0_2
        s_branch .LBB0_3
    .LBB0_2:
        s_nop 4
        v_accvgpr_write_b32 a3, 0
    .LBB0_3:
        s_andn2_b64 vcc, exec, s[2:3]
        v_accvgpr_read_b32 v7, a3
        s_endpgm
    .Lfunc_end0:
    """)
    assert len(viol) >= 1 and any(v[3] < v[4] for v in viol)


def test_accepts_enough_wait_states_and_srcc_chains():
    viol = _check("""
        v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], 0
        v_mfma_f32_16x16x32_bf16 a[0:3], v[8:11], v[12:15], a[0:3]
        s_nop 7
        v_accvgpr_read_b32 v20, a0
        v_mfma_f32_16x16x4_f32 a[4:7], v1, v2, 0
        s_cbranch_vccnz .LBB0_1
        s_nop 7
    .LBB0_1:
        s_nop 7
        v_accvgpr_read_b32 v21, a4
        s_endpgm
    .Lfunc_end0:
    """)
    assert viol == []


def test_flags_a_too_early_read_in_one_block():
    viol = _check("""
        v_mfma_f32_16x16x4_f32 v[0:3], v10, v11, 0
        s_nop 3
        v_add_f32_e32 v20, v1, v20
        s_endpgm
    .Lfunc_end0:
    """)
    assert len(viol) == 1 and viol[0][3] == 4


def test_library_kernels_have_no_early_reads():
    viol = isa_check.check_sources()
    for v in viol[:20]:
        print(f"{v[0]}: {v[1][:90]}: mfma line {v[2]}, access line {v[3]}, {v[4]} < {v[5]} wait states")
    assert viol == [], f"{len(viol)} MFMA result(s) read too early"
