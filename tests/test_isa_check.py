"""The build-time hazard check around the kernels' inline-asm LDS copies.

isa_check scans generated device assembly for two gfx9-family rules the
compiler does not apply to inline asm: 5 wait states between a VALU write of
an SGPR and a VMEM read of it (the copy's base address), and 1 wait state
between an SALU write of m0 and an LDS copy.  The snippets below plant each
violation (straight-line, through a branch, through a carry-out operand) and
the clean forms beside them; the last test runs the check on the assembly the
build generated, when it is present.
"""

import glob
import os

import pytest

from exact_tiled_attention_prefill_amd.isa_check import check_asm, valu_sgpr_writes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def kernel(body):
    return "_Zk:\n" + "\n".join("\t" + line if not line.startswith(".") else line for line in body) + "\n"


def rules(asm):
    return sorted(r for _, _, r in check_asm(asm))


SGPR = "SGPR base written by VALU < 5 wait states before"
M0 = "m0 written by SALU < 1 wait state before"


def test_clean_copy_passes():
    asm = kernel(["s_add_u32 s2, s4, s6", "s_mov_b32 m0, s5", "s_nop 0", "global_load_lds_dwordx4 v1, s[2:3]"])
    assert check_asm(asm) == []


def test_m0_written_right_before_copy_is_flagged():
    asm = kernel(["s_mov_b32 m0, s5", "global_load_lds_dwordx4 v1, s[2:3]"])
    assert rules(asm) == [M0]


def test_m0_rule_applies_to_the_vgpr_address_form():
    asm = kernel(["s_movk_i32 m0, 0x1000", "global_load_lds_dwordx4 v[2:3], off nt"])
    assert rules(asm) == [M0]


def test_readlane_restoring_the_base_is_flagged():
    # the pattern the compiler produced when it spilled a copy's base to a VGPR lane
    asm = kernel(["s_mov_b64 s[0:1], -1", "v_readlane_b32 s0, v247, 2", "s_mov_b32 m0, s86",
                  "v_readlane_b32 s1, v247, 3", "s_nop 0", "global_load_lds_dwordx4 v144, s[0:1]"])
    assert rules(asm) == [SGPR]


def test_five_wait_states_after_the_write_are_enough():
    ok = kernel(["v_readfirstlane_b32 s3, v7", "s_nop 3", "s_mov_b32 m0, s5", "s_nop 0",
                 "global_load_lds_dwordx4 v1, s[2:3]"])
    assert check_asm(ok) == []  # 4 + 1 + 1 wait states between
    short = kernel(["v_readfirstlane_b32 s3, v7", "s_nop 2", "s_nop 0", "global_load_lds_dwordx4 v1, s[2:3]"])
    assert rules(short) == [SGPR]  # 3 + 1


def test_write_before_a_branch_into_the_copy_block_is_flagged():
    asm = kernel(["v_readfirstlane_b32 s2, v0", "s_branch .LBB0_2", "s_endpgm", ".LBB0_2:",
                  "s_mov_b32 m0, s5", "s_nop 0", "global_load_lds_dwordx4 v1, s[2:3]"])
    assert rules(asm) == [SGPR]


def test_fall_through_is_not_followed_past_an_unconditional_branch():
    asm = kernel([".LBB0_1:", "v_readfirstlane_b32 s2, v0", "s_branch .LBB0_3", ".LBB0_2:",
                  "s_mov_b32 m0, s5", "s_nop 0", "global_load_lds_dwordx4 v1, s[2:3]", ".LBB0_3:", "s_endpgm"])
    assert check_asm(asm) == []  # .LBB0_2 has no predecessor here


def test_carry_out_into_the_base_is_a_write():
    assert valu_sgpr_writes("v_add_co_u32_e64 v1, s[2:3], v2, v3") == {2, 3}
    asm = kernel(["v_add_co_u32_e64 v1, s[2:3], v2, v3", "s_mov_b32 m0, s5", "s_nop 0",
                  "global_load_lds_dwordx4 v1, s[2:3]"])
    assert rules(asm) == [SGPR]


def test_a_valu_reading_the_base_is_not_a_write():
    assert valu_sgpr_writes("v_add_u32_e32 v1, s2, v2") == set()
    assert valu_sgpr_writes("v_writelane_b32 v247, s2, 0") == set()
    asm = kernel(["v_add_u32_e32 v1, s2, v2", "s_mov_b32 m0, s5", "s_nop 0", "global_load_lds_dwordx4 v1, s[2:3]"])
    assert check_asm(asm) == []


def test_loop_back_edge_is_followed_without_looping_forever():
    asm = kernel([".LBB0_1:", "s_mov_b32 m0, s5", "s_nop 0", "global_load_lds_dwordx4 v1, s[2:3]",
                  "v_readfirstlane_b32 s2, v0", "s_cbranch_scc1 .LBB0_1", "s_endpgm"])
    assert rules(asm) == [SGPR]  # the write at the loop's end reaches the copy at its top


@pytest.mark.parametrize("name", ["prefill_bf16", "backward_bf16", "decode"])
def test_built_device_code_is_clean(name):
    path = os.path.join(ROOT, "_build", name + ".s")
    if not os.path.exists(path):
        pytest.skip("no generated assembly (run the build first)")
    with open(path) as f:
        asm = f.read()
    assert "global_load_lds_dwordx4" in asm
    assert check_asm(asm) == []


def test_generated_assembly_lists_every_library_source():
    from exact_tiled_attention_prefill_amd.build import SOURCES
    built = {os.path.basename(p)[:-2] for p in glob.glob(os.path.join(ROOT, "_build", "*.s"))}
    if not built:
        pytest.skip("no generated assembly (run the build first)")
    assert {s[:-4] for s in SOURCES} <= built
