"""The hazard scan of tests/mfma_asm_check.py on small hand-written listings (no compiler, no
GPU): each rule it applies to the head-size-128 kernel's assembly is shown to pass a correct
sequence and to flag the same sequence with one wait state too few."""
from tests import mfma_asm_check as chk


def asm(*lines):
    """Lines as one inline-asm block of the compiler's output."""
    return [";;#ASMSTART", *lines, ";;#ASMEND"]


# an O^T MFMA into the fixed accumulators and an S^T MFMA into arch registers, as the
# kernel writes them (inline asm)
MFMA_O = asm("\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]")
MFMA_S = asm("\tv_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], a[128:131], 0")


def nops(n):
    """n wait states as s_nop instructions (s_nop k counts k + 1)."""
    out = []
    while n > 0:
        k = min(n, 8)
        out.append(f"\ts_nop {k - 1}")
        n -= k
    return out


def test_vector_read_of_an_mfma_result_needs_13_wait_states():
    read = "\tv_max3_f32 v40, v16, v17, v18"
    assert not chk.check(MFMA_S + nops(chk.MFMA_WS) + [read])
    found = chk.check(MFMA_S + nops(chk.MFMA_WS - 1) + [read])
    assert any("access of an MFMA result" in m for _, m in found)


def test_vector_write_feeding_an_mfma_needs_2_wait_states():
    write = "\tv_cvt_pk_bf16_f32 v4, v40, v41"
    assert not chk.check([write] + nops(chk.VALU_WS) + MFMA_O)
    found = chk.check([write] + nops(chk.VALU_WS - 1) + MFMA_O)
    assert any("vector result" in m for _, m in found)


def test_an_mfma_may_chain_on_its_own_accumulator_at_once():
    assert not chk.check(MFMA_O + MFMA_O)


def test_an_mfma_result_is_never_an_a_or_b_operand():
    use = asm("\tv_mfma_f32_32x32x16_bf16 v[32:47], v[16:19], a[128:131], 0")
    found = chk.check(MFMA_S + nops(20) + use)
    assert any("A/B operand" in m for _, m in found)


def test_compiler_instructions_must_not_write_the_fixed_accumulators():
    assert any("fixed accumulator" in m for _, m in chk.check(["\tv_accvgpr_write_b32 a3, v0"]))
    # the same instruction inside inline asm is the kernel's own and allowed
    assert not chk.check(asm("\tv_accvgpr_write_b32 a3, v0"))
    # registers past the fixed range are the compiler's
    assert not chk.check(["\tv_accvgpr_write_b32 a140, v0"])


def test_a_forward_branch_carries_its_pending_hazards_to_the_target():
    # taken branch skips the wait states on the fall-through path
    lines = MFMA_S + ["\ts_cbranch_scc1 .LBB0_2"] + nops(chk.MFMA_WS) + [
        ".LBB0_2:", "\tv_max3_f32 v40, v16, v17, v18"]
    found = chk.check(lines)
    assert any("access of an MFMA result" in m for _, m in found)
    # with the wait states before the branch both paths are clean
    lines = MFMA_S + nops(chk.MFMA_WS) + ["\ts_cbranch_scc1 .LBB0_2", "\ts_nop 0",
                                            ".LBB0_2:", "\tv_max3_f32 v40, v16, v17, v18"]
    assert not chk.check(lines)


def test_a_loop_back_edge_needs_the_wait_states_behind_the_last_mfma():
    loop = [".LBB0_1:"] + MFMA_O + ["\ts_cbranch_scc1 .LBB0_1"]
    assert any("back edge" in m for _, m in chk.check(loop))
    loop = [".LBB0_1:"] + MFMA_O + nops(chk.MFMA_WS) + ["\ts_cbranch_scc1 .LBB0_1"]
    assert not chk.check(loop)


def test_the_rescale_asm_counts_as_reading_every_fixed_accumulator():
    rescale = asm("\t.rept 64", "\tv_accvgpr_read_b32 v1, a[d128_r]", "\t.endr")
    assert not chk.check(MFMA_O + nops(chk.MFMA_WS) + rescale)
    found = chk.check(MFMA_O + nops(chk.MFMA_WS - 1) + rescale)
    assert any("rescale" in m for _, m in found)
