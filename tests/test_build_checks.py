"""The build's checks of the generated attention code, on small hand-written
assembly listings: each must flag the hazard it exists for and pass the safe
form of the same sequence.  (Host logic only; nothing is compiled.)"""

from gated_gqa_causal_amd import build as b


def _lines(text):
    return [ln for ln in text.strip("\n").splitlines()]


# ---- a compiler-issued MFMA's result read by inline asm ---------------------

def test_asm_read_of_builtin_mfma_result_too_soon_is_refused():
    asm = _lines("""
    v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]
    s_nop 7
    ;;#ASMSTART
    v_cvt_pk_bf16_f32 v0, 0, v3
    ;;#ASMEND
    """)
    probs = b._check_asm_reads_of_mfma_results("k", asm)
    assert len(probs) == 1 and "8 wait states" in probs[0]


def test_asm_read_after_enough_wait_states_passes():
    asm = _lines("""
    v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]
    s_nop 7
    s_nop 7
    v_mov_b32 v40, v41
    v_mov_b32 v42, v43
    v_mov_b32 v44, v45
    ;;#ASMSTART
    v_cvt_pk_bf16_f32 v0, 0, v3
    ;;#ASMEND
    """)
    assert b._check_asm_reads_of_mfma_results("k", asm) == []


def test_compiler_read_and_unrelated_asm_are_not_flagged():
    asm = _lines("""
    v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]
    v_cvt_pk_bf16_f32 v1, v2, s0
    ;;#ASMSTART
    v_max3_f32 v30, v31, v32, v33
    ;;#ASMEND
    """)
    # The compiler guards its own read (v2); the asm reads no result register.
    assert b._check_asm_reads_of_mfma_results("k", asm) == []


def test_agpr_result_and_branch_end_the_scan():
    agpr = _lines("""
    v_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[24:27], a[0:15]
    ;;#ASMSTART
    v_cvt_pk_bf16_f32 v0, 0, v3
    ;;#ASMEND
    """)
    assert b._check_asm_reads_of_mfma_results("k", agpr) == []
    branch = _lines("""
    v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]
    s_branch .LBB0_3
    ;;#ASMSTART
    v_cvt_pk_bf16_f32 v0, 0, v3
    ;;#ASMEND
    """)
    assert b._check_asm_reads_of_mfma_results("k", branch) == []


def test_scan_continues_through_a_label():
    asm = _lines("""
    v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]
.LBB0_2:
    ;;#ASMSTART
    v_cvt_pk_bf16_f32 v0, 0, v3
    ;;#ASMEND
    """)
    assert len(b._check_asm_reads_of_mfma_results("k", asm)) == 1


def test_short_path_through_a_taken_branch_is_refused():
    # The fall-through is long enough; the branch target is reached after
    # three wait states and reads the result at once.
    asm = _lines("""
    v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]
    s_and_b64 vcc, exec, s[4:5]
    s_cbranch_vccnz .LBB0_7
    s_nop 7
    s_nop 7
    s_nop 7
.LBB0_7:
    ;;#ASMSTART
    v_max3_f32 v30, v0, v1, v2
    ;;#ASMEND
    """)
    probs = b._check_asm_reads_of_mfma_results("k", asm)
    assert len(probs) == 1 and "after 2 wait states" in probs[0]
    # The same through an unconditional branch to a label further down.
    jump = _lines("""
    v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]
    s_branch .LBB0_9
    s_nop 7
    s_nop 7
    s_nop 7
.LBB0_9:
    ;;#ASMSTART
    v_max3_f32 v30, v0, v1, v2
    ;;#ASMEND
    """)
    assert len(b._check_asm_reads_of_mfma_results("k", jump)) == 1


def test_taken_branch_with_enough_wait_states_passes():
    asm = _lines("""
    v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]
    s_cbranch_vccnz .LBB0_7
    s_waitcnt vmcnt(4)
    s_barrier
.LBB0_7:
    s_nop 7
    s_nop 7
    s_nop 4
    ;;#ASMSTART
    v_max3_f32 v30, v0, v1, v2
    ;;#ASMEND
    """)
    assert b._check_asm_reads_of_mfma_results("k", asm) == []


def test_a_later_mfma_of_the_chain_takes_over_the_count():
    # The read is far from the chain's first MFMA and close to its last: one
    # finding, against the last.
    asm = _lines("""
    v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], 0
    s_nop 7
    s_nop 7
    s_nop 7
    v_mfma_f32_32x32x16_bf16 v[0:15], v[28:31], v[32:35], v[0:15]
    ;;#ASMSTART
    v_max3_f32 v30, v0, v1, v2
    ;;#ASMEND
    """)
    probs = b._check_asm_reads_of_mfma_results("k", asm)
    assert len(probs) == 1 and "v[28:31]" in probs[0] and "after 0 wait states" in probs[0]


# ---- a VALU result feeding an inline-asm MFMA operand ------------------------

def test_valu_result_into_inline_mfma_operand():
    bad = _lines("""
    v_mov_b32 v21, v50
    ;;#ASMSTART
    v_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[24:27], a[0:15]
    ;;#ASMEND
    """)
    assert len(b._check_inline_mfma_operands("k", bad)) == 1
    ok = _lines("""
    v_mov_b32 v21, v50
    s_nop 2
    ;;#ASMSTART
    v_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[24:27], a[0:15]
    ;;#ASMEND
    """)
    assert b._check_inline_mfma_operands("k", ok) == []


# ---- M0 written right before an LDS copy ------------------------------------

def test_m0_write_before_lds_copy():
    bad = _lines("""
    s_mov_b32 m0, s4
    global_load_lds_dwordx4 v1, s[2:3] offset:1024
    """)
    assert len(b._check_m0_before_lds_copy("k", bad)) == 1
    ok = _lines("""
    s_mov_b32 m0, s4
    s_nop 0
    global_load_lds_dwordx4 v1, s[2:3] offset:1024
    """)
    assert b._check_m0_before_lds_copy("k", ok) == []


def test_register_operand_parser():
    assert b._regs("v[4:7]") == {4, 5, 6, 7}
    assert b._regs("v9") == {9}
    assert b._regs("a[0:15]") == set()
    assert b._regs("s0") == set()


# ---- packed fp32 arithmetic ----------------------------------------------------

def test_packed_fp32_arithmetic_is_refused():
    bad = _lines("""
    v_pk_mul_f32 v[0:1], v[2:3], v[4:5]
    v_pk_fma_f32 v[6:7], v[2:3], v[4:5], v[6:7]
    v_pk_add_f32 v[8:9], v[2:3], v[4:5] op_sel_hi:[1,1]
    """)
    assert len(b._check_no_packed_fp32("k", bad)) == 3
    ok = _lines("""
    v_pk_mov_b32 v[0:1], v[2:3], v[4:5] op_sel:[0,1]
    v_pk_add_f16 v0, v1, v2
    v_cvt_pk_bf16_f32 v3, v4, v5
    v_mul_f32_e32 v6, v7, v8
    """)
    assert b._check_no_packed_fp32("k", ok) == []


# ---- a VALU-written SGPR address read by an LDS copy --------------------------

def test_lds_copy_right_after_readfirstlane_of_its_address_is_refused():
    asm = _lines("""
    v_readfirstlane_b32 s8, v3
    s_mov_b32 m0, s20
    ;;#ASMSTART
    s_nop 0
    global_load_lds_dwordx4 v97, s[8:9] offset:0
    ;;#ASMEND
    """)
    probs = b._check_vmem_sgpr_after_valu("k", asm)
    assert len(probs) == 1 and "2 wait states" in probs[0]


def test_lds_copy_after_salu_address_or_enough_wait_states_passes():
    salu = _lines("""
    v_readfirstlane_b32 s8, v3
    s_lshl_b32 s10, s8, 14
    s_add_u32 s12, s4, s10
    s_addc_u32 s13, s5, 0
    global_load_lds_dwordx4 v97, s[12:13] offset:0
    """)
    # The copy reads s[12:13], written by SALU instructions only.
    assert b._check_vmem_sgpr_after_valu("k", salu) == []
    padded = _lines("""
    v_readlane_b32 s8, v3, 5
    s_nop 4
    global_load_lds_dwordx4 v97, s[8:9] offset:0x400
    """)
    assert b._check_vmem_sgpr_after_valu("k", padded) == []
    label = _lines("""
.LBB0_4:
    global_load_lds_dword v97, s[8:9]
    """)
    assert len(b._check_vmem_sgpr_after_valu("k", label)) == 1

