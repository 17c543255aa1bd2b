"""CPU tests of the build's check of the compiler's per-kernel resource report: the GEMM
kernels' LDS copies pad their own SGPR wait states in inline assembly, which holds only if no
GEMM kernel spills an SGPR (a restore would be an unpadded VALU write), so the build must stop
on such a spill and pass everything else."""
import pytest

from block_scaled_matrix_amd import _build


def report(kernel, sgpr_spill, vgpr_spill=0, src="k_gemm_mx.hip"):
    pre = f"remark: block_scaled_matrix_amd/csrc/{src}:240:0:"
    tag = " [-Rpass-analysis=kernel-resource-usage]"
    return "\n".join([f"{pre} Function Name: {kernel}{tag}", f"{pre}     TotalSGPRs: 92{tag}",
                      f"{pre}     SGPRs Spill: {sgpr_spill}{tag}", f"{pre}     VGPRs Spill: {vgpr_spill}{tag}"])


def test_gemm_kernel_with_sgpr_spill_stops_the_build():
    text = report("kern_a", 0, 7) + "\n" + report("kern_b", 3)
    with pytest.raises(RuntimeError, match="kern_b spills SGPRs"):
        _build.check_report("k_gemm_mx.hip", text)


def test_clean_report_passes_and_keeps_real_warnings():
    text = "\n".join([report("kern_a", 0, 16), "warning: unknown target feature packed-fp32-ops",
                      "k_gemm_dense.hip:12:3: warning: unused variable 'x'"])
    assert _build.check_report("k_gemm_dense.hip", text) == ["k_gemm_dense.hip:12:3: warning: unused variable 'x'"]


def test_spill_outside_the_gemm_sources_is_allowed():
    # kernels without the padded LDS copies (box copies, diagnostics) may spill SGPRs
    assert _build.check_report("k_tile.hip", report("k_box_load", 4, src="k_tile.hip")) == []


def test_build_asks_the_compiler_for_the_report():
    assert _build.REPORT == "-Rpass-analysis=kernel-resource-usage"


# --- the assembly audit (block_scaled_matrix_amd/_asm_audit.py) on hand-written gfx950 snippets

from block_scaled_matrix_amd import _asm_audit  # noqa: E402


def kernel(*body):
    return "\n".join(["\t.text", "kern:"] + ["\t" + x for x in body] + ["\ts_endpgm", ".Lfunc_end0:"])


def test_copy_right_after_the_readfirstlane_of_its_base_is_flagged():
    text = kernel("v_readfirstlane_b32 s4, v1", "v_readfirstlane_b32 s5, v2", "s_mov_b32 m0, s6",
                  "global_load_lds_dwordx4 v3, s[4:5]")
    bad = _asm_audit.audit(text)
    assert any("1 wait states after a VALU write of its SGPR base" in x for x in bad), bad
    assert any("no wait state after the write of M0" in x for x in bad), bad


def test_padded_copy_passes():
    text = kernel("v_readfirstlane_b32 s4, v1", "v_readfirstlane_b32 s5, v2", "s_nop 4", "s_mov_b32 m0, s6",
                  "s_nop 0", "global_load_lds_dwordx4 v3, s[4:5]", "global_load_lds_dword v4, off")
    assert _asm_audit.audit(text) == []


def test_short_path_through_a_branch_is_found():
    # the fall-through path is long enough, the branch to the label is not
    text = kernel("v_readfirstlane_b32 s4, v1", "v_readfirstlane_b32 s5, v1", "s_cbranch_scc1 .LBB0_2",
                  "s_nop 7", "s_nop 7", ".LBB0_2:", "s_mov_b32 m0, s6", "s_nop 0",
                  "global_load_lds_dwordx4 v3, s[4:5]")
    bad = _asm_audit.audit(text)
    assert len(bad) == 1 and "3 wait states after a VALU write of its SGPR base" in bad[0], bad
    # a loop back edge: the write at the bottom of the loop reaches the copy at its top
    loop = [".LBB0_1:", "s_mov_b32 m0, s6", "s_nop 0", "global_load_lds_dwordx4 v3, s[4:5]", "s_nop 7",
            "v_readfirstlane_b32 s4, v1", "s_cbranch_scc0 .LBB0_1"]
    bad = _asm_audit.audit(kernel("s_nop 7", *loop))
    assert len(bad) == 1 and "3 wait states after a VALU write of its SGPR base" in bad[0], bad
    assert _asm_audit.audit(kernel("s_nop 7", loop[0], "s_nop 1", *loop[1:])) == []


def test_mfma_reading_a_fresh_conversion_is_flagged_and_two_wait_states_pass():
    cvt = "v_cvt_scalef32_pk32_bf16_fp6 v[0:15], v[16:21], v22"
    mfma = "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[24:27], a[0:15]"
    bad = _asm_audit.audit(kernel(cvt, mfma))
    assert len(bad) == 1 and "0 wait states after a VALU write of its A/B VGPRs" in bad[0], bad
    assert len(_asm_audit.audit(kernel(cvt, "s_nop 0", mfma))) == 1
    assert _asm_audit.audit(kernel(cvt, "s_nop 1", mfma)) == []
    # an MFMA writing the registers is not a VALU write for this rule
    assert _asm_audit.audit(kernel("v_mfma_f32_16x16x32_bf16 v[4:7], v[8:11], v[12:15], v[4:7]", mfma)) == []


def test_reading_an_mfma_result_too_soon_is_flagged():
    mfma = "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"   # 8 passes: 11 wait states
    bad = _asm_audit.audit(kernel(mfma, "s_nop 7", "v_accvgpr_read_b32 v0, a3"))
    assert len(bad) == 1 and "8 wait states after an MFMA wrote what it reads (needs 11)" in bad[0], bad
    assert _asm_audit.audit(kernel(mfma, "s_nop 7", "s_nop 2", "v_accvgpr_read_b32 v0, a3")) == []
    # a store of the result counts as a read; an untouched register does not
    assert len(_asm_audit.audit(kernel(mfma, "ds_write_b128 v1, a[0:3]"))) == 1
    assert _asm_audit.audit(kernel(mfma, "v_accvgpr_read_b32 v0, a16")) == []
    # the 16x16x32 shape (4 passes) needs 7
    m16 = "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]"
    assert len(_asm_audit.audit(kernel(m16, "s_nop 5", "v_accvgpr_read_b32 v0, a1"))) == 1
    assert _asm_audit.audit(kernel(m16, "s_nop 6", "v_accvgpr_read_b32 v0, a1")) == []


def test_block_scaled_mfma_passes_follow_the_operand_formats():
    fp8 = "v_mfma_scale_f32_32x32x64_f8f6f4 a[0:15], v[0:7], v[8:15], a[0:15], v16, v17 op_sel_hi:[0,0,0]"
    fp4 = "v_mfma_scale_f32_32x32x64_f8f6f4 a[0:15], v[0:3], v[8:11], a[0:15], v16, v17 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
    mixed = "v_mfma_scale_f32_32x32x64_f8f6f4 a[0:15], v[0:7], v[8:11], a[0:15], v16, v17 op_sel_hi:[0,0,0] blgp:4"
    wait = ["s_nop 7", "s_nop 7", "s_nop 1"]                      # 18 wait states
    assert len(_asm_audit.audit(kernel(fp8, *wait, "v_accvgpr_read_b32 v0, a3"))) == 1   # needs 19
    assert _asm_audit.audit(kernel(fp4, *wait, "v_accvgpr_read_b32 v0, a3")) == []       # needs 11
    assert len(_asm_audit.audit(kernel(mixed, *wait, "v_accvgpr_read_b32 v0, a3"))) == 1
