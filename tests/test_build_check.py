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
