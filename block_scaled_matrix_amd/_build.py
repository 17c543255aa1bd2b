"""Builds libbsm.so (the gfx950 HIP library) in place with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import tempfile

try:
    from . import _asm_audit
except ImportError:  # run as a script
    import _asm_audit

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbsm.so")
SOURCES = ["bsm_api.hip", "k_tile.hip", "k_gemm_dense.hip", "k_gemm_mx.hip", "k_gemm_mx_any.hip",
           "k_gemm_mx_mn_a.hip", "k_gemm_mx_mn_b.hip", "k_gemm_mx_mn_ab.hip", "k_diag.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -packed-fp32-ops: never emit packed fp32 arithmetic (v_pk_*_f32).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# The GEMM kernels' LDS copies read SGPR operands that inline assembly pads for itself
# (gemm_common.hpp, sgpr_base): that padding holds only if the compiler never spills and
# restores an SGPR, so their per-kernel resource report is checked for SGPR spills.
REPORT = "-Rpass-analysis=kernel-resource-usage"


def check_report(src: str, stderr: str) -> list:
    """Reads hipcc's output for one source: raises if a GEMM kernel spills SGPRs, returns the
    warnings worth showing (the host pass's note about the packed-fp32 feature excluded)."""
    kernel, shown = "?", []
    for line in stderr.splitlines():
        if "Function Name:" in line:
            kernel = line.split("Function Name:")[1].split()[0]
        elif "SGPRs Spill:" in line:
            if src.startswith("k_gemm") and int(line.split("SGPRs Spill:")[1].split()[0]):
                raise RuntimeError(f"{src}: kernel {kernel} spills SGPRs")
        elif "warning" in line and "packed-fp32-ops" not in line:
            shown.append(line)
    return shown


def _compile(src: str, obj: str) -> None:
    """Compiles one source. The GEMM sources keep their gfx950 assembly (-save-temps, which
    leaves the generated code unchanged), and the build stops if it misses a wait state that
    inline assembly must provide itself (_asm_audit)."""
    audit = src.startswith("k_gemm")
    with tempfile.TemporaryDirectory(prefix="bsm_asm_") as tmp:
        cmd = [HIPCC, *FLAGS, REPORT, *(["-save-temps"] if audit else []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        for line in check_report(src, r.stderr):
            print(line)
        if audit:
            asm = os.path.join(tmp, src[:-len(".hip")] + "-hip-amdgcn-amd-amdhsa-gfx950.s")
            with open(asm) as f:
                bad = _asm_audit.audit(f.read())
            if bad:
                raise RuntimeError(f"{src}: {len(bad)} missing wait state(s) in the assembly, e.g. {bad[0]}")


def build(jobs: int = min(8, os.cpu_count() or 4)) -> str:
    """Compile every source for gfx950 and link libbsm.so next to this file."""
    with tempfile.TemporaryDirectory(prefix="bsm_build_") as tmp:
        objs = [os.path.join(tmp, s.replace(".hip", ".o")) for s in SOURCES]
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(_compile, SOURCES, objs))
        out = LIB + ".tmp"
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
