"""Benchmark of the block-scaled tile-matrix hot path on one MI355X.

One step runs every row of the hot path once, on seeded synthetic inputs already
resident in HBM, on one HIP stream:
  box_copy   bf16 16381x8190 (8192-element pitch), (128,64) boxes, 128-byte swizzle:
             load every box into LDS, store it to a second tensor, add-reduce it into a third
  gemm_bf16  M=N=K=8192 bf16, A K-major, B MN-major, accumulate onto float32 D
  gemm_mxfp8 M=N=8192, K=16384, E4M3 + E8M0 scales per 32 K, fresh D
  gemm_mxfp4 M=16384, N=8192, K=8192, E2M1 + E8M0 scales per 32 K, neg_a, fresh D
  add_one    the (2,32,3,4) float32 tile plus one
Prints one JSON line. `value` is the step's GEMM work (sum of 2*M*N*K of the three
GEMMs) divided by the measured step time; every kernel's own rate and roofline
fraction is in `per_kernel`, from HIP events on the launch stream.

`roofline.traffic` is the dominant kernel's measured HBM bytes per launch, read from
the committed counter summary profiles/hbm_traffic_bench_step.md (rocprofv3 FETCH_SIZE
and WRITE_SIZE, calibrated against a plain copy of known size, see --copy-calibration);
it is null when the kernel's sources no longer hash to the ones the counters were
taken with.

Rows widened beyond the step, timed after it on their own (same stream, HIP events) and
reported under `widened` (not part of `value`):
  gather4    four-row gathers from a bf16 65536x4096 table, (1,64) boxes, 128-byte swizzle,
             rows four at a time from a seeded permutation, 1 048 576 issues (512 MiB of images)
  scatter4   the images scattered to the rows of a second permutation (a row permutation of
             the table)
  box_load_rank3   a bf16 (64, 2048, 2048) tensor into (2, 64, 128) box images at element
             strides (1, 2, 1), the 32 x 32 x 16 boxes given as repeat axes (one call)
  gemm_e4m3_e2m1   block-scaled M=N=8192, K=16384, A E4M3, B E2M1 (mixed widths), fresh D
  gemm_e2m3_e2m3   block-scaled M=N=8192, K=16384, both FP6 E2M3, fresh D
  box_copy_only    the box-copy workload's call with the store alone (dst only: read src and
             write dst, 2 x 268 320 780 bytes)
  box_reduce_only  the same call with the reduce-add alone (dst_add only: read src, read and
             write dst_add, 3 x 268 320 780 bytes)
(the mixed pair runs at the 8-bit MFMA rate, peak 5033.2 TFLOP/s; FP6 pairs at the 4-bit
rate, peak 10066.3 TFLOP/s)

`context` holds reference points that are not part of the path, timed the same way after the
step: torch.mm (hipBLASLt) on the bf16 workload's shape with a fresh bf16 output, the vendor's fp8
GEMMs through torch._scaled_mm on the MXFP8 workload's codes (per-tensor scales with a float32
output, and E8M0 block scales with a bf16 output), and the ceilings the rows run against.

--epilogue silu_affine fuses the scalar epilogue f(x) = x / (1 + exp(-x)) * 2 + 1 (the example call
of "Explicit CUDA tile patterns", Scalar compositions) into the three GEMMs' stores (bsm_gemm_ewise, bsm_gemm_block_scale_ewise); the
rest of the step is unchanged, and config.epilogue names it.

--copy-calibration runs only the calibration copy: the float32 add-scalar kernel over a
1 GiB buffer (1 GiB read + 1 GiB written per launch), three launches.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"hbm_GBs": 8000.0, "bf16_TFs": 2516.6, "fp8_TFs": 5033.2, "fp4_TFs": 10066.3}
# The MFMA each GEMM row executes, and that instruction's dense peak. Block-scaled pairings
# with wide product ranges (any 8-bit operand) sum exact products with the bf16 MFMA, so
# their rate is bounded by the bf16 peak; `frac` stays against the format's own MFMA peak.
INSTRUCTION = {
    "gemm_bf16": ("v_mfma_f32_16x16x32_bf16", "bf16_TFs"),
    "gemm_mxfp8": ("v_mfma_f32_32x32x16_bf16 (exact products)", "bf16_TFs"),
    "gemm_mxfp4": ("v_mfma_scale_f32_32x32x64_f8f6f4 (fp4)", "fp4_TFs"),
    "gemm_mxfp8_fastacc": ("v_mfma_scale_f32_32x32x64_f8f6f4 (fp8)", "fp8_TFs"),
    "gemm_e4m3_e2m1": ("v_mfma_f32_32x32x16_bf16 (exact products)", "bf16_TFs"),
    "gemm_e2m3_e2m3": ("v_mfma_scale_f32_32x32x64_f8f6f4 (fp6)", "fp4_TFs"),
}

# Source files each kernel is built from (their hash ties a counter summary to the code).
_CSRC = os.path.join("block_scaled_matrix_amd", "csrc")
KERNEL_SOURCES = {
    "box_copy": ["k_tile.hip", "bsm_device.hpp"],
    "gemm_bf16": ["k_gemm_dense.hip", "gemm_common.hpp", "bsm_device.hpp"],
    "gemm_mxfp8": ["k_gemm_mx_any.hip", "gemm_mx_any.hpp", "gemm_common.hpp", "bsm_device.hpp"],
    "gemm_mxfp8_fastacc": ["k_gemm_mx.hip", "gemm_common.hpp", "bsm_device.hpp"],
    "gemm_mxfp4": ["k_gemm_mx.hip", "gemm_common.hpp", "bsm_device.hpp"],
    "add_one": ["k_tile.hip", "bsm_device.hpp"],
    "gather4": ["k_tile.hip", "bsm_device.hpp"],
    "scatter4": ["k_tile.hip", "bsm_device.hpp"],
    "box_load_rank3": ["k_tile.hip", "bsm_device.hpp"],
    "gemm_e4m3_e2m1": ["k_gemm_mx_any.hip", "gemm_mx_any.hpp", "gemm_common.hpp", "bsm_device.hpp"],
    "gemm_e2m3_e2m3": ["k_gemm_mx_any.hip", "gemm_mx_any.hpp", "gemm_common.hpp", "bsm_device.hpp"],
    "box_copy_only": ["k_tile.hip", "bsm_device.hpp"],
    "box_reduce_only": ["k_tile.hip", "bsm_device.hpp"],
}
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_bench_step.md")
MFMA_SUMMARY = os.path.join(ROOT, "profiles", "mfma_busy_bench_step.md")
CALIB_BYTES = 1 << 30
EPILOGUE_ARGS = (2.0, 1.0)   # silu_affine scale, bias


def source_hash(kernel):
    """Hash of a kernel's sources with comments and blank lines removed: an edit to the code
    makes the committed counter figures stale, an edit to its comments does not."""
    import re

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, _CSRC, f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        lines = [ln.rstrip() for ln in re.sub(r"//[^\n]*", "", text).split("\n") if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter summary, if it matches the code."""
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            for line in fh:
                # machine-readable rows: "traffic: <kernel> <bytes per launch> <source hash>"
                parts = line.split()
                if len(parts) == 4 and parts[0] == "traffic:" and parts[1] == kernel:
                    return int(parts[2]) if parts[3] == source_hash(kernel) else None
    except OSError:
        return None
    return None


def measured_mfma(kernel):
    """(MFMA busy fraction, clock GHz) from the committed counter summary, if it matches the code."""
    try:
        with open(MFMA_SUMMARY) as fh:
            for line in fh:
                # machine-readable rows: "mfma: <kernel> <busy fraction> <clock GHz> <source hash>"
                parts = line.split()
                if len(parts) == 5 and parts[0] == "mfma:" and parts[1] == kernel:
                    return (float(parts[2]), float(parts[3])) if parts[4] == source_hash(kernel) else None
    except OSError:
        return None
    return None


CALIB_K = 1 << 20   # the LDS-DMA calibration: one 256 x 256 output tile over K = 2^20 bf16


def copy_calibration():
    """Kernels of known HBM traffic for calibrating the byte counters: the float32 add-scalar copy
    (coalesced 16-byte loads and stores; 1 GiB read + 1 GiB written per launch, three launches),
    and a one-workgroup dense GEMM M = N = 256, K = 2^20 whose operands arrive only through the
    GEMMs' direct HBM->LDS copies (global_load_lds): A and B are read exactly once (512 MiB each,
    1 GiB in all) and 256 KiB of D is written."""
    import torch

    import block_scaled_matrix_amd as bsm

    n = CALIB_BYTES // 4
    src = torch.zeros(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        bsm.bsm_tile_add_scalar_f32(src, dst, n, 1.0)
    torch.cuda.synchronize()
    del src, dst
    A = torch.zeros(256 * CALIB_K, dtype=torch.int16, device="cuda")
    B = torch.zeros_like(A)
    D = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    bsm.bsm_gemm(256, 256, CALIB_K, "bf16", A, CALIB_K, "k", B, CALIB_K, "k", D, 256, 0, 0, 0)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": ["add_scalar_f32", "gemm_bf16 256x256x2^20 (global_load_lds)"],
                      "bytes_read": [CALIB_BYTES, 2 * 256 * CALIB_K * 2], "bytes_written": [CALIB_BYTES, 256 * 256 * 4],
                      "launches": [3, 1]}), flush=True)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def make_inputs():
    import numpy as np
    import torch

    from block_scaled_matrix_amd import workloads as W

    sha = {}

    def dev(a, name=None):
        a = np.ascontiguousarray(a)
        if name is not None:
            sha[name] = hashlib.sha256(a.view(np.uint8).reshape(-1)).hexdigest()[:16]
        return torch.from_numpy(a).cuda()

    def put(prefix, g):
        return {k: (dev(v, f"{prefix}.{k}") if isinstance(v, np.ndarray) else v) for k, v in g.items()}

    t0 = time.time()
    inp = {"sha256": sha}
    bc = W.box_copy_bf16()
    inp["box"] = put("box_copy", bc)
    log(f"box_copy inputs {time.time() - t0:.1f}s")
    g = W.gemm_bf16()
    inp["bf16"] = put("gemm_bf16", g)
    log(f"gemm_bf16 inputs {time.time() - t0:.1f}s")
    g = W.mxfp8()
    inp["fp8"] = put("mxfp8", g)
    inp["fp8"]["D"] = torch.empty((g["M"], g["N"]), dtype=torch.float32, device="cuda")
    log(f"mxfp8 inputs {time.time() - t0:.1f}s")
    g = W.mxfp4()
    inp["fp4"] = put("mxfp4", g)
    inp["fp4"]["D"] = torch.empty((g["M"], g["N"]), dtype=torch.float32, device="cuda")
    log(f"mxfp4 inputs {time.time() - t0:.1f}s")
    inp["add"] = dev(W.add_one_tile(), "add_one.A")
    inp["add_out"] = torch.empty_like(inp["add"])
    g = W.gather4_bf16()
    n = len(g["gather"])
    raw = torch.empty(n * 1024 + 1024, dtype=torch.uint8, device="cuda")   # 1024-byte aligned images
    off = (-raw.data_ptr()) % 1024
    inp["g4"] = {"rows": g["rows"], "cols": g["cols"], "width": g["width"], "n": n, "table": dev(g["table"]),
                 "gather": dev(g["gather"].reshape(-1)), "scatter": dev(g["scatter"].reshape(-1)),
                 "images": raw[off:off + n * 1024], "dst": torch.empty((g["rows"], g["cols"]), dtype=torch.int16,
                                                                       device="cuda")}
    log(f"gather4 inputs {time.time() - t0:.1f}s")
    for key, (af, bf, seed) in {"mix": ("e4m3", "e2m1", 21), "fp6": ("e2m3", "e2m3", 22)}.items():
        g = W.mx_pair(seed, 8192, 8192, 16384, af, bf)
        inp[key] = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in g.items()}
        inp[key]["D"] = torch.empty((8192, 8192), dtype=torch.float32, device="cuda")
    log(f"mixed / fp6 GEMM inputs {time.time() - t0:.1f}s")
    b3 = W.box_rank3_bf16()
    inp["b3"] = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in b3.items()}
    n3 = int(np.prod(b3["repeats"]))
    img3 = 2 * 32 * 128 * 2                     # (2, 32, 128) bf16 image, already a multiple of 128 bytes
    raw3 = torch.empty(n3 * img3 + 1024, dtype=torch.uint8, device="cuda")
    off3 = (-raw3.data_ptr()) % 1024
    inp["b3"]["images"] = raw3[off3:off3 + n3 * img3]
    log(f"rank-3 box inputs {time.time() - t0:.1f}s")
    return inp


def kernels(inp, epilogue="none"):
    """(name, launch callable, work, unit, peak) for each row of the step."""
    import block_scaled_matrix_amd as bsm

    if epilogue == "none":
        gemm, gemm_bs = bsm.bsm_gemm, bsm.bsm_gemm_block_scale
    else:
        ew = bsm.ewise_desc(epilogue, *EPILOGUE_ARGS)
        gemm = lambda *a: bsm.bsm_gemm_ewise(*a, ew=ew)
        gemm_bs = lambda *a: bsm.bsm_gemm_block_scale_ewise(*a, ew=ew)

    b = inp["box"]
    rows, cols, pitch = b["rows"], b["cols"], b["pitch"]
    st = (pitch * 2, 2)
    td = lambda t: bsm.tensor_desc(t, "bf16", (rows, cols), st)
    src, dst, add = td(b["src"]), td(b["dst"]), td(b["dst_add"])
    box = bsm.box_desc(b["box"], (1, 1), 3, 0)
    box_bytes = 4 * rows * cols * 2            # read src + write dst + read/write dst_add (logical elements)

    g = inp["bf16"]
    M, N, K = g["M"], g["N"], g["K"]
    f8, f4 = inp["fp8"], inp["fp4"]
    ks = [
        ("box_copy", lambda: bsm.bsm_tile_box_copy(src, dst, add, box), box_bytes, "GB/s", PEAK["hbm_GBs"]),
        ("gemm_bf16", lambda: gemm(M, N, K, "bf16", g["A"], K, "k", g["B"], N, "n", g["D0"], N, 0, 0, 1),
         2.0 * M * N * K, "TFLOP/s", PEAK["bf16_TFs"]),
        ("gemm_mxfp8", lambda: gemm_bs(
            f8["M"], f8["N"], f8["K"], "e4m3", f8["A"], f8["lda"], f8["SFA"], f8["ld_sfa"], "e4m3", f8["B"], f8["ldb"],
            f8["SFB"], f8["ld_sfb"], f8["D"], f8["N"], 0, 0, 0), 2.0 * f8["M"] * f8["N"] * f8["K"], "TFLOP/s",
         PEAK["fp8_TFs"]),
        ("gemm_mxfp4", lambda: gemm_bs(
            f4["M"], f4["N"], f4["K"], "e2m1", f4["A"], f4["lda"], f4["SFA"], f4["ld_sfa"], "e2m1", f4["B"], f4["ldb"],
            f4["SFB"], f4["ld_sfb"], f4["D"], f4["N"], 1, 0, 0), 2.0 * f4["M"] * f4["N"] * f4["K"], "TFLOP/s",
         PEAK["fp4_TFs"]),
        ("add_one", lambda: bsm.bsm_tile_add_scalar_f32(inp["add"], inp["add_out"], 768, 1.0), 2 * 768 * 4, "GB/s",
         PEAK["hbm_GBs"]),
    ]
    return ks


def widened(inp):
    """(name, launch callable, work, unit, peak) for the rows timed beside the step."""
    import block_scaled_matrix_amd as bsm

    g = inp["g4"]
    rows, cols, n = g["rows"], g["cols"], g["n"]
    box = bsm.box_desc((1, g["width"]), (1, 1), 3, 0)
    src = bsm.tensor_desc(g["table"], "bf16", (rows, cols), (cols * 2, 2))
    dst = bsm.tensor_desc(g["dst"], "bf16", (rows, cols), (cols * 2, 2))
    nbytes = 2 * rows * cols * 2                 # every table byte read once and written once (as image bytes)

    def mx(key, call=bsm.bsm_gemm_block_scale):
        x = inp[key]
        return lambda: call(x["M"], x["N"], x["K"], x["fmt"], x["A"], x["lda"], x["SFA"], x["ld_sfa"], x["b_fmt"],
                            x["B"], x["ldb"], x["SFB"], x["ld_sfb"], x["D"], x["N"], 0, 0, 0)
    flops = 2.0 * 8192 * 8192 * 16384
    b3 = inp["b3"]
    d3 = b3["dims"]
    t3 = bsm.tensor_desc(b3["x"], "bf16", d3, (d3[1] * d3[2] * 2, d3[2] * 2, 2))
    bx3 = bsm.box_desc(b3["box"], b3["estr"], 0, 0)
    bytes3 = 2 * (d3[0] * d3[1] // 2 * d3[2] * 2)   # the sampled half of the rows read, written as images
    b = inp["box"]
    brows, bcols, bpitch = b["rows"], b["cols"], b["pitch"]
    btd = lambda t: bsm.tensor_desc(t, "bf16", (brows, bcols), (bpitch * 2, 2))
    bbox = bsm.box_desc(b["box"], (1, 1), 3, 0)
    belem = brows * bcols * 2                    # bytes of one tensor's logical elements
    return [
        ("box_copy_only", lambda: bsm.bsm_tile_box_copy(btd(b["src"]), btd(b["dst"]), None, bbox), 2 * belem, "GB/s",
         PEAK["hbm_GBs"]),
        ("box_reduce_only", lambda: bsm.bsm_tile_box_copy(btd(b["src"]), None, btd(b["dst_add"]), bbox), 3 * belem,
         "GB/s", PEAK["hbm_GBs"]),
        ("box_load_rank3", lambda: bsm.bsm_tile_box_load_steps(t3, bx3, b3["coords"], b3["repeats"], b3["steps"],
                                                               b3["images"]), bytes3, "GB/s", PEAK["hbm_GBs"]),
        ("gather4", lambda: bsm.bsm_tile_gather4(src, box, g["gather"], n, g["images"]), nbytes, "GB/s",
         PEAK["hbm_GBs"]),
        ("scatter4", lambda: bsm.bsm_tile_scatter4(dst, box, g["scatter"], n, g["images"]), nbytes, "GB/s",
         PEAK["hbm_GBs"]),
        ("gemm_e4m3_e2m1", mx("mix"), flops, "TFLOP/s", PEAK["fp8_TFs"]),
        ("gemm_e2m3_e2m3", mx("fp6"), flops, "TFLOP/s", PEAK["fp4_TFs"]),
        # the MXFP8 workload through the fast-accumulation call (scaled fp8 MFMA, its 2^-13
        # block window: outside the stated bound on these operands)
        ("gemm_mxfp8_fastacc", mx("fp8", bsm.bsm_gemm_block_scale_fastacc), 2.0 * 8192 * 8192 * 16384, "TFLOP/s",
         PEAK["fp8_TFs"]),
    ]


def vendor_fp8(inp, steps, stream):
    """Context rows: the vendor library's fp8 GEMMs (torch._scaled_mm -> hipBLASLt) on the MXFP8
    workload's operand codes, as reference points outside the path: per-tensor unit scales with a
    float32 output, and the E8M0 block scales with a bfloat16 output (its block-scaled path writes
    only bf16 or f16). The first also reports its sum on a 16-row sample against a float64 torch
    (CPU) product of the decoded codes, under the 1e-5 * sum|ab| bound: the scaled fp8 MFMA's
    block window shows there too. Rows whose call the installed torch does not support are left
    out."""
    import torch

    f8 = inp["fp8"]
    M, N, K = f8["M"], f8["N"], f8["K"]
    try:
        A = f8["A"].view(torch.float8_e4m3fn).reshape(M, K)
        B = f8["B"].view(torch.float8_e4m3fn).reshape(N, K)
        one = torch.ones((), device="cuda")
        SA = f8["SFA"].view(torch.float8_e8m0fnu).reshape(M, -1)[:, :K // 32]
        SB = f8["SFB"].view(torch.float8_e8m0fnu).reshape(N, -1)[:, :K // 32]
    except (AttributeError, RuntimeError) as e:
        log(f"vendor fp8 rows skipped: {e}")
        return {}
    rows = [("torch_scaled_mm_fp8", lambda: torch._scaled_mm(A, B.t(), scale_a=one, scale_b=one,
                                                             out_dtype=torch.float32),
             "hipBLASLt fp8 GEMM through torch._scaled_mm on the MXFP8 workload's E4M3 codes, per-tensor unit "
             "scales (not block-scaled), float32 output"),
            ("torch_scaled_mm_mxfp8", lambda: torch._scaled_mm(A, B.t(), scale_a=SA.contiguous(),
                                                               scale_b=SB.contiguous(), out_dtype=torch.bfloat16),
             "hipBLASLt block-scaled fp8 GEMM through torch._scaled_mm on the MXFP8 workload (E8M0 scales passed "
             "as (rows, K/32)), bfloat16 output (the only widths its block-scaled path writes)")]
    out = {}
    flop = 2.0 * M * N * K
    for name, fn, note in rows:
        try:
            fn()
            torch.cuda.synchronize()
        except (RuntimeError, ValueError, TypeError) as e:
            log(f"{name} (context) skipped: {str(e)[:200]}")
            continue
        ms = time_launches([(name, fn, flop, "TFLOP/s", PEAK["fp8_TFs"])], steps, stream)[0]
        out[name] = rate_entry(ms, flop, "TFLOP/s", PEAK["fp8_TFs"])
        out[name]["note"] = note
        log(f"{name} (context): {ms:.4f} ms  {out[name]['achieved']:.1f} TFLOP/s")
    if "torch_scaled_mm_fp8" in out:
        r = 16
        D = rows[0][1]()[:r].double().cpu()
        a = A[:r].cpu().to(torch.float64)
        b = B.cpu().to(torch.float64)
        ref, bound = a @ b.T, a.abs() @ b.abs().T
        ratio = ((D - ref).abs() / bound)
        out["torch_scaled_mm_fp8"]["parity_sample"] = {
            "sample": f"rows 0..{r - 1}, all columns, against float64 torch (CPU) on the decoded codes",
            "tol_sum_abs_ab": 1e-5, "n_bad": int((ratio > 1e-5).sum()), "worst_err_over_sum_abs_ab": ratio.max().item()}
    return out


MFMA_LOOP = {"bf16": (800, 32768), "e4m3": (400, 131072), "e2m1": (800, 131072)}   # iters, FLOP per MFMA
LOOP_WGS = 1024
UNRAGGED_ROWS = 16256      # 127 box rows of 128: no ragged edge along either axis


def ceilings(inp):
    """(name, launch, work, unit, peak, note) of the diagnostic rows in `context`."""
    import torch

    import block_scaled_matrix_amd as bsm

    b = inp["box"]
    rows, cols, pitch = b["rows"], b["cols"], b["pitch"]
    n = rows * pitch                                   # every element of the three buffers, padding included
    st = (pitch * 2, 2)
    td = lambda t: bsm.tensor_desc(t, "bf16", (UNRAGGED_ROWS, pitch), st)
    box = bsm.box_desc(b["box"], (1, 1), 3, 0)
    out = inp.setdefault("loop_out", torch.empty(LOOP_WGS * 256, dtype=torch.float32, device="cuda"))
    rows_ = [
        ("stream_mix_bf16", lambda: bsm.bsm_debug_stream_mix_bf16(b["src"], b["dst"], b["dst_add"], n), 4 * 2 * n,
         "GB/s", PEAK["hbm_GBs"], "the box copy's traffic mix (read src, write dst, read and write dst_add) on the "
         "three flat 16381 x 8192 bf16 buffers, 16-byte non-temporal accesses, no boxes: the stream ceiling of the mix"),
        ("box_copy_unragged", lambda: bsm.bsm_tile_box_copy(td(b["src"]), td(b["dst"]), td(b["dst_add"]), box),
         4 * UNRAGGED_ROWS * pitch * 2, "GB/s", PEAK["hbm_GBs"],
         "bsm_tile_box_copy on a 16256 x 8192 view of the same buffers ((128, 64) boxes, 128-byte swizzle): "
         "the workload's kernel with no ragged box row or column"),
    ]
    for kind, peak in (("bf16", PEAK["bf16_TFs"]), ("e4m3", PEAK["fp8_TFs"]), ("e2m1", PEAK["fp4_TFs"])):
        iters, fl = MFMA_LOOP[kind]
        rows_.append((f"mfma_loop_{kind}", (lambda k=kind, it=iters: bsm.bsm_debug_mfma_loop(k, LOOP_WGS, it, out)),
                      float(LOOP_WGS * 4 * iters * 16 * fl), "TFLOP/s", peak,
                      f"back-to-back {kind} MFMAs on random register operands, 16 accumulators per wave, "
                      f"{LOOP_WGS} workgroups x {iters} iterations, no memory traffic: the matrix-pipe ceiling "
                      "under the clock the device holds for that load"))
    return rows_


def time_launches(ks, steps, stream):
    """Average HIP-event time (ms) of each launch in ks over `steps` rounds, on `stream`."""
    import torch

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ks]
          for _ in range(steps)]
    for s in range(steps):
        for i, (_, fn, *_) in enumerate(ks):
            ev[s][i][0].record(stream)
            fn()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    return [sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)) / steps for i in range(len(ks))]


def rate_entry(ms, work, unit, peak, name=None):
    rate = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
    e = {"ms": round(ms, 4), "achieved": round(rate, 1), "unit": unit, "peak": peak,
         "frac": round(rate / peak, 4), "work_per_launch": work}
    if name in INSTRUCTION:
        ins, key = INSTRUCTION[name]
        e["instruction"], e["instruction_peak"] = ins, PEAK[key]
        e["instruction_frac"] = round(rate / PEAK[key], 4)
    return e


def cpu_baseline(inp):
    """The oracle, as it stands, on a bounded sample of the same workloads. Its rows also give
    the GPU's parity on that sample: each call is launched once more on fresh outputs (the timed
    steps accumulate into the bf16 D and the reduce-add target) and compared element by element
    with the oracle, under the bound each row states (bf16: 2e-3 * sum|ab|, block scaled:
    1e-5 * sum|ab|, both plus half an ulp of the float32 result; box copy: bit for bit)."""
    import numpy as np
    import torch

    import block_scaled_matrix_amd as bsm
    from block_scaled_matrix_amd import workloads as W
    from oracle import oracle as O

    O.lib()
    flops = 0.0
    t_gemm = 0.0
    parity = {}
    per_cfg = {}

    def timed(name, rows, fl, t):
        per_cfg[name] = {"rows": rows, "s": round(t, 2), "TFLOP/s": fl / t / 1e12}

    def gemm_parity(name, D, ref, bound, tol, sample):
        nb, _, worst = O.check_gemm(np.ascontiguousarray(D, np.float32), ref, bound, tol)
        parity[name] = {"sample": sample, "tol_sum_abs_ab": tol, "n_bad": nb, "worst_err_over_sum_abs_ab": worst}

    # row counts sized for about 10-15 s of the oracle's time on 16 host cores
    rows_bf16, rows_fp8, rows_fp4 = 64, 16, 32
    g = W.gemm_bf16()
    rows = rows_bf16
    t0 = time.perf_counter()
    ref, bound = O.gemm(g["M"], g["N"], g["K"], "bf16", g["A"], g["K"], "k", g["B"], g["N"], "n", g["D0"], g["N"], 0,
                        0, 1, 0, rows)
    dt = time.perf_counter() - t0
    t_gemm += dt
    flops += 2.0 * rows * g["N"] * g["K"]
    timed("gemm_bf16", rows, 2.0 * rows * g["N"] * g["K"], dt)
    x = inp["bf16"]
    D = torch.from_numpy(g["D0"][:rows].copy()).cuda()   # the first rows of D0, accumulated once
    bsm.bsm_gemm(rows, x["N"], x["K"], "bf16", x["A"], x["K"], "k", x["B"], x["N"], "n", D, x["N"], 0, 0, 1)
    gemm_parity("gemm_bf16", D.cpu().numpy(), ref, bound, 2e-3, f"rows 0..{rows - 1}, all columns")
    del g
    g = W.mxfp8()
    rows = rows_fp8
    t0 = time.perf_counter()
    ref, bound = O.gemm_block_scale(g["M"], g["N"], g["K"], "e4m3", g["A"], g["K"], g["SFA"], g["ld_sfa"], "e4m3",
                                    g["B"], g["K"], g["SFB"], g["ld_sfb"], None, 0, 0, 0, 0, 0, rows)
    dt = time.perf_counter() - t0
    t_gemm += dt
    flops += 2.0 * rows * g["N"] * g["K"]
    timed("gemm_mxfp8", rows, 2.0 * rows * g["N"] * g["K"], dt)
    x = inp["fp8"]
    x["D"].fill_(float("nan"))
    bsm.bsm_gemm_block_scale(x["M"], x["N"], x["K"], "e4m3", x["A"], x["lda"], x["SFA"], x["ld_sfa"], "e4m3", x["B"],
                             x["ldb"], x["SFB"], x["ld_sfb"], x["D"], x["N"], 0, 0, 0)
    gemm_parity("gemm_mxfp8", x["D"][:rows].cpu().numpy(), ref, bound, 1e-5, f"rows 0..{rows - 1}, all columns")
    x["D"].fill_(float("nan"))
    bsm.bsm_gemm_block_scale_fastacc(x["M"], x["N"], x["K"], "e4m3", x["A"], x["lda"], x["SFA"], x["ld_sfa"], "e4m3",
                                     x["B"], x["ldb"], x["SFB"], x["ld_sfb"], x["D"], x["N"], 0, 0, 0)
    gemm_parity("gemm_mxfp8_fastacc", x["D"][:rows].cpu().numpy(), ref, bound, 1e-5,
                f"rows 0..{rows - 1}, all columns (fast accumulation: not expected within the bound)")
    del g
    g = W.mxfp4()
    rows = rows_fp4
    t0 = time.perf_counter()
    ref, bound = O.gemm_block_scale(g["M"], g["N"], g["K"], "e2m1", g["A"], g["K"], g["SFA"], g["ld_sfa"], "e2m1",
                                    g["B"], g["K"], g["SFB"], g["ld_sfb"], None, 0, 1, 0, 0, 0, rows)
    dt = time.perf_counter() - t0
    t_gemm += dt
    flops += 2.0 * rows * g["N"] * g["K"]
    timed("gemm_mxfp4", rows, 2.0 * rows * g["N"] * g["K"], dt)
    x = inp["fp4"]
    x["D"].fill_(float("nan"))
    bsm.bsm_gemm_block_scale(x["M"], x["N"], x["K"], "e2m1", x["A"], x["lda"], x["SFA"], x["ld_sfa"], "e2m1", x["B"],
                             x["ldb"], x["SFB"], x["ld_sfb"], x["D"], x["N"], 1, 0, 0)
    gemm_parity("gemm_mxfp4", x["D"][:rows].cpu().numpy(), ref, bound, 1e-5, f"rows 0..{rows - 1}, all columns")
    del g
    # box round trip on a 1024-row band of the copy workload (128 boxes wide)
    b = W.box_copy_bf16(rows=1024)
    st = (b["pitch"] * 2, 2)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ds, dd, da = dev(b["src"]), dev(b["dst"]), dev(b["dst_add"])
    td = lambda t: bsm.tensor_desc(t, "bf16", (1024, b["cols"]), st)
    bsm.bsm_tile_box_copy(td(ds), td(dd), td(da), bsm.box_desc(b["box"], (1, 1), 3, 0))
    t0 = time.perf_counter()
    O.box_copy_grid(b["src"], b["dst"], b["dst_add"], "bf16", (1024, b["cols"]), st, b["box"], (1, 1), 3, 0)
    t_box = time.perf_counter() - t0
    box_gbs = 4 * 1024 * b["cols"] * 2 / t_box / 1e9
    same = (np.array_equal(dd.cpu().numpy(), b["dst"]), np.array_equal(da.cpu().numpy(), b["dst_add"]))
    parity["box_copy"] = {"sample": "a 1024x8190 band (128 boxes wide), store and reduce-add, padding included",
                          "bit_exact": bool(all(same))}
    base = {"value": flops / t_gemm / 1e12, "unit": "TFLOP/s", "cores": O.num_threads(), "kind": "oracle",
            "host": host_cpu(),
            "sample": f"GEMM rows: bf16 {rows_bf16} of 8192, mxfp8 {rows_fp8} of 8192, mxfp4 {rows_fp4} of 16384 "
                      f"(full N and K), "
                      f"{t_gemm:.1f} s; box copy on a 1024x8190 band: {box_gbs:.3f} GB/s in {t_box:.1f} s",
            "box_copy_GBs": box_gbs,
            "per_config": dict(per_cfg, box_copy={"rows": 1024, "s": round(t_box, 2), "GB/s": box_gbs})}
    return base, parity


def host_cpu():
    """The host CPU the oracle ran on: its model name and the cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "cores_allowed": len(os.sched_getaffinity(0))}


# rocprofv3 kernel names -> bench row names (first match wins). Two k_box_copy2d groups are
# told apart by their grid: the workload's (16381 rows) has more workgroups than the
# unragged 16256-row view.
NAME_RULES = [
    (r"k_gemm_dense<4, true, false, true>", "gemm_bf16"),
    (r"k_gemm_mx_any<0, 0, false, false, true>", "gemm_mxfp8"),
    (r"k_gemm_mx<0, 0, 0, false>", "gemm_mxfp8_fastacc"),
    (r"k_gemm_mx<4, 4, 4, false>", "gemm_mxfp4"),
    (r"k_gemm_mx_any<0, 4, false, false, true>", "gemm_e4m3_e2m1"),
    (r"k_gemm_mx_any<2, 2, false, false, false>", "gemm_e2m3_e2m3"),
    (r"k_row4<false>", "gather4"),
    (r"k_row4<true>", "scatter4"),
    (r"k_box_load\(", "box_load_rank3"),
    (r"k_add_scalar_f32", "add_one"),
    (r"k_stream_mix_bf16", "stream_mix_bf16"),
    (r"k_mfma_loop<4>", "mfma_loop_bf16"),
    (r"k_mfma_loop<6>", "mfma_loop_e4m3"),
    (r"k_mfma_loop<7>", "mfma_loop_e2m1"),
    (r"k_box_copy2d<0, true>", "box_copy_only"),
    (r"k_box_copy2d<4, false>", "box_reduce_only"),
    (r"k_box_copy2d<4, true>", "box_copy*"),
]
# Algorithmic HBM bytes per launch of the GEMMs: operands once, D written (and read when
# accumulating), scales once.
ALG_BYTES = {
    "gemm_bf16": 2 * 8192 * 8192 * 2 + 2 * 8192 * 8192 * 4,
    "gemm_mxfp8": 2 * 8192 * 16384 + 2 * 8192 * 512 + 8192 * 8192 * 4,
    "gemm_mxfp8_fastacc": 2 * 8192 * 16384 + 2 * 8192 * 512 + 8192 * 8192 * 4,
    "gemm_mxfp4": 16384 * 4096 + 8192 * 4096 + 16384 * 256 + 8192 * 256 + 16384 * 8192 * 4,
    "gemm_e4m3_e2m1": 8192 * 16384 + 8192 * 8192 + 2 * 8192 * 512 + 8192 * 8192 * 4,
    "gemm_e2m3_e2m3": 2 * 8192 * 12288 + 2 * 8192 * 512 + 8192 * 8192 * 4,
}
# Work per launch (FLOP or algorithmic bytes), the same figures the timed run uses.
STATIC_WORK = {
    "box_copy": (4 * 16381 * 8190 * 2, "GB/s", PEAK["hbm_GBs"]),
    "box_copy_unragged": (4 * UNRAGGED_ROWS * 8192 * 2, "GB/s", PEAK["hbm_GBs"]),
    "box_copy_only": (2 * 16381 * 8190 * 2, "GB/s", PEAK["hbm_GBs"]),
    "box_reduce_only": (3 * 16381 * 8190 * 2, "GB/s", PEAK["hbm_GBs"]),
    "stream_mix_bf16": (4 * 2 * 16381 * 8192, "GB/s", PEAK["hbm_GBs"]),
    "gemm_bf16": (2.0 * 8192 ** 3, "TFLOP/s", PEAK["bf16_TFs"]),
    "gemm_mxfp8": (2.0 * 8192 * 8192 * 16384, "TFLOP/s", PEAK["fp8_TFs"]),
    "gemm_mxfp8_fastacc": (2.0 * 8192 * 8192 * 16384, "TFLOP/s", PEAK["fp8_TFs"]),
    "gemm_mxfp4": (2.0 * 16384 * 8192 * 8192, "TFLOP/s", PEAK["fp4_TFs"]),
    "gemm_e4m3_e2m1": (2.0 * 8192 * 8192 * 16384, "TFLOP/s", PEAK["fp8_TFs"]),
    "gemm_e2m3_e2m3": (2.0 * 8192 * 8192 * 16384, "TFLOP/s", PEAK["fp4_TFs"]),
    "gather4": (2 * 65536 * 4096 * 2, "GB/s", PEAK["hbm_GBs"]),
    "scatter4": (2 * 65536 * 4096 * 2, "GB/s", PEAK["hbm_GBs"]),
    "box_load_rank3": (2 * (64 * 2048 // 2 * 2048 * 2), "GB/s", PEAK["hbm_GBs"]),
    "add_one": (2 * 768 * 4, "GB/s", PEAK["hbm_GBs"]),
}
for _k, (_it, _fl) in MFMA_LOOP.items():
    STATIC_WORK[f"mfma_loop_{_k}"] = (float(LOOP_WGS * 4 * _it * 16 * _fl), "TFLOP/s",
                                      PEAK[{"bf16": "bf16_TFs", "e4m3": "fp8_TFs", "e2m1": "fp4_TFs"}[_k]])


def _profile_groups(rows, steps):
    """rows: (kernel name, grid, start, end, extra) per dispatch. Groups them by (bench name, grid),
    keeps each group's last `steps` dispatches (the timed launches: the bench issues every row's
    untimed launches first) and returns {bench name: [(start, end, extra), ...]}, plus a log."""
    import re
    groups = {}
    for name, grid, t0, t1, extra in rows:
        bench = None
        for rx, bn in NAME_RULES:
            if re.search(rx, name):
                bench = bn
                break
        if bench is None:
            continue
        groups.setdefault((bench, grid), []).append((t0, t1, extra, name))
    boxes = sorted((g for g in groups if g[0] == "box_copy*"), key=lambda g: -g[1])
    out, names = {}, {}
    for key, lst in groups.items():
        bench = key[0]
        if bench == "box_copy*":
            bench = "box_copy" if key == boxes[0] else "box_copy_unragged"
        lst.sort()
        kept = lst[-steps:] if steps else lst
        out[bench] = [(a, b, e) for a, b, e, _ in kept]
        names[bench] = (lst[0][3], key[1], len(lst), len(kept))
    return out, names


def summarize(dirs, steps, calib=None):
    """Markdown summaries of rocprofv3 CSV output (kernel trace and/or counter collection)
    under `dirs`, over each row's timed launches only (its last `steps` dispatches)."""
    import csv
    import glob

    def rd(pattern):
        fs = []
        for d in dirs:
            fs += glob.glob(os.path.join(d, "**", pattern), recursive=True)
        out = []
        for f in fs:
            with open(f) as fh:
                out += list(csv.DictReader(fh))
        return out

    trace = rd("*kernel_trace.csv")
    if trace:
        rows = [(r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
                 int(r["Start_Timestamp"]), int(r["End_Timestamp"]), None) for r in trace]
        g, names = _profile_groups(rows, steps)
        print("| bench name | kernel | workgroups | launches (kept / all) | mean us | min us | max us | achieved | frac |")
        print("|---|---|---|---|---|---|---|---|---|")
        for bench in sorted(g, key=lambda b: -sum(e - s for s, e, _ in g[b])):
            d = [(e - s) / 1e3 for s, e, _ in g[bench]]
            mean = sum(d) / len(d)
            kname, grid, nall, nkept = names[bench]
            work, unit, peak = STATIC_WORK.get(bench, (None, "", None))
            ach = f"{work / (mean * 1e-6) / (1e12 if unit == 'TFLOP/s' else 1e9):.1f} {unit}" if work else ""
            frac = f"{work / (mean * 1e-6) / (1e12 if unit == 'TFLOP/s' else 1e9) / peak:.4f}" if work else ""
            print(f"| {bench} | `{kname[:60]}` | {grid // 256} | {nkept} / {nall} | {mean:.1f} | {min(d):.1f} | "
                  f"{max(d):.1f} | {ach} | {frac} |")
    # counters: one rocprofv3 pass per directory (each pass its own process); per row, the mean
    # of each counter over its timed dispatches, merged over the passes
    means, durs, kept = {}, {}, {}
    for d in dirs:
        cc = rd_dir(d)
        if not cc:
            continue
        per = {}
        for r in cc:
            key = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
            per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
        g, _ = _profile_groups([(k[0], k[1], k[2], k[3], v) for k, v in per.items()], steps)
        for bench, lst in g.items():
            for c in {c for x in lst for c in x[2]}:
                means.setdefault(bench, {})[c] = sum(x[2].get(c, 0.0) for x in lst) / len(lst)
            durs.setdefault(bench, []).append(sum(e - s for s, e, _ in lst) / len(lst))
            kept[bench] = len(lst)
    if means:
        cal = {"FETCH_SIZE": 1.0, "WRITE_SIZE": 1.0}
        if calib:
            # true KiB per dispatch of each calibration kernel, per counter
            truth = {"FETCH_SIZE": {"k_add_scalar_f32": CALIB_BYTES / 1024, "k_gemm_dense": 2 * 256 * CALIB_K * 2 / 1024},
                     "WRITE_SIZE": {"k_add_scalar_f32": CALIB_BYTES / 1024, "k_gemm_dense": 256 * 256 * 4 / 1024}}
            print("| counter | calibration kernel | dispatches | counter KiB (mean) | true KiB | true / counter |")
            print("|---|---|---|---|---|---|")
            for c, dirc in calib.items():
                for kern, true_kib in truth[c].items():
                    vals = [float(r["Counter_Value"]) for r in rd_dir(dirc)
                            if r["Counter_Name"] == c and kern in r["Kernel_Name"]]
                    if not vals:
                        continue
                    f = true_kib / (sum(vals) / len(vals))
                    if kern == "k_add_scalar_f32":
                        cal[c] = f
                    print(f"| {c} | {kern} | {len(vals)} | {sum(vals) / len(vals):.0f} | {true_kib:.0f} | {f:.4f} |")
            print("\nfactors applied below (the plain copy's): " + ", ".join(f"{c} {v:.4f}" for c, v in cal.items()) +
                  "\n")
        counters = sorted({c for v in means.values() for c in v})
        print("| bench name | launches kept | mean us | " + " | ".join(counters) + " | derived |")
        print("|---|---|---|" + "---|" * len(counters) + "---|")
        machine = []
        for bench in sorted(means):
            mean = means[bench]
            dur = sum(durs[bench]) / len(durs[bench])   # ns
            der = []
            if mean.get("GRBM_GUI_ACTIVE", 0) > 0:
                cyc = mean["GRBM_GUI_ACTIVE"] / 8
                clock = cyc / dur
                der.append(f"clock {clock:.2f} GHz")
                if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                    busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cyc)
                    der.append(f"MFMA busy {busy:.3f}")
                    if bench in KERNEL_SOURCES and busy > 0:
                        machine.append(f"mfma: {bench} {busy:.4f} {clock:.4f} {source_hash(bench)}")
            if "SQ_LDS_BANK_CONFLICT" in mean and "SQ_LDS_IDX_ACTIVE" in mean:
                act, con = mean["SQ_LDS_IDX_ACTIVE"], mean["SQ_LDS_BANK_CONFLICT"]
                der.append(f"conflict ratio {con / max(act - con, 1):.3f}")
            if "SQ_WAIT_INST_LDS" in mean and mean.get("SQ_WAVE_CYCLES", 0) > 0:
                der.append(f"LDS-issue wait {4 * mean['SQ_WAIT_INST_LDS'] / mean['SQ_WAVE_CYCLES']:.3f}")
            if "FETCH_SIZE" in mean and "WRITE_SIZE" in mean:
                b = int(round((mean["FETCH_SIZE"] * cal["FETCH_SIZE"] + mean["WRITE_SIZE"] * cal["WRITE_SIZE"]) * 1024))
                alg = STATIC_WORK.get(bench)
                if alg and alg[1] == "GB/s":
                    der.append(f"HBM bytes {b} ({b / alg[0]:.2f}x algorithmic)")
                elif bench in ALG_BYTES:
                    der.append(f"HBM bytes {b} ({b / ALG_BYTES[bench]:.2f}x algorithmic {ALG_BYTES[bench]})")
                else:
                    der.append(f"HBM bytes {b}")
                if bench in KERNEL_SOURCES:
                    machine.append(f"traffic: {bench} {b} {source_hash(bench)}")
            print(f"| {bench} | {kept[bench]} | {dur / 1e3:.1f} | " + " | ".join(f"{mean.get(c, 0.0):.4g}" for c in counters) +
                  " | " + "; ".join(der) + " |")
        if machine:
            print("\nMachine-readable rows for bench.py (mfma: kernel, MFMA busy, clock GHz, source hash; traffic: "
                  "kernel, HBM bytes per launch, source hash; the hash covers the kernel's sources without "
                  "comments):\n\n```")
            print("\n".join(machine))
            print("```")


def rd_dir(d):
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            out += list(csv.DictReader(fh))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--epilogue", choices=["none", "silu_affine"], default="none",
                    help="scalar epilogue fused into the GEMMs' stores")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the plain copy of known size used to calibrate the HBM byte counters")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="print markdown summaries of rocprofv3 CSV output under DIR (kernel trace, counters) over "
                         "each row's timed launches (the last --steps dispatches of each kernel); no GPU needed")
    ap.add_argument("--calib-fetch", metavar="DIR", help="with --summarize: FETCH_SIZE run of --copy-calibration")
    ap.add_argument("--calib-write", metavar="DIR", help="with --summarize: WRITE_SIZE run of --copy-calibration")
    args = ap.parse_args()
    if args.summarize:
        calib = {}
        if args.calib_fetch:
            calib["FETCH_SIZE"] = args.calib_fetch
        if args.calib_write:
            calib["WRITE_SIZE"] = args.calib_write
        summarize(args.summarize, args.steps, calib or None)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); every workload here fits one MI355X and "
              "no multi-GPU path is part of this library.", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_scaled_matrix_amd as bsm
    bsm.lib()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    inp = make_inputs()
    ks = kernels(inp, args.epilogue)
    stream = torch.cuda.current_stream()

    def step():
        for _, fn, *_ in ks:
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ks]
          for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        for i, (_, fn, *_) in enumerate(ks):
            ev[s][i][0].record(stream)
            fn()
            ev[s][i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    log(f"timed {args.steps} steps: {ms_total:.2f} ms (wall {wall * 1e3:.1f} ms)")

    per = {}
    for i, (name, _, work, unit, peak) in enumerate(ks):
        ms = sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)) / args.steps
        rate = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        per[name] = rate_entry(ms, work, unit, peak, name)
        per[name]["traffic"] = measured_traffic(name)
        mf = measured_mfma(name)
        if mf is not None:   # counter figures of the same kernel sources (profiles/mfma_busy_bench_step.md)
            per[name]["mfma_busy"], per[name]["clock_ghz"] = mf
        log(f"{name}: {ms:.4f} ms  {rate:.1f} {unit}  ({100 * rate / peak:.1f}% of {peak})")
    wk = widened(inp)
    for _, fn, *_ in wk:
        fn()
    torch.cuda.synchronize()
    wide = {}
    for (name, _, work, unit, peak), ms in zip(wk, time_launches(wk, args.steps, stream)):
        wide[name] = rate_entry(ms, work, unit, peak, name)
        wide[name]["traffic"] = measured_traffic(name)
        mf = measured_mfma(name)
        if mf is not None:
            wide[name]["mfma_busy"], wide[name]["clock_ghz"] = mf
        log(f"{name} (widened): {ms:.4f} ms  {wide[name]['achieved']:.1f} {unit}")
    # context, not part of the path: the vendor library (torch.mm -> hipBLASLt) on the bf16
    # workload's shape, fresh output, B as stored (K, N); timed the same way after the step
    g = inp["bf16"]
    A16 = g["A"].view(torch.bfloat16).reshape(g["M"], g["K"])
    B16 = g["B"].view(torch.bfloat16).reshape(g["K"], g["N"])
    mm = [("torch_mm_bf16", lambda: torch.mm(A16, B16), 2.0 * g["M"] * g["N"] * g["K"], "TFLOP/s", PEAK["bf16_TFs"])]
    mm[0][1]()
    torch.cuda.synchronize()
    context = {"torch_mm_bf16": rate_entry(time_launches(mm, args.steps, stream)[0], *mm[0][2:])}
    context["torch_mm_bf16"]["note"] = ("hipBLASLt through torch.mm, bf16 8192^3, fresh bf16 output, no accumulation: "
                                        "a vendor-library reference point, not part of the step")
    log(f"torch_mm_bf16 (context): {context['torch_mm_bf16']['ms']:.4f} ms  {context['torch_mm_bf16']['achieved']:.1f} TFLOP/s")
    context.update(vendor_fp8(inp, args.steps, stream))
    # the ceilings the rows run against, measured with the library's diagnostic kernels on the
    # same device in the same run (not part of the step)
    ck = ceilings(inp)
    for _, fn, *_ in ck:
        fn()
    torch.cuda.synchronize()
    for (name, _, work, unit, peak, note), ms in zip(ck, time_launches(ck, args.steps, stream)):
        context[name] = rate_entry(ms, work, unit, peak)
        context[name]["note"] = note
        context[name]["traffic"] = measured_traffic(name)
        mf = measured_mfma(name)
        if mf is not None:
            context[name]["mfma_busy"], context[name]["clock_ghz"] = mf
        log(f"{name} (context): {ms:.4f} ms  {context[name]['achieved']:.1f} {unit}")
    dom = max((n for n in per if n != "add_one"), key=lambda n: per[n]["ms"])
    d = per[dom]
    gemm_flops = sum(k[2] for k in ks if k[0].startswith("gemm"))
    value = gemm_flops / (ms_step * 1e-3) / 1e12

    cpu = parity = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) and parity on its sample ...")
        cpu, parity = cpu_baseline(inp)
        log(f"cpu baseline: {cpu}")
        log(f"parity: {parity}")

    out = {
        "metric": "GEMM TFLOP/s (% MFMA peak) bf16/MXFP8/MXFP4; box-copy GB/s (% HBM)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 / e4m3 / e2m1 operands, f32 accumulate; bf16 box copy", "data": "synthetic",
        "config": {"workload": "box_copy bf16 16381x8190 (128,64) swz128 + gemm bf16 8192^3 (B MN-major, accum) + "
                               "mxfp8 8192x8192x16384 + mxfp4 16384x8192x8192 (neg_a) + add_one (2,32,3,4)",
                   "seeds": {"box_copy": 2, "gemm_bf16": 3, "mxfp8": 4, "mxfp4": 5},
                   "epilogue": args.epilogue if args.epilogue == "none" else
                   f"{args.epilogue}(scale {EPILOGUE_ARGS[0]:g}, bias {EPILOGUE_ARGS[1]:g})"},
        "inputs_sha256": inp["sha256"],
        "per_kernel": per,
        "widened": wide,
        "context": context,
        "roofline": dict({"kernel": dom, "bound": "hbm" if d["unit"] == "GB/s" else "mfma", "achieved": d["achieved"],
                          "peak": d["peak"], "unit": d["unit"], "frac": d["frac"], "traffic": measured_traffic(dom)},
                         **{k: d[k] for k in ("instruction", "instruction_peak", "instruction_frac") if k in d}),
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
