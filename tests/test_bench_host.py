"""Host side of bench.py (no GPU): the one-GPU rule, the work and byte figures the rates
and roofline fractions use, and the profile summaries over the timed launches only."""
import contextlib
import csv
import io
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

BF16_KERNEL = "void bsm::(anonymous namespace)::k_gemm_dense<4, true, false, true>(bsm::GemmArgs, int, int)"
MX4_KERNEL = "void bsm::(anonymous namespace)::k_gemm_mx<4, 4, 4, false>(bsm::GemmArgs, int, int)"
BOX_KERNEL = "void bsm::k_box_copy2d<4, true>(bsm::Copy2D)"
COPY_ONLY_KERNEL = "void bsm::k_box_copy2d<0, true>(bsm::Copy2D)"
REDUCE_ONLY_KERNEL = "void bsm::k_box_copy2d<4, false>(bsm::Copy2D)"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_work_and_byte_figures():
    # units of work of the bench step, as the method defines them: 2 M N K per GEMM, 4 bytes per
    # logical element per fused box pass (read src, write dst, read and write the reduce target)
    assert bench.STATIC_WORK["gemm_bf16"][0] == 2 * 8192 ** 3 == 1099511627776
    assert bench.STATIC_WORK["gemm_mxfp8"][0] == bench.STATIC_WORK["gemm_mxfp4"][0] == 2199023255552
    assert bench.STATIC_WORK["box_copy"][0] == 1073283120 == 4 * 16381 * 8190 * 2
    # algorithmic HBM bytes: operands once, scales once, D written (and read when accumulating)
    assert bench.ALG_BYTES["gemm_bf16"] == 805306368
    assert bench.ALG_BYTES["gemm_mxfp8"] == 545259520
    assert bench.ALG_BYTES["gemm_mxfp4"] == 643825664
    # each rate is priced against its own format's published peak
    assert bench.STATIC_WORK["gemm_mxfp8"][2] == bench.PEAK["fp8_TFs"]
    assert bench.STATIC_WORK["gemm_mxfp4"][2] == bench.PEAK["fp4_TFs"]
    assert bench.STATIC_WORK["box_copy"][2] == bench.PEAK["hbm_GBs"]


def test_profile_groups_keep_the_timed_launches():
    # 3 warm-up and 5 timed launches of the bf16 GEMM (1000 ns, then 900 ns each), the box copy
    # on the workload's grid and on the smaller unragged view, and a kernel no rule names
    rows = [(BF16_KERNEL, 1024 * 256, 10 * i, 10 * i + (1000 if i < 3 else 900), None) for i in range(8)]
    rows += [(BOX_KERNEL, 32768 * 256, 100 + i, 150 + i, None) for i in range(3)]
    rows += [(BOX_KERNEL, 32512 * 256, 200 + i, 240 + i, None) for i in range(3)]
    # the store-only and reduce-add-only forms of the workload's call: same grid, own kernels
    rows += [(COPY_ONLY_KERNEL, 32768 * 256, 300 + i, 330 + i, None) for i in range(2)]
    rows += [(REDUCE_ONLY_KERNEL, 32768 * 256, 400 + i, 445 + i, None) for i in range(2)]
    rows += [("void other_kernel()", 64, 0, 5, None)]
    groups, names = bench._profile_groups(rows, 5)
    assert sorted(groups) == ["box_copy", "box_copy_only", "box_copy_unragged", "box_reduce_only", "gemm_bf16"]
    assert [e - s for s, e, _ in groups["box_copy_only"]] == [30] * 2
    assert [e - s for s, e, _ in groups["box_reduce_only"]] == [45] * 2
    assert [e - s for s, e, _ in groups["gemm_bf16"]] == [900] * 5
    assert names["gemm_bf16"][2:] == (8, 5)
    assert [e - s for s, e, _ in groups["box_copy"]] == [50] * 3
    assert [e - s for s, e, _ in groups["box_copy_unragged"]] == [40] * 3


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def _summary(dirs, steps, calib=None):
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        bench.summarize(dirs, steps, calib)
    return out.getvalue()


def test_summarize_kernel_trace(tmp_path):
    # two warm-up launches of 1.2 ms and two timed ones of 0.9 and 1.1 ms: mean 1.0 ms over
    # the timed pair, so 1.0995e12 FLOP / 1 ms = 1099.5 TFLOP/s, 0.4369 of 2516.6
    head = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"]
    durs = [1_200_000, 1_200_000, 900_000, 1_100_000]
    rows, t = [], 0
    for d in durs:
        rows.append([BF16_KERNEL, 1024 * 256, 1, 1, t, t + d])
        t += d + 1000
    _write_csv(str(tmp_path / "trace" / "run_kernel_trace.csv"), head, rows)
    text = _summary([str(tmp_path / "trace")], 2)
    line = next(l for l in text.splitlines() if l.startswith("| gemm_bf16 "))
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[2] == "1024" and cells[3] == "2 / 4"
    assert (cells[4], cells[5], cells[6]) == ("1000.0", "900.0", "1100.0")
    assert cells[7] == "1099.5 TFLOP/s" and cells[8] == "0.4369"


def test_summarize_counters(tmp_path):
    # one timed dispatch of the fp4 GEMM lasting 600 us: GRBM_GUI_ACTIVE sums 8 XCDs, so
    # 7.2e6 / 8 = 9e5 cycles in 600 us is 1.5 GHz, and 5.4e8 MFMA-busy cycles over 1024 SIMDs
    # x 9e5 cycles is 0.5859 busy; the machine row carries both with the sources' hash
    head = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp", "Counter_Name",
            "Counter_Value"]
    rows = []
    for i, (t0, dur) in enumerate([(0, 700_000), (1_000_000, 600_000)]):
        for name, val in (("GRBM_GUI_ACTIVE", 7.2e6), ("SQ_VALU_MFMA_BUSY_CYCLES", 5.4e8)):
            rows.append([i, MX4_KERNEL, 2048 * 256, t0, t0 + dur, name, val])
    _write_csv(str(tmp_path / "mfma" / "run_counter_collection.csv"), head, rows)
    text = _summary([str(tmp_path / "mfma")], 1)
    line = next(l for l in text.splitlines() if l.startswith("| gemm_mxfp4 "))
    assert "| 1 | 600.0 |" in line
    assert "clock 1.50 GHz; MFMA busy 0.586" in line
    assert f"mfma: gemm_mxfp4 0.5859 1.5000 {bench.source_hash('gemm_mxfp4')}" in text


@pytest.mark.parametrize("bench_name", ["gemm_bf16", "gemm_mxfp8", "gemm_mxfp4", "box_copy"])
def test_committed_profiles_match_the_sources(bench_name):
    """The traffic rows the bench line reports come from the committed counter summary, and
    only while the kernel sources hash as they did when the counters were taken."""
    with open(os.path.join(ROOT, "profiles", "hbm_traffic_bench_step.md")) as fh:
        rows = [l.split() for l in fh if l.startswith("traffic: ")]
    hashes = {r[1]: r[3] for r in rows}
    assert hashes.get(bench_name) == bench.source_hash(bench_name)


def test_host_cpu_names_the_model_and_the_allowed_cores():
    h = bench.host_cpu()
    assert isinstance(h["model"], str) and h["model"]
    assert h["cores_allowed"] == len(os.sched_getaffinity(0)) >= 1
