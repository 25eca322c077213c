"""Host logic of bench.py (no GPU): the counter summary that turns rocprofv3
FETCH_SIZE / WRITE_SIZE csv output into bytes per launch, and the
kernel-source digests that decide whether those figures still apply.

The csv files here are synthetic, written in rocprofv3's column layout with
counter values chosen so every expected figure is known exactly.
"""
import csv
import json
import os

import pytest

import bench

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(d, counter, dispatches):
    """dispatches: [(kernel name, [per-instance KiB values])]; the counter
    value of a dispatch is split over instances (the summary adds them)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (name, vals) in enumerate(dispatches):
            for v in vals:
                w.writerow({c: 0 for c in COLS} | {
                    "Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": 256,
                    "Counter_Name": counter, "Counter_Value": v})
                # another counter's row in the same file must be ignored
                w.writerow({c: 0 for c in COLS} | {
                    "Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": 256,
                    "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 1e9})


def step_dispatches(kib_of):
    """One step's nvfp4 dispatches in launch order; each launch's dispatches
    share its KiB equally (two counter instances each)."""
    out = []
    for name, cnt in bench.STEP_LAUNCHES:
        for _ in range(cnt):
            per = kib_of[name] / cnt
            out.append(("nvfp4::kernel_for_" + name, [per / 2, per / 2]))
    return out


@pytest.fixture
def dirs(tmp_path):
    kib = {name: 1000.0 * (i + 1) for i, (name, _) in enumerate(bench.STEP_LAUNCHES)}
    steps = 3
    fetch = step_dispatches(kib) * steps
    write = step_dispatches({k: v / 10 for k, v in kib.items()}) * steps
    # routing dispatches before the steps are not part of any launch
    fetch = [("nvfp4::route_topk_kernel", [5.0])] + fetch
    write = [("nvfp4::route_topk_kernel", [5.0])] + write
    d = {k: str(tmp_path / k) for k in ("f", "w", "cf", "cw", "df", "dw")}
    write_csv(d["f"], "FETCH_SIZE", fetch)
    write_csv(d["w"], "WRITE_SIZE", write)
    # calibration: the copy of 1 GiB reads as 2^19 KiB (factor 2) and writes
    # as 2^20 KiB (factor 1); a smaller non-library dispatch is ignored
    write_csv(d["cf"], "FETCH_SIZE", [("copyBuffer", [2.0 ** 19]), ("small", [10.0])])
    write_csv(d["cw"], "WRITE_SIZE", [("copyBuffer", [2.0 ** 20]), ("small", [10.0])])
    dec = []
    for i, _ in enumerate(bench.DECODE_ROWS):
        dec += [("void nvfp4::gemm_skinny_kernel<...>", [100.0 * (i + 1)])] * bench.DECODE_REPS
    for name, kern in bench.EXTRA_COUNTER_ROWS:
        dec += [("nvfp4::%s(nvfp4::GemmArgs)" % kern, [7000.0])] * bench.DECODE_REPS
    write_csv(d["df"], "FETCH_SIZE", dec)
    write_csv(d["dw"], "WRITE_SIZE", [(n, [v[0] / 2]) for n, v in dec])
    return d, kib, tmp_path


def test_pmc_summary_bytes_per_launch(dirs):
    d, kib, tmp = dirs
    out = bench.pmc_summary(d["f"], d["w"], d["cf"], d["cw"], d["df"], d["dw"],
                            path=str(tmp / "traffic.json"))
    assert out["calibration"]["FETCH_SIZE"]["factor"] == pytest.approx(2.0)
    assert out["calibration"]["WRITE_SIZE"]["factor"] == pytest.approx(1.0)
    for name, _ in bench.STEP_LAUNCHES:
        e = out["kernels"][name]
        assert e["fetch_bytes"] == round(kib[name] * 1024 * 2)
        assert e["write_bytes"] == round(kib[name] / 10 * 1024)
        assert e["bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"]
        assert e["source_digest"] == bench.kernel_digest(name)
    for i, name in enumerate(bench.DECODE_ROWS):
        e = out["kernels"][name]
        assert e["fetch_bytes"] == round(100.0 * (i + 1) * 1024 * 2)
        assert e["write_bytes"] == round(50.0 * (i + 1) * 1024)
    e = out["kernels"]["grouped_gemm_up_swiglu"]
    assert e["fetch_bytes"] == round(7000.0 * 1024 * 2) and e["write_bytes"] == round(3500.0 * 1024)
    assert json.load(open(tmp / "traffic.json")) == out


def test_pmc_summary_rejects_partial_steps(dirs, tmp_path):
    d, kib, tmp = dirs
    bad = str(tmp_path / "partial")
    write_csv(bad, "FETCH_SIZE", step_dispatches(kib)[:-1])
    with pytest.raises(SystemExit):
        bench.pmc_summary(bad, d["w"], d["cf"], d["cw"], path=str(tmp / "t.json"))


def test_kernel_digest_follows_its_sources():
    # every launch's digest is built from files that exist, and launches built
    # from the same files share it
    for name in bench.KERNEL_SOURCES:
        assert len(bench.kernel_digest(name)) == 16
    assert bench.kernel_digest("gemm_dense") == bench.kernel_digest("grouped_gemm_down")
    assert bench.kernel_digest("gemm_dense") != bench.kernel_digest("quantize_rows_dense")
    assert bench.kernel_digest("decode_gemm_dense") != bench.kernel_digest("gemm_dense")


def test_gemm_and_quantizer_byte_counts():
    # closed forms of the algorithmic bytes the bench divides by
    assert bench.quant_rows_bytes(4096, 2560) == 4096 * 2560 * 2 + 4096 * 1280 + 4096 * 160 + 4096 * 4
    assert bench.quant_rows_bytes(32768, 768, amax_in=True) == 64749568
    # one read of the bf16 weight: the same bytes as dequantizing it back
    assert bench.quant_weight_bytes(128, 1536, 2048) == 1031799296
    assert bench.gemm_bytes(4096, 4096, 9728, 2560, 1) == \
        4096 * (1280 + 160 + 4) + 9728 * (1280 + 160) + 4 + 4096 * 9728 * 4
