"""Host-side checks of bench.py (CPU only): the algorithmic byte counts its
rooflines use, the per-launch HBM traffic summary built from rocprofv3
counter files, and the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_match_the_measurement_plan():
    """Per-token quantize of X 4096x2560, two-pass weight quantize of W
    9728x2560 and the dense / down GEMM traffic as the plan states them; the
    up-projection reads each of its 4096 unique A rows once (row_index reuse),
    so its A term is 4096 rows, not the 32768 routed ones."""
    assert bench.quant_rows_bytes(4096, 2560) == 26886144
    assert bench.quant_rows_bytes(32768, 768, amax_in=True) == 64749568
    assert bench.quant_weight_bytes(1, 9728, 2560) == 113623044
    assert bench.quant_weight_bytes(128, 1536, 2048) == 1837105664
    assert bench.gemm_bytes(4096, 4096, 9728, 2560, 1) == 179306500
    assert bench.gemm_bytes(32768, 32768, 2048, 768, 128) == 395969024
    up = bench.gemm_bytes(4096, 32768, 1536, 2048, 128)
    # A: 4096 rows x (1024 code + 128 scale + 4 S) bytes; B: 128 x 1536 x 1152
    # plus 128 expert scales; Y: 32768 x 1536 fp32
    assert up == 4096 * 1156 + 128 * 1536 * 1152 + 128 * 4 + 32768 * 1536 * 4 == 432554496


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                          "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            # two counter instances per dispatch (summed by the reader)
            for half in (0.25, 0.75):
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": 256,
                            "Counter_Name": counter, "Counter_Value": value * half})


def _step_rows(scale):
    rows = [("route_topk_kernel(nvfp4)", 1.0)]  # setup routing: ignored
    for step in range(3):
        for j, (name, cnt) in enumerate(bench.STEP_LAUNCHES):
            for c in range(cnt):
                rows.append(("void nvfp4::k%d(...)" % j, scale * (j + 1) * (c + 1)))
    return rows


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path):
    cal_kib = bench.CALIB_BYTES / 1024.0
    _write_counters(str(tmp_path / "cf"), "FETCH_SIZE", [("copyBuffer", cal_kib / 2)])
    _write_counters(str(tmp_path / "cw"), "WRITE_SIZE", [("fill", cal_kib), ("copyBuffer", cal_kib)])
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", _step_rows(10.0))
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", _step_rows(1.0))
    out = bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                            str(tmp_path / "cw"), path=str(tmp_path / "t.json"))
    assert out["calibration"]["FETCH_SIZE"]["factor"] == pytest.approx(2.0)
    assert out["calibration"]["WRITE_SIZE"]["factor"] == pytest.approx(1.0)
    for j, (name, cnt) in enumerate(bench.STEP_LAUNCHES):
        kib = (j + 1) * sum(c + 1 for c in range(cnt))  # summed over the launch's dispatches
        k = out["kernels"][name]
        assert k["fetch_bytes"] == round(10.0 * kib * 1024 * 2.0)
        assert k["write_bytes"] == round(1.0 * kib * 1024)
        assert k["source_digest"] == bench.kernel_digest(name)
    assert json.load(open(tmp_path / "t.json")) == out


def test_pmc_summary_rejects_a_partial_step(tmp_path):
    cal_kib = bench.CALIB_BYTES / 1024.0
    _write_counters(str(tmp_path / "cf"), "FETCH_SIZE", [("copyBuffer", cal_kib)])
    _write_counters(str(tmp_path / "cw"), "WRITE_SIZE", [("copyBuffer", cal_kib)])
    rows = _step_rows(1.0)[:-1]
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", rows)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", rows)
    with pytest.raises(SystemExit):
        bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                          str(tmp_path / "cw"), path=str(tmp_path / "t.json"))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
