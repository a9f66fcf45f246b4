"""Host logic of the rocprofv3 summaries: counter calibration, per-kernel HBM bytes, MFMA busy.

Synthetic counter files in rocprofv3's CSV layout stand in for a profiled run; the expected
figures follow from the stated formulas by hand.
"""
import csv
import os

import bench
from io_aware_tiled_fattn_amd import profiling

COPY = "void at::native::elementwise_kernel<128, 4>(int, copy)"
KERN = "fattn::(anonymous namespace)::fwd_kernel<Bf16, 128, 256, 128, 2, true, false, false, false>(fattn::(anonymous namespace)::FwdArgs)"


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _row(did, name, grid, counter, value):
    return {"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
            "Counter_Value": value}


def _run_dir(tmp_path):
    copy_grid = 128 * 2**20 // 8
    # the copy moves 256 MiB each way; FETCH_SIZE reads half of that (in KiB), WRITE_SIZE all of it
    fetch = [_row(1, COPY, copy_grid, "FETCH_SIZE", 128 * 1024),
             _row(2, KERN, 524288, "FETCH_SIZE", 1000.0), _row(2, KERN, 524288, "FETCH_SIZE", 500.0),
             _row(3, KERN, 524288, "FETCH_SIZE", 1500.0)]
    write = [_row(1, COPY, copy_grid, "WRITE_SIZE", 256 * 1024),
             _row(2, KERN, 524288, "WRITE_SIZE", 64.0), _row(3, KERN, 524288, "WRITE_SIZE", 64.0)]
    # GRBM_GUI_ACTIVE is summed over 8 XCDs: 8 * 1000 cycles; MFMA busy cycles over 1024 SIMDs
    mfma = [_row(2, KERN, 524288, "SQ_VALU_MFMA_BUSY_CYCLES", 512000.0), _row(2, KERN, 524288, "GRBM_GUI_ACTIVE", 8000.0),
            _row(3, KERN, 524288, "SQ_VALU_MFMA_BUSY_CYCLES", 256000.0), _row(3, KERN, 524288, "GRBM_GUI_ACTIVE", 8000.0)]
    _write(str(tmp_path / "fetch" / "run_counter_collection.csv"), fetch)
    _write(str(tmp_path / "write" / "run_counter_collection.csv"), write)
    _write(str(tmp_path / "mfma" / "run_counter_collection.csv"), mfma)
    return str(tmp_path)


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path):
    run = _run_dir(tmp_path)
    tr, fc, wc = profiling.traffic(run)
    assert abs(fc - 0.5) < 1e-12 and abs(wc - 1.0) < 1e-12
    (rec,) = tr
    assert rec["grid"] == 524288
    # per dispatch: (1000 + 500) and 1500 KiB counted, i.e. 3000 KiB true; mean over the two
    assert abs(rec["fetch_bytes"] - 3000 * 1024) < 1e-6
    assert abs(rec["write_bytes"] - 64 * 1024) < 1e-6


def test_mfma_busy_is_the_mean_over_dispatches(tmp_path):
    run = _run_dir(tmp_path)
    busy = profiling.mfma_busy(run)
    key = (profiling.short_name(KERN), 524288)
    # 512000 / (1000 * 1024) = 0.5 and 256000 / (1000 * 1024) = 0.25
    assert abs(busy[key] - 0.375) < 1e-12
    assert profiling.mfma_busy(str(tmp_path / "nothing")) is None


def test_roofline_traffic_fields():
    out = bench.traffic_fields({"fetch_bytes": 1.5e8, "write_bytes": 6.7e7, "mfma_busy": 0.4234})
    assert out["traffic"] == 217_000_000
    assert out["traffic_fetch_bytes"] == 150_000_000 and out["traffic_write_bytes"] == 67_000_000
    assert out["mfma_busy"] == 0.4234
    assert "mfma_busy" not in bench.traffic_fields({"fetch_bytes": 1.0, "write_bytes": 2.0})

