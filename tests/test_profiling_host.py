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



DKDV = ("fattn::(anonymous namespace)::bwd_dkdv_pair_kernel<Bf16, 128, true, false, false, false>"
        "(fattn::(anonymous namespace)::BwdArgs)")


def _write_timed(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    keys = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=keys)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_stall_table_clock_busy_and_shares(tmp_path):
    # one dK/dV launch of 100 us at 2000 MHz: 200,000 cycles per XCD, GRBM_GUI_ACTIVE summed over
    # the 8 XCDs; half of the 1024 SIMDs' cycles with the MFMA unit busy
    ns = 100_000
    cyc = 200_000
    t = lambda did, c, v: {"Dispatch_Id": did, "Kernel_Name": DKDV, "Grid_Size": 524288, "Counter_Name": c,
                           "Counter_Value": v, "Start_Timestamp": 1000, "End_Timestamp": 1000 + ns}
    sq1 = [t(1, "SQ_WAVE_CYCLES", 1000.0), t(1, "SQ_ACTIVE_INST_ANY", 350.0), t(1, "SQ_WAIT_ANY", 300.0),
           t(1, "SQ_WAIT_INST_ANY", 340.0), t(1, "SQ_ACTIVE_INST_VALU", 180.0), t(1, "SQ_ACTIVE_INST_LDS", 70.0),
           t(1, "SQ_WAIT_INST_LDS", 50.0), t(1, "SQ_BUSY_CYCLES", 1.0), t(1, "GRBM_GUI_ACTIVE", 8.0 * cyc)]
    sq2 = [t(2, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * cyc), t(2, "SQ_VALU_MFMA_COEXEC_CYCLES", 0.1 * 1024 * cyc),
           t(2, "SQ_INSTS_MFMA", 1000.0), t(2, "SQ_INSTS_VALU", 5000.0), t(2, "SQ_INSTS_LDS", 2000.0),
           t(2, "SQ_INSTS_SALU", 2500.0), t(2, "SQ_LDS_BANK_CONFLICT", 0.0), t(2, "SQ_LDS_IDX_ACTIVE", 1.0),
           t(2, "GRBM_GUI_ACTIVE", 8.0 * cyc)]
    _write_timed(str(tmp_path / "sq1" / "run_counter_collection.csv"), sq1)
    _write_timed(str(tmp_path / "sq2" / "run_counter_collection.csv"), sq2)
    (r,) = profiling.stall_table(str(tmp_path))
    assert r["label"].startswith("dK/dV") and r["calls"] == 2
    assert abs(r["us"] - 100.0) < 1e-9 and abs(r["mhz"] - 2000.0) < 1e-9
    assert abs(r["mfma_busy"] - 0.5) < 1e-12 and abs(r["coexec"] - 0.1) < 1e-12
    assert abs(r["issuing"] - 0.35) < 1e-12 and abs(r["wait_any"] - 0.3) < 1e-12
    assert abs(r["wait_issue"] - 0.34) < 1e-12 and abs(r["lds_wait"] - 0.05) < 1e-12
    assert abs(r["valu_per_mfma"] - 4.0) < 1e-12 and abs(r["lds_per_mfma"] - 2.0) < 1e-12
    assert abs(r["salu_per_mfma"] - 2.5) < 1e-12
    # 4 dK/dV GEMMs at B=2 H=16 N=4096 d=128, causal, in 100 us; the peak scales with the clock
    flops = 2 * 4.0 * 2 * 16 * 4096 * 4096 * 128 / 2
    assert abs(r["tflops"] - flops / 1e-4 / 1e12) < 1e-6
    assert abs(r["frac_clock"] - r["frac_nominal"] * 2400 / 2000) < 1e-12
    profiling.write_stalls(str(tmp_path), str(tmp_path / "out"))
    assert os.path.exists(str(tmp_path / "out" / "stalls_b2h16n4096d128_causal_bf16.md"))


def test_kernel_times_are_split_by_grid(tmp_path):
    path = tmp_path / "trace" / "run_kernel_trace.csv"
    os.makedirs(os.path.dirname(str(path)), exist_ok=True)
    with open(str(path), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X",
                                          "Grid_Size_Y", "Grid_Size_Z"])
        w.writeheader()
        for grid, dur in ((262144, 100), (262144, 300), (524288, 1000)):
            w.writerow({"Kernel_Name": KERN, "Start_Timestamp": 0, "End_Timestamp": dur, "Grid_Size_X": grid,
                        "Grid_Size_Y": 1, "Grid_Size_Z": 1})
    rows = {r["grid"]: r for r in profiling.kernel_stats_by_grid(str(tmp_path))}
    assert rows[262144]["calls"] == 2 and abs(rows[262144]["avg_us"] - 0.2) < 1e-12
    assert rows[524288]["calls"] == 1 and abs(rows[524288]["pct"] - 1000 / 14) < 1e-9


def test_gemm_summary_row_and_timings(tmp_path):
    # one library GEMM launch of 800 us at 2000 MHz with the MFMA unit busy 70% of the SIMD cycles
    ns, cyc = 800_000, 1_600_000
    name = "Cijk_Ailk_Bljk_BBS_BH_MT256x256x64"
    t = lambda did, c, v: {"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": 65536, "Counter_Name": c,
                           "Counter_Value": v, "Start_Timestamp": 0, "End_Timestamp": ns}
    sq1 = [t(1, c, 1.0) for c in ("SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                                  "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS")]
    sq1.append(t(1, "GRBM_GUI_ACTIVE", 8.0 * cyc))
    sq2 = [t(2, "SQ_VALU_MFMA_BUSY_CYCLES", 0.7 * 1024 * cyc), t(2, "SQ_VALU_MFMA_COEXEC_CYCLES", 0.0),
           t(2, "SQ_INSTS_MFMA", 100.0), t(2, "SQ_INSTS_VALU", 150.0), t(2, "SQ_INSTS_LDS", 40.0),
           t(2, "SQ_INSTS_SALU", 10.0), t(2, "SQ_LDS_BANK_CONFLICT", 0.0), t(2, "GRBM_GUI_ACTIVE", 8.0 * cyc)]
    _write_timed(str(tmp_path / "sq1" / "run_counter_collection.csv"), sq1)
    _write_timed(str(tmp_path / "sq2" / "run_counter_collection.csv"), sq2)
    times = tmp_path / "time.jsonl"
    times.write_text('noise\n{"gemm": "bf16 8192x8192x8192", "ms": 0.8, "tflops": 1374.4, "frac_of_peak": 0.5461}\n')
    (r,) = profiling.write_gemm(str(tmp_path), str(tmp_path / "out"), str(times))
    assert abs(r["mhz"] - 2000.0) < 1e-9 and abs(r["mfma_busy"] - 0.7) < 1e-12
    assert abs(r["tflops"] - 2.0 * 8192 ** 3 / 8e-4 / 1e12) < 1e-6
    assert abs(r["valu_per_mfma"] - 0.5) < 1e-12
    text = (tmp_path / "out" / "gemm_ceiling_bf16_hipblaslt.md").read_text()
    assert "| bf16 8192x8192x8192 | 0.8000 | 1374.4 | 54.6% |" in text
