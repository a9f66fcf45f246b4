"""Summaries of rocprofv3 output for the attention kernels (kernel times and HBM traffic).

Usage, after the profiled runs of bench.py described in ``COMMANDS`` have written their
CSV files under ``<run_dir>``::

    python -m io_aware_tiled_fattn_amd.profiling <run_dir> <profiles_dir>

writes ``kernel_times_<workload>.md``, ``hbm_traffic_<workload>.md`` and ``traffic.json`` into
``profiles_dir``. HBM bytes come from the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch),
each scaled by what the same counter reads for a plain elementwise copy of known size
(256 MiB read + 256 MiB written) run in the same process. ``traffic.json`` records a hash of the
kernel sources, so a reader can tell when the numbers no longer describe the built kernels.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
KERNEL_SOURCES = ("fattn_device.hpp", "fattn_fwd.hip", "fattn_bwd.hip", "fattn_splitkv.hip",
                  "fattn_kouter.hip")
DECODE_KERNELS = ("splitkv_kernel", "combine_kernel")
COPY_BYTES = 256 * 2**20  # the calibration copy reads and writes this many bytes each

COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {run}/trace -o run -- "
             "python -u bench.py --steps 10 --warmup 3 --no-cpu-baseline --clock-warmup-s 0.5",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {run}/fetch -o run -- "
             "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy "
             "--clock-warmup-s 0 --decode 6",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {run}/write -o run -- "
             "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy "
             "--clock-warmup-s 0 --decode 6",
    "mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d {run}/mfma -o run -- "
            "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --clock-warmup-s 0 --decode 6",
}


# Where the cycles of the step kernels go: two SQ counter passes over bench.py's kernel pass
# (each pass at most 8 SQ counters, plus GRBM_GUI_ACTIVE for the engine clock).
STALL_COUNTERS = {
    "sq1": "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
           "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE",
    "sq2": "SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_INSTS_VALU SQ_INSTS_MFMA "
           "SQ_INSTS_LDS SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_SALU GRBM_GUI_ACTIVE",
}
STALL_COMMANDS = {
    key: "rocprofv3 --pmc " + ctrs + " --output-format csv -d {run}/" + key + " -o run -- "
         "python -u bench.py --kernel-pass"
    for key, ctrs in STALL_COUNTERS.items()
}
# Algorithmic FLOPs per launch of the step kernels at B=2 H=16 N=4096 d=128 causal (B=4 for the
# prefill forward), per the stated convention (each GEMM 2 N^2 d per head, halved for causal).
_F5 = 4.0 * 2 * 16 * 4096 * 4096 * 128 / 2


# HBM bytes versus N for the forward and the backward (evidence that traffic stays O(N d)).
SWEEP_COMMANDS = {
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {run}/fetch -o run -- "
             "python -u bench.py --n-sweep",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {run}/write -o run -- "
             "python -u bench.py --n-sweep",
    "mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d {run}/mfma -o run -- "
            "python -u bench.py --n-sweep",
}


def source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    k = kernel.replace("fattn::(anonymous namespace)::", "").replace("fattn::", "")
    k = k.replace("(unsigned short const*, unsigned short const*, float*, long long)", "")
    for args in ("FwdArgs", "BwdArgs", "SplitArgs", "CombineArgs", "KoArgs", "OwArgs"):
        k = k.replace(f"((anonymous namespace)::{args})", "")
    return k.replace("void ", "").strip()


def _find(run_dir, sub, suffix):
    d = os.path.join(run_dir, sub)
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def kernel_stats(run_dir):
    rows = list(csv.DictReader(open(_find(run_dir, "trace", "kernel_stats.csv"))))
    out = []
    for r in rows:
        out.append({"kernel": short_name(r["Name"]), "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return out


def _counter_per_dispatch(path, counter):
    per = collections.defaultdict(float)
    meta = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = int(r["Dispatch_Id"])
        per[key] += float(r["Counter_Value"])
        meta[key] = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
    return per, meta


def traffic(run_dir):
    fetch, fmeta = _counter_per_dispatch(_find(run_dir, "fetch", "counter_collection.csv"), "FETCH_SIZE")
    write, wmeta = _counter_per_dispatch(_find(run_dir, "write", "counter_collection.csv"), "WRITE_SIZE")

    def calib(per, meta):
        vals = [v for k, v in per.items() if "elementwise" in meta[k][0] and meta[k][1] == 128 * 2**20 // 8]
        vals = [v for v in vals if v > 1000]
        if not vals:
            raise RuntimeError("calibration copy not found")
        return (sum(vals) / len(vals)) * 1024 / COPY_BYTES  # counter bytes per true byte

    fc, wc = calib(fetch, fmeta), calib(write, wmeta)
    groups = collections.defaultdict(lambda: {"fetch": [], "write": []})
    for k, v in fetch.items():
        name, grid = fmeta[k]
        if "elementwise" in name or "fill" in name.lower():
            continue
        groups[(name, grid)]["fetch"].append(v * 1024 / fc)
    for k, v in write.items():
        name, grid = wmeta[k]
        if "elementwise" in name or "fill" in name.lower():
            continue
        groups[(name, grid)]["write"].append(v * 1024 / wc)
    out = []
    for (name, grid), g in sorted(groups.items()):
        if not g["fetch"] or not g["write"]:
            continue
        out.append({"kernel": name, "grid": grid,
                    "fetch_bytes": sum(g["fetch"]) / len(g["fetch"]),
                    "write_bytes": sum(g["write"]) / len(g["write"])})
    return out, fc, wc


def mfma_busy(run_dir):
    """Per-(kernel, grid) mean fraction of SIMD cycles with the MFMA unit busy:
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); GRBM_GUI_ACTIVE is summed
    over the 8 XCDs. None when the run has no such counter pass."""
    try:
        path = _find(run_dir, "mfma", "counter_collection.csv")
    except FileNotFoundError:
        return None
    busy, bmeta = _counter_per_dispatch(path, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui, _ = _counter_per_dispatch(path, "GRBM_GUI_ACTIVE")
    per = collections.defaultdict(list)
    for k, v in busy.items():
        if gui.get(k):
            per[bmeta[k]].append(v / (gui[k] / 8.0 * 1024.0))
    return {key: sum(v) / len(v) for key, v in per.items()}


def kernel_stats_by_grid(run_dir):
    """Per-(kernel, grid) launch counts and durations from the kernel trace."""
    path = _find(run_dir, "trace", "kernel_trace.csv")
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        grid = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)
        per[(short_name(r["Kernel_Name"]), grid)].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    total = sum(sum(v) for v in per.values()) or 1
    out = []
    for (name, grid), v in sorted(per.items()):
        out.append({"kernel": name, "grid": grid, "calls": len(v), "avg_us": sum(v) / len(v) / 1e3,
                    "min_us": min(v) / 1e3, "max_us": max(v) / 1e3, "pct": 100.0 * sum(v) / total})
    return out


def _per_dispatch(path):
    """{dispatch: {"kernel", "grid", "ns", counter: value}} from one counter-collection CSV."""
    out = {}
    for r in csv.DictReader(open(path)):
        d = out.setdefault(int(r["Dispatch_Id"]), {"kernel": short_name(r["Kernel_Name"]),
                                                  "grid": int(r["Grid_Size"]),
                                                  "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


# the step kernels whose counters the stall summary reports: (label, signature, grid, FLOPs)
STALL_KERNELS = (
    ("forward, prefill B=4", "fwd_kernel<Bf16, 128, 256, 128, 2, true, false, false, false>", 1048576 // 2, 2 * _F5),
    ("forward, step B=2", "fwd_kernel<Bf16, 128, 256, 128, 2, true, false, false, false>", 262144, _F5),
    ("dK/dV (wave pairs)", "bwd_dkdv_pair_kernel<Bf16, 128, true, false, false, false>", 524288, 2 * _F5),
    ("dQ, computing D (in fattn_bwd)", "bwd_dq_kernel<Bf16, 128, true, false, false, false, true>", 262144, 1.5 * _F5),
    ("dQ, D given (stage entry point)", "bwd_dq_kernel<Bf16, 128, true, false, false, false, false>", 262144, 1.5 * _F5),
    ("forward, dropout p = 0.1", "fwd_kernel<Bf16, 128, 256, 128, 2, true, false, true, false>", 262144, _F5),
    ("dK/dV, dropout p = 0.1", "bwd_dkdv_pair_kernel<Bf16, 128, true, false, true, false>", 524288, 2 * _F5),
    ("dQ, dropout p = 0.1", "bwd_dq_kernel<Bf16, 128, true, false, true, false, true>", 262144, 1.5 * _F5),
    ("forward, block-sparse", "fwd_kernel<Bf16, 128, 128, 64, 2, true, false, false, true>", 262144, 0.0),
    ("dK/dV, block-sparse", "bwd_dkdv_pair_kernel<Bf16, 128, true, false, false, true>", 524288, 0.0),
    ("dQ, block-sparse", "bwd_dq_kernel<Bf16, 128, true, false, false, true, true>", 262144, 0.0),
)


# The one-wave-per-SIMD forward ablation (microbench/fwd_one_wave.py, after build --tools) beside
# the library forward, on the B=4 H=16 N=4096 d=128 causal prefill.
ONE_WAVE_KERNELS = (
    ("library forward (two waves per SIMD)", "fwd_kernel<Bf16, 128, 256, 128, 2, true, false, false, false>",
     524288, 2 * _F5),
    ("one wave per SIMD, compiler order", "fwd_one_wave_kernel<Bf16, 3, true, 0>", 262144, 2 * _F5),
    ("one wave per SIMD, fixed slots", "fwd_one_wave_kernel<Bf16, 3, true, 1>", 262144, 2 * _F5),
    ("one wave per SIMD, fixed slots, 4 stages", "fwd_one_wave_kernel<Bf16, 4, true, 1>", 262144, 2 * _F5),
)
ONE_WAVE_COMMANDS = {
    key: "rocprofv3 --pmc " + ctrs + " --output-format csv -d {run}/" + key + " -o run -- "
         "python -u io_aware_tiled_fattn_amd/microbench/fwd_one_wave.py --timing-only"
    for key, ctrs in STALL_COUNTERS.items()
}


def stall_table(run_dir, peak_tflops=2516.6, max_mhz=2400.0, kernels=None):
    """Per step kernel: time, engine clock, MFMA busy, and where the waves' cycles go, from the
    two SQ counter passes (STALL_COMMANDS)."""
    d1 = _per_dispatch(_find(run_dir, "sq1", "counter_collection.csv"))
    d2 = _per_dispatch(_find(run_dir, "sq2", "counter_collection.csv"))
    rows = []
    for label, sig, grid, flops in (kernels or STALL_KERNELS):
        a = [v for v in d1.values() if v["kernel"].startswith(sig) and v["grid"] == grid]
        b = [v for v in d2.values() if v["kernel"].startswith(sig) and v["grid"] == grid]
        if not a or not b:
            continue
        mean = lambda xs, k: sum(x[k] for x in xs) / len(xs)
        ns = (mean(a, "ns") + mean(b, "ns")) / 2
        cyc = mean(b, "GRBM_GUI_ACTIVE") / 8.0  # GRBM_GUI_ACTIVE is summed over the 8 XCDs
        mhz = cyc / (ns * 1e-3)
        wave = mean(a, "SQ_WAVE_CYCLES")
        mfma = mean(b, "SQ_INSTS_MFMA")
        row = {"label": label, "kernel": sig, "grid": grid, "calls": len(a) + len(b), "us": ns / 1e3,
               "mhz": mhz,
               "mfma_busy": mean(b, "SQ_VALU_MFMA_BUSY_CYCLES") / (1024.0 * cyc),
               "coexec": mean(b, "SQ_VALU_MFMA_COEXEC_CYCLES") / (1024.0 * cyc),
               "issuing": mean(a, "SQ_ACTIVE_INST_ANY") / wave,
               "wait_any": mean(a, "SQ_WAIT_ANY") / wave,
               "wait_issue": mean(a, "SQ_WAIT_INST_ANY") / wave,
               "valu_active": mean(a, "SQ_ACTIVE_INST_VALU") / wave,
               "lds_active": mean(a, "SQ_ACTIVE_INST_LDS") / wave,
               "lds_wait": mean(a, "SQ_WAIT_INST_LDS") / wave,
               "bank_conflict": mean(b, "SQ_LDS_BANK_CONFLICT"),
               "valu_per_mfma": (mean(b, "SQ_INSTS_VALU") - mfma) / mfma if mfma else None,
               "lds_per_mfma": mean(b, "SQ_INSTS_LDS") / mfma if mfma else None,
               "salu_per_mfma": mean(b, "SQ_INSTS_SALU") / mfma if mfma else None}
        if flops:
            tf = flops / (ns * 1e-9) / 1e12
            row["tflops"] = tf
            row["frac_nominal"] = tf / peak_tflops
            row["frac_clock"] = tf / (peak_tflops * mhz / max_mhz)
        rows.append(row)
    return rows


STEP_CLOCK_NOTE = ("The counter also runs through each dispatch's own set-up: the 12 us rowsum kernel of "
                   "the same passes reads as 3.8 GHz, so some 18 to 28 thousand cycles per dispatch are "
                   "not kernel time. The clock of a 130-280 us kernel therefore reads 3-10% high (the "
                   "clock-adjusted fractions are lower bounds), and the 57-110 us block-sparse kernels "
                   "read above the 2400 MHz maximum.")


def write_stalls(run_dir, prof_dir, workload="b2h16n4096d128_causal_bf16", kernels=None, commands=None,
                 title=None, runs_note=None, name=None, clock_note=STEP_CLOCK_NOTE):
    os.makedirs(prof_dir, exist_ok=True)
    rows = stall_table(run_dir, kernels=kernels)
    pct = lambda x: "—" if x is None else f"{x:.1%}"
    num = lambda x, f="{:.2f}": "—" if x is None else f.format(x)
    title = title or f"Where the step kernels' cycles go — {workload} (and the B=4 prefill forward)"
    runs_note = runs_note or ("Every figure is the mean over the kernel's launches in the pass (bench.py "
                              "--kernel-pass runs each three times after 0.5 s of warm-up).")
    lines = [f"# {title}\n",
             "Commands (from the repository root, on an MI355X; RUN is an output folder):\n"]
    for key in ("sq1", "sq2"):
        lines.append("    " + (commands or STALL_COMMANDS)[key].format(run="RUN"))
    lines += ["", runs_note,
              "- Engine clock = GRBM_GUI_ACTIVE / 8 XCDs / kernel duration (the counter runs at the "
              "engine clock and is summed over the XCDs). The nominal peak (2516.6 TFLOP/s) assumes "
              "2400 MHz; the clock-adjusted fraction divides by the peak at the measured clock. "
              + clock_note,
              "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles); co-issue = "
              "SQ_VALU_MFMA_COEXEC_CYCLES (a VALU instruction issued while the MFMA unit was busy) on "
              "the same base.",
              "- Wave-time shares (each over SQ_WAVE_CYCLES, all in quad-cycles summed over waves): "
              "issuing = SQ_ACTIVE_INST_ANY, waiting = SQ_WAIT_ANY (for a dependency, a count or a "
              "barrier), waiting for an issue slot = SQ_WAIT_INST_ANY, VALU = SQ_ACTIVE_INST_VALU, "
              "LDS = SQ_ACTIVE_INST_LDS, LDS issue wait = SQ_WAIT_INST_LDS. Two waves share each "
              "SIMD, so a wave waits for an issue slot whenever the other one issues.",
              "- Instruction mix per MFMA from SQ_INSTS_VALU (less the MFMAs), SQ_INSTS_LDS and "
              "SQ_INSTS_SALU.", "",
              "| kernel | us | clock MHz | TFLOP/s | of nominal peak | of clock-adjusted peak | MFMA busy | co-issue | bank-conflict cycles |",
              "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['label']} (`{r['kernel']}`) | {r['us']:.1f} | {r['mhz']:.0f} | "
                     f"{num(r.get('tflops'), '{:.0f}')} | {pct(r.get('frac_nominal'))} | {pct(r.get('frac_clock'))} | "
                     f"{pct(r['mfma_busy'])} | {pct(r['coexec'])} | {r['bank_conflict']:.0f} |")
    lines += ["", "| kernel | issuing | waiting | waiting for an issue slot | VALU | LDS | LDS issue wait | VALU / MFMA | LDS / MFMA | SALU / MFMA |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['label']} | {pct(r['issuing'])} | {pct(r['wait_any'])} | {pct(r['wait_issue'])} | "
                     f"{pct(r['valu_active'])} | {pct(r['lds_active'])} | {pct(r['lds_wait'])} | "
                     f"{num(r['valu_per_mfma'])} | {num(r['lds_per_mfma'])} | {num(r['salu_per_mfma'])} |")
    with open(os.path.join(prof_dir, name or f"stalls_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return rows


def write_one_wave(run_dir, prof_dir):
    """Counter summary of the one-wave forward ablation beside the library forward."""
    return write_stalls(
        run_dir, prof_dir, kernels=ONE_WAVE_KERNELS, commands=ONE_WAVE_COMMANDS,
        title="One wave per SIMD against two: forward B=4 H=16 N=4096 d=128 causal bf16",
        runs_note=("Every figure is the mean over the kernel's launches in the pass (fwd_one_wave.py "
                   "--timing-only runs each variant 155 times per shape after 0.5 s of warm-up; only "
                   "the B=4 launches are listed). In the one-wave kernels a SIMD holds one wave, so "
                   "'waiting for an issue slot' there is time the wave's next instruction waits for "
                   "its own unit (MFMA, VALU, LDS) to accept it."),
        name="stalls_fwd_one_wave_b4h16n4096d128_causal_bf16.md",
        clock_note=("The counter also runs through each dispatch's own set-up (some 18 to 28 thousand "
                    "cycles, measured on the step kernels' passes), so the clocks of these 250-360 us "
                    "kernels read 2-5% high."))


# The vendor's bf16 GEMM (torch.mm, which on ROCm runs a hipBLASLt kernel) on 8192^3, for the
# clock and MFMA-busy fraction an MFMA-bound kernel without any softmax work reaches on this GPU.
GEMM_N = 8192
GEMM_KERNELS = (("hipBLASLt bf16 GEMM 8192 x 8192 x 8192", "Cijk_Ailk_Bljk_BBS", GEMM_N * GEMM_N // 1024,
                 2.0 * GEMM_N ** 3),)
GEMM_COMMANDS = {
    key: "rocprofv3 --pmc " + ctrs + " --output-format csv -d {run}/" + key + " -o run -- "
         f"python -u io_aware_tiled_fattn_amd/microbench/gemm_ceiling.py --sizes {GEMM_N}"
    for key, ctrs in STALL_COUNTERS.items()
}


def write_gemm(run_dir, prof_dir, times_path=None):
    """Counter summary of the library GEMM (GEMM_KERNELS), plus the timed sizes of
    gemm_ceiling.py when its JSON lines are given."""
    name = "gemm_ceiling_bf16_hipblaslt.md"
    rows = write_stalls(
        run_dir, prof_dir, kernels=GEMM_KERNELS, commands=GEMM_COMMANDS,
        title="The vendor's bf16 GEMM on the same GPU: a practical ceiling for MFMA-bound kernels",
        runs_note=("Every figure is the mean over the GEMM kernel's launches in the pass (gemm_ceiling.py "
                   f"--sizes {GEMM_N}: a second of untimed calls, then five blocks of 20 timed ones, all counted). "
                   "torch.mm on ROCm runs a hipBLASLt (Tensile) kernel; the row is matched by its name "
                   "prefix and grid."),
        name=name,
        clock_note=("The counter also runs through each dispatch's own set-up (some 18 to 28 thousand "
                    "cycles, measured on the attention kernels' passes), so the clock of this 760 us "
                    "kernel reads about 1% high."))
    if times_path:
        res = [json.loads(x) for x in open(times_path) if x.startswith("{")]
        lines = ["", "Timed with HIP events (`python -u io_aware_tiled_fattn_amd/microbench/gemm_ceiling.py`, "
                 "median of five blocks of 20 calls after a second of warm-up):", "",
                 "| GEMM | ms per call | TFLOP/s | of the 2516.6 TFLOP/s nominal peak |", "|---|---|---|---|"]
        for r in res:
            lines.append(f"| {r['gemm']} | {r['ms']:.4f} | {r['tflops']:.1f} | {r['frac_of_peak']:.1%} |")
        with open(os.path.join(prof_dir, name), "a") as f:
            f.write("\n".join(lines) + "\n")
    return rows


def _is_decode(kernel):
    return any(kernel.startswith(d) for d in DECODE_KERNELS)


DECODE_WORKLOAD = "decode_b8h32nk16384d128_bf16"


# bench.py's per-kernel HIP-event times (kernel_ms) for the step workload, and the kernels they time
# (its dQ figure times the stage entry point, the instance that reads D)
LIVE_KERNELS = {
    "dkdv": "bwd_dkdv_pair_kernel<Bf16, 128, true, false, false, false>",
    "dq": "bwd_dq_kernel<Bf16, 128, true, false, false, false, false>",
}


def _live_vs_trace(run_dir, stats):
    """Lines comparing bench.py's live kernel times with the trace, when the run directory holds
    the JSON line of a plain bench.py run made on the same box (``bench.json``)."""
    path = os.path.join(run_dir, "bench.json")
    if not os.path.exists(path):
        return []
    with open(path) as f:
        live = json.loads(f.read().strip().splitlines()[-1])
    out = ["", "The same box, a plain `python bench.py` run just before the trace: its HIP-event times "
           "per launch beside the trace's average (the trace's average for a kernel that runs only "
           "the step workload):", "", "| kernel | bench.py live ms | trace avg ms |", "|---|---|---|"]
    for key, sig in LIVE_KERNELS.items():
        tr = [s_ for s_ in stats if s_["kernel"].startswith(sig)]
        if key in live.get("kernel_ms", {}) and tr:
            out.append(f"| `{sig}` | {live['kernel_ms'][key]:.4f} | {tr[0]['avg_us'] / 1e3:.4f} |")
    roof = live.get("roofline", {})
    if roof:
        out += ["", f"bench.py roofline on that run: `{roof.get('kernel')}`, {roof.get('achieved')} "
                f"{roof.get('unit')} of {roof.get('peak')} (frac {roof.get('frac')})."]
    return out


def write_summaries(run_dir, prof_dir, workload="b2h16n4096d128_causal_bf16"):
    os.makedirs(prof_dir, exist_ok=True)
    stats = kernel_stats_by_grid(run_dir)
    tr, fc, wc = traffic(run_dir)
    busy = mfma_busy(run_dir)
    for t in tr:
        t["mfma_busy"] = busy.get((t["kernel"], t["grid"])) if busy else None
    cmd_note = "Commands (from the repository root, on an MI355X; RUN is an output folder):\n\n"
    titles = {
        workload: (f"bench.py step workload ({workload}), the B=4 forward and the K-outer ablation",
                   "The forward kernel's calls mix the B=2 (step), B=4 (prefill, every tile) and "
                   "B=1 H=32 N=16384 (long-context) workloads; bench.py times each live with HIP "
                   "events. The dK/dV and dQ kernels run the step workload only (the dQ instance "
                   "that also computes D is the one fattn_bwd runs). `ko_kernel` is the K-outer ablation on "
                   "the step's forward shape, one launch per 128-key block (32 per call), so its "
                   "per-launch figures are 1/32 of a call."),
        DECODE_WORKLOAD: ("bench.py split-KV decode workloads (B=8 H=32 Nk=16384 d=128 bf16, "
                          "Nq = 1 and Nq = 16, one shared cache)",
                          "The partial kernel's calls mix Nq = 1 and Nq = 16 (same grid); the "
                          "counter runs (HBM traffic) run the Nq = 1 workload only."),
    }
    for wl, (title, note) in titles.items():
        pick = (lambda k: _is_decode(k)) if wl == DECODE_WORKLOAD else (lambda k: not _is_decode(k))
        lines = [f"# Kernel times — {title}\n",
                 cmd_note + "    " + COMMANDS["trace"].format(run="RUN") + "\n",
                 "One row per (kernel, grid): the grid (threads) tells the workloads apart.\n",
                 "| kernel | grid | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|---|"]
        for s in stats:
            if pick(s["kernel"]):
                lines.append(f"| `{s['kernel']}` | {s['grid']} | {s['calls']} | {s['avg_us']:.1f} | {s['min_us']:.1f} | "
                             f"{s['max_us']:.1f} | {s['pct']:.1f} |")
        lines.append("\n" + note + " % time is over every kernel of the run.")
        if wl != DECODE_WORKLOAD:
            lines += _live_vs_trace(run_dir, stats)
        with open(os.path.join(prof_dir, f"kernel_times_{wl}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")

        cmds = "    " + COMMANDS["fetch"].format(run="RUN") + "\n    " + COMMANDS["write"].format(run="RUN")
        if busy:
            cmds += "\n    " + COMMANDS["mfma"].format(run="RUN")
        lines = [f"# HBM traffic per launch — {title}\n",
                 cmd_note + cmds + "\n",
                 f"Calibration (elementwise copy, 256 MiB read + 256 MiB written): FETCH_SIZE reads "
                 f"{fc:.3f} x true bytes, WRITE_SIZE reads {wc:.3f} x; the figures below are divided by "
                 f"those factors." + (" MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs "
                                      "x 1024 SIMDs), from the third run.\n" if busy else "\n"),
                 "| kernel | grid | fetched MiB | written MiB | MFMA busy |", "|---|---|---|---|---|"]
        for t in tr:
            if pick(t["kernel"]):
                mb = f"{t['mfma_busy']:.1%}" if t.get("mfma_busy") is not None else "—"
                lines.append(f"| `{t['kernel']}` | {t['grid']} | {t['fetch_bytes'] / 2**20:.1f} | "
                             f"{t['write_bytes'] / 2**20:.1f} | {mb} |")
        with open(os.path.join(prof_dir, f"hbm_traffic_{wl}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    with open(os.path.join(prof_dir, "traffic.json"), "w") as f:
        json.dump({"source_hash": source_hash(), "fetch_factor": fc, "write_factor": wc,
                   "kernels": tr}, f, indent=1)
    return stats, tr


def _fit_exponent(ns, ys):
    """Least-squares slope of log(y) against log(N)."""
    import math
    xs = [math.log(n) for n in ns]
    ls = [math.log(y) for y in ys]
    mx, my = sum(xs) / len(xs), sum(ls) / len(ls)
    return sum((x - mx) * (y - my) for x, y in zip(xs, ls)) / sum((x - mx) ** 2 for x in xs)


def write_sweep(run_dir, prof_dir, times=None, bh=16, d=128):
    """profiles/hbm_scaling_fwd_bwd_bh16d128_bf16.md from the three sweep runs (fetch, write, mfma)."""
    tr, fc, wc = traffic(run_dir)
    mfma = mfma_busy(run_dir) or {}
    rows = []
    bwd = collections.defaultdict(dict)  # (N, causal) -> {"dkdv": record, "dq": record}
    for t in tr:
        name = t["kernel"]
        targs = name[name.index("<") + 1:name.index(">")].split(", ") if "<" in name else []
        if name.startswith("bwd_dkdv_pair_kernel") and targs[3:6] == ["false"] * 3:
            bwd[(t["grid"] // 512 * 128 // bh, targs[2] == "true")]["dkdv"] = t
        elif name.startswith("bwd_dq_kernel") and targs[3:7] == ["false", "false", "false", "true"]:
            bwd[(t["grid"] // 512 * 256 // bh, targs[2] == "true")]["dq"] = t
    for t in tr:
        if not t["kernel"].startswith("fwd_kernel"):
            continue
        n = t["grid"] // 512 * 256 // bh  # 256 query rows per 512-thread work-group
        causal = ", true, false, false, false>" in t["kernel"]
        rows.append({"N": n, "causal": causal, "fetch": t["fetch_bytes"], "write": t["write_bytes"],
                     "mfma_busy": mfma.get((t["kernel"], t["grid"]))})
    rows.sort(key=lambda r: (r["causal"], r["N"]))
    lines = ["# HBM bytes versus N — forward and backward, B=1 H=16 d=128 bf16\n",
             "Commands (from the repository root, on an MI355X; RUN is an output folder):\n"]
    for key in ("fetch", "write", "mfma"):
        lines.append("    " + SWEEP_COMMANDS[key].format(run="RUN"))
    lines += ["", f"Counters calibrated on a 256 MiB + 256 MiB copy (FETCH_SIZE x{fc:.3f}, WRITE_SIZE x{wc:.3f}). "
              "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs).", "",
              "Forward (256 x 128 tiles):", "",
              "| causal | N | HBM read MiB | HBM written MiB | Q+K+V+O+LSE MiB | N x N score matrix MiB (bf16) | MFMA busy |",
              "|---|---|---|---|---|---|---|"]
    for r in rows:
        io = (4 * r["N"] * d * 2 + 4 * r["N"]) * bh / 2**20
        nn = r["N"] * r["N"] * 2 * bh / 2**20
        mb = f"{r['mfma_busy']:.1%}" if r["mfma_busy"] is not None else "—"
        lines.append(f"| {r['causal']} | {r['N']} | {r['fetch'] / 2**20:.1f} | {r['write'] / 2**20:.1f} | "
                     f"{io:.1f} | {nn:.0f} | {mb} |")
    lines.append("")
    for causal in (False, True):
        sel = [r for r in rows if r["causal"] == causal]
        if len(sel) >= 2:
            e = _fit_exponent([r["N"] for r in sel], [r["fetch"] + r["write"] for r in sel])
            lines.append(f"Fitted exponent of HBM bytes in N (causal={causal}): {e:.3f} "
                         f"(the score matrix would grow with exponent 2).")
    brows = sorted((k, v) for k, v in bwd.items() if "dkdv" in v and "dq" in v)
    if brows:
        lines += ["", "Backward (`fattn_bwd`: the dQ kernel, which also computes D = rowsum(dO∘O), then "
                  "the dK/dV kernel), same runs. The one-pass minimum reads Q, K, V, O, dO once and "
                  "writes dQ, dK, dV once: 8 N d 2 B per head, plus the float32 LSE and D.", "",
                  "| causal | N | dQ read MiB | dK/dV read MiB | written MiB | one-pass MiB | N x N score matrix MiB (bf16) | MFMA busy dQ / dK/dV |",
                  "|---|---|---|---|---|---|---|---|"]
        totals = {False: [], True: []}
        for (n, causal), v in brows:
            dq_, kv_ = v["dq"], v["dkdv"]
            wr = dq_["write_bytes"] + kv_["write_bytes"]
            one = (8 * n * d * 2 + 12 * n) * bh
            mb = lambda r: f"{mfma[(r['kernel'], r['grid'])]:.1%}" if (r["kernel"], r["grid"]) in mfma else "—"
            lines.append(f"| {causal} | {n} | {dq_['fetch_bytes'] / 2**20:.1f} | {kv_['fetch_bytes'] / 2**20:.1f} | "
                         f"{wr / 2**20:.1f} | {one / 2**20:.1f} | {n * n * 2 * bh / 2**20:.0f} | {mb(dq_)} / {mb(kv_)} |")
            totals[causal].append((n, dq_["fetch_bytes"] + kv_["fetch_bytes"] + wr))
        lines.append("")
        for causal in (False, True):
            sel = sorted(totals[causal])
            if len(sel) >= 2:
                e = _fit_exponent([x[0] for x in sel], [x[1] for x in sel])
                lines.append(f"Fitted exponent of the backward's HBM bytes in N (causal={causal}): {e:.3f}.")
    if times:
        lines += ["", "Times from the same command's timed blocks (HIP events):", "",
                  "| pass | causal | N | ms | TFLOP/s |", "|---|---|---|---|---|"]
        for t in times:
            lines.append(f"| {t.get('kind', 'fwd')} | {t['causal']} | {t['N']} | {t['ms']} | {t['tflops']} |")
    with open(os.path.join(prof_dir, "hbm_scaling_fwd_bwd_bh16d128_bf16.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return rows


def load_traffic(prof_dir):
    """Per-(kernel, grid) HBM bytes if they were measured on the current kernel sources."""
    path = os.path.join(prof_dir, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_hash") != source_hash():
        return None
    return {(k["kernel"], k["grid"]): k for k in data["kernels"]}


if __name__ == "__main__":
    if sys.argv[1] == "sweep":
        times = None
        if len(sys.argv) > 4:
            with open(sys.argv[4]) as f:
                times = json.loads(f.read().strip().splitlines()[-1])["runs"]
        for r in write_sweep(sys.argv[2], sys.argv[3], times):
            print(r)
        sys.exit(0)
    if sys.argv[1] == "onewave":
        for r in write_one_wave(sys.argv[2], sys.argv[3]):
            print(r)
        sys.exit(0)
    if sys.argv[1] == "gemm":
        for r in write_gemm(sys.argv[2], sys.argv[3], sys.argv[4] if len(sys.argv) > 4 else None):
            print(r)
        sys.exit(0)
    if sys.argv[1] == "stalls":
        for r in write_stalls(sys.argv[2], sys.argv[3]):
            print(r)
        sys.exit(0)
    run = sys.argv[1]
    prof = sys.argv[2] if len(sys.argv) > 2 else os.path.join(os.path.dirname(HERE), "profiles")
    s, t = write_summaries(run, prof)
    for x in s:
        print(x)
    for x in t:
        print(x)
