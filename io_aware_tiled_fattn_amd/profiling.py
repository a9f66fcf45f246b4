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
    for args in ("FwdArgs", "BwdArgs", "SplitArgs", "CombineArgs", "KoArgs"):
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
    stats = kernel_stats(run_dir)
    tr, fc, wc = traffic(run_dir)
    busy = mfma_busy(run_dir)
    for t in tr:
        t["mfma_busy"] = busy.get((t["kernel"], t["grid"])) if busy else None
    cmd_note = "Commands (from the repository root, on the GPU box; RUN is an output folder):\n\n"
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
                 "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
        for s in stats:
            if pick(s["kernel"]):
                lines.append(f"| `{s['kernel']}` | {s['calls']} | {s['avg_us']:.1f} | {s['min_us']:.1f} | "
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
             "Commands (from the repository root, on the GPU box; RUN is an output folder):\n"]
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
    run = sys.argv[1]
    prof = sys.argv[2] if len(sys.argv) > 2 else os.path.join(os.path.dirname(HERE), "profiles")
    s, t = write_summaries(run, prof)
    for x in s:
        print(x)
    for x in t:
        print(x)
