"""What the vendor's own bf16 GEMM reaches on this GPU: a practical ceiling for MFMA-bound kernels.

Run: python io_aware_tiled_fattn_amd/microbench/gemm_ceiling.py [--sizes 4096,8192,16384] [--reps 20]

Times torch.mm on square bf16 matrices (row-major, contiguous; on ROCm torch sends these to
hipBLASLt) with HIP events on the current stream, after a second of untimed calls to bring the
engine clock to its loaded level. Each size is timed as the median of five blocks of `reps` calls.
Prints one JSON line per size: time per call, TFLOP/s (2 M N K per call) and the fraction of the
2516.6 TFLOP/s nominal dense bf16 peak (256 CUs x 4 SIMDs x 1024 FLOP per cycle x 2.4 GHz).
Under rocprofv3 counter passes the same calls give the library kernel's engine clock and MFMA
busy fraction, for comparison with the attention kernels' counters.
"""
import argparse
import json
import sys
import time

import torch

PEAK_BF16_TFLOPS = 2516.6


def time_mm(n, reps):
    g = torch.Generator(device="cuda").manual_seed(n)
    a = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    t_end = time.perf_counter() + 1.0
    while time.perf_counter() < t_end:
        for _ in range(4):
            torch.mm(a, b, out=c)
        torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.mm(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / reps)
    ms = sorted(ts)[2]
    # spot check: one output element against a float64 dot product of the same bf16 inputs
    ref = (a[n // 3].double() * b[:, n // 5].double()).sum().item()
    got = c[n // 3, n // 5].double().item()
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"gemm": f"bf16 {n}x{n}x{n}", "ms": round(ms, 4), "tflops": round(tf, 1),
            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "check_abs_err": abs(got - ref),
            "check_ref": ref}


def main(argv):
    ap = argparse.ArgumentParser()
    ap.add_argument("--sizes", default="4096,8192,16384")
    ap.add_argument("--reps", type=int, default=20)
    a = ap.parse_args(argv)
    for n in (int(s) for s in a.sizes.split(",")):
        print(json.dumps(time_mm(n, a.reps)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
