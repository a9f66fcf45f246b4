"""Benchmark: attention forward/backward TFLOP/s on one MI355X at N=4096, d=128 (bf16, causal).

A step is one pass of the whole hot path over one batch: fattn_fwd then fattn_bwd (rowsum(dO*O),
dK/dV, dQ) on the training-shaped workload B=2, H=16, N=4096, d=128 (causal, bf16; Q, K, V, dO
iid N(0,1) from a seed). FLOPs per step follow the stated convention: forward 4*B*H*N^2*d halved
for causal, backward 2.5x the forward. The forward alone is also timed on the prefill workload
B=4, H=16, N=4096, and the split-KV forward on the decode workloads (B=8, H=32, d=128, one or
16 queries per head against a 16384-key cache), reported in GB/s against the HBM peak.

Timing: HIP events on the stream the kernels are launched on (torch's current stream), after
warm-up, inputs resident in HBM. Every kernel of the step is also timed on its own (one launch
per call), which gives the dominant kernel's per-launch time for the roofline object. Prints ONE
JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks: bf16 MFMA 2.5 PFLOP/s (256 CU x 2.4 GHz x 4096 FLOP/clk/CU),
# HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


def traffic_fields(rec):
    """Roofline fields from one profiles/traffic.json record: ``traffic`` is the kernel's HBM bytes
    per launch (FETCH_SIZE + WRITE_SIZE, each scaled by the calibration copy's reading), with its
    two parts and, when that counter pass was taken, the MFMA-busy fraction."""
    out = {"traffic": round(rec["fetch_bytes"] + rec["write_bytes"]),
           "traffic_fetch_bytes": round(rec["fetch_bytes"]), "traffic_write_bytes": round(rec["write_bytes"]),
           "traffic_source": "profiles/traffic.json"}
    if rec.get("mfma_busy") is not None:
        out["mfma_busy"] = round(rec["mfma_busy"], 4)
    return out


def flops_fwd(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def _upload(inp, torch):
    import numpy as np

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    return tuple(up(inp.bits[n]) if n in inp.bits else None for n in ("q", "k", "v", "do"))


def _upload_named(inp, names, torch):
    import numpy as np
    return tuple(torch.from_numpy(np.ascontiguousarray(inp.bits[n]).view(np.int16)).view(torch.bfloat16).cuda()
                 for n in names)


def _time_calls(fn, steps, warmup, torch, min_warm_s=0.05):
    """Mean ms per call of fn over `steps` calls, timed with HIP events on the current stream,
    after `warmup` calls (continued for at least min_warm_s, so the clock stays at its steady
    value when the timed calls start)."""
    t_end = time.perf_counter() + min_warm_s
    n = 0
    while n < warmup or time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per call


def cpu_oracle_baseline(budget_s: float = 20.0):
    """Time the float64 oracle on a bounded sample of the step's workload (host cores)."""
    import fattn_inputs as fi
    from oracle import attention as att
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    w = fi.WORKLOADS[5]
    inp = fi.make_inputs((1, 1, w.N, w.d), "bf16", 5, with_do=True)
    t0 = time.perf_counter()
    heads = 0
    while True:
        att.forward(inp.q, inp.k, inp.v, w.scale, True)
        att.backward(inp.q, inp.k, inp.v, inp.do, w.scale, True)
        heads += 1
        if time.perf_counter() - t0 > budget_s / 2 or heads >= w.B * w.H:
            break
    total = time.perf_counter() - t0
    dt = total / heads
    fl = flops_fwd(1, 1, w.N, w.d, True) * 3.5
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": model,
            "sample": f"{heads} of the 32 (b,h) slices of B=2,H=16,N=4096,d=128 causal (the same "
                      f"slice's inputs each time): fp64 forward + backward, {total:.1f} s in all, "
                      f"{dt:.2f} s per slice (the oracle evaluates full rows, i.e. non-causal work, "
                      f"but is credited the causal FLOP count)"}


SWEEP_N = (1024, 2048, 4096, 8192, 16384)
FWD_TILES = ((64, 64), (64, 128), (128, 64), (128, 128), (256, 64), (256, 128))


def n_sweep(torch, fa):
    """Forward and backward at N = 1024 .. 16384 (B=1, H=16, d=128, bf16), causal and non-causal:
    three launches each (for counter runs) and a timed block each; then a 256 MiB + 256 MiB
    calibration copy."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)
    out = {"workload": "forward and backward, B=1 H=16 d=128 bf16, N sweep", "runs": []}
    for N in SWEEP_N:
        q, k, v, do = (torch.randn(1, 16, N, 128, device="cuda", dtype=torch.bfloat16, generator=gen)
                       for _ in range(4))
        o, lse = torch.empty_like(q), torch.empty(1, 16, N, device="cuda")
        for causal in (False, True):
            for _ in range(3):
                fa.forward(q, k, v, causal=causal, out=o, lse=lse)
            torch.cuda.synchronize()
            ms = _time_calls(lambda: fa.forward(q, k, v, causal=causal, out=o, lse=lse), 10, 2, torch)
            out["runs"].append({"kind": "fwd", "N": N, "causal": causal, "ms": round(ms, 4),
                                "tflops": round(flops_fwd(1, 16, N, 128, causal) / (ms * 1e-3) / 1e12, 1)})
            ws = torch.empty(fa.fattn_bwd_workspace_size(1, 16, N, 128, 2), dtype=torch.uint8, device="cuda")
            for _ in range(3):
                fa.backward(q, k, v, o, do, lse, causal=causal, workspace=ws)
            torch.cuda.synchronize()
            ms = _time_calls(lambda: fa.backward(q, k, v, o, do, lse, causal=causal, workspace=ws), 5, 1, torch)
            out["runs"].append({"kind": "bwd", "N": N, "causal": causal, "ms": round(ms, 4),
                                "tflops": round(2.5 * flops_fwd(1, 16, N, 128, causal) / (ms * 1e-3) / 1e12, 1)})
            del ws
        del q, k, v, do, o, lse
    src = torch.ones(128 * 2**20, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps(out), flush=True)
    return 0


def kernel_pass(torch, fa, fi, reps=3):
    """Each kernel of the step a few times, for counter passes (rocprofv3 --pmc ...): the causal
    forward on the prefill (B=4) and step (B=2) workloads, the backward's stage entry points and
    fattn_bwd on the step workload, the dropout and block-sparse forward and backward on the
    step's shape, the long-context forward (B=1 H=32 N=16384) with both masks, then a
    256 MiB + 256 MiB calibration copy. Inputs are the seeded workloads' own."""
    w5 = fi.WORKLOADS[5]
    B, H, N, d = w5.shape
    q, k, v, do = _upload(fi.workload_inputs(5), torch)
    o, lse = fa.forward(q, k, v, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dvec = torch.empty(B * H * N, dtype=torch.float32, device="cuda")
    q3, k3, v3, _ = _upload(fi.workload_inputs(3), torch)
    o3, l3 = fa.forward(q3, k3, v3, causal=True)
    torch.cuda.synchronize()
    t_end = time.perf_counter() + 0.5  # steady clocks before the counted launches
    while time.perf_counter() < t_end:
        fa.forward(q3, k3, v3, causal=True, out=o3, lse=l3)
        fa.backward(q, k, v, o, do, lse, causal=True)
        torch.cuda.synchronize()
    for _ in range(reps):
        fa.forward(q3, k3, v3, causal=True, out=o3, lse=l3)
        fa.forward(q, k, v, causal=True, out=o, lse=lse)
        fa.backward_stages(q, k, v, o, do, lse, dq, dk, dv, dvec, causal=True)
        fa.backward(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv)
    # the variants on the step's shape: dropout (p = 0.1) and block-sparse (blocks kept with
    # p = 1/4 plus the diagonal), as bench.py times them
    bmask = torch.from_numpy(fi.block_mask(B, H, N // 128, 0.25, 5)).cuda()
    for _ in range(reps):
        fa.forward(q, k, v, causal=True, out=o, lse=lse, p_drop=0.1, seed=1234)
        fa.backward(q, k, v, o, do, lse, causal=True, p_drop=0.1, seed=1234, dq=dq, dk=dk, dv=dv)
        fa.forward_blocksparse(q, k, v, bmask, causal=True, out=o, lse=lse)
        fa.backward_blocksparse(q, k, v, o, do, lse, bmask, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    del q3, k3, v3, o3, l3
    q4, k4, v4, _ = _upload(fi.workload_inputs(4), torch)
    o4, l4 = fa.forward(q4, k4, v4, causal=True)
    for causal in (True, False):
        for _ in range(reps):
            fa.forward(q4, k4, v4, causal=causal, out=o4, lse=l4)
    torch.cuda.synchronize()
    del q4, k4, v4, o4, l4
    src = torch.ones(128 * 2**20, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"kernel_pass": "done", "reps": reps}), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--clock-warmup-s", type=float, default=1.0,
                    help="seconds of untimed fwd+bwd steps before any timing, to reach steady clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", default="6,7",
                    help="split-KV decode workloads to time (comma-separated ids, or 'none')")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB read + 256 MiB write elementwise copy, so HBM "
                         "byte counters can be scaled by a kernel of known traffic")
    ap.add_argument("--n-sweep", action="store_true",
                    help="only run the forward and the backward at N = 1024 .. 16384 (B=1, H=16, d=128, bf16, causal and "
                         "non-causal) a few times each, plus the calibration copy, for the HBM-bytes-vs-N "
                         "counters; prints one JSON line with the per-N times")
    ap.add_argument("--kernel-pass", action="store_true",
                    help="only run each step kernel (and the long-context forward, and a calibration "
                         "copy) a few times, for rocprofv3 counter passes; prints one JSON line")
    a = ap.parse_args(argv)
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the kernels shard over (batch, head) with no "
              "communication, so runs on more than one GPU are not provided", file=sys.stderr)
        return 2

    import torch
    import fattn_inputs as fi
    import io_aware_tiled_fattn_amd as fa
    from io_aware_tiled_fattn_amd import profiling

    fa.lib()
    if a.n_sweep:
        return n_sweep(torch, fa)
    if a.kernel_pass:
        return kernel_pass(torch, fa, fi)
    w5, w3 = fi.WORKLOADS[5], fi.WORKLOADS[3]
    B, H, N, d = w5.shape

    # Training-shaped step: forward + backward.
    inp5 = fi.workload_inputs(5)
    q, k, v, do = _upload(inp5, torch)
    del inp5
    o, lse = fa.forward(q, k, v, causal=True)
    ws = torch.empty(fa.fattn_bwd_workspace_size(B, H, N, d, fa.FATTN_BF16), dtype=torch.uint8, device="cuda")
    dvec = ws[: 4 * B * H * N].view(torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa.backward(q, k, v, o, do, lse, causal=True, workspace=ws)

    # Prefill-shaped forward inputs (B=4), uploaded now so no host work sits between timings.
    inp3 = fi.workload_inputs(3)
    q3, k3, v3, _ = _upload(inp3, torch)
    del inp3
    o3, l3 = fa.forward(q3, k3, v3, causal=True)

    # Decode workloads: one key/value cache shared by both, each with its own queries.
    dec = {}
    dec_ids = [] if a.decode == "none" else [int(x) for x in a.decode.split(",")]
    if dec_ids:
        kv = fi.decode_workload_inputs(dec_ids[0], with_q=False)
        kc, vc = _upload_named(kv, ("k", "v"), torch)
        del kv
        for ident in dec_ids:
            wd = fi.DECODE_WORKLOADS[ident]
            (qd,) = _upload_named(fi.decode_workload_inputs(ident, with_kv=False), ("q",), torch)
            S = fa.fattn_splitkv_num_splits(wd.B, wd.H, wd.Nq, wd.Nk, wd.d)
            wsd = torch.empty(fa.fattn_fwd_splitkv_workspace_size(wd.B, wd.H, wd.Nq, wd.Nk, wd.d, S),
                              dtype=torch.uint8, device="cuda")
            od, ld = fa.forward_splitkv(qd, kc, vc, causal=True, num_splits=S, workspace=wsd)
            op = torch.empty((S, wd.B, wd.H, wd.Nq, wd.d), dtype=torch.float32, device="cuda")
            lp = torch.empty((S, wd.B, wd.H, wd.Nq), dtype=torch.float32, device="cuda")
            dec[ident] = (wd, qd, S, wsd, od, ld, op, lp)

    # Bring the GPU to its steady clock before anything is timed: the engine clock ramps up over
    # the first few hundred milliseconds of sustained MFMA work, and a short warm-up under-reports.
    def step():
        fa.forward(q, k, v, causal=True, out=o, lse=lse)
        fa.backward(q, k, v, o, do, lse, causal=True, workspace=ws, dq=dq, dk=dk, dv=dv)

    t_end = time.perf_counter() + a.clock_warmup_s
    while time.perf_counter() < t_end:
        for _ in range(50):
            step()
        torch.cuda.synchronize()

    T = lambda fn: _time_calls(fn, a.steps, a.warmup, torch)
    st = lambda stages: (lambda: fa.backward_stages(q, k, v, o, do, lse, dq, dk, dv, dvec, causal=True,
                                                    stages=stages))
    ms = {
        "fwd": T(lambda: fa.forward(q, k, v, causal=True, out=o, lse=lse)),
        "pre": T(st((0,))),
        "dkdv": T(st((1,))),
        "dq": T(st((2,))),
        "bwd": T(lambda: fa.backward(q, k, v, o, do, lse, causal=True, workspace=ws)),
    }

    ms_step = T(step)

    # The same step captured once as a HIP graph and replayed: the three kernel launches without
    # the host's per-call work in between.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    step_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(step_graph):
        step()
    torch.cuda.synchronize()
    ms_step_graph = T(step_graph.replay)

    # Ablation: the same forward in the K-outer loop order (one launch per key block, query tile
    # and running state reloaded from HBM on every visit).
    ws_ko = torch.empty(fa.fattn_fwd_kouter_workspace_size(B, H, N, d, fa.FATTN_BF16), dtype=torch.uint8,
                        device="cuda")
    o_ko, l_ko = torch.empty_like(q), torch.empty_like(lse)
    ms_kouter = T(lambda: fa.forward_kouter(q, k, v, causal=True, out=o_ko, lse=l_ko, workspace=ws_ko))
    del ws_ko, o_ko, l_ko

    # Block-sparse forward on the step's shape: 128 x 128 blocks kept with probability 1/4, plus
    # the diagonal, under the causal mask.
    import numpy as np
    nbk = N // 128
    bmask_np = fi.block_mask(B, H, nbk, 0.25, 5)
    bmask = torch.from_numpy(bmask_np).cuda()
    ms_bs = T(lambda: fa.forward_blocksparse(q, k, v, bmask, causal=True, out=o, lse=lse))
    # and its backward (on the block-sparse forward's O and LSE)
    ms_bs_bwd = T(lambda: fa.backward_blocksparse(q, k, v, o, do, lse, bmask, causal=True, workspace=ws))
    # allowed (query, key) pairs: full blocks below the diagonal, half (with the diagonal) on it
    tri = np.tril(np.ones((nbk, nbk), bool), -1)
    pairs_bs = float((bmask_np.astype(bool) & tri).sum() * 128 * 128
                     + np.diagonal(bmask_np, axis1=2, axis2=3).astype(bool).sum() * 128 * 129 // 2)
    f_bs = 4.0 * d * pairs_bs
    density = pairs_bs / (B * H * N * (N + 1) / 2)
    fa.forward(q, k, v, causal=True, out=o, lse=lse)  # leave the step's O and LSE in place

    # Dropout (p = 0.1) on the same step: forward and backward with the Philox keep mask.
    p_drop, seed = 0.1, 1234
    ms_drop_fwd = T(lambda: fa.forward(q, k, v, causal=True, out=o, lse=lse, p_drop=p_drop, seed=seed))
    ms_drop_bwd = T(lambda: fa.backward(q, k, v, o, do, lse, causal=True, workspace=ws, p_drop=p_drop, seed=seed))

    # Prefill-shaped forward (B=4), default tile, then every tile the d = 128 forward supports.
    ms_fwd3 = T(lambda: fa.forward(q3, k3, v3, causal=True, out=o3, lse=l3))
    tile_ms = {}
    for br, bc in FWD_TILES:
        tile_ms[(br, bc)] = T(lambda: fa.forward(q3, k3, v3, causal=True, Br=br, Bc=bc, out=o3, lse=l3))
    del q3, k3, v3, o3, l3

    # Long-context forward (B=1 H=32 N=16384 d=128), both masks.
    inp4 = fi.workload_inputs(4)
    q4, k4, v4, _ = _upload(inp4, torch)
    del inp4
    o4, l4 = torch.empty_like(q4), torch.empty(q4.shape[:3], dtype=torch.float32, device="cuda")
    ms_fwd4 = {c: T(lambda: fa.forward(q4, k4, v4, causal=c, out=o4, lse=l4)) for c in (True, False)}
    del q4, k4, v4, o4, l4

    tr_all = profiling.load_traffic(os.path.join(ROOT, "profiles"))

    # Split-KV decode: whole path (partials + merge), and each kernel on its own.
    decode = {}
    for ident, (wd, qd, S, wsd, od, ld, op, lp) in dec.items():
        causal = True  # with the queries at the end of the sequence (bottom-right alignment)
        t_all = T(lambda: fa.forward_splitkv(qd, kc, vc, causal=causal, num_splits=S, out=od, lse=ld,
                                             workspace=wsd))
        t_part = T(lambda: fa.forward_partial(qd, kc, vc, S, causal=causal, o_parts=op, lse_parts=lp))
        t_comb = T(lambda: fa.combine(op, lp, dtype=torch.bfloat16, out=od, lse=ld))
        bh = wd.B * wd.H
        kv_b = 2 * bh * wd.Nk * wd.d * 2
        q_b = bh * wd.Nq * wd.d * 2
        out_b = bh * wd.Nq * (wd.d * 2 + 4)
        part_b = S * bh * wd.Nq * (wd.d + 1) * 4
        gbs = lambda nbytes, t_ms: nbytes / (t_ms * 1e-3) / 1e9
        dtraffic = {"traffic": None}
        if tr_all and ident == 6:
            sig_d = "splitkv_kernel<Bf16, 128, 32, "
            grid_d = bh * ((wd.Nq + 31) // 32) * S * 64
            for (kname, kgrid), rec in tr_all.items():
                if kname.startswith(sig_d) and kgrid == grid_d:
                    dtraffic = traffic_fields(rec)
        path_gbs = gbs(kv_b + q_b + out_b, t_all)
        part_gbs = gbs(kv_b + q_b + part_b, t_part)
        decode[f"w{ident}"] = {
            "workload": f"{wd.name}: B={wd.B} H={wd.H} Nq={wd.Nq} Nk={wd.Nk} d={wd.d} causal",
            "num_splits": S, "ms": round(t_all, 4), "GB_s": round(path_gbs, 1),
            "frac_of_hbm_peak": round(path_gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": kv_b + q_b + out_b,
            "kernel_ms": {"partial": round(t_part, 4), "combine": round(t_comb, 4)},
            "roofline": {"kernel": "splitkv_kernel (partials)", "bound": "hbm",
                         "achieved": round(part_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(part_gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_launch": kv_b + q_b + part_b, **dtraffic,
                         "ms_per_launch": round(t_part, 4)},
        }
    dec.clear()
    if dec_ids:
        del kc, vc

    if a.calibrate_copy:
        src = torch.ones(128 * 2**20, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    tf = lambda f, t: f / (t * 1e-3) / 1e12
    f_fwd = flops_fwd(B, H, N, d, True)
    f_step = 3.5 * f_fwd
    value = tf(f_step, ms_step)

    # Algorithmic FLOPs per launch of each matmul kernel (causal halves every GEMM), each GEMM
    # 2*N^2*d per head: forward 2 (S, PV); dK/dV 4 (S, dP, dV, dK); dQ 3 (S, dP, dQ). Grids in
    # threads: 512 per work-group; forward and dQ 256 rows per group, dK/dV 128 keys.
    kernels = {
        "fwd": ("fwd_kernel", f_fwd, 1024 * 256, "fwd_kernel<Bf16, 128, 256, 128, 2, true, false, false, false>"),
        "dkdv": ("bwd_dkdv_pair_kernel", 2 * f_fwd, 1024 * 512,
                 "bwd_dkdv_pair_kernel<Bf16, 128, true, false, false, false>"),
        "dq": ("bwd_dq_kernel", 1.5 * f_fwd, 1024 * 256, "bwd_dq_kernel<Bf16, 128, true, false, false, false, false>"),
    }
    dom = max(kernels, key=lambda k_: ms[k_])
    name, fl, grid, sig = kernels[dom]
    achieved = tf(fl, ms[dom])
    traffic = {"traffic": None}
    if tr_all:
        for (kname, kgrid), rec in tr_all.items():
            if kname.startswith(sig) and kgrid == grid:
                traffic = traffic_fields(rec)
    roof = {"kernel": f"{sig} on B=2,H=16,N=4096", "bound": "mfma",
            "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), **traffic,
            "ms_per_launch": round(ms[dom], 4), "algorithmic_tflop_per_launch": round(fl / 1e12, 4)}

    f3 = flops_fwd(w3.B, w3.H, w3.N, w3.d, True)
    fwd3_tf = tf(f3, ms_fwd3)
    bwd_tf = tf(2.5 * f_fwd, ms["bwd"])
    result = {
        "metric": "attention fwd/bwd TFLOP/s and % of MI355X bf16 MFMA peak at N=4096, d=128",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_graph": {"ms_per_step": round(ms_step_graph, 4), "tflops": round(tf(f_step, ms_step_graph), 1),
                       "note": "the same step captured as one HIP graph and replayed"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "training step fwd+bwd, B=2 H=16 N=4096 d=128 causal",
                   "B": B, "H": H, "N": N, "d": d, "causal": True},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"workload": "B=4 H=16 N=4096 d=128 causal", "ms": round(ms_fwd3, 4),
                "tflops": round(fwd3_tf, 1), "frac_of_peak": round(fwd3_tf / PEAK_BF16_TFLOPS, 4),
                "tile_default": "256x128",
                "tiles": {f"{br}x{bc}": {"ms": round(t_, 4), "tflops": round(tf(f3, t_), 1)}
                          for (br, bc), t_ in tile_ms.items()}},
        "fwd_long": {f"{'causal' if c else 'noncausal'}": {
                         "workload": f"B=1 H=32 N=16384 d=128 {'causal' if c else 'non-causal'}",
                         "ms": round(t_, 4), "tflops": round(tf(flops_fwd(1, 32, 16384, 128, c), t_), 1),
                         "frac_of_peak": round(tf(flops_fwd(1, 32, 16384, 128, c), t_) / PEAK_BF16_TFLOPS, 4)}
                     for c, t_ in ms_fwd4.items()},
        "bwd": {"workload": "B=2 H=16 N=4096 d=128 causal", "ms": round(ms["bwd"], 4),
                "tflops": round(bwd_tf, 1), "frac_of_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
                "workspace_bytes": ws.numel()},
        "kernel_ms": {k_: round(t, 4) for k_, t in ms.items()},
        "roofline": roof,
    }
    ko_launches = (N + 127) // 128
    ko = {"workload": "B=2 H=16 N=4096 d=128 causal, K-outer order (FA-1), 256 x 128 tiles",
          "ms": round(ms_kouter, 4), "tflops": round(tf(f_fwd, ms_kouter), 1),
          "time_vs_q_outer": round(ms_kouter / ms["fwd"], 2), "launches": ko_launches}
    if tr_all:
        recs = [r for (kn, _), r in tr_all.items() if kn.startswith("ko_kernel<Bf16, 128, 256, 128, true>")]
        if recs:
            ko["hbm_bytes_per_call"] = {"fetch": round(recs[0]["fetch_bytes"] * ko_launches),
                                        "write": round(recs[0]["write_bytes"] * ko_launches),
                                        "source": "profiles/traffic.json (per-launch mean x launches)"}
        fw = [r for (kn, g), r in tr_all.items() if kn.startswith(kernels["fwd"][3]) and g == kernels["fwd"][2]]
        if fw:
            ko["q_outer_hbm_bytes_per_call"] = {"fetch": round(fw[0]["fetch_bytes"]),
                                                "write": round(fw[0]["write_bytes"])}
    result["ablation_kouter"] = ko
    result["blocksparse"] = {"workload": "B=2 H=16 N=4096 d=128 causal, 128x128 blocks kept with p = 1/4 "
                                         "plus the diagonal",
                             "ms": round(ms_bs, 4), "allowed_fraction_of_causal_pairs": round(density, 4),
                             "tflops_on_allowed_pairs": round(tf(f_bs, ms_bs), 1),
                             "time_vs_dense": round(ms_bs / ms["fwd"], 3),
                             "bwd_ms": round(ms_bs_bwd, 4),
                             "bwd_tflops_on_allowed_pairs": round(tf(2.5 * f_bs, ms_bs_bwd), 1),
                             "bwd_time_vs_dense": round(ms_bs_bwd / ms["bwd"], 3)}
    result["dropout"] = {"workload": "B=2 H=16 N=4096 d=128 causal, p = 0.1 (Philox4x32-10 keep mask)",
                         "fwd_ms": round(ms_drop_fwd, 4), "bwd_ms": round(ms_drop_bwd, 4),
                         "fwd_tflops": round(tf(f_fwd, ms_drop_fwd), 1),
                         "bwd_tflops": round(tf(2.5 * f_fwd, ms_drop_bwd), 1),
                         "fwd_time_vs_plain": round(ms_drop_fwd / ms["fwd"], 2),
                         "bwd_time_vs_plain": round(ms_drop_bwd / ms["bwd"], 2)}
    if decode:
        result["decode"] = decode
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_oracle_baseline()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
