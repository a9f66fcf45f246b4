"""One-wave-per-SIMD forward ablation against the library forward, on the GPU.

Build first: python -m io_aware_tiled_fattn_amd.build --tools (makes libfwd_one_wave.so here).
Run:         python io_aware_tiled_fattn_amd/microbench/fwd_one_wave.py [--timing-only]

Checks the ablation kernel against fattn_fwd on ragged, causal, negative-scale, zero-scale and
rising-logit inputs (the last force the lazy rescale), then times both on the prefill and
long-context shapes (B=4 H=16 N=4096 causal; B=2 H=16 N=4096 causal; B=1 H=32 N=16384 causal and
non-causal; d=128 bf16) with HIP events on the launch stream. Prints one JSON line per result.
"""
import ctypes
import json
import os
import sys
import time

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import io_aware_tiled_fattn_amd as fa  # noqa: E402

VARIANTS = ((3, 0), (3, 1), (4, 1))  # (K/V stages, schedule: 0 = compiler order, 1 = fixed slots)


def load():
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    ow = ctypes.CDLL(os.path.join(HERE, "libfwd_one_wave.so"), mode=ctypes.RTLD_LOCAL)
    ow.fwd_one_wave.argtypes = [vp, vp, vp, vp, vp, i, i, i, f, i, i, i, vp]
    return ow, fa.lib()


def main(argv):
    ow, lib = load()
    st = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: t.data_ptr()

    def ref(q, k, v, sc, causal):
        B, H, N, _ = q.shape
        o = torch.empty_like(q)
        lse = torch.empty(B, H, N, device="cuda")
        assert lib.fattn_fwd(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), B, H, N, 128, sc, causal, 2, st) == 0
        return o, lse

    def one(q, k, v, sc, causal, ns, sched, o=None, lse=None):
        B, H, N, _ = q.shape
        if o is None:
            o = torch.full_like(q, float("nan"))
            lse = torch.full((B, H, N), float("nan"), device="cuda")
        rc = ow.fwd_one_wave(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), B, H, N, sc, causal, ns, sched, st)
        assert rc == 0, rc
        return o, lse

    torch.manual_seed(0)
    worst = 0.0
    if "--timing-only" not in argv:
        cases = [(1, 8, 64, 1, 1.0), (1, 8, 100, 1, 1.0), (1, 8, 256, 0, 1.0), (2, 8, 1000, 1, 1.0),
                 (2, 8, 1000, 0, 1.0), (1, 8, 4096, 1, -1.0), (1, 8, 777, 0, 0.0), (2, 4, 321, 1, 1.0)]
        for B, H, N, causal, sgn in cases:
            q, k, v = (torch.randn(B, H, N, 128, device="cuda").to(torch.bfloat16) for _ in range(3))
            sc = sgn * 128 ** -0.5
            ro, rl = ref(q, k, v, sc, causal)
            for ns, sched in VARIANTS:
                mo, ml = one(q, k, v, sc, causal, ns, sched)
                torch.cuda.synchronize()
                d_o = (mo.float() - ro.float()).abs().max().item()
                d_l = (ml - rl).abs().max().item()
                worst = max(worst, d_o)
                print(json.dumps({"check": [B, H, N, causal, sgn], "ns": ns, "sched": sched, "o_max_abs_diff": d_o,
                                  "lse_max_abs_diff": d_l}), flush=True)
        for causal in (0, 1):  # logits that grow along the keys: the reference max moves often
            B, H, N = 1, 8, 2048
            q = torch.randn(B, H, N, 128, device="cuda")
            ramp = (torch.arange(N, device="cuda").float() / 128.0)[None, None, :, None]
            k = torch.randn(B, H, N, 128, device="cuda") + ramp * q.mean(2, keepdim=True).sign()
            v = torch.randn(B, H, N, 128, device="cuda")
            q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
            ro, rl = ref(q, k, v, 128 ** -0.5, causal)
            for ns, sched in VARIANTS:
                mo, ml = one(q, k, v, 128 ** -0.5, causal, ns, sched)
                torch.cuda.synchronize()
                d_o = (mo.float() - ro.float()).abs().max().item()
                worst = max(worst, d_o)
                print(json.dumps({"check": "rising logits", "causal": causal, "ns": ns, "sched": sched,
                                  "o_max_abs_diff": d_o, "lse_max_abs_diff": (ml - rl).abs().max().item(),
                                  "lse_range": [rl.min().item(), rl.max().item()]}), flush=True)

    def timeit(fn, reps=30):
        for _ in range(5):
            fn()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps)
        return sorted(ts)[2]

    for B, H, N, causal in ((4, 16, 4096, 1), (2, 16, 4096, 1), (1, 32, 16384, 1), (1, 32, 16384, 0)):
        q, k, v = (torch.randn(B, H, N, 128, device="cuda").to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty(B, H, N, device="cuda")
        sc = 128 ** -0.5
        flops = 4 * B * H * N * N * 128 / (2 if causal else 1)
        t0 = time.time()
        while time.time() - t0 < 0.5:  # warm clocks
            lib.fattn_fwd(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), B, H, N, 128, sc, causal, 2, st)
        res = {"shape": {"B": B, "H": H, "N": N, "causal": causal}}
        ms = timeit(lambda: lib.fattn_fwd(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), B, H, N, 128, sc, causal, 2, st))
        res["library"] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1)}
        for ns, sched in VARIANTS:
            ms = timeit(lambda: one(q, k, v, sc, causal, ns, sched, o, lse))
            res[f"one_wave_ns{ns}_sched{sched}"] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1)}
        print(json.dumps(res), flush=True)
    print(json.dumps({"worst_o_max_abs_diff": worst}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
