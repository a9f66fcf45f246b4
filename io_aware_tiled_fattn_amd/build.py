"""Build libfattn.so for gfx950 with hipcc (no GPU needed: hipcc cross-compiles).

Usage: python -m io_aware_tiled_fattn_amd.build [--verbose] [--resource-usage] [--tools]

--tools also builds the stand-alone measurement programs under microbench/ (not part of the
library; each writes its own executable beside its source).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libfattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["fattn_api.cpp", "fattn_fwd.hip", "fattn_bwd.hip", "fattn_splitkv.hip", "fattn_kouter.hip",
           "fattn_noalloc.hip"]

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: the softmax reads them every tile, and AGPR<->VGPR copies
    # cost both instructions and registers
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libfattn needs the ROCm toolchain")


def _compile(src, hipcc, extra, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{text}")
    return obj, text


MICROBENCH = os.path.join(HERE, "microbench")
TOOLS = ["issue_rates.hip", "atomic_rates.hip", "stream_rates.hip"]  # stand-alone measurement programs, on request
# measurement libraries, on request: the one-wave forward ablation keeps its MFMA results in AGPRs,
# so it is built without the VGPR-form flag
TOOL_LIBS = ["fwd_one_wave.hip"]


def _build_tool(src, hipcc, verbose):
    exe = os.path.join(MICROBENCH, os.path.splitext(src)[0])
    cmd = [hipcc, *[c for c in COMMON if c != "-fPIC"], os.path.join(MICROBENCH, src), "-o", exe + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
    os.replace(exe + ".tmp", exe)


def _build_tool_lib(src, hipcc, verbose):
    out = os.path.join(MICROBENCH, "lib" + os.path.splitext(src)[0] + ".so")
    flags = [c for c in COMMON if c not in ("-mllvm", "-amdgpu-mfma-vgpr-form")]
    cmd = [hipcc, *flags, "-shared", os.path.join(MICROBENCH, src), "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, resource_usage: bool = False, tools: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, hipcc, extra, verbose), SOURCES))
    for _, text in results:
        if text.strip() and (verbose or resource_usage):
            print(text)
    tmp = OUT + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    if tools:
        for src in TOOLS:
            if os.path.exists(os.path.join(MICROBENCH, src)):
                _build_tool(src, hipcc, verbose)
        for src in TOOL_LIBS:
            if os.path.exists(os.path.join(MICROBENCH, src)):
                _build_tool_lib(src, hipcc, verbose)
    return OUT


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("--tools", action="store_true", help="also build the microbench/ programs")
    a = ap.parse_args(argv)
    print(build(a.verbose, a.resource_usage, a.tools))


if __name__ == "__main__":
    sys.exit(main())
