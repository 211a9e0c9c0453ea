"""Build the HIP library libcompressed_linear.so in-tree for gfx950.

    python -m compressed_linear_amd.build [--jobs N] [--verbose]

Every source compiles with hipcc to an object under compressed_linear_amd/_build/
and links into compressed_linear_amd/libcompressed_linear.so.  Always rebuilds.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcompressed_linear.so")
ARCH = os.environ.get("CL_OFFLOAD_ARCH", "gfx950")

SOURCES = ["pack.cpp", "runtime.hip", "decode.hip", "aux.hip", "prefill.hip", "fit.hip", "fit_lowrank.cpp", "probe.hip",
           "decode_lut3.hip", "decode_lut4.hip", "decode_int4.hip", "decode_int4_24.hip",
           "decode_int8.hip", "decode_int8_bm.hip",
           "decode_rows_lut3.hip", "decode_rows_lut4.hip", "decode_rows_int4.hip", "decode_rows_int4_24.hip",
           "decode_rows_int8.hip",
           "decode_stream_lut3.hip", "decode_stream_lut4.hip", "decode_stream_int4.hip", "decode_stream_int4_24.hip",
           "decode_stream_int8.hip",
           "decode_mfma_lut3.hip", "decode_mfma_lut4.hip", "decode_mfma_int4.hip", "decode_mfma_int4_24.hip",
           "decode_mfma_int8.hip", "decode_mfma_int8_bm.hip",
           "prefill_lut3.hip", "prefill_lut4.hip", "prefill_int.hip", "prefill_lr.hip"]

LIBS = ["-lrocblas"]  # the Naive-LoRA fitter's products with the residual

COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-result",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-x", "hip"] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs + LIBS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
    sys.exit(0)
