"""Build the gfx950 HIP library libgemm_f16.so in-tree with hipcc.

Three translation units: csrc/gemm_f16.hip (every GEMM kernel instantiation and
the C ABI of include/gemm_f16.h), csrc/softmax.hip (the row softmax, C ABI in
include/softmax_f16.h) and csrc/attention.hip (the attention forward pass, C ABI
in include/attention_f16.h).  Flags: gfx950 only, -O3, no
fast-math, packed-fp32 VALU instructions disabled, a pragma-unroll threshold
high enough for the fully unrolled MFMA schedules.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libgemm_f16.so")
SOURCES = [os.path.join(CSRC, f) for f in ("gemm_f16.hip", "softmax.hip", "attention.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("common.h", "tile_pipe_kernel.h", "skinny_kernel.h")] + [
    os.path.join(INCLUDE, "gemm_f16.h"), os.path.join(INCLUDE, "softmax_f16.h"), os.path.join(INCLUDE, "attention_f16.h")
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_cmd(out: str, save_temps_dir: str | None = None) -> list[str]:
    cmd = [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++20", "-shared", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the fenced MFMA schedules are fully unrolled loops of a few thousand instructions; a refused
        # unroll leaves the fragment and accumulator arrays in scratch memory
        "-mllvm", "-pragma-unroll-threshold=200000",
        "-I" + INCLUDE, "-I" + CSRC, "-o", out,
    ] + SOURCES
    if save_temps_dir:
        cmd.insert(1, "-save-temps=obj")
    return cmd


def build(verbose: bool = False, save_temps_dir: str | None = None) -> str:
    """Compile libgemm_f16.so next to this file (always rebuilds)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cwd = save_temps_dir or PKG_DIR
    if save_temps_dir:
        os.makedirs(save_temps_dir, exist_ok=True)
    cmd = compile_cmd(tmp, save_temps_dir)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None, help="directory for the .s / .bc intermediates")
    a = ap.parse_args()
    print(build(verbose=True, save_temps_dir=a.save_temps))
