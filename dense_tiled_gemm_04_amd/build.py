"""Build the gfx950 HIP library libgemm_f16.so in-tree with hipcc.

Four translation units: csrc/gemm_f16.hip (every GEMM kernel instantiation and
the C ABI of include/gemm_f16.h), csrc/softmax.hip (the row softmax, C ABI in
include/softmax_f16.h) and csrc/attention.hip (the attention forward pass, C ABI
in include/attention_f16.h), csrc/calibration.hip (the MFMA throughput
calibration, C ABI in include/calibration_f16.h).  Flags: gfx950 only, -O3, no
fast-math, packed-fp32 VALU instructions disabled, a pragma-unroll threshold
high enough for the fully unrolled MFMA schedules.

The units compile in parallel to objects, which are then linked.  Each compile
asks for the compiler's per-kernel resource remarks (VGPRs, AGPRs, scratch,
occupancy, LDS); they are written to _build/kernel_resources.json, and the
build fails if any kernel of the shipped library uses scratch memory (a
register spill would otherwise show up only as a slowdown).  Before a built
library replaces the old one, its gfx950 code is disassembled and checked for
wait-state hazards around the inline-asm copies and MFMAs, which the compiler
does not guard (asm_check.py); a hazard fails the build.
"""
from __future__ import annotations

import concurrent.futures
import json
import os
import re
import shutil
import subprocess
import sys

try:
    from . import asm_check
except ImportError:  # run as a script from the package directory
    import asm_check

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libgemm_f16.so")
RESOURCES_PATH = os.path.join(BUILD_DIR, "kernel_resources.json")
SOURCES = [os.path.join(CSRC, f) for f in ("gemm_f16.hip", "softmax.hip", "attention.hip", "calibration.hip")]


# Sources each kernel family is built from: a change to any of them voids what was measured on that family's
# kernels (HBM traffic records, timeline builds).
KERNEL_SOURCES = {
    "gemm": ["common.h", "tile_pipe_kernel.h", "skinny_kernel.h", "skinny_splitk_kernel.h", "pingpong_kernel.h",
             "gemm_f16.hip", "config_table.inc"],
    "softmax": ["common.h", "softmax.hip"],
    "attention": ["common.h", "attention.hip"],
}


def source_digest(family: str = "gemm") -> str:
    """sha256 over the named sources of one kernel family (file names and contents, in name order)."""
    import hashlib

    h = hashlib.sha256()
    for f in sorted(KERNEL_SOURCES[family]):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def base_flags() -> list[str]:
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the fenced MFMA schedules are fully unrolled loops of a few thousand instructions; a refused
        # unroll leaves the fragment and accumulator arrays in scratch memory
        "-mllvm", "-pragma-unroll-threshold=200000",
        "-I" + INCLUDE, "-I" + CSRC,
    ]


def compile_cmd(out: str, save_temps_dir: str | None = None) -> list[str]:
    """One hipcc command that compiles every source straight into the shared library `out`."""
    cmd = [hipcc()] + base_flags() + ["-shared", "-o", out] + SOURCES
    if save_temps_dir:
        cmd.insert(1, "-save-temps=obj")
    return cmd


_REMARK_NAME = re.compile(r"remark: Function Name: (\S+)")
_REMARK_FIELD = re.compile(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\S+) \[-Rpass-analysis=kernel-resource-usage\]")


def parse_resource_remarks(text: str) -> list[dict]:
    """Per-kernel records from the compiler's -Rpass-analysis=kernel-resource-usage remarks."""
    rows, cur = [], None
    for line in text.splitlines():
        m = _REMARK_NAME.search(line)
        if m:
            cur = {"kernel": m.group(1)}
            rows.append(cur)
            continue
        m = _REMARK_FIELD.search(line)
        if m and cur is not None:
            key, val = m.group(1).strip(), m.group(2)
            cur[key] = int(val) if re.fullmatch(r"-?\d+", val) else val
    return rows


def scratch_users(rows: list[dict]) -> list[dict]:
    """Kernels with scratch memory: spilled VGPRs or any other scratch use.  (SGPR spills go to lanes of a
    VGPR, not to memory; they are recorded but allowed.)"""
    return [r for r in rows if int(r.get("ScratchSize [bytes/lane]", 0)) > 0 or int(r.get("VGPRs Spill", 0)) > 0]


def _compile_object(src: str, obj: str, defines: list[str]) -> tuple[str, str]:
    cmd = [hipcc()] + base_flags() + defines + ["-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, cwd=PKG_DIR, capture_output=True, text=True)
    if r.returncode != 0:
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "remark:" not in l)
        raise RuntimeError("hipcc failed on %s:\n%s" % (os.path.basename(src), err[-6000:]))
    return src, r.stderr


def build_library(out: str, sources: list[str], defines: list[str] | None = None, allow_scratch: bool = False,
                  resources_path: str | None = None, verbose: bool = False) -> list[dict]:
    """Compile `sources` in parallel and link them into the shared library `out`.  Returns the per-kernel
    resource records; raises if a kernel uses scratch memory unless allow_scratch."""
    defines = defines or []
    os.makedirs(BUILD_DIR, exist_ok=True)
    tag = "%s.%d" % (os.path.splitext(os.path.basename(out))[0], os.getpid())
    objs = [os.path.join(BUILD_DIR, "%s.%s.o" % (tag, os.path.splitext(os.path.basename(s))[0])) for s in sources]
    rows = []
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(sources)) as ex:
            futs = [ex.submit(_compile_object, s, o, defines) for s, o in zip(sources, objs)]
            for f in futs:
                src, stderr = f.result()
                for r in parse_resource_remarks(stderr):
                    r["source"] = os.path.basename(src)
                    rows.append(r)
        bad = scratch_users(rows)
        if bad and not allow_scratch:
            raise RuntimeError("kernels using scratch memory (register spills):\n" + "\n".join(
                "  %s: %s bytes/lane, %s VGPRs spilled" % (r["kernel"], r.get("ScratchSize [bytes/lane]"),
                                                           r.get("VGPRs Spill")) for r in bad))
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, cwd=PKG_DIR, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stderr[-4000:])
        try:
            n = asm_check.check_library(tmp)
        except Exception:
            os.remove(tmp)
            raise
        if verbose:
            print("wait-state check: %d MFMA and vector-memory instructions, no hazard" % n, flush=True)
        os.replace(tmp, out)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    if resources_path:
        with open(resources_path, "w") as f:
            json.dump(rows, f, indent=1)
    return rows


def build(verbose: bool = False, save_temps_dir: str | None = None) -> str:
    """Compile libgemm_f16.so next to this file (always rebuilds)."""
    if save_temps_dir:
        # one serial compile that keeps the .s / .bc intermediates
        os.makedirs(save_temps_dir, exist_ok=True)
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        cmd = compile_cmd(tmp, save_temps_dir)
        r = subprocess.run(cmd, cwd=save_temps_dir, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + r.stderr[-6000:])
        os.replace(tmp, LIB_PATH)
        return LIB_PATH
    rows = build_library(LIB_PATH, SOURCES, resources_path=RESOURCES_PATH, verbose=verbose)
    if verbose:
        sg = sum(1 for r in rows if int(r.get("SGPRs Spill", 0)) > 0)
        print("%d kernels, none using scratch (%d with SGPRs spilled to VGPR lanes); resources in %s"
              % (len(rows), sg, RESOURCES_PATH), flush=True)
    return LIB_PATH


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None, help="directory for the .s / .bc intermediates")
    a = ap.parse_args()
    print(build(verbose=True, save_temps_dir=a.save_temps))
