"""Offline configuration sweep of the gfx950 fp16 GEMM library.

This plays the part of the tutorial's autotuner. That autotuner has a search
space over tile sizes, K-block, pipeline depth and thread count, drops the
configurations that exceed the shared-memory budget, then compiles, benches,
validates and caches each one (news article on TileLang kernel design,
paragraph on autotuning; blog post "Designing High-Performance GPU Kernels
with TileLang", section "Step 5"). Here the search happens once, offline, on
the target GPU, and its outcome is compiled into the library. There is no JIT.

Steps:

1. ``space()`` enumerates kernel configurations. The tile kernel's knobs are
   block tile, K-block, waves, LDS stages, tile-order group, barrier slot,
   copy stride, loader (LDS-DMA, buffer LDS-DMA or registers), MFMA shape,
   read spreading and waves per SIMD; the skinny kernel's are rows per
   workgroup and stages. ``valid()`` mirrors the kernels' static_asserts and
   applies the budgets: at most 160 KiB of LDS per workgroup (per CU when two
   workgroups share one), and the 512 registers per lane (VGPR + AGPR) shared
   by the waves of a SIMD.
2. ``--build`` writes the whole space into a config-table include and
   compiles ``libgemm_f16_sweep.so`` from the library's own sources, with
   -DGEMM_F16_CONFIG_TABLE pointing at that include.
3. ``--run`` (on the GPU) times every configuration on each sweep workload
   through the C ABI entry ``gemm_f16_with_config``: launches back to back
   after a warm-up, timed in ~1 ms chunks between HIP events (median chunk). It checks each output against a float32
   PyTorch reference on sampled rows; that check is a screen only, and the
   library's parity tests compare with the CPU oracle. One JSON record per
   (config, workload) is appended to the results file, and a restarted run
   skips the records already there.
4. ``--select`` picks, for each shape class the dispatcher knows (skinny
   M <= 16/32/64; LDS-DMA huge (several rounds of 256x256 tiles per CU),
   big (about one round) or small; buffer LDS-DMA (unaligned, K % 8 == 0)
   big or small; register loader (K % 8 != 0) big or small), the
   configuration with the lowest geometric-mean time over that class's
   workloads. It writes csrc/config_table.inc with just those configurations
   and a Markdown summary of the measurements.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import subprocess
import sys
import time

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
TABLE = os.path.join(CSRC, "config_table.inc")
SWEEP_LIB = os.path.join(PKG_DIR, "libgemm_f16_sweep.so")
SWEEP_TABLE = os.path.join(PKG_DIR, "_build", "sweep_space.inc")
WARM_MS = 50.0   # back-to-back work before a configuration's timed chunks

LDS_PER_CU = 160 * 1024
REGS_PER_LANE = 512      # VGPR + AGPR per SIMD lane, shared by the waves resident on the SIMD
SK_BN, SK_BK, SK_WAVES = 64, 128, 4   # skinny kernel constants (csrc/skinny_kernel.h)
SKS_BN = 256                           # split-K skinny panel width (csrc/skinny_splitk_kernel.h)


@dataclasses.dataclass(frozen=True)
class Tile:
    bm: int
    bn: int
    bk: int
    wm: int
    wn: int
    stages: int
    group: int
    bslot: int
    dstride: int
    loader: str          # "dma" | "buf" | "reg"
    cslot: int = 0
    wpe: int = 1         # waves per SIMD; a workgroup of wm*wn waves puts wm*wn/4 on each SIMD, so a CU holds
                         # wpe / (wm*wn/4) workgroups (4 waves: wpe workgroups; 8 waves at wpe 2: one)
    mf: int = 32         # MFMA shape: 32 -> 32x32x16, 16 -> 16x16x32
    spread: int = 0      # schedule flags: 1 LDS reads spread evenly over a k-step's slots, 2 A refilled in
                         # place (one A fragment set), 4 MFMAs as asm on accumulators pinned to AGPRs,
                         # 8 copies of stage kt+STAGES issued right after stage kt's barrier, 16 (with 2) the
                         # next k-step's B reads front-loaded, 32 C staged through LDS and written with
                         # row-contiguous 16-byte stores, 64 (with 32) those stores non-temporal, 128 the A ring
                         # one stage deeper than the B ring
    bt: int = 0          # B given transposed (Bt[N][K])

    kind = "tile"

    @property
    def name(self) -> str:
        n = "%s_%dx%dx%d_w%dx%d_s%d_g%d_b%d_d%d" % (self.loader, self.bm, self.bn, self.bk, self.wm, self.wn,
                                                   self.stages, self.group, self.bslot, self.dstride)
        if self.loader == "reg":
            n += "_c%d" % self.cslot
        n += "_o%d" % self.wpe if self.wpe != 1 else ""
        n += "_m16" if self.mf == 16 else ""
        n += "_ip" if self.spread & 2 else ("_sp" if self.spread & 1 else "")
        n += "_pa" if self.spread & 4 else ""
        n += "_ea" if self.spread & 8 else ""
        n += "_fb" if self.spread & 16 else ""
        n += "_le" if self.spread & 32 else ""
        n += "_nt" if self.spread & 64 else ""
        n += "_ax" if self.spread & 128 else ""
        return n + ("_bt" if self.bt else "")

    # derived quantities, as in TilePipeCfg (csrc/tile_pipe_kernel.h)
    @property
    def lds_bytes(self) -> int:
        a_stages = self.stages + (1 if self.spread & 128 else 0)   # deeper A ring
        return a_stages * self.bm * self.bk * 2 + self.stages * self.bk * self.bn * 2

    def derived(self):
        nw = self.wm * self.wn
        wtm, wtn = self.bm // self.wm, self.bn // self.wn
        tm, tn = wtm // self.mf, wtn // self.mf
        ca, cb = self.bk // 8, self.bn // 8
        ksteps = self.bk // (16 if self.mf == 32 else 32)
        a_ins = self.bm * ca // 64 // nw
        b_ins = (self.bn * ca if self.bt else self.bk * cb) // 64 // nw
        return dict(nw=nw, wtm=wtm, wtn=wtn, tm=tm, tn=tn, ca=ca, cb=cb, ksteps=ksteps, a_ins=a_ins, b_ins=b_ins,
                    per_stage=a_ins + b_ins, nmma=tm * tn, nrd=tm + (tn if self.bt else 2 * tn),
                    nacc=self.mf * self.mf // 64)

    def macro(self) -> str:
        return "TILE_CFG(%d, %d, %d, %d, %d, %d, %d, %d, %d, %s, %d, %d, %d, %d, %d, \"%s\")" % (
            self.bm, self.bn, self.bk, self.wm, self.wn, self.stages, self.group, self.bslot, self.dstride,
            {"dma": "LOAD_DMA", "buf": "LOAD_BUF", "reg": "LOAD_REG"}[self.loader], self.cslot, self.wpe, self.mf,
            self.spread, self.bt, self.name)


@dataclasses.dataclass(frozen=True)
class Skinny:
    mb: int
    stages: int
    bt: int = 0          # B given transposed (Bt[N][K])
    krot: int = 0        # K stages walked from stage (workgroup mod KT)
    a16: int = 0         # A copied by 16-byte LDS-DMA (else 4-byte)

    kind = "skinny"
    loader = "lds_dma"

    @property
    def name(self) -> str:
        return "skinny_m%d_s%d" % (16 * self.mb, self.stages) + ("_r" if self.krot else "") + \
            ("_a16" if self.a16 else "") + ("_bt" if self.bt else "")

    @property
    def lds_bytes(self) -> int:
        return self.stages * (16 * self.mb * SK_BK * 2 + SK_BK * SK_BN * 2)

    def macro(self) -> str:
        return "SKINNY_CFG(%d, %d, %d, %d, %d, \"%s\")" % (self.mb, self.stages, self.bt, self.krot, self.a16, self.name)


@dataclasses.dataclass(frozen=True)
class SplitK:
    """The split-K skinny path (csrc/skinny_splitk_kernel.h), B[K][N] only: 256-column panels over `splits`
    contiguous K ranges (512-byte row segments of B), fp32 partial sums in a workspace, then a reduce kernel
    that sums the ranges in order and applies the epilogue."""
    mb: int
    stages: int
    bk: int = 32
    splits: int = 4

    kind = "splitk"
    loader = "lds_dma"
    bt = 0

    @property
    def name(self) -> str:
        return "splitk_m%d_s%d_k%d_x%d" % (16 * self.mb, self.stages, self.bk, self.splits)

    @property
    def lds_bytes(self) -> int:
        return self.stages * (16 * self.mb * self.bk * 2 + self.bk * SKS_BN * 2)

    def macro(self) -> str:
        return "SPLITK_CFG(%d, %d, %d, %d, \"%s\")" % (self.mb, self.stages, self.bk, self.splits, self.name)


@dataclasses.dataclass(frozen=True)
class PingPong:
    """The ping-pong schedule (csrc/pingpong_kernel.h): a 256x256 tile on 8 waves in two groups, one wave of
    each per SIMD, taking turns between the 64 back-to-back MFMAs of a 64-deep stage and the LDS reads and
    copies of their next one, two stages in LDS (128 KiB); staged epilogue; whole tiles only."""
    group: int = 4
    bt: int = 0
    nt: int = 1          # non-temporal C stores

    kind = "tile"
    loader = "dma"
    bm, bn, bk, wm, wn, stages, wpe, mf = 256, 256, 64, 2, 4, 2, 2, 16

    @property
    def spread(self) -> int:
        return 256 | 32 | (64 if self.nt else 0)

    @property
    def name(self) -> str:
        return "pp_256x256x64_w2x4_g%d" % self.group + ("_nt" if self.nt else "") + ("_bt" if self.bt else "")

    @property
    def lds_bytes(self) -> int:
        return 2 * (256 * 64 * 2 + 64 * 256 * 2)

    def macro(self) -> str:
        return "PINGPONG_CFG(%d, %d, %d, \"%s\")" % (self.group, self.bt, self.nt, self.name)


def pow2(x: int) -> bool:
    return x > 0 and (x & (x - 1)) == 0


def valid(c) -> bool:
    """The kernels' static_asserts plus the LDS and register budgets."""
    if isinstance(c, PingPong):   # one fixed shape, within budget by construction (static_asserts)
        return c.group in (1, 4, 8) and c.lds_bytes <= LDS_PER_CU
    if isinstance(c, SplitK):
        b_ins = c.bk * SKS_BN * 2 // 16 // (SK_WAVES * 64)
        a_ins = 16 * c.mb * c.bk * 2 // 4 // (SK_WAVES * 64)
        return (c.bk % 32 == 0 and c.stages >= 2 and c.splits >= 2 and (c.stages - 2) * (a_ins + b_ins) <= 63
                and c.lds_bytes <= LDS_PER_CU)
    if isinstance(c, Skinny):
        b_ins = SK_BK * SK_BN * 2 // 16 // (SK_WAVES * 64)
        a_ins = 16 * c.mb * SK_BK * 2 // (16 if c.a16 else 4) // (SK_WAVES * 64)
        return c.stages >= 2 and (c.stages - 2) * (a_ins + b_ins) <= 63 and c.lds_bytes <= LDS_PER_CU
    if c.mf not in (16, 32) or c.loader not in ("dma", "buf", "reg"):
        return False
    d = c.derived()
    if d["ksteps"] % 2 or d["wtm"] % c.mf or d["wtn"] % c.mf or d["tm"] < 1 or d["tn"] < 1:
        return False
    if not 0 <= c.spread <= 255 or (c.spread & 2 and d["tm"] < 2) or (c.spread & 16 and not c.spread & 2):
        return False
    # LDS epilogue: the C tile fits in the stage buffers, power-of-two 16-byte chunks per sub-tile row;
    # non-temporal C stores only with it
    rch = d["wtn"] // 8
    if c.spread & 32 and not (c.bm * c.bn * 2 <= c.lds_bytes and ((pow2(rch) and 4 <= rch <= 64) or rch == 12)):
        return False
    if c.spread & 64 and not c.spread & 32:
        return False
    # deeper A ring: ring loaders, early copies, in-place A, two B stages
    if c.spread & 128 and not (c.loader in ("dma", "buf") and c.spread & 8 and c.spread & 2 and c.stages == 2):
        return False
    cb_ok = pow2(d["cb"]) or (d["cb"] % 8 == 0 and (c.bn * 2) % 256 == 128)   # e.g. BN = 192
    if not (pow2(d["ca"]) and cb_ok and d["cb"] >= 4):
        return False
    if (c.bm * d["ca"]) % (64 * d["nw"]) or ((c.bn * d["ca"]) if c.bt else (c.bk * d["cb"])) % (64 * d["nw"]):
        return False
    ps = d["per_stage"]
    if c.stages < 2 or ps * (c.stages - 1) > 63:
        return False
    # wpe is waves per SIMD; a workgroup of nw waves puts nw / 4 of them on each SIMD
    if d["nw"] % 4 or c.wpe % (d["nw"] // 4) or c.lds_bytes * (c.wpe // (d["nw"] // 4)) > LDS_PER_CU:
        return False
    last = (d["ksteps"] - 1) * d["nmma"] + c.bslot
    if not (0 <= c.bslot and c.bslot + 1 < d["nmma"]):
        return False
    if c.spread & 8:   # early copies: ring loaders, all issued after the barrier within the stage
        if c.loader == "reg" or not (c.dstride >= 1 and last + 1 + (ps - 1) * c.dstride < d["ksteps"] * d["nmma"]):
            return False
    elif not (c.dstride >= 1 and (ps - 1) * c.dstride < last):
        return False
    if c.loader == "reg":
        if c.stages != 2 or c.cslot < 0 or c.cslot + ps > last + 1:
            return False
        if c.cslot + (ps - 1) * c.dstride >= d["ksteps"] * d["nmma"]:
            return False
    # registers per lane: accumulators, two fragment sets, staging (register loader), one copy offset per
    # chunk (plus the k offset of each A chunk for the buffer loader) and ~48 of addressing and temporaries
    # (the compiler's resource report of the eight-wave 256x256 kernels: 80-92 VGPRs beside 128 AGPRs).  With one wave per SIMD the accumulators sit in the 256 AGPRs and the
    # rest must fit the 256 VGPRs; with more waves all of it shares 512 / waves.
    acc = d["tm"] * d["tn"] * d["nacc"]
    frags = (1 if c.spread & 2 else 2) * d["tm"] * 4 + 2 * d["tn"] * 4
    stg = 4 * ps if c.loader == "reg" else 0
    rest = frags + stg + ps + (d["a_ins"] if c.loader == "buf" else 0) + 48
    if c.wpe == 1:
        return acc <= REGS_PER_LANE // 2 and rest <= REGS_PER_LANE // 2
    return acc + rest <= REGS_PER_LANE // c.wpe


def space() -> list:
    out = []
    for g in (4, 8):
        for bs in (1, 3):
            for ds in (1, 2):
                out.append(Tile(256, 256, 64, 2, 2, 2, g, bs, ds, "dma"))
    for st in (2, 3):
        out.append(Tile(256, 128, 64, 2, 2, st, 4, 3, 2, "dma"))
        out.append(Tile(128, 256, 64, 2, 2, st, 4, 3, 2, "dma"))
    for st in (2, 3, 4):
        out.append(Tile(128, 128, 64, 2, 2, st, 4, 1, 1, "dma"))
    out.append(Tile(128, 128, 64, 2, 2, 2, 4, 1, 1, "dma", wpe=2))
    out.append(Tile(128, 128, 128, 2, 2, 2, 4, 1, 1, "dma"))
    for bs, ds in ((3, 3), (8, 4), (8, 2)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=1))
    out.append(Tile(256, 256, 64, 2, 2, 2, 8, 8, 4, "dma", mf=16, spread=1))
    out.append(Tile(128, 128, 64, 2, 2, 3, 4, 3, 2, "dma", mf=16, spread=1))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 8, 4, "reg", mf=16, spread=1))
    for ds in (1, 2):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, ds, "reg"))
    out.append(Tile(256, 128, 64, 2, 2, 2, 4, 3, 2, "reg"))
    out.append(Tile(128, 256, 64, 2, 2, 2, 4, 3, 2, "reg"))
    for wpe in (1, 2):
        out.append(Tile(128, 128, 64, 2, 2, 2, 4, 1, 1, "reg", wpe=wpe))
    # 192-wide tiles: 3001 columns are 16 tiles of 192 (one full round of 256 tiles at 256 x 192)
    out.append(Tile(256, 192, 64, 2, 2, 2, 4, 1, 2, "reg"))
    out.append(Tile(128, 192, 64, 2, 2, 2, 4, 1, 1, "reg", wpe=2))
    out.append(Tile(256, 192, 64, 2, 2, 2, 4, 1, 2, "dma"))
    out.append(Tile(128, 128, 128, 2, 2, 2, 4, 1, 1, "reg", wpe=2))
    # buffer LDS-DMA (unaligned and ragged shapes with K % 8 == 0): the shapes of the best aligned ones
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 1, "buf"))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 8, 2, "buf", mf=16, spread=1))
    out.append(Tile(256, 192, 64, 2, 2, 2, 4, 1, 2, "buf"))
    out.append(Tile(256, 128, 64, 2, 2, 3, 4, 3, 2, "buf"))
    out.append(Tile(128, 256, 64, 2, 2, 3, 4, 3, 2, "buf"))
    for st in (3, 4):
        out.append(Tile(128, 128, 64, 2, 2, st, 4, 1, 1, "buf"))
    out.append(Tile(128, 128, 64, 2, 2, 3, 4, 3, 2, "buf", mf=16, spread=1))
    out.append(Tile(128, 192, 64, 2, 2, 3, 4, 1, 1, "buf"))
    # tile-order ablation of the two large-tile schedules: no swizzle (g0), XCD remap only (g1)
    for g in (0, 1, 8):
        out.append(Tile(256, 256, 64, 2, 2, 2, g, 8, 2, "dma", mf=16, spread=1))
    for g in (0, 1):
        out.append(Tile(256, 256, 64, 2, 2, 2, g, 3, 1, "dma"))
    # B given transposed (Bt[N][K], a linear layer's weight): the shapes of the best plain schedules
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 8, 2, "dma", mf=16, spread=1, bt=1))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 1, "dma", bt=1))
    out.append(Tile(128, 128, 64, 2, 2, 3, 4, 1, 1, "dma", bt=1))
    out.append(Tile(128, 128, 64, 2, 2, 3, 4, 3, 2, "dma", mf=16, spread=1, bt=1))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 1, "buf", bt=1))
    out.append(Tile(128, 192, 64, 2, 2, 3, 4, 1, 1, "buf", bt=1))
    out.append(Tile(128, 128, 64, 2, 2, 3, 4, 1, 1, "buf", bt=1))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 2, "reg", bt=1))
    out.append(Tile(128, 128, 64, 2, 2, 2, 4, 1, 1, "reg", wpe=2, bt=1))
    # accumulators pinned to AGPRs (asm MFMAs): the 16x16 schedules then keep their accumulators in place
    for bs, ds in ((8, 2), (8, 4), (3, 3)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=5))
    for bs, ds in ((8, 2), (8, 4), (16, 2), (24, 2), (32, 2), (3, 2)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=6))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 8, 2, "buf", mf=16, spread=6))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 1, "dma", spread=6))
    # copies of stage kt+2 issued right after stage kt's barrier (16x16 schedules: 128 MFMA slots per stage)
    for bs, ds in ((24, 1), (32, 1), (40, 1), (16, 2), (24, 2), (32, 2)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=14))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 24, 2, "buf", mf=16, spread=14))
    # ... and the next k-step's B fragments read first
    for bs, ds, fl in ((24, 2, 22), (16, 2, 22), (24, 1, 30), (32, 1, 30), (16, 2, 30), (24, 2, 30)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=fl))
    for bs, ds in ((8, 2), (16, 2), (24, 2), (32, 2)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=6, bt=1))
    for bs, ds in ((24, 1), (24, 2), (32, 1)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=14, bt=1))
    for bs, ds, fl in ((24, 2, 22), (24, 1, 30), (16, 2, 30)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=fl, bt=1))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 8, 2, "buf", mf=16, spread=6, bt=1))
    for bs, ds in ((3, 1), (3, 2)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", spread=4))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 2, "dma", spread=6))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 8, 2, "buf", mf=16, spread=5))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 1, "buf", spread=4))
    out.append(Tile(128, 128, 64, 2, 2, 3, 4, 1, 1, "dma", spread=4))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 8, 2, "dma", mf=16, spread=5, bt=1))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 8, 4, "dma", mf=16, spread=5, bt=1))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 1, "dma", spread=4, bt=1))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 8, 2, "buf", mf=16, spread=5, bt=1))
    # C staged through LDS and written with row-contiguous 16-byte stores (+32), non-temporal (+96): the
    # schedules of every loader and B layout that lead their classes
    for le in (32, 96):
        for bs, ds, fl in ((24, 2, 14), (16, 2, 14), (24, 1, 14), (32, 2, 14)):
            out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=fl + le))
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, 24, 2, "buf", mf=16, spread=14 + le))
        for bs, ds in ((16, 2), (24, 2), (24, 1)):
            out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=30 + le, bt=1))
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 1, "buf", spread=le, bt=1))
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 2, "reg", spread=le))
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, 3, 2, "reg", spread=le, bt=1))
        for st, fl in ((3, 4), (4, 0), (3, 0)):
            out.append(Tile(128, 128, 64, 2, 2, st, 4, 1, 1, "dma", spread=fl + le))
            out.append(Tile(128, 128, 64, 2, 2, st, 4, 1, 1, "dma", spread=fl + le, bt=1))
            out.append(Tile(128, 128, 64, 2, 2, st, 4, 1, 1, "buf", spread=fl + le))
    # 256x192 tiles on the 16x16 schedules: 3001 columns are 16 tiles of 192, so 4095x3001 fills the 256 CUs
    # in one round (256x256 tiles leave 64 idle)
    for ld in ("buf", "dma"):
        for bs, ds in ((8, 2), (16, 2), (16, 1), (24, 1)):
            for le in (0, 32, 96):
                out.append(Tile(256, 192, 64, 2, 2, 2, 4, bs, ds, ld, mf=16, spread=14 + le))
    # ... and for B given transposed (ragged Bt), plain or with front-loaded B reads
    for bs, ds in ((8, 2), (16, 2), (16, 1)):
        for fl in (14, 30):
            out.append(Tile(256, 192, 64, 2, 2, 2, 4, bs, ds, "buf", mf=16, spread=fl + 96, bt=1))
    # barrier slot and copy stride around the chosen large-tile schedule, with the staged epilogue
    for bs, ds in ((8, 2), (32, 1), (40, 1)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=14 + 96))
    # A ring one stage deeper than B's (160 KiB at 256x256x64): A copies get two stages to land
    for bs, ds in ((8, 2), (16, 2), (32, 2)):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, ds, "dma", mf=16, spread=14 + 96 + 128))
    out.append(Tile(256, 256, 64, 2, 2, 2, 4, 16, 2, "dma", mf=16, spread=30 + 96 + 128, bt=1))
    # ... and with front-loaded B reads for B[K][N] as well
    for bs in (8, 16):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, 2, "dma", mf=16, spread=30 + 96 + 128))
    # eight-wave 256x256 tiles (two waves per SIMD, 128x64 or 64x128 per wave): one wave's MFMAs can cover
    # the other's waits, for 50% more fragment reads per MFMA
    for wm, wn in ((2, 4), (4, 2)):
        for bs in (4, 12):
            out.append(Tile(256, 256, 64, wm, wn, 2, 4, bs, 2, "dma", wpe=2, mf=16, spread=14 + 96))
        out.append(Tile(256, 256, 64, wm, wn, 2, 4, 8, 2, "dma", wpe=2, mf=16, spread=30 + 96, bt=1))
    # ... their barrier slot, copy stride and flags (32 MFMA slots per k-step)
    for bs, ds in ((0, 2), (8, 2), (16, 2), (4, 1), (12, 1), (20, 1), (4, 3)):
        out.append(Tile(256, 256, 64, 2, 4, 2, 4, bs, ds, "dma", wpe=2, mf=16, spread=14 + 96))
    out.append(Tile(256, 256, 64, 2, 4, 2, 4, 4, 2, "dma", wpe=2, mf=16, spread=30 + 96))
    out.append(Tile(256, 256, 64, 2, 4, 2, 4, 4, 2, "dma", wpe=2, mf=16, spread=14 + 32))
    for bs, ds in ((4, 2), (12, 2), (16, 2), (8, 1)):
        out.append(Tile(256, 256, 64, 2, 4, 2, 4, bs, ds, "dma", wpe=2, mf=16, spread=30 + 96, bt=1))
    out.append(Tile(256, 256, 64, 2, 4, 2, 4, 8, 2, "dma", wpe=2, mf=16, spread=14 + 96, bt=1))
    # wider copy strides (the copies of a stage spread over more of its slots)
    for bs, ds in ((0, 3), (8, 3), (0, 4)):
        out.append(Tile(256, 256, 64, 2, 4, 2, 4, bs, ds, "dma", wpe=2, mf=16, spread=14 + 96))
    for bs, ds in ((4, 3), (8, 3), (0, 4)):
        out.append(Tile(256, 256, 64, 2, 4, 2, 4, bs, ds, "dma", wpe=2, mf=16, spread=30 + 96, bt=1))
    # flags around the stride-3 schedules: front-loaded B for B[K][N], plain B reads for Bt, cached C stores
    for bs in (4, 8):
        out.append(Tile(256, 256, 64, 2, 4, 2, 4, bs, 3, "dma", wpe=2, mf=16, spread=30 + 96))
    out.append(Tile(256, 256, 64, 2, 4, 2, 4, 4, 3, "dma", wpe=2, mf=16, spread=14 + 32))
    out.append(Tile(256, 256, 64, 2, 4, 2, 4, 4, 3, "dma", wpe=2, mf=16, spread=14 + 96, bt=1))
    out.append(Tile(256, 256, 64, 2, 4, 2, 4, 4, 3, "dma", wpe=2, mf=16, spread=30 + 32, bt=1))
    # eight waves with A's ring one stage deeper than B's (3 A + 2 B buffers, exactly 160 KiB): the A copies of
    # stage kt+3 go out during stage kt, so they have two stages to land
    for bs, ds in ((4, 2), (4, 3), (8, 2), (8, 3)):
        out.append(Tile(256, 256, 64, 2, 4, 2, 4, bs, ds, "dma", wpe=2, mf=16, spread=14 + 96 + 128))
    for bs, ds in ((4, 3), (8, 2)):
        out.append(Tile(256, 256, 64, 2, 4, 2, 4, bs, ds, "dma", wpe=2, mf=16, spread=30 + 96 + 128, bt=1))
    # eight waves for the buffer loader (unaligned shapes): 256x192 tiles on 4x2 waves (64x96 per wave, 12-chunk
    # epilogue rows) for the ragged class, 256x256 on 2x4 waves for the big unaligned class
    for bs, ds in ((4, 3), (8, 2), (0, 3)):
        out.append(Tile(256, 192, 64, 4, 2, 2, 4, bs, ds, "buf", wpe=2, mf=16, spread=14 + 32))
        out.append(Tile(256, 192, 64, 4, 2, 2, 4, bs, ds, "buf", wpe=2, mf=16, spread=30 + 96, bt=1))
    for bs, ds in ((4, 3), (8, 2)):
        out.append(Tile(256, 256, 64, 2, 4, 2, 4, bs, ds, "buf", wpe=2, mf=16, spread=14 + 32))
    # the ping-pong schedule (two wave groups alternating MFMAs and loads)
    for bt in (0, 1):
        for nt in (0, 1):
            out.append(PingPong(4, bt, nt))
    # the same large schedules with the copies issued as buffer loads (the vendor's copy form)
    for bs in (8, 16):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, 2, "buf", mf=16, spread=14 + 96))
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, 2, "buf", mf=16, spread=30 + 96, bt=1))
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, 2, "buf", mf=16, spread=30 + 96 + 128, bt=1))
    # front-loaded B reads (the B-transposed winner's flag) with the staged epilogue, for B[K][N]
    for bs in (8, 16, 32):
        out.append(Tile(256, 256, 64, 2, 2, 2, 4, bs, 2, "dma", mf=16, spread=30 + 96))
    for bt in (0, 1):
        for mb, sts in ((1, (4, 6, 8)), (2, (4, 6)), (4, (3, 5))):
            for st in sts:
                for kr in (0, 1):
                    out.append(Skinny(mb, st, bt, kr))
    # A by 16-byte copies (a quarter of the A copy instructions)
    for bt in (0, 1):
        for mb, sts in ((1, (3, 4, 6, 8)), (2, (3, 4, 6)), (4, (3, 5))):
            for st in sts:
                for kr in (0, 1):
                    out.append(Skinny(mb, st, bt, kr, a16=1))
    # split-K over 256-column panels (B[K][N]): four K ranges put 256 workgroups on N = 16384
    for mb, sts in ((1, (4, 6, 8)), (2, (4, 6)), (4, (4,))):
        for st in sts:
            for bk in (32, 64):
                for sp in (2, 4):
                    out.append(SplitK(mb, st, bk, sp))
    # eight-wave 256x256 tiles on 32x32x16 MFMAs (half the operand register reads per FLOP of 16x16x32)
    for bt in (0, 1):
        for fl in (0, 4, 6):
            for bs, ds in ((2, 2), (4, 2), (4, 3)):
                out.append(Tile(256, 256, 64, 2, 4, 2, 4, bs, ds, "dma", wpe=2, spread=fl + 96, bt=bt))
        for bs, ds in ((2, 2), (4, 2), (4, 3)):
            out.append(Tile(256, 256, 64, 4, 2, 2, 4, bs, ds, "dma", wpe=2, spread=6 + 96, bt=bt))
    # two workgroups per CU: 256x128 and 128x256 tiles at BK = 32 on four waves (128x64 or 64x128 per wave,
    # 32x32 MFMAs, 48 or 72 KiB of LDS each), so that one workgroup's epilogue can run beside the other's K loop
    for bm, bn in ((256, 128), (128, 256)):
        for st in (2, 3):
            for fl in (96, 4 + 96, 14 + 96):
                for bs, ds in ((1, 1), (3, 2), (4, 2)):
                    out.append(Tile(bm, bn, 32, 2, 2, st, 4, bs, ds, "dma", wpe=2, spread=fl))
    return [c for c in out if valid(c)]


CLASSES = ["SEL_SKINNY16", "SEL_SKINNY32", "SEL_SKINNY64", "SEL_DMA_HUGE", "SEL_DMA_BIG", "SEL_DMA_SMALL",
           "SEL_BUF_BIG", "SEL_BUF_SMALL", "SEL_REG_BIG", "SEL_REG_SMALL",
           "SEL_BT_BIG", "SEL_BT_SMALL", "SEL_BT_BUF", "SEL_BT_REG",
           "SEL_BT_SKINNY16", "SEL_BT_SKINNY32", "SEL_BT_SKINNY64"]


def class_of(c, cls: str) -> bool:
    """Whether configuration c may serve shape class cls.  The skinny classes
    (M <= 16/32/64, aligned) accept any skinny kernel with enough rows and any
    LDS-DMA tile configuration; the dispatcher falls back if it cannot run.
    The buffer classes (unaligned, K % 8 == 0) accept the buffer and the
    register loader, which both run every call of the class."""
    if cls.startswith("SEL_SKINNY") or cls.startswith("SEL_BT_SKINNY"):
        bt = cls.startswith("SEL_BT_")
        if c.kind in ("skinny", "splitk"):
            return bool(c.bt) == bt and 16 * c.mb >= int(cls.split("SKINNY")[1])
        return c.loader == "dma" and bool(c.bt) == bt
    if c.kind != "tile":
        return False
    if cls.startswith("SEL_BT_"):   # B transposed: LDS-DMA (big/small), buffer or register loader
        if not c.bt:
            return False
        kind = cls[len("SEL_BT_"):]
        return c.loader == {"BIG": "dma", "SMALL": "dma", "BUF": "buf", "REG": "reg"}[kind] or \
            (kind == "BUF" and c.loader == "reg")
    if c.bt:
        return False
    if "_BUF_" in cls:
        return c.loader in ("buf", "reg")
    return c.loader == cls.split("_")[1].lower()


def emit_table(configs: list, sel: dict, path: str, header: str) -> None:
    lines = ["// " + l for l in header.splitlines()]
    lines += ["#define GEMM_F16_CONFIGS \\"]
    for i, c in enumerate(configs):
        lines.append("    %s%s  /* %d */" % (c.macro(), "," if i + 1 < len(configs) else "", i)
                     + (" \\" if i + 1 < len(configs) else ""))
    for cls in CLASSES:
        lines.append("#define %s %d" % (cls, sel[cls]))
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def finalists(table_path: str = TABLE) -> list:
    """A focused re-sweep: the configurations of the current table plus their
    LDS-epilogue variants (names with _le / _le_nt added), as far as the space
    holds them."""
    import re

    keep = set(re.findall(r'"([^"]+)"\)', open(table_path).read()))
    return [c for c in space() if c.name in keep or c.name.replace("_le_nt", "").replace("_le", "") in keep]


def build_sweep_lib(verbose: bool = True, configs: list | None = None) -> str:
    from dense_tiled_gemm_04_amd import build as libbuild

    configs = space() if configs is None else configs
    sel = {}
    for cls in CLASSES:
        # the sweep launches forced configurations only; a class without a member points at entry 0
        sel[cls] = next((i for i, c in enumerate(configs) if class_of(c, cls)), 0)
    emit_table(configs, sel, SWEEP_TABLE, "Sweep space (generated by sweep.py --build); not the product table.")
    if verbose:
        print("%d configurations; compiling %s" % (len(configs), SWEEP_LIB), flush=True)
    t = time.time()
    # only the GEMM unit; scratch is allowed here (a spilling configuration is merely slow), and reported
    rows = libbuild.build_library(SWEEP_LIB, [os.path.join(PKG_DIR, "csrc", "gemm_f16.hip")],
                                  defines=["-DGEMM_F16_CONFIG_TABLE=\"%s\"" % SWEEP_TABLE], allow_scratch=True,
                                  resources_path=os.path.join(PKG_DIR, "_build", "sweep_kernel_resources.json"))
    if verbose:
        for r in libbuild.scratch_users(rows):
            print("uses scratch (%s bytes/lane): %s" % (r.get("ScratchSize [bytes/lane]"), r["kernel"]), flush=True)
        print("built in %.0f s" % (time.time() - t), flush=True)
    return SWEEP_LIB


# ---------------------------------------------------------------------------
# workloads of the sweep: name -> (workload id or shape spec, classes it scores)
# ---------------------------------------------------------------------------
def sweep_workloads():
    import workloads as wl

    W = wl.WORKLOADS
    out = []
    out.append(("gemm_4096", W["gemm_4096"], {}, ["SEL_DMA_BIG"]))
    out.append(("mlp_up_8192x16384x4096", W["mlp_up_8192x16384x4096"], {}, ["SEL_DMA_HUGE"]))
    out.append(("gemm_256", W["gemm_256"], {}, ["SEL_DMA_SMALL"]))
    out.append(("gemm_2048", dataclasses.replace(W["gemm_4096"], name="gemm_2048", M=2048, N=2048, K=2048, seed=5),
                {}, ["SEL_DMA_SMALL"]))
    out.append(("ragged_4095x3001x1000", W["ragged_4095x3001x1000"], {}, ["SEL_BUF_SMALL"]))
    out.append(("gemm_4096_offset1", W["gemm_4096"], {"offset": 1}, ["SEL_BUF_BIG"]))
    # K % 8 != 0: only the register loader runs these
    out.append(("ragged_4095x3001x1004", dataclasses.replace(W["ragged_4095x3001x1000"], name="ragged_k1004",
                                                             K=1004, seed=6), {}, ["SEL_REG_SMALL"]))
    out.append(("gemm_4096x4096x4092", dataclasses.replace(W["gemm_4096"], name="gemm_k4092", K=4092, seed=7),
                {}, ["SEL_REG_BIG"]))
    # B given transposed (Bt[N][K])
    out.append(("gemm_4096_bt", W["gemm_4096"], {"bt": True}, ["SEL_BT_BIG"]))
    out.append(("mlp_up_8192x16384x4096_bt", W["mlp_up_8192x16384x4096"], {"bt": True}, ["SEL_BT_BIG"]))
    out.append(("gemm_2048_bt", dataclasses.replace(W["gemm_4096"], name="gemm_2048", M=2048, N=2048, K=2048, seed=5),
                {"bt": True}, ["SEL_BT_SMALL"]))
    out.append(("ragged_4095x3001x1000_bt", W["ragged_4095x3001x1000"], {"bt": True}, ["SEL_BT_BUF"]))
    out.append(("ragged_4095x3001x1004_bt", dataclasses.replace(W["ragged_4095x3001x1000"], name="ragged_k1004",
                                                                K=1004, seed=6), {"bt": True}, ["SEL_BT_REG"]))
    # HBM-bound: B (256 MiB) is rotated over 3 copies so the 256 MB Infinity Cache cannot serve it
    out.append(("skinny_16x16384x8192", W["skinny_16x16384x8192"], {"rotate": 3}, ["SEL_SKINNY16"]))
    out.append(("skinny_32x16384x8192", dataclasses.replace(W["skinny_16x16384x8192"], name="skinny_32", M=32),
                {"rotate": 3}, ["SEL_SKINNY32"]))
    out.append(("skinny_64x16384x8192", dataclasses.replace(W["skinny_16x16384x8192"], name="skinny_64", M=64),
                {"rotate": 3}, ["SEL_SKINNY64"]))
    # the same with B given transposed: decode through a linear layer's weight
    out.append(("skinny_16x16384x8192_bt", W["skinny_16x16384x8192"], {"rotate": 3, "bt": True}, ["SEL_BT_SKINNY16"]))
    out.append(("skinny_32x16384x8192_bt", dataclasses.replace(W["skinny_16x16384x8192"], name="skinny_32", M=32),
                {"rotate": 3, "bt": True}, ["SEL_BT_SKINNY32"]))
    out.append(("skinny_64x16384x8192_bt", dataclasses.replace(W["skinny_16x16384x8192"], name="skinny_64", M=64),
                {"rotate": 3, "bt": True}, ["SEL_BT_SKINNY64"]))
    return out


def _reference_rows(A, B, bias, epilogue, rows):
    """float32 PyTorch reference of the sampled output rows (a screen, not the oracle)."""
    import torch

    r = A[rows].float() @ B.float()
    if epilogue != "none":
        r = r + bias.float()
    if epilogue == "bias_gelu":
        r = torch.nn.functional.gelu(r)
    return r


def run(results_path: str, lib_path: str = SWEEP_LIB, iters: int = 20, only: str | None = None,
        repeat: int = 1) -> None:
    import ctypes
    import numpy as np
    import torch
    import workloads as wl

    lib = ctypes.CDLL(lib_path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.gemm_f16_with_config.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, i32, vp]
    lib.gemm_f16_with_config.restype = i32
    lib.gemm_f16_bt_with_config.argtypes = [i32, i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, i32, vp]
    lib.gemm_f16_bt_with_config.restype = i32
    lib.gemm_f16_config_info.argtypes = [i32, ctypes.c_char_p, i32]
    n_cfg = lib.gemm_f16_num_configs()
    infos = []
    for i in range(n_cfg):
        buf = ctypes.create_string_buffer(1024)
        lib.gemm_f16_config_info(i, buf, 1024)
        infos.append(json.loads(buf.value.decode()))
    done = set()
    if os.path.exists(results_path):
        for line in open(results_path):
            try:
                rec = json.loads(line)
                done.add((rec["config"], rec["workload"]))
            except ValueError:
                pass
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    epi_ids = {"none": 0, "bias": 1, "bias_gelu": 2}
    out = open(results_path, "a")
    for name, w, opts, classes in sweep_workloads():
        if only and name not in only.split(","):
            continue
        A, B, bias = wl.make_inputs(w)
        off = opts.get("offset", 0)

        def place(x):
            t = torch.empty(x.size + off, dtype=torch.float16, device=dev)
            t[off:] = torch.from_numpy(np.ascontiguousarray(x).reshape(-1)).to(dev)
            return t[off:].view(*x.shape)

        bt = opts.get("bt", False)
        dA = place(A)
        # the kernels get Bt[N][K] for the transposed workloads; the reference keeps B[K][N]
        dBs = [place(np.ascontiguousarray(B.T) if bt else B) for _ in range(opts.get("rotate", 1))]
        dB = dBs[0].t().contiguous() if bt else dBs[0]
        db = place(bias) if bias is not None else None
        cbuf = torch.empty(w.M * w.N + off, dtype=torch.float16, device=dev)
        dC = cbuf[off:].view(w.M, w.N)
        rng = np.random.default_rng(0)
        rows = sorted(set(list(range(min(w.M, 16))) + list(range(max(0, w.M - 16), w.M)) +
                      list(rng.integers(0, w.M, 32))))
        ref = _reference_rows(dA, dB, db, w.epilogue, rows)
        refh = ref.half().float()
        epi = epi_ids[w.epilogue]
        if bt:
            call = lambda *a: lib.gemm_f16_bt_with_config(a[0], a[1], a[2], a[3], a[4], w.K, a[5], w.K, a[6],
                                                          a[7], w.N, a[8], a[9])
        else:
            call = lib.gemm_f16_with_config

        def time_config(i):
            """Sustained time per launch of config i, as the benchmark sees it: launches back to back (the
            benchmark puts no event between them), since the power limit sets the clock within milliseconds
            and the gaps of per-launch events would let the card rest.  From a short idle: >= WARM_MS of
            warm-up (the controller boosts, throttles and settles within ~40 ms), then >= 25 ms in chunks of
            ~1 ms between event pairs.  Returns the sorted per-launch chunk times
            (us) and leaves C written from the first copy of B, or None if the config cannot run the call."""
            def args(r=0):
                return (i, w.M, w.N, w.K, dA.data_ptr(), dBs[r % len(dBs)].data_ptr(),
                        db.data_ptr() if db is not None else None, dC.data_ptr(), epi, stream.cuda_stream)
            st = call(*args())
            if st == 6:  # GEMM_ERR_UNSUPPORTED: this config cannot run this call
                return None
            if st != 0:
                raise RuntimeError("config %s on %s: status %d" % (infos[i]["name"], name, st))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for r in range(3):
                call(*args(r + 1))
            e1.record(stream)
            torch.cuda.synchronize()
            t_one = max(e0.elapsed_time(e1) / 3, 1e-3)   # ms
            time.sleep(0.02)
            for r in range(int(math.ceil(WARM_MS / t_one))):
                call(*args(r + 1))
            per = max(1, int(round(1.0 / t_one)))        # launches per chunk
            evs = []
            r = 0
            for _c in range(max(iters, int(math.ceil(25.0 / (per * t_one))))):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(per):
                    call(*args(r + 1))
                    r += 1
                e1.record(stream)
                evs.append((e0, e1))
            call(*args(0))   # the screened output comes from the first copy of B
            torch.cuda.synchronize()
            return sorted(a.elapsed_time(b) * 1e3 / per for a, b in evs)

        # With repeat > 1 the configurations are timed round-robin, repeat times each, so that a slow drift
        # of the card's clock spreads over all of them; a record holds the median of the rounds' medians.
        todo = [i for i, info in enumerate(infos) if (info["name"], name) not in done]
        rounds = {i: [] for i in todo}
        screen = {}
        for rep in range(repeat):
            for i in todo:
                if i in screen and screen[i] is None:
                    continue
                us = time_config(i)
                if us is None:
                    screen[i] = None
                    continue
                rounds[i].append((us[len(us) // 2], us[0]))
                if rep == 0:
                    got = dC[rows].float()
                    diff = (got - refh)
                    rel = float(diff.norm() / refh.norm()) if float(refh.norm()) > 0 else float(diff.norm())
                    mx = float((diff.abs() / (1 + refh.abs())).max())
                    screen[i] = (rel, mx, bool(rel <= 2e-3 and mx <= 1e-2 and not torch.isnan(got).any()))
        for i in todo:
            if screen.get(i) is None:
                continue
            info = infos[i]
            rel, mx, ok = screen[i]
            meds = sorted(m for m, _ in rounds[i])
            med = meds[len(meds) // 2]
            rec = {"config": info["name"], "idx": i, "workload": name, "classes": classes, "median_us": med,
                   "min_us": min(m for _, m in rounds[i]), "tflops": 2.0 * w.M * w.N * w.K / med / 1e6,
                   "rel_fro_vs_fp32": rel, "max_elem_vs_fp32": mx, "ok": ok, "info": info}
            if repeat > 1:
                rec["round_medians_us"] = [m for m, _ in rounds[i]]
            out.write(json.dumps(rec) + "\n")
            out.flush()
            print("%-28s %-48s %9.1f us %7.1f TF %s" % (name, info["name"], med, rec["tflops"],
                                                        "ok" if ok else "FAIL rel=%.2e" % rel), flush=True)
        del dA, dB, dBs, db, cbuf, dC
        torch.cuda.empty_cache()
    out.close()


def scratch_configs(resources_path: str = os.path.join(PKG_DIR, "_build", "sweep_kernel_resources.json")) -> set:
    """Names of the configurations whose kernels used scratch memory in the last sweep build (none if unknown)."""
    import re

    if not os.path.exists(resources_path) or not os.path.exists(SWEEP_TABLE):
        return set()
    rows = json.load(open(resources_path))
    bad_sym = [r["kernel"] for r in rows if r.get("ScratchSize [bytes/lane]", 0) or r.get("VGPRs Spill", 0)]
    out = set()
    for c in space():
        if c.kind != "tile" or isinstance(c, PingPong):
            continue
        args = [c.bm, c.bn, c.bk, c.wm, c.wn, c.stages, c.group]
        tail = [c.bslot, c.dstride, {"dma": 0, "reg": 1, "buf": 2}[c.loader], c.cslot, c.wpe, c.mf, c.spread, c.bt]
        for sym in bad_sym:
            v = [int(x) for x in re.findall(r"Li(-?\d+)E", sym)]
            if "gemm_tile_pipe_kernel" in sym and v[:7] == args and v[8:16] == tail:
                out.add(c.name)
    return out


def select(results_path: str, table_path: str = TABLE, summary_path: str | None = None, note: str = "") -> dict:
    recs = [json.loads(l) for l in open(results_path) if l.strip()]
    # classes come from the current workload table, so a reclassification needs no new measurements
    wl_classes = {name: classes for name, _w, _o, classes in sweep_workloads()}
    for r in recs:
        r["classes"] = wl_classes.get(r["workload"], r["classes"])
    by_name = {c.name: c for c in space()}
    spilled = scratch_configs()
    chosen, scores = {}, {}
    for cls in CLASSES:
        wls = sorted({r["workload"] for r in recs if cls in r["classes"]})
        best = None
        for name, c in by_name.items():
            if not class_of(c, cls) or name in spilled:
                continue
            ts = [r["median_us"] for r in recs if r["config"] == name and r["workload"] in wls]
            oks = [r["ok"] for r in recs if r["config"] == name and r["workload"] in wls]
            if len(ts) != len(wls) or not all(oks) or not ts:
                continue
            g = math.exp(sum(math.log(t) for t in ts) / len(ts))
            if best is None or g < best[0]:
                best = (g, name)
        if best is None:
            raise RuntimeError("no valid configuration measured for %s" % cls)
        chosen[cls] = best[1]
        scores[cls] = best[0]
    names = []
    for cls in CLASSES:
        if chosen[cls] not in names:
            names.append(chosen[cls])
    configs = [by_name[n] for n in names]
    sel = {cls: names.index(chosen[cls]) for cls in CLASSES}
    emit_table(configs, sel, table_path,
               "Generated by dense_tiled_gemm_04_amd/sweep.py --select from the sweep results\n"
               "(%s). Do not edit by hand; rerun the sweep." % os.path.basename(results_path))
    if summary_path:
        lines = ["# Offline sweep of the tile and skinny kernels", "",
                 "Per (configuration, workload) on one MI355X: launches back to back, as in bench.py; after >= %.0f ms of "
                 "warm-up (records of runs before the warm-up was raised from 5 ms: the clock was still recovering "
                 "then), >= 25 ms in ~1 ms chunks between HIP events, median chunk time per launch; the skinny" % WARM_MS,
                 "workloads rotate 3 copies of B so the Infinity Cache cannot serve it;",
                 "outputs screened against a float32 PyTorch reference on sampled rows (parity proper is the",
                 "oracle tests). Command: `python -m dense_tiled_gemm_04_amd.sweep --run RESULTS` on the GPU, then",
                 "`--select RESULTS` here."] + ([""] + note.splitlines() if note else []) + ["", "## Chosen per shape class", "",
                 "| class | configuration | geo-mean us |", "|---|---|---|"]
        for cls in CLASSES:
            lines.append("| %s | %s | %.1f |" % (cls, chosen[cls], scores[cls]))
        lines += ["", "## All measurements", "", "| workload | configuration | median us | TFLOP/s | screen |",
                  "|---|---|---|---|---|"]
        for r in sorted(recs, key=lambda r: (r["workload"], r["median_us"])):
            lines.append("| %s | %s | %.1f | %.1f | %s |" % (r["workload"], r["config"], r["median_us"], r["tflops"],
                                                             "ok" if r["ok"] else "FAIL"))
        with open(summary_path, "w") as f:
            f.write("\n".join(lines) + "\n")
    return chosen


def ablation(results_path: str, out_path: str) -> None:
    """Markdown tables of the tile-order and pipeline-depth ablations from the sweep results: each row is one
    schedule with only the ablated knob varied (the tutorial's use_swizzle switch and num_stages)."""
    recs = [json.loads(l) for l in open(results_path) if l.strip()]
    t = {(r["config"], r["workload"]): r for r in recs if r.get("ok")}
    by_name = {c.name: c for c in space()}
    lines = ["# Ablations: tile order (swizzle) and LDS stages", "",
             "Back-to-back launches timed in ~1 ms chunks over >= 25 ms (after the warm-up of the record's run), median chunk, per cell on one "
             "MI355X, from the same sweep records as the",
             "configuration table (`python -m dense_tiled_gemm_04_amd.sweep --run RESULTS` on the GPU, then",
             "`--ablation RESULTS`).", "",
             "## Tile order", "",
             "g0: row-major tile order, no XCD remap (swizzle off). g1: XCD-contiguous remap, row-major.",
             "g4 / g8: XCD remap plus a grouped raster of 4 / 8 tile-rows (swizzle on).", ""]
    wls = ["gemm_4096", "mlp_up_8192x16384x4096", "gemm_2048", "gemm_4096_offset1"]
    lines += ["| schedule | workload | g0 us | g1 us | g4 us | g8 us |", "|---|---|---|---|---|---|"]
    bases = sorted({c.name.replace("_g%d_" % c.group, "_gX_") for c in by_name.values()
                    if c.kind == "tile" and c.group == 0})
    for base in bases:
        for w in wls:
            cells = []
            for g in (0, 1, 4, 8):
                r = t.get((base.replace("_gX_", "_g%d_" % g), w))
                cells.append("%.1f" % r["median_us"] if r else "-")
            if cells.count("-") < 3:
                lines.append("| %s | %s | %s |" % (base, w, " | ".join(cells)))
    lines += ["", "## LDS stages", "", "Same schedule, 2, 3 or 4 LDS stages (where the LDS budget allows).", "",
              "| schedule | workload | s2 us | s3 us | s4 us |", "|---|---|---|---|---|"]
    fams = sorted({c.name.replace("_s%d_" % c.stages, "_sX_") for c in by_name.values()
                   if c.kind == "tile" and c.loader != "reg"})
    for fam in fams:
        for w in wls + ["ragged_4095x3001x1000"]:
            cells = []
            for st in (2, 3, 4):
                r = t.get((fam.replace("_sX_", "_s%d_" % st), w))
                cells.append("%.1f" % r["median_us"] if r else "-")
            if cells.count("-") <= 1:
                lines.append("| %s | %s | %s |" % (fam, w, " | ".join(cells)))
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--list", action="store_true", help="print the sweep space")
    ap.add_argument("--build", action="store_true", help="compile libgemm_f16_sweep.so with the whole space")
    ap.add_argument("--finalists", action="store_true",
                    help="with --build/--list: only the current table's configurations and their LDS-epilogue "
                         "variants; with --select: say so in the summary")
    ap.add_argument("--subset", default=None, metavar="REGEX",
                    help="with --build/--list: add the configurations of the space whose names match REGEX (alone: "
                         "only those)")
    ap.add_argument("--run", metavar="RESULTS", help="time every configuration (GPU); JSONL, resumable")
    ap.add_argument("--only", default=None, help="comma-separated sweep workload names for --run")
    ap.add_argument("--repeat", type=int, default=1,
                    help="--run: time the configurations round-robin this many times per workload")
    ap.add_argument("--select", metavar="RESULTS", help="pick per-class defaults, write csrc/config_table.inc")
    ap.add_argument("--summary", default=None, help="Markdown summary path for --select")
    ap.add_argument("--note", default="", help="extra paragraph for the --select summary")
    ap.add_argument("--ablation", metavar="RESULTS", help="write the tile-order / stages ablation tables")
    ap.add_argument("--ablation-out", default=os.path.join(ROOT, "profiles",
                                                           "ablation__tile_order_and_stages__gemm_workloads.md"))
    a = ap.parse_args()
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    chosen = finalists() if a.finalists else ([] if a.subset else space())
    if a.subset:
        import re

        chosen += [c for c in space() if re.search(a.subset, c.name) and c not in chosen]
    if a.list:
        for c in chosen:
            print("%-50s lds=%6d" % (c.name, c.lds_bytes))
    if a.build:
        build_sweep_lib(configs=chosen)
    if a.run:
        run(a.run, only=a.only, repeat=a.repeat)
    if a.select:
        note = ("Focused re-sweep (`--build --finalists%s`, then `--run`): the configurations of the table in force "
                "before it, plus\ntheir variants with C staged through LDS (`_le`) and with non-temporal C stores "
                "(`_le_nt`)%s." % (" --subset '%s'" % a.subset if a.subset else "",
                                   ", and the configurations of the space matching `%s`" % a.subset if a.subset else "")
                ) if a.finalists else ""
        note = "\n".join(x for x in (note, a.note) if x)
        print(json.dumps(select(a.select, summary_path=a.summary, note=note), indent=1))
    if a.ablation:
        ablation(a.ablation, a.ablation_out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
