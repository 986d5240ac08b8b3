"""The compiler's per-kernel resource report of the shipped library (written by
dense_tiled_gemm_04_amd/build.py from -Rpass-analysis=kernel-resource-usage).

A register spill would only show up as a slowdown, so the build refuses kernels
with scratch memory; this checks the recorded report again, and that every tile
kernel fits the waves per SIMD its template asks for (the eight-wave 256x256
tiles need their 128 accumulators and everything else within 256 registers)."""
import json
import os
import re

import pytest

from dense_tiled_gemm_04_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.RESOURCES_PATH), reason="library not built here")

# template parameters of gemm_tile_pipe_kernel, in order
TILE_PARAMS = ["BM", "BN", "BK", "WM", "WN", "STAGES", "GROUP_M", "EPI", "BSLOT", "DSTRIDE", "LOADER", "CSLOT",
               "WPE", "MF", "SPREAD", "BT"]


def rows():
    return json.load(open(build.RESOURCES_PATH))


def test_report_covers_every_kernel_family():
    names = [r["kernel"] for r in rows()]
    for fam in ("gemm_tile_pipe_kernel", "gemm_skinny_kernel", "vector_add_f32", "softmax", "flash_attn"):
        assert any(fam in n for n in names), fam


def test_no_kernel_uses_scratch():
    bad = [r["kernel"] for r in rows() if r.get("ScratchSize [bytes/lane]", 0) or r.get("VGPRs Spill", 0)]
    assert not bad, bad


def test_tile_kernels_reach_their_waves_per_simd():
    n = 0
    for r in rows():
        if "gemm_tile_pipe_kernel" not in r["kernel"]:
            continue
        vals = [int(v) for v in re.findall(r"Li(-?\d+)E", r["kernel"])][:len(TILE_PARAMS)]
        p = dict(zip(TILE_PARAMS, vals))
        assert r["Occupancy [waves/SIMD]"] >= p["WPE"], (p, r)
        if p["WPE"] == 2:  # two waves share the 512 registers of a SIMD lane
            assert r["VGPRs"] + r["AGPRs"] <= 256, (p, r)
        n += 1
    assert n >= 10
