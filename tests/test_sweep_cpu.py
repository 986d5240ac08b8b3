"""The offline sweep's host logic: search space, budget filter, table emission
and per-class selection (no GPU; synthetic timing records)."""
import json
import os
import re

import pytest

from dense_tiled_gemm_04_amd import sweep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_budget_filter():
    # 256x256x64 double-buffered: 128 KiB of LDS, fits; three stages: 192 KiB, rejected
    assert sweep.valid(sweep.Tile(256, 256, 64, 2, 2, 2, 4, 3, 2, "dma"))
    assert not sweep.valid(sweep.Tile(256, 256, 64, 2, 2, 3, 4, 3, 2, "dma"))
    # two 128x128x64 double-buffered workgroups per CU: 2 x 64 KiB fits; 2 x 96 KiB does not
    assert sweep.valid(sweep.Tile(128, 128, 64, 2, 2, 2, 4, 1, 1, "dma", wpe=2))
    assert not sweep.valid(sweep.Tile(128, 128, 64, 2, 2, 3, 4, 1, 1, "dma", wpe=2))
    # 256 accumulators per lane cannot share a SIMD with a second wave
    assert not sweep.valid(sweep.Tile(256, 256, 64, 2, 2, 2, 4, 3, 2, "dma", wpe=2))
    # skinny: M <= 16 with 8 stages uses the whole 160 KiB; 9 would not fit
    assert sweep.valid(sweep.Skinny(1, 8)) and not sweep.valid(sweep.Skinny(1, 9))
    # split-K skinny: stages of 32 k-rows x 256 columns (16 KiB) plus 1 KiB of A per 16 rows; 64 rows at
    # BK = 64 and 4 stages is exactly 160 KiB, 5 stages is not; at least two K ranges; BK a multiple of 32
    assert sweep.SplitK(4, 4, 64, 4).lds_bytes == 160 * 1024 and sweep.valid(sweep.SplitK(4, 4, 64, 4))
    assert not sweep.valid(sweep.SplitK(4, 5, 64, 4))
    assert not sweep.valid(sweep.SplitK(1, 4, 32, 1)) and not sweep.valid(sweep.SplitK(1, 4, 48, 4))
    # at M = 16, BK = 32 a stage is 17 KiB: nine fit in the LDS, ten do not
    assert sweep.valid(sweep.SplitK(1, 9, 32, 4)) and not sweep.valid(sweep.SplitK(1, 10, 32, 4))


def test_eight_wave_budget_rules():
    # eight waves (2 x 4) put two on each SIMD: wpe must be a multiple of 2, and wpe 2 means one workgroup per CU
    t = dict(bm=256, bn=256, bk=64, wm=2, wn=4, stages=2, group=4, bslot=4, dstride=3, loader="dma", mf=16,
             spread=110)
    assert sweep.valid(sweep.Tile(**t, wpe=2))
    assert not sweep.valid(sweep.Tile(**t, wpe=1))
    # wpe 4 would put two such workgroups (2 x 128 KiB of LDS) on one CU
    assert not sweep.valid(sweep.Tile(**t, wpe=4))
    # the 4 x 2 layout (64 x 128 per wave) needs two B fragment sets of 8: past the 256 registers per lane
    assert not sweep.valid(sweep.Tile(**dict(t, wm=4, wn=2), wpe=2))
    # three stages of 256 x 256 x 64 (192 KiB) exceed the LDS of the CU even for one workgroup
    assert not sweep.valid(sweep.Tile(**dict(t, stages=3), wpe=2))
    # a workgroup whose wave count is not a multiple of the 4 SIMDs is rejected
    assert not sweep.valid(sweep.Tile(256, 256, 64, 2, 3, 2, 4, 4, 3, "dma", wpe=2, mf=16, spread=110))


def test_schedule_constraints_mirror_kernel():
    # barrier slot must leave room in the last k-step for the next stage's reads
    assert not sweep.valid(sweep.Tile(128, 128, 64, 2, 2, 2, 4, 3, 1, "dma"))   # 4 MFMAs per k-step
    # every copy must be issued before the stage's barrier
    assert not sweep.valid(sweep.Tile(128, 128, 64, 2, 2, 2, 4, 1, 4, "dma"))
    # register loader is double-buffered only
    assert not sweep.valid(sweep.Tile(128, 128, 64, 2, 2, 3, 4, 1, 1, "reg"))
    # odd number of k16-steps per stage breaks the fragment ping-pong
    assert not sweep.valid(sweep.Tile(128, 128, 16, 2, 2, 2, 4, 1, 1, "dma"))


def test_schedule_flags_in_names_and_limits():
    # schedule flags: 1 spread reads, 2 in-place A refill (needs two MFMA rows per wave), 4 pinned accumulators
    t = sweep.Tile(256, 256, 64, 2, 2, 2, 4, 16, 2, "dma", mf=16, spread=6)
    assert t.name.endswith("_m16_ip_pa") and sweep.valid(t)
    assert sweep.Tile(256, 256, 64, 2, 2, 2, 4, 8, 2, "dma", mf=16, spread=5).name.endswith("_m16_sp_pa")
    assert not sweep.valid(sweep.Tile(64, 128, 64, 2, 2, 2, 4, 1, 1, "dma", spread=2))   # one 32-row MFMA per wave
    assert not sweep.valid(sweep.Tile(256, 256, 64, 2, 2, 2, 4, 3, 1, "dma", spread=8))
    assert sweep.Skinny(2, 6, 1).name == "skinny_m32_s6_bt"
    assert sweep.Skinny(1, 4, 1, 1).name == "skinny_m16_s4_r_bt"
    assert sweep.Skinny(2, 4, 0, 1, a16=1).name == "skinny_m32_s4_r_a16"
    # 16-byte A copies: 2 per lane and stage at 32 rows (8 with 4-byte copies); 8 stages of M <= 16 still fit
    assert sweep.valid(sweep.Skinny(1, 8, a16=1)) and not sweep.valid(sweep.Skinny(1, 9, a16=1))


def test_lds_epilogue_flags():
    # 32: C staged through the stage buffers (the whole fp16 tile must fit in them), 64: non-temporal C stores,
    # only together with 32
    t = sweep.Tile(256, 256, 64, 2, 2, 2, 4, 24, 2, "dma", mf=16, spread=14 + 96)
    assert t.name.endswith("_m16_ip_pa_ea_le_nt") and sweep.valid(t)
    assert sweep.valid(sweep.Tile(128, 128, 64, 2, 2, 3, 4, 1, 1, "dma", spread=32))
    assert sweep.Tile(256, 256, 64, 2, 2, 2, 4, 16, 2, "dma", mf=16, spread=30 + 32, bt=1).name.endswith("_fb_le_bt")
    assert not sweep.valid(sweep.Tile(256, 256, 64, 2, 2, 2, 4, 24, 2, "dma", mf=16, spread=14 + 64))
    # a 256x256 tile (128 KiB of fp16) does not fit in two 32-deep stages (96 KiB)
    assert not sweep.valid(sweep.Tile(256, 256, 32, 2, 2, 2, 4, 3, 1, "dma", spread=32))
    # 192-wide tiles: 12 chunks per sub-tile row, the one non-power-of-two row the epilogue swizzle handles
    assert sweep.valid(sweep.Tile(256, 192, 64, 2, 2, 2, 4, 16, 2, "buf", mf=16, spread=14 + 96))
    # the finalists of a re-sweep are the table's configurations and their epilogue variants, all in the space
    fin = sweep.finalists()
    names = {c.name for c in fin}
    assert all(sweep.valid(c) for c in fin)
    for n in names:
        base = n.replace("_le_nt", "").replace("_le", "")
        assert base in names or n in names


def test_space_is_valid_and_unique():
    sp = sweep.space()
    assert len(sp) >= 20
    names = [c.name for c in sp]
    assert len(set(names)) == len(names)
    assert all(sweep.valid(c) for c in sp)
    assert all(c.lds_bytes <= 160 * 1024 for c in sp)
    for cls in sweep.CLASSES:
        assert any(sweep.class_of(c, cls) for c in sp), cls


def _table_entries(path):
    src = open(path).read()
    tiles = re.findall(r'(?<!PINGPONG_)TILE_CFG\(([^)]*)\)', src)
    skinny = re.findall(r'SKINNY_CFG\(([^)]*)\)', src)
    splitk = re.findall(r'SPLITK_CFG\(([^)]*)\)', src)
    pingpong = re.findall(r'PINGPONG_CFG\(([^)]*)\)', src)
    sel = dict(re.findall(r'#define (SEL_\w+) (\d+)', src))
    return tiles + [("pp", x) for x in pingpong], skinny + [("splitk", x) for x in splitk], \
        {k: int(v) for k, v in sel.items()}


def test_product_table_entries_are_in_budget():
    tiles, skinny, sel = _table_entries(os.path.join(ROOT, "dense_tiled_gemm_04_amd", "csrc", "config_table.inc"))
    n = len(tiles) + len(skinny)
    assert set(sel) == set(sweep.CLASSES) and all(0 <= v < n for v in sel.values())
    for t in tiles:
        if isinstance(t, tuple):  # a ping-pong entry: group, B transposed, non-temporal C, name
            f = [x.strip() for x in t[1].split(",")]
            c = sweep.PingPong(int(f[0]), int(f[1]), int(f[2]))
            assert sweep.valid(c) and f[3].strip('"') == c.name
            continue
        f = [x.strip() for x in t.split(",")]
        c = sweep.Tile(*map(int, f[:9]), f[9][len("LOAD_"):].lower(), int(f[10]), int(f[11]),
                       int(f[12]), int(f[13]), int(f[14]))
        assert sweep.valid(c), c
        assert f[15].strip('"') == c.name
    for s in skinny:
        if isinstance(s, tuple):  # a split-K entry: MB, stages, BK, ranges, name
            f = [x.strip() for x in s[1].split(",")]
            c = sweep.SplitK(*map(int, f[:4]))
            assert sweep.valid(c) and f[4].strip('"') == c.name
            continue
        f = [x.strip() for x in s.split(",")]
        c = sweep.Skinny(int(f[0]), int(f[1]), int(f[2]), int(f[3]), a16=int(f[4]))
        assert sweep.valid(c), c
        assert f[5].strip('"') == c.name


def test_select_picks_fastest_valid_per_class(tmp_path):
    sp = sweep.space()
    recs = []
    # synthetic timings: time grows with the config's position, except one clear winner per class
    winners = {}
    spilled = sweep.scratch_configs()   # never selected; which ones spill depends on the last sweep build
    for cls in sweep.CLASSES:
        winners[cls] = [c for c in sp if sweep.class_of(c, cls) and c.name not in spilled][-1].name
    for name, w, opts, classes in sweep.sweep_workloads():
        for i, c in enumerate(sp):
            if not any(sweep.class_of(c, cls) for cls in classes):
                continue
            t = 100.0 + i
            if any(winners[cls] == c.name for cls in classes):
                t = 10.0
            recs.append({"config": c.name, "workload": name, "classes": classes, "median_us": t, "ok": True,
                         "tflops": 1.0})
    # a faster configuration whose output failed the screen must never be chosen
    bad = [c for c in sp if sweep.class_of(c, "SEL_DMA_BIG")][0].name
    for r in recs:
        if r["config"] == bad and "SEL_DMA_BIG" in r["classes"]:
            r["median_us"], r["ok"] = 1.0, False
    res = tmp_path / "res.jsonl"
    res.write_text("\n".join(json.dumps(r) for r in recs) + "\n")
    table = tmp_path / "table.inc"
    chosen = sweep.select(str(res), table_path=str(table), summary_path=str(tmp_path / "s.md"))
    for cls in sweep.CLASSES:
        assert chosen[cls] == winners[cls], cls
    tiles, skinny, sel = _table_entries(str(table))
    assert len(tiles) + len(skinny) == len(set(chosen.values()))
    assert (tmp_path / "s.md").read_text().count("|") > 10
