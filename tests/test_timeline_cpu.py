"""Host logic of the tile kernel's timeline tool (dense_tiled_gemm_04_amd/timeline.py) on synthetic stamps."""
import numpy as np

from dense_tiled_gemm_04_amd import timeline


def _stamps(nwg=16, waves=8):
    # workgroup w on XCD w % 8 at (1.6 + 0.02 * xcd) GHz; loop of 144000 shader cycles; prologue 2 us at that
    # clock, epilogue 4 us at 2.2 GHz; all start at real time 1000 (10 ns ticks)
    s = np.zeros((nwg, waves, 8), dtype=np.int64)
    for w in range(nwg):
        ghz = 1.6 + 0.02 * (w % 8)
        loop_ns = 144000 / ghz
        r = [10000.0, 10000.0 + 2000.0, 10000.0 + 2000.0 + loop_ns, 10000.0 + 2000.0 + loop_ns + 4000.0]
        t = [5e6, 5e6 + 2000 * ghz, 5e6 + 2000 * ghz + 144000, 5e6 + 2000 * ghz + 144000 + 4000 * 2.2]
        for wave in range(waves):
            s[w, wave, 0:4] = np.round(t)
            s[w, wave, 4:8] = np.round(np.array(r) / 10.0)
    return s


def test_summary_recovers_clock_loop_and_xcd_ends():
    s = _stamps()
    s[3, 5, 7] += 150  # wave 5 of workgroup 3 completes its C stores 1.5 us after wave 0
    out = timeline.summarise(s, 16, 8)
    # the workgroup's epilogue runs to its last wave's stores; wave 0's own stays 4 us
    assert abs(out["epilogue_us"][-1] - 5.5) < 0.02 and abs(out["epilogue_wave0_us"][-1] - 4.0) < 0.02
    assert out["loop_kcycles"][2] == 144.0
    assert abs(out["loop_clock_GHz"][0] - 1.6) < 2e-3 and abs(out["loop_clock_GHz"][-1] - 1.74) < 2e-3
    assert abs(out["prologue_us"][2] - 2.0) < 0.02 and abs(out["epilogue_us"][2] - 4.0) < 0.02
    assert abs(out["epilogue_clock_GHz"][2] - 2.2) < 2e-3
    xs = out["per_xcd"]
    assert [x["xcd"] for x in xs] == list(range(8)) and all(x["workgroups"] == 2 for x in xs)
    # the slowest XCD (0, 1.6 GHz) ends last: 2 + 90 + 4 us
    assert abs(xs[0]["last_end_us"] - 96.0) < 0.02 and abs(out["span_us"] - 96.0) < 0.02
    assert xs[7]["last_end_us"] < xs[0]["last_end_us"]


def test_stale_or_missing_timeline_build_is_reported_not_used(tmp_path, monkeypatch):
    import bench

    lib = tmp_path / "libgemm_f16_timeline.so"
    monkeypatch.setattr(timeline, "TIMELINE_LIB", str(lib))
    ok, why = timeline.available()
    assert not ok and "no timeline build" in why
    lib.write_bytes(b"")
    (tmp_path / "libgemm_f16_timeline.so.sha256").write_text("0" * 64 + "\n")
    ok, why = timeline.available()
    assert not ok and "older than the GEMM sources" in why
    # bench reports the reason instead of a clock, and never raises
    r = bench.timeline_clock(None, None, 0, 0, None, 0, 0, None, {"name": "x"})
    assert r == {"note": why}
