"""Timeline of the tile GEMM kernel from clock stamps taken inside it.

A diagnostic, not part of the product path.  `--build` compiles the GEMM unit
with -DGK_TIMELINE=1 into _build/libgemm_f16_timeline.so (same kernels, same
configuration table, plus per-wave stamps: shader clock `s_memtime` and the
100 MHz `s_memrealtime` counter at kernel entry, after the prologue's barrier,
after the K loop and after the C stores have completed).  `--run` (GPU) times
the shipped library and the timeline build on the same inputs, checks that
their outputs are bit-identical, and summarises one launch taken after >= 60 ms
of back-to-back launches:
  * per workgroup: prologue and K loop durations (wave 0), and the epilogue from
    the end of wave 0's K loop to the completion of the last wave's C stores
    (waves store their parts of C independently), with wave 0's own beside it;
  * the shader clock during the K loop (stamp cycles over stamp time), and the
    loop's length in shader cycles;
  * per XCD (workgroup w runs on XCD w mod 8): clock, loop time and when its
    last workgroup ended.

    python -m dense_tiled_gemm_04_amd.timeline --build
    python -m dense_tiled_gemm_04_amd.timeline --run timeline.json [--markdown timeline.md]
"""
from __future__ import annotations

import argparse
import json
import os
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
TIMELINE_LIB = os.path.join(PKG_DIR, "_build", "libgemm_f16_timeline.so")
RESOURCES = os.path.join(PKG_DIR, "_build", "timeline_kernel_resources.json")

# (name, M, N, K, epilogue): the 4096^3 product, the MLP up-projection with bias + GELU, the ragged shape with bias
WORKLOADS = (("gemm_4096", 4096, 4096, 4096, 0), ("mlp_up_8192x16384x4096", 8192, 16384, 4096, 2),
             ("ragged_4095x3001x1000", 4095, 3001, 1000, 1))


def build(verbose: bool = True) -> str:
    from dense_tiled_gemm_04_amd import build as libbuild

    # the stamps' registers push a few register-loader kernels into scratch; those are never measured here
    # (run() refuses a configuration whose kernel uses scratch in the timeline build)
    rows = libbuild.build_library(TIMELINE_LIB, [os.path.join(PKG_DIR, "csrc", "gemm_f16.hip")],
                                  defines=["-DGK_TIMELINE=1"], allow_scratch=True, resources_path=RESOURCES,
                                  verbose=verbose)
    with open(TIMELINE_LIB + ".sha256", "w") as f:
        f.write(libbuild.source_digest("gemm") + "\n")
    if verbose:
        for r in libbuild.scratch_users(rows):
            print("uses scratch in the timeline build: %s" % r["kernel"], flush=True)
    return TIMELINE_LIB


def available() -> tuple:
    """(True, None) when the timeline build exists and was built from the current GEMM sources, else
    (False, reason)."""
    from dense_tiled_gemm_04_amd import build as libbuild

    if not os.path.exists(TIMELINE_LIB) or not os.path.exists(TIMELINE_LIB + ".sha256"):
        return False, "no timeline build (python -m dense_tiled_gemm_04_amd.timeline --build)"
    if open(TIMELINE_LIB + ".sha256").read().strip() != libbuild.source_digest("gemm"):
        return False, "the timeline build is older than the GEMM sources"
    return True, None


_LIB = None


def _load():
    import ctypes

    global _LIB
    if _LIB is None:
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib = ctypes.CDLL(TIMELINE_LIB)
        lib.gemm_f16.argtypes = [i64, i64, i64, vp, vp, vp, vp, i32, vp]
        lib.gemm_f16.restype = i32
        lib.gemm_f16_with_config.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, i32, vp]
        lib.gemm_f16_with_config.restype = i32
        lib.gemm_f16_select_config.argtypes = [i64, i64, i64, vp, vp, vp, vp, i32]
        lib.gemm_f16_select_config.restype = i32
        lib.gemm_f16_config_info.argtypes = [i32, ctypes.c_char_p, i32]
        lib.gemm_f16_timeline_buffer.argtypes = [vp]
        _LIB = lib
    return _LIB


def _config(idx: int) -> dict:
    import ctypes

    b = ctypes.create_string_buffer(1024)
    _load().gemm_f16_config_info(idx, b, 1024)
    return json.loads(b.value.decode())


def config_index(name: str) -> int:
    lib = _load()
    for i in range(lib.gemm_f16_num_configs()):
        if _config(i)["name"] == name:
            return i
    raise KeyError(name)


def measure(torch, M: int, N: int, K: int, epi: int, A: int, B: int, bias, C: int, stream, warm_ms: float = 60.0,
            config: int | None = None) -> dict:
    """Stamps of one launch of the timeline build of the tile kernel (B[K][N], device pointers A, B, bias, C),
    taken after >= warm_ms of back-to-back launches of it on `stream`; the default configuration unless
    `config` (an index of the table) is given.  Returns summarise() plus the configuration's name and the K
    loop's MFMA share: MFMA cycles per SIMD (BM x BN x (K stages x BK) x 2 FLOP over 4 SIMDs at 1024 FLOP per
    SIMD-cycle) over the loop's median shader cycles."""
    lib = _load()
    idx = config if config is not None else lib.gemm_f16_select_config(M, N, K, A, B, bias, C, epi)
    info = _config(idx)
    if info["kind"] != "tile" or info["spread"] & 256:
        return {"config": info["name"], "note": "not a gemm_tile_pipe_kernel configuration: no stamps"}
    tmpl = [info["bm"], info["bn"], info["bk"], info["waves_m"], info["waves_n"], info["stages"], info["group_m"],
            epi, info["bslot"], info["dstride"], {"dma": 0, "reg": 1, "buf": 2}[info["loader"]], info["cslot"],
            info["waves_per_simd"], info["mfma"], info["spread"], info["b_transposed"]]
    sym = "gemm_tile_pipe_kernelI" + "".join("Li%dE" % v for v in tmpl)
    if any(sym in k for k in _spilling_tile_kernels()):
        return {"config": info["name"], "note": "this configuration spills in the timeline build: not measured"}
    waves = info["waves_m"] * info["waves_n"]
    nwg = ((M + info["bm"] - 1) // info["bm"]) * ((N + info["bn"] - 1) // info["bn"])
    stamps = torch.zeros(nwg * waves * 8, dtype=torch.int64, device=torch.device("cuda:0"))
    sh = stream.cuda_stream

    def launch():
        st = lib.gemm_f16_with_config(idx, M, N, K, A, B, bias, C, epi, sh)
        if st != 0:
            raise RuntimeError("timeline build: gemm_f16_with_config status %d" % st)

    lib.gemm_f16_timeline_buffer(stamps.data_ptr())
    try:
        # the first launch of the timeline build also loads its code object: keep it out of the launch time
        # that sizes the warm-up (a short warm-up would leave the stamped launch in the controller's early dip)
        launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        one_ms = max(e0.elapsed_time(e1) / 3, 1e-3)
        for _ in range(max(1, int(warm_ms / one_ms))):
            launch()
        torch.cuda.synchronize()
    finally:
        lib.gemm_f16_timeline_buffer(None)
    s = stamps.cpu().numpy().reshape(nwg, waves, 8)
    out = summarise(s, nwg, waves)
    kt = (K + info["bk"] - 1) // info["bk"]
    mfma_cycles = info["bm"] * info["bn"] * kt * info["bk"] * 2 / (4 * 1024)
    out["config"] = info["name"]
    out["loop_mfma_share"] = round(mfma_cycles / (out["loop_kcycles"][2] * 1e3), 3)
    return out


def _spilling_tile_kernels() -> list:
    rows = json.load(open(RESOURCES)) if os.path.exists(RESOURCES) else []
    return [r["kernel"] for r in rows if "gemm_tile_pipe_kernel" in r["kernel"] and
            (int(r.get("ScratchSize [bytes/lane]", 0)) or int(r.get("VGPRs Spill", 0)))]


def _pct(x, ps=(0, 10, 50, 90, 100)):
    import numpy as np

    return [round(float(np.percentile(x, p)), 3) for p in ps]


def summarise(stamps, nwg: int, waves: int) -> dict:
    """stamps: int64 [nwg, waves, 8] = shader clock at points 0-3, real-time counter (10 ns) at points 0-3."""
    import numpy as np

    t = stamps[:, :, 0:4].astype(np.float64)
    r = stamps[:, :, 4:8].astype(np.float64) * 10.0   # ns
    r0 = r[:, :, 0].min()
    w0t, w0r = t[:, 0, :], r[:, 0, :]
    loop_ns = w0r[:, 2] - w0r[:, 1]
    loop_cyc = w0t[:, 2] - w0t[:, 1]
    out = {
        "span_us": round(float((r[:, :, 3].max() - r0) / 1e3), 2),
        "start_us": _pct((r[:, :, 0].min(axis=1) - r0) / 1e3),
        "prologue_us": _pct((w0r[:, 1] - w0r[:, 0]) / 1e3),
        "loop_us": _pct(loop_ns / 1e3),
        "loop_kcycles": _pct(loop_cyc / 1e3),
        "loop_clock_GHz": _pct(loop_cyc / loop_ns),
        "epilogue_us": _pct((r[:, :, 3].max(axis=1) - w0r[:, 2]) / 1e3),
        "epilogue_wave0_us": _pct((w0r[:, 3] - w0r[:, 2]) / 1e3),
        "epilogue_clock_GHz": _pct((w0t[:, 3] - w0t[:, 2]) / (w0r[:, 3] - w0r[:, 2])),
        "end_us": _pct((r[:, :, 3].max(axis=1) - r0) / 1e3),
        "percentiles": [0, 10, 50, 90, 100],
        "per_xcd": [],
    }
    xcd = np.arange(nwg) % 8
    for x in range(8):
        m = xcd == x
        if not m.any():
            continue
        out["per_xcd"].append({
            "xcd": x, "workgroups": int(m.sum()),
            "loop_clock_GHz": round(float(np.median(loop_cyc[m] / loop_ns[m])), 3),
            "loop_us": round(float(np.median(loop_ns[m]) / 1e3), 2),
            "last_end_us": round(float((r[m, :, 3].max() - r0) / 1e3), 2),
        })
    return out


def run(out_path: str, markdown: str | None = None, extra: list | None = None) -> dict:
    """Measure WORKLOADS with the default configurations, then `extra` runs: (name, M, N, K, epilogue,
    configuration name or None), with B[K][N] as allocated (row stride N: aligned when N % 8 == 0)."""
    import ctypes

    import torch

    sys.path.insert(0, ROOT)
    from dense_tiled_gemm_04_amd import build as libbuild

    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    shipped = ctypes.CDLL(libbuild.LIB_PATH)
    shipped.gemm_f16.argtypes = [i64, i64, i64, vp, vp, vp, vp, i32, vp]
    shipped.gemm_f16.restype = i32
    shipped.gemm_f16_with_config.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, i32, vp]
    shipped.gemm_f16_with_config.restype = i32
    lib_t = _load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    results = {}
    runs = [w + (None,) for w in WORKLOADS] + list(extra or [])
    for name, M, N, K, epi, forced in runs:
        print("workload %s" % name, flush=True)
        g = torch.Generator().manual_seed(1)
        A = (torch.rand(M, K, generator=g) * 2 - 1).half().to(dev)
        B = (torch.rand(K, N, generator=g) * 2 - 1).half().to(dev)
        bias = (torch.randn(N, generator=g) * 0.1).half().to(dev)
        C = {k: torch.empty(M, N, dtype=torch.float16, device=dev) for k in ("shipped", "timeline")}
        pb = bias.data_ptr() if epi else None
        idx = config_index(forced) if forced else \
            lib_t.gemm_f16_select_config(M, N, K, A.data_ptr(), B.data_ptr(), pb, C["timeline"].data_ptr(), epi)

        def call(which):
            L = shipped if which == "shipped" else lib_t
            st = L.gemm_f16_with_config(idx, M, N, K, A.data_ptr(), B.data_ptr(), pb, C[which].data_ptr(), epi,
                                        stream.cuda_stream)
            assert st == 0, st

        def timed(which, n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                call(which)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n * 1e3   # us per launch

        times = {"shipped": [], "timeline": []}
        for _rep in range(3):
            for which in times:
                one = timed(which, 3)
                timed(which, max(1, int(60e3 / one)))             # >= 60 ms back to back
                times[which].append(round(timed(which, max(20, int(25e3 / one))), 2))
        res = measure(torch, M, N, K, epi, A.data_ptr(), B.data_ptr(), pb, C["timeline"].data_ptr(), stream,
                      config=idx)
        res.update({"us_per_launch": times, "outputs_identical": bool(torch.equal(C["shipped"], C["timeline"]))})
        results[name] = res
        print(json.dumps({name: {k: v for k, v in res.items() if k != "per_xcd"}}), flush=True)
        for row in res.get("per_xcd", []):
            print("   ", json.dumps(row), flush=True)
    with open(out_path, "w") as f:
        json.dump(results, f, indent=1)
    if markdown:
        write_markdown(results, markdown)
    return results


def write_markdown(results: dict, path: str) -> None:
    lines = []
    for name, r in results.items():
        lines += ["### %s (`%s`)" % (name, r["config"]), "",
                  "µs per launch (three rounds of ≥ 60 ms warm-up + ≥ 25 ms timed): shipped %s, timeline build %s; "
                  "outputs bit-identical: %s. K loop MFMA share: %s." % (
                      r["us_per_launch"]["shipped"], r["us_per_launch"]["timeline"], r["outputs_identical"],
                      r.get("loop_mfma_share")), "",
                  "| quantity (percentiles over workgroups: 0/10/50/90/100) | values |", "|---|---|"]
        for k in ("start_us", "prologue_us", "loop_us", "loop_kcycles", "loop_clock_GHz", "epilogue_us",
                  "epilogue_wave0_us", "epilogue_clock_GHz", "end_us"):
            lines.append("| %s | %s |" % (k, " / ".join("%g" % v for v in r[k])))
        lines += ["| span of the launch (first entry to last C store) | %g µs |" % r["span_us"], "",
                  "| XCD | workgroups | K-loop clock GHz | K loop µs (median) | last workgroup ends µs |",
                  "|---:|---:|---:|---:|---:|"]
        for x in r["per_xcd"]:
            lines.append("| %d | %d | %.3f | %.2f | %.2f |" % (x["xcd"], x["workgroups"], x["loop_clock_GHz"],
                                                              x["loop_us"], x["last_end_us"]))
        lines.append("")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--build", action="store_true", help="compile the timeline build of the GEMM unit")
    ap.add_argument("--run", metavar="OUT_JSON", help="measure on the GPU and write the summary")
    ap.add_argument("--markdown", default=None, help="with --run: also write the tables as Markdown")
    ap.add_argument("--extra", action="append", default=[], metavar="NAME:M:N:K:EPI:CONFIG",
                    help="with --run: one more case with a forced configuration of the table (repeatable)")
    a = ap.parse_args()
    if a.build:
        print(build())
    if a.run:
        extra = []
        for e in a.extra:
            f = e.split(":")
            extra.append((f[0], int(f[1]), int(f[2]), int(f[3]), int(f[4]), f[5]))
        run(a.run, a.markdown, extra)
    return 0


if __name__ == "__main__":
    sys.exit(main())
