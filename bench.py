#!/usr/bin/env python3
"""Benchmark of the MI355X fp16 GEMM (+ fused bias / GELU) library.

One "step" is one call of the library's C entry point gemm_f16 on one batch of
synthetic, seeded input already resident in HBM: the whole hot path (tile
scheduling, LDS staging, MFMA main loop, fused epilogue, single write of C).
The default workload is the 4096^3 fp16 GEMM (the headline shape of the
TileLang tutorial's blog post, sections "performance" and "Step 4").

Prints ONE JSON line:
  value     = TFLOP/s = 2*M*N*K / (time per step)
  roofline  = the dominant kernel against MI355X's published peak (dense fp16
              MFMA 2.5 PFLOP/s, or HBM 8 TB/s for the skinny workload), its
              duration measured here with HIP events on the launch stream;
              traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE
              counters (profiles/), null if the kernel sources changed since.
  cpu_baseline = the CPU oracle (fp64, all host threads) on a bounded sample.
  context   = the vendor BLAS in the same process (sequential and interleaved),
              the settled rate under the power limiter (context.sustained:
              >= 50 ms of warm-up, then >= 25 ms of launches in ~1 ms chunks,
              median chunk), the library's own event-median helper
              gemm_f16_time, the sha256 of every input, a status per workload,
              and (GEMM workloads, unless --no-context) the fused bias+GELU MLP
              up-projection and the skinny HBM-bound shape measured the same
              way under context.workloads.

--workload softmax_* benchmarks the library's row softmax instead (one step =
one softmax_rows_f16 call over the whole matrix; value in GB/s of X read plus Y
written, against the HBM peak; copies of X rotated past the Infinity Cache).
--workload attn_* benchmarks the attention forward pass (one step = one
flash_attn_fwd_f16 call; value in TFLOP/s counting 4*D per allowed query-key
pair, against the MFMA peak; PyTorch's fused SDPA timed alongside).
--b-transposed stores the GEMM's B as Bt[N][K] (a linear layer's weight) and
calls gemm_f16_bt; torch.nn.functional.linear on the same tensors is the
comparison.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
# minimum back-to-back work before a timed region: after idle the power controller boosts the clock for ~2 ms,
# throttles hard at ~3-8 ms and settles after 30-40 ms (bench.py --clock-series)
WARMUP_MS = 50.0


def kernel_family(workload: str) -> str:
    return "softmax" if workload.startswith("softmax") else "attention" if workload.startswith("attn") else "gemm"


def kernel_source_digest(family: str = "gemm") -> str:
    """Digest of a kernel family's sources (a change voids that family's recorded traffic)."""
    from dense_tiled_gemm_04_amd import build as libbuild

    return libbuild.source_digest(family)


def interleaved_ms(torch, stream, ours, theirs, launch_ms: float, rounds: int = 6, chunk_ms: float = 2.0):
    """Ours against the vendor's on equal terms: alternating chunks of ~chunk_ms of back-to-back launches of
    each step function, every chunk between its own pair of HIP events on the launch stream, after one untimed
    round.  The power limiter sets the clock within milliseconds, so a vendor loop timed right after ours runs
    on a hotter card than ours did; alternating puts both through the same states.  Returns the median ms per
    launch of each side's chunks."""
    n = max(1, int(round(chunk_ms / max(launch_ms, 1e-3))))
    evs = ([], [])
    i = 0
    for r in range(rounds + 1):
        for k, f in enumerate((ours, theirs)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                f(i)
                i += 1
            e1.record(stream)
            if r > 0:
                evs[k].append((e0, e1))
    torch.cuda.synchronize()

    def med(pairs):
        t = sorted(a.elapsed_time(b) / n for a, b in pairs)
        return t[len(t) // 2]
    return med(evs[0]), med(evs[1])


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch recorded from rocprofv3 counters, if still valid."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_sha256") != kernel_source_digest(kernel_family(workload)) or \
            rec.get("kernel") != kernel:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def per_core_gflops(target_s: float = 1.0) -> float:
    """The oracle on the whole 256^3 workload with one thread, repeated for about target_s: a per-core rate."""
    import oracle
    import workloads
    w = workloads.WORKLOADS["gemm_256"]
    A, B, bias = workloads.make_inputs(w)
    n, t = 0, time.perf_counter()
    while True:
        oracle.gemm(A, B, bias, w.epilogue, threads=1)
        n += 1
        dt = time.perf_counter() - t
        if dt >= target_s:
            return round(n * w.flops / dt / 1e9, 3)


def cpu_baseline(w, A, B, bias, target_s: float = 15.0):
    """Time the CPU oracle on the first R rows of the workload (full K, all N).

    R grows geometrically until one run takes at least a second, then is sized
    from that rate for about ``target_s`` seconds of CPU work (capped at M).
    """
    import numpy as np
    import oracle

    threads = oracle.max_threads()
    rows, dt = 0, 0.0
    r = min(w.M, 16)
    while True:
        t = time.perf_counter()
        oracle.gemm(np.ascontiguousarray(A[:r]), B, bias, w.epilogue, threads=threads)
        rows, dt = r, time.perf_counter() - t
        if dt >= 1.0 or r >= w.M:
            break
        r = min(w.M, r * 4)
    if dt < target_s and rows < w.M:
        r = int(min(w.M, max(rows, rows * target_s / max(dt, 1e-6))))
        t = time.perf_counter()
        oracle.gemm(np.ascontiguousarray(A[:r]), B, bias, w.epilogue, threads=threads)
        rows, dt = r, time.perf_counter() - t
    flops = 2.0 * rows * w.N * w.K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "per_core_GFLOPs": per_core_gflops(),
        "kind": "oracle",
        "sample": "rows 0..%d of C (%d x %d outputs, full K=%d, epilogue %s), fp64 oracle, %.2f s wall"
                  % (rows - 1, rows, w.N, w.K, w.epilogue, dt),
    }


CALIB_ELEMS = 64 * 1024 * 1024  # fp32 elements per vector: 256 MiB each for a, b and c


def hbm_calibration(g, torch) -> int:
    """c = a + b over 3 x 256 MiB fp32 buffers: each launch reads exactly 512 MiB and writes 256 MiB."""
    dev = torch.device("cuda:0")
    a = torch.ones(CALIB_ELEMS, dtype=torch.float32, device=dev)
    b = torch.ones(CALIB_ELEMS, dtype=torch.float32, device=dev)
    c = torch.empty_like(a)
    for _ in range(3):
        g.vector_add(a, b, out=c)
    torch.cuda.synchronize()
    assert bool((c == 2.0).all())
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(20):
        g.vector_add(a, b, out=c)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 20 * 1e3
    print(json.dumps({"calibration": "vector_add_f32", "elems": CALIB_ELEMS, "launches": 23,
                      "read_bytes_per_launch": 8 * CALIB_ELEMS, "write_bytes_per_launch": 4 * CALIB_ELEMS,
                      "avg_launch_us": round(us, 2), "GBps": round(12 * CALIB_ELEMS / us / 1e3, 1)}),
          flush=True)
    return 0


class PowerSampler:
    """Board power and shader clock of the GPU in use, sampled from its amdgpu hwmon files (power1_average or
    power1_input in microwatts, freq1_input in Hz) by a host thread every `period_s`.  The card is the one whose
    PCI address matches torch's device 0; failing that, every card is sampled and the one whose power rose the
    most is reported.  Readings are None where the files cannot be read."""

    def __init__(self, torch, period_s: float = 0.01):
        import glob
        import threading
        self.period_s = period_s
        self.cards = {}
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            hw = sorted(glob.glob(dev + "/hwmon/hwmon*"))
            if not hw:
                continue
            pw = next((hw[0] + "/" + f for f in ("power1_average", "power1_input") if os.path.exists(hw[0] + "/" + f)),
                      None)
            fr = hw[0] + "/freq1_input" if os.path.exists(hw[0] + "/freq1_input") else None
            if pw:
                self.cards[os.path.basename(os.path.realpath(dev))] = (pw, fr)
        self.match = None
        try:
            p = torch.cuda.get_device_properties(0)
            bus = getattr(p, "pci_bus_id", None)
            if bus is not None:
                for addr in self.cards:
                    if int(addr.split(":")[1], 16) == int(bus):
                        self.match = addr
        except Exception:
            pass
        self.samples = {a: [] for a in self.cards}
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                return float(f.read().strip())
        except (OSError, ValueError):
            return None

    def _run(self):
        while not self._stop.is_set():
            for a, (pw, fr) in self.cards.items():
                self.samples[a].append((self._read(pw), self._read(fr) if fr else None))
            time.sleep(self.period_s)

    def idle(self):
        return {a: self._read(pw) for a, (pw, fr) in self.cards.items()}

    def __enter__(self):
        self._idle = self.idle()
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self) -> dict:
        def med(v):
            v = sorted(x for x in v if x is not None)
            return v[len(v) // 2] if v else None
        if not self.cards:
            return {"card": None, "note": "no readable amdgpu hwmon power file"}
        rise = {a: (med([p for p, _ in self.samples[a]]) or 0) - (self._idle.get(a) or 0) for a in self.cards}
        card = self.match or max(rise, key=rise.get)
        pw = med([p for p, _ in self.samples[card]])
        fr = med([f for _, f in self.samples[card]])
        return {"card": card, "matched_by": "pci bus" if self.match else "largest power rise",
                "samples": len(self.samples[card]), "board_power_W": round(pw / 1e6, 1) if pw else None,
                "idle_power_W": round(self._idle[card] / 1e6, 1) if self._idle.get(card) else None,
                "sclk_GHz_hwmon": round(fr / 1e9, 3) if fr else None}


def clock_series(g, torch, ms_total: float = 80.0) -> int:
    """How the power controller sets the clock under sustained load: after 0.5 s idle, ms_total of back-to-back
    launches of the 4096^3 GEMM and of the MLP up-projection in ~1 ms chunks between HIP events; prints one
    JSON line per run with the time per launch of every chunk and the chunk's end time."""
    import numpy as np
    import workloads

    lib = g.load()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    for name in ("gemm_4096", "mlp_up_8192x16384x4096"):
        w = workloads.WORKLOADS[name]
        A, B, bias = workloads.make_inputs(w)
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        db = torch.from_numpy(bias).cuda() if bias is not None else None
        dC = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
        epi = g.EPILOGUES[w.epilogue]

        def step():
            st = lib.gemm_f16(w.M, w.N, w.K, dA.data_ptr(), dB.data_ptr(), db.data_ptr() if db is not None else None,
                              dC.data_ptr(), epi, sh)
            if st != 0:
                raise g.GemmError(st)
        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        per = max(1, int(round(1.0 / max(e0.elapsed_time(e1), 1e-3))))
        n = int(ms_total / max(per * e0.elapsed_time(e1), 1e-3)) + 1
        time.sleep(0.5)
        evs = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(per):
                step()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) / per * 1e3 for a, b in evs]
        end_ms = np.cumsum([u * per / 1e3 for u in us])
        print(json.dumps({"clock_series": name, "launches_per_chunk": per,
                          "us_per_launch": [round(u, 1) for u in us], "chunk_end_ms": [round(float(t), 2) for t in end_ms]}),
              flush=True)
        del dA, dB, dC
    return 0


def mfma_calibration(g, torch, seconds: float = 0.4) -> int:
    """The practical MFMA ceiling under the board power limit: the register-only MFMA loop on all 256 CUs (two
    waves per SIMD, 8 independent chains each) run back to back for `seconds`, for each MFMA shape; then the
    shipped 4096^3 GEMM the same way.  Prints one JSON line per run: FLOP/s from HIP events (median launch),
    the clock the loop ran at (s_memtime against the 100 MHz s_memrealtime), board power from hwmon, FLOP/J."""
    import numpy as np
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    wgs = 256
    stamps = torch.zeros((wgs, 4), dtype=torch.int64, device=dev)
    sink = torch.zeros(wgs * 512, dtype=torch.float32, device=dev)
    lines = []
    for shape in (16, 32):
        def launch(iters):
            st = g.mfma_calibration_raw(shape, iters, wgs, stamps.data_ptr(), sink.data_ptr(), sh)
            if st != 0:
                raise g.GemmError(st)
        # size one launch at ~20 ms from a short probe
        launch(2000)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch(2000)
        e1.record(stream)
        torch.cuda.synchronize()
        iters = max(1000, int(2000 * 20.0 / max(e0.elapsed_time(e1), 1e-3)))
        n = max(5, int(seconds * 1e3 / 20.0))
        evs = []
        with PowerSampler(torch) as ps:
            for _ in range(n):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                launch(iters)
                b.record(stream)
                evs.append((a, b))
            torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs[1:])
        t = ms[len(ms) // 2]
        flops = g.mfma_calibration_flops(shape, iters, wgs)
        st = stamps.cpu().numpy().astype(np.float64)
        clk = np.median((st[:, 1] - st[:, 0]) / ((st[:, 3] - st[:, 2]) / 100e6)) / 1e9
        pw = ps.summary()
        tf = flops / (t * 1e-3) / 1e12
        lines.append({"calibration": "mfma_f16_%dx%dx%d" % ((16, 16, 32) if shape == 16 else (32, 32, 16)),
                      "workgroups": wgs, "waves_per_simd": 2, "iters": iters, "launches": n,
                      "median_launch_ms": round(t, 3), "TFLOPs": round(tf, 1), "frac_of_spec": round(tf / PEAK_FP16_TFLOPS, 4),
                      "sclk_GHz_memtime": round(float(clk), 3),
                      "TFLOPs_at_2.4GHz_per_sclk": round(tf * 2.4 / float(clk), 1), "power": pw,
                      "GFLOP_per_J": round(tf * 1e3 / pw["board_power_W"], 1) if pw.get("board_power_W") else None})
    # the shipped 4096^3 GEMM, back to back for the same time
    w = workloads.WORKLOADS["gemm_4096"]
    A, B, _ = workloads.make_inputs(w)
    dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    dC = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    lib = g.load()
    step = lambda: lib.gemm_f16(w.M, w.N, w.K, dA.data_ptr(), dB.data_ptr(), None, dC.data_ptr(), 0, sh)
    for _ in range(50):
        step()
    torch.cuda.synchronize()
    per = 10
    chunks = []
    with PowerSampler(torch) as ps:
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(per):
                step()
            b.record(stream)
            chunks.append((a, b))
            if len(chunks) % 20 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) / per for a, b in chunks)
    t = ms[len(ms) // 2]
    tf = w.flops / (t * 1e-3) / 1e12
    pw = ps.summary()
    cfg = g.config_info(g.select_config_raw(w.M, w.N, w.K, dA.data_ptr(), dB.data_ptr(), None, dC.data_ptr(), 0))
    lines.append({"calibration": "gemm_4096 (shipped kernel, back to back)", "kernel": cfg["name"],
                  "launches": per * len(chunks), "median_launch_ms": round(t, 4), "TFLOPs": round(tf, 1),
                  "frac_of_spec": round(tf / PEAK_FP16_TFLOPS, 4), "power": pw,
                  "GFLOP_per_J": round(tf * 1e3 / pw["board_power_W"], 1) if pw.get("board_power_W") else None})
    for l in lines:
        print(json.dumps(l), flush=True)
    return 0


def cpu_baseline_softmax(w, X, target_s: float = 10.0):
    """Time the CPU oracle's row softmax on the first R rows (R grown as for the GEMM sample)."""
    import numpy as np
    import oracle

    threads = oracle.max_threads()
    r, rows, dt = min(w.rows, 64), 0, 0.0
    while True:
        t = time.perf_counter()
        oracle.softmax_rows(np.ascontiguousarray(X[:r]), threads=threads)
        rows, dt = r, time.perf_counter() - t
        if dt >= 1.0 or r >= w.rows:
            break
        r = min(w.rows, r * 4)
    if dt < target_s and rows < w.rows:
        r = int(min(w.rows, max(rows, rows * target_s / max(dt, 1e-6))))
        t = time.perf_counter()
        oracle.softmax_rows(np.ascontiguousarray(X[:r]), threads=threads)
        rows, dt = r, time.perf_counter() - t
    passes = 1
    if rows == w.rows and dt < target_s:
        # the whole matrix takes less than the target: repeat it for a steadier figure
        passes = max(1, int(target_s / max(dt, 1e-6)))
        t = time.perf_counter()
        for _ in range(passes):
            oracle.softmax_rows(X, threads=threads)
        dt = (time.perf_counter() - t) / passes
    return {"value": 4.0 * rows * w.cols / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "rows 0..%d of Y (%d x %d outputs), fp64 oracle, %.3f s wall per pass, %d pass(es)"
                      % (rows - 1, rows, w.cols, dt, passes)}


def bench_softmax(args, g, torch, w) -> int:
    """Row softmax: X copies rotated (the 256 MB Infinity Cache must not serve them), HIP events on the
    launch stream around exactly `steps` launches."""
    import workloads

    X = workloads.make_softmax_input(w)
    rotate = args.rotate if args.rotate is not None else 3
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dXs = [torch.from_numpy(X).to(dev) for _ in range(rotate)]
    dY = torch.empty_like(dXs[0])
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    pXs, pY = [x.data_ptr() for x in dXs], dY.data_ptr()
    lib = g.load()

    def step(i):
        st = lib.softmax_rows_f16(w.rows, w.cols, pXs[i % rotate], pY, sh)
        if st != 0:
            raise g.GemmError(st)

    n_warm, _ = warm_up(torch, stream, step, args.warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = w.algorithmic_bytes / (ms * 1e-3) / 1e9

    for i in range(5):
        torch.softmax(dXs[i % rotate], dim=-1)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_t = max(10, min(args.steps, 100))
    t0.record(stream)
    for i in range(n_t):
        torch.softmax(dXs[i % rotate], dim=-1)
    t1.record(stream)
    torch.cuda.synchronize()
    torch_ms = t0.elapsed_time(t1) / n_t
    il_ours, il_torch = interleaved_ms(torch, stream, step, lambda i: torch.softmax(dXs[i % rotate], dim=-1), ms)

    kernel = "softmax_" + g.softmax_path(w.rows, w.cols)
    roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "traffic": load_traffic(w.name, kernel), "kernel": kernel,
            "algorithmic_bytes_per_launch": w.algorithmic_bytes, "avg_launch_us": ms * 1e3}
    cpu = None if args.no_cpu_baseline else cpu_baseline_softmax(w, X)
    out = {
        "metric": "fp16 row softmax GB/s (X read + Y written once) + % of MI355X HBM peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in/out, f32 arithmetic",
        "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "cols": w.cols,
                   "inputs": "seeded numpy draws (%s), X copies rotated: %d" % (w.note, rotate)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "context": {"warmup_launches": n_warm, "torch_softmax_ms": round(torch_ms, 6),
                    "torch_GBps": round(w.algorithmic_bytes / (torch_ms * 1e-3) / 1e9, 1),
                    "interleaved": {"ours_ms": round(il_ours, 6), "torch_ms": round(il_torch, 6),
                                    "torch_over_ours": round(il_torch / il_ours, 3)}},
    }
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline_attention(w, Q, K, V, target_s: float = 10.0):
    """Time the CPU oracle on the first R query rows of (batch 0, head 0) and beyond (R grown as above)."""
    import numpy as np
    import oracle

    threads = oracle.max_threads()
    total = w.B * w.H * w.Nq
    r, rows, dt = min(total, 64), 0, 0.0
    while True:
        idx = np.arange(r, dtype=np.int64)
        t = time.perf_counter()
        oracle.attention_rows(Q, K, V, idx, causal=w.causal, threads=threads)
        rows, dt = r, time.perf_counter() - t
        if dt >= 1.0 or r >= total:
            break
        r = min(total, r * 4)
    if dt < target_s and rows < total:
        r = int(min(total, max(rows, rows * target_s / max(dt, 1e-6))))
        idx = np.arange(r, dtype=np.int64)
        t = time.perf_counter()
        oracle.attention_rows(Q, K, V, idx, causal=w.causal, threads=threads)
        rows, dt = r, time.perf_counter() - t
    flops = 0
    for flat in range(rows):
        i = flat % w.Nq
        flops += 4 * w.D * (min(i + 1, w.Nkv) if w.causal else w.Nkv)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "query rows 0..%d in (batch, head, row) order, all keys, fp64 oracle, %.2f s wall"
                      % (rows - 1, dt)}


# kernels of the attention forward pass (flash_attn_fwd_f16_kernel); auto is the library's default dispatch
ATTN_KERNELS = {"auto": 0, "block_serial": 1, "pipelined": 2}


def bench_attention(args, g, torch, w) -> int:
    """Attention forward: Q, K, V resident in HBM, HIP events on the launch stream around `steps` launches."""
    import math
    import workloads

    Q, K, V = workloads.make_attention_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dQ, dK, dV = (torch.from_numpy(x).to(dev) for x in (Q, K, V))
    dO = torch.empty_like(dQ)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    lib = g.load()
    scale = 1.0 / math.sqrt(w.D)
    ptrs = (dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), dO.data_ptr())

    kernel_id = ATTN_KERNELS[args.attn_kernel]
    kernel_name = args.attn_kernel if args.attn_kernel != "auto" else ("pipelined" if w.D == 128 else "block_serial")

    def step():
        st = lib.flash_attn_fwd_f16_kernel(w.B, w.H, w.Nq, w.Nkv, w.D, *ptrs, 1 if w.causal else 0, scale, kernel_id, sh)
        if st != 0:
            raise g.GemmError(st)

    n_warm, _ = warm_up(torch, stream, lambda i: step(), args.warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = w.flops / (ms * 1e-3) / 1e12

    # context: PyTorch's scaled dot-product attention on the same tensors, fused backends only
    torch_ms, backend, il = None, None, None
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            f = lambda: torch.nn.functional.scaled_dot_product_attention(dQ, dK, dV, is_causal=w.causal)
            for _ in range(3):
                f()
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n_t = max(5, min(args.steps, 50))
            t0.record(stream)
            for _ in range(n_t):
                f()
            t1.record(stream)
            torch.cuda.synchronize()
            torch_ms = t0.elapsed_time(t1) / n_t
            backend = "flash/efficient"
            il = interleaved_ms(torch, stream, lambda i: step(), lambda i: f(), ms)
    except RuntimeError as e:
        backend = "unavailable: %s" % str(e).splitlines()[0][:120]

    roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / PEAK_FP16_TFLOPS, "traffic": load_traffic(w.name, "flash_attn_fwd"),
            "kernel": "flash_attn_fwd", "algorithmic_flops_per_launch": w.flops,
            "algorithmic_bytes_per_launch": w.algorithmic_bytes, "avg_launch_us": ms * 1e3}
    cpu = None if args.no_cpu_baseline else cpu_baseline_attention(w, Q, K, V)
    out = {
        "metric": "fp16 attention forward TFLOP/s (4*D per allowed query-key pair) + % of MI355X MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in/out, f32 accumulate and softmax",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nkv": w.Nkv, "D": w.D, "causal": w.causal,
                   "attention_kernel": kernel_name,
                   "inputs": "seeded numpy draws, Q, K, V ~ N(0, 1) (%s)" % w.note},
        "roofline": roof,
        "cpu_baseline": cpu,
        "context": {"warmup_launches": n_warm, "torch_sdpa_ms": round(torch_ms, 6) if torch_ms else None, "torch_sdpa_backend": backend,
                    "torch_tflops": round(w.flops / (torch_ms * 1e-3) / 1e12, 3) if torch_ms else None,
                    "interleaved": {"ours_ms": round(il[0], 6), "torch_ms": round(il[1], 6),
                                    "torch_over_ours": round(il[1] / il[0], 3)} if il else None},
    }
    print(json.dumps(out), flush=True)
    return 0


def warm_up(torch, stream, step, warmup: int):
    """Untimed launches before a timed region: the `warmup` requested, extended until >= WARMUP_MS of
    back-to-back work has run, so that the timed launches see the clock the card settles at rather than its
    ramp out of idle.  step(i) launches once.  Returns (launches run, their ms per launch estimate)."""
    step(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(1, 4):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    one_ms = max(e0.elapsed_time(e1) / 3, 1e-3)
    n_warm = max(warmup, int(math.ceil(WARMUP_MS / one_ms)))
    for i in range(n_warm):
        step(i)
    torch.cuda.synchronize()
    return 4 + n_warm, one_ms


def sustained_ms(torch, stream, step, launch_ms: float, warm_ms: float = WARMUP_MS, total_ms: float = 25.0,
                 chunk_ms: float = 1.0) -> dict:
    """The settled rate under the power limiter: >= warm_ms of untimed back-to-back launches, then >= total_ms of
    launches timed in chunks of ~chunk_ms, each chunk between its own pair of HIP events on the launch stream.
    Returns the median, p10 and p90 over the chunks of the time per launch (ms)."""
    per = max(1, int(round(chunk_ms / max(launch_ms, 1e-3))))
    chunks = max(5, int(round(total_ms / max(per * launch_ms, 1e-3))))
    i = 0
    for _ in range(max(1, int(round(warm_ms / max(launch_ms, 1e-3))))):
        step(i)
        i += 1
    evs = []
    for _ in range(chunks):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(per):
            step(i)
            i += 1
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) / per for a, b in evs)
    q = lambda f: t[min(len(t) - 1, int(f * len(t)))]
    return {"ms": t[len(t) // 2], "p10_ms": q(0.1), "p90_ms": q(0.9), "chunks": chunks, "launches_per_chunk": per,
            "warmup_ms": warm_ms}


def gemm_workload_inputs(w):
    """Seeded inputs of a GEMM workload plus the sha256 of their bits (numpy streams are not promised stable
    across versions, so the digest records what was actually used)."""
    import workloads
    A, B, bias = workloads.make_inputs(w)
    return A, B, bias, workloads.input_digest(A, B, bias)


def measure_gemm(g, torch, w, A, B, bias, steps: int, warmup: int, bt: bool = False, rotate: int | None = None,
                 config: int | None = None, vendor: bool = True) -> dict:
    """One GEMM workload on the GPU: `steps` launches timed between one pair of HIP events on the launch stream
    after `warmup` untimed ones (synchronised on both sides), then the settled rate, the library's own
    event-median helper and (optionally) the vendor BLAS in the same process."""
    import numpy as np

    hbm_bound = w.flops / w.algorithmic_bytes < 100.0
    rotate = rotate if rotate is not None else (3 if hbm_bound else 1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dA = torch.from_numpy(A).to(dev)
    Bdev = np.ascontiguousarray(B.T) if bt else B
    dBs = [torch.from_numpy(Bdev).to(dev) for _ in range(rotate)]
    db = torch.from_numpy(bias).to(dev) if bias is not None else None
    dC = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    epi = g.EPILOGUES[w.epilogue]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    pA, pC = dA.data_ptr(), dC.data_ptr()
    pBs = [b.data_ptr() for b in dBs]
    pb = db.data_ptr() if db is not None else None
    lib = g.load()
    if bt:
        ld = (w.K, w.K, w.N)  # lda, ldb (row length of Bt), ldc
        cfg_idx = config if config is not None else \
            g.select_config_bt_raw(w.M, w.N, w.K, pA, ld[0], pBs[0], ld[1], pb, pC, ld[2], epi)
    else:
        cfg_idx = config if config is not None else g.select_config_raw(w.M, w.N, w.K, pA, pBs[0], pb, pC, epi)
    cfg = g.config_info(cfg_idx)

    def step(i):
        if bt:
            st = lib.gemm_f16_bt_with_config(cfg_idx, w.M, w.N, w.K, pA, ld[0], pBs[i % rotate], ld[1], pb, pC,
                                             ld[2], epi, sh) if config is not None else \
                lib.gemm_f16_bt(w.M, w.N, w.K, pA, ld[0], pBs[i % rotate], ld[1], pb, pC, ld[2], epi, sh)
        else:
            st = lib.gemm_f16_with_config(cfg_idx, w.M, w.N, w.K, pA, pBs[i % rotate], pb, pC, epi, sh) \
                if config is not None else lib.gemm_f16(w.M, w.N, w.K, pA, pBs[i % rotate], pb, pC, epi, sh)
        if st != 0:
            raise g.GemmError(st)

    t_start = time.perf_counter()
    n_warm, one_ms = warm_up(torch, stream, step, warmup)
    warm_s = time.perf_counter() - t_start
    # timed region: synchronised on both sides, HIP events on the launch stream
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    out = {"w": w, "bt": bt, "rotate": rotate, "hbm_bound": hbm_bound, "ms": ms, "cfg": cfg, "warm_s": warm_s,
           "warmup_launches": n_warm, "warmup_ms": round(n_warm * one_ms, 2),
           "finite": bool(torch.isfinite(dC).all().item())}
    out["sustained"] = sustained_ms(torch, stream, step, ms)
    if not bt and not hbm_bound:
        out["clock"] = timeline_clock(torch, w, pA, pBs[0], pb, pC, epi, stream, cfg)
    if hbm_bound and rotate > 1:
        # the same launches on one copy of B, which the Infinity Cache then partly serves: labelled, never `value`
        e0.record(stream)
        for i in range(steps):
            step(0)
        e1.record(stream)
        torch.cuda.synchronize()
        out["warm_unrotated_ms"] = e0.elapsed_time(e1) / steps
    # the library's own timing entry point (median of event-bracketed launches); it takes one B, so only where
    # B is not rotated (a single 256 MiB B would be partly served from the Infinity Cache)
    if not bt and rotate == 1:
        st, med = g.gemm_f16_time_raw(w.M, w.N, w.K, pA, pBs[0], pb, pC, epi, 51, sh,
                                      config=-1 if config is None else config)
        out["helper_median_ms"] = med if st == 0 else None
    if vendor:
        # the vendor BLAS on the same tensors (torch.matmul, or F.linear for Bt; + bias + gelu eagerly if fused)
        def torch_step(i):
            c = torch.nn.functional.linear(dA, dBs[i % rotate]) if bt else torch.matmul(dA, dBs[i % rotate])
            if w.epilogue == "bias":
                c = c + db
            elif w.epilogue == "bias_gelu":
                c = torch.nn.functional.gelu(c + db)
            return c
        for i in range(5):
            torch_step(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        n_t = max(10, min(steps, 100))
        t0.record(stream)
        for i in range(n_t):
            torch_step(i)
        t1.record(stream)
        torch.cuda.synchronize()
        out["torch_ms"] = t0.elapsed_time(t1) / n_t
        out["interleaved"] = interleaved_ms(torch, stream, step, torch_step, ms)
    del dA, dBs, db, dC
    torch.cuda.empty_cache()
    return out


def timeline_clock(torch, w, pA, pB, pb, pC, epi, stream, cfg) -> dict:
    """The shader clock and MFMA share of the tile kernel's K loop, from clock stamps inside a timeline build of
    the same kernel (dense_tiled_gemm_04_amd/timeline.py), one launch after 60 ms of back-to-back launches of it
    on the same inputs; or a note saying why there is none.  The spec ceilings assume 2.4 GHz."""
    try:
        from dense_tiled_gemm_04_amd import timeline

        ok, why = timeline.available()
        if not ok:
            return {"note": why}
        r = timeline.measure(torch, w.M, w.N, w.K, epi, pA, pB, pb, pC, stream,
                             config=timeline.config_index(cfg["name"]))
        if "note" in r:
            return {"note": r["note"]}
        clk = r["loop_clock_GHz"]
        return {"loop_GHz_median": clk[2], "loop_GHz_min": clk[0], "loop_GHz_max": clk[-1],
                "per_xcd_loop_GHz": [x["loop_clock_GHz"] for x in r["per_xcd"]],
                "loop_mfma_share": r["loop_mfma_share"], "launch_span_us": r["span_us"],
                "source": "s_memtime against s_memrealtime stamps inside a GK_TIMELINE build of the same kernel"}
    except Exception as e:  # a diagnostic: never fails the benchmark
        return {"note": "timeline measurement failed: %s" % e}


def roofline_of(m: dict) -> dict:
    w = m["w"]
    ms = m["ms"]
    tflops = w.flops / (ms * 1e-3) / 1e12
    gbs = w.algorithmic_bytes / (ms * 1e-3) / 1e9
    traffic = load_traffic(w.name + ("_bt" if m["bt"] else ""), m["cfg"]["name"])
    if m["hbm_bound"]:
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_FP16_TFLOPS, "traffic": traffic}
    roof["kernel"] = m["cfg"]["name"]
    roof["algorithmic_flops_per_launch"] = w.flops
    roof["algorithmic_bytes_per_launch"] = w.algorithmic_bytes
    roof["avg_launch_us"] = ms * 1e3
    if "clock" in m:
        roof["sclk"] = m["clock"]
    return roof


def context_line(m: dict) -> dict:
    """Figures of one measured workload for the context object: timed steps, settled rate, roofline fractions."""
    w = m["w"]
    roof = roofline_of(m)
    sus = m["sustained"]
    peak = roof["peak"]
    per = (lambda t: w.algorithmic_bytes / (t * 1e-3) / 1e9) if m["hbm_bound"] else \
        (lambda t: w.flops / (t * 1e-3) / 1e12)
    out = {"status": "ok" if m["finite"] else "fail: non-finite output", "kernel": roof["kernel"],
           "ms_per_step": round(m["ms"], 6), "value": round(roof["achieved"], 3), "unit": roof["unit"],
           "frac": round(roof["frac"], 4), "bound": roof["bound"], "traffic": roof["traffic"],
           "sustained": {"ms_per_launch": round(sus["ms"], 6), "p10_ms": round(sus["p10_ms"], 6),
                         "p90_ms": round(sus["p90_ms"], 6), "value": round(per(sus["ms"]), 3),
                         "frac": round(per(sus["ms"]) / peak, 4), "chunks": sus["chunks"],
                         "launches_per_chunk": sus["launches_per_chunk"]},
           "b_layout": "Bt[N][K]" if m["bt"] else "B[K][N]", "rotated_B_copies": m["rotate"]}
    if "sclk" in roof:
        out["sclk"] = roof["sclk"]
    if m.get("helper_median_ms") is not None:
        out["gemm_f16_time_median_ms"] = round(m["helper_median_ms"], 6)
    if "warm_unrotated_ms" in m:
        t = m["warm_unrotated_ms"]
        out["warm_unrotated"] = {"ms_per_launch": round(t, 6), "GBps": round(per(t), 1),
                                 "note": "one copy of B for every launch, partly served from the Infinity Cache"}
    if "torch_ms" in m:
        out["torch_ms"] = round(m["torch_ms"], 6)
        if m["hbm_bound"]:
            out["torch_GBps"] = round(per(m["torch_ms"]), 1)
        il = m["interleaved"]
        out["interleaved"] = {"ours_ms": round(il[0], 6), "torch_ms": round(il[1], 6),
                              "torch_over_ours": round(il[1] / il[0], 3)}
    return out


# workloads measured beside the headline one, under "context": the metric's fused MLP and the skinny HBM-bound shape
CONTEXT_WORKLOADS = ["mlp_up_8192x16384x4096", "skinny_16x16384x8192"]


def report(g, torch) -> int:
    """The pages' report utility (latency, throughput and error per kernel) as one table over every workload:
    ours and the torch comparator each timed after >= 50 ms of back-to-back launches (median of ~1 ms chunks),
    the rate against the MI355X peak, and the relative Frobenius error of our output against a float32
    reference computed with torch on the GPU (a sanity check like the pages' `check`; parity against the oracle
    is the test suite's).  Prints a Markdown table, then one JSON line with the same rows."""
    import numpy as np
    import torch.nn.functional as F

    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    lib = g.load()

    def ok(st):
        if st != 0:
            raise g.GemmError(st)

    def settled(step):
        step(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(1, 4):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return sustained_ms(torch, stream, step, max(e0.elapsed_time(e1) / 3, 1e-3))["ms"]

    def rel_fro(got, ref):
        d = got.float() - ref
        return float(torch.linalg.vector_norm(d) / torch.linalg.vector_norm(ref))

    rows = []

    def row(name, path, ms, torch_ms, err, flops=None, nbytes=None, comparator=""):
        if flops is not None:
            rate, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
            frac = rate / PEAK_FP16_TFLOPS
        else:
            rate, unit = nbytes / (ms * 1e-3) / 1e9, "GB/s"
            frac = rate / PEAK_HBM_GBS
        rows.append({"workload": name, "path": path, "ours_us": round(ms * 1e3, 2), "rate": round(rate, 1),
                     "unit": unit, "frac_of_peak": round(frac, 4), "torch": comparator,
                     "torch_us": round(torch_ms * 1e3, 2), "torch_over_ours": round(torch_ms / ms, 3),
                     "rel_fro_vs_fp32": float("%.3g" % err)})
        print("report: %s %s done" % (name, path), file=sys.stderr, flush=True)

    for wname, w in workloads.WORKLOADS.items():
        A, B, bias = workloads.make_inputs(w)
        hbm = w.flops / w.algorithmic_bytes < 100.0
        rot = 3 if hbm else 1
        dA = torch.from_numpy(A).to(dev)
        db = torch.from_numpy(bias).to(dev) if bias is not None else None
        for bt in ((False, True) if wname in ("gemm_4096", "mlp_up_8192x16384x4096") else (False,)):
            dBs = [torch.from_numpy(np.ascontiguousarray(B.T) if bt else B).to(dev) for _ in range(rot)]
            out = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
            pBs = [t.data_ptr() for t in dBs]
            pA, pC, pb, epi = dA.data_ptr(), out.data_ptr(), db.data_ptr() if db is not None else None, \
                g.EPILOGUES[w.epilogue]

            def ours(i):  # the C ABI directly, as in the bench lines (the torch binding adds host time per call)
                ok(lib.gemm_f16_bt(w.M, w.N, w.K, pA, w.K, pBs[i % rot], w.K, pb, pC, w.N, epi, sh) if bt else
                   lib.gemm_f16(w.M, w.N, w.K, pA, pBs[i % rot], pb, pC, epi, sh))

            ms = settled(ours)

            def vendor(i):
                y = F.linear(dA, dBs[i % rot]) if bt else torch.matmul(dA, dBs[i % rot])
                if w.epilogue != "none":
                    y = y + db
                if w.epilogue == "bias_gelu":
                    y = F.gelu(y)
                return y

            tms = settled(vendor)
            g.gemm_f16(dA, dBs[0], db, w.epilogue, out=out, b_transposed=bt)
            ref = dA.float() @ (dBs[0].float().t() if bt else dBs[0].float())
            if w.epilogue != "none":
                ref += db.float()
            if w.epilogue == "bias_gelu":
                ref = F.gelu(ref)
            err = rel_fro(out, ref)
            del ref
            cfg = g.config_info(g.select_config(dA, dBs[0], db, w.epilogue, out=out, b_transposed=bt))["name"]
            row(wname + (" (Bt)" if bt else ""), cfg, ms, tms, err,
                flops=None if hbm else w.flops, nbytes=w.algorithmic_bytes if hbm else None,
                comparator=("F.linear" if bt else "matmul") + {"none": "", "bias": " + add",
                                                                "bias_gelu": " + add + gelu"}[w.epilogue])
            del dBs, out
        del dA, db, A, B, bias
    for wname, w in workloads.SOFTMAX_WORKLOADS.items():
        X = workloads.make_softmax_input(w)
        rot = 3 if X.nbytes >= (64 << 20) else 1
        dXs = [torch.from_numpy(X).to(dev) for _ in range(rot)]
        out = torch.empty_like(dXs[0])
        pXs, pY = [t.data_ptr() for t in dXs], out.data_ptr()
        ms = settled(lambda i: ok(g.softmax_rows_raw(w.rows, w.cols, pXs[i % rot], pY, sh)))
        tms = settled(lambda i: torch.softmax(dXs[i % rot], dim=-1))
        g.softmax_f16(dXs[0], out=out)
        err = rel_fro(out, torch.softmax(dXs[0].float(), dim=-1))
        row(wname, "softmax " + g.softmax_path(*X.shape), ms, tms, err, nbytes=w.algorithmic_bytes,
            comparator="torch.softmax")
        del dXs, out, X
    for wname, w in workloads.ATTENTION_WORKLOADS.items():
        Q, K, V = (torch.from_numpy(x).to(dev) for x in workloads.make_attention_inputs(w))
        out = torch.empty_like(Q)
        ptrs = (Q.data_ptr(), K.data_ptr(), V.data_ptr(), out.data_ptr())
        ms = settled(lambda i: ok(g.flash_attn_raw(w.B, w.H, w.Nq, w.Nkv, w.D, *ptrs, w.causal,
                                                   1.0 / math.sqrt(w.D), sh)))
        tms = settled(lambda i: F.scaled_dot_product_attention(Q, K, V, is_causal=w.causal))
        g.flash_attn(Q, K, V, causal=w.causal, out=out)
        # float32 reference, one (batch, head) slab at a time; the transposed operand is made contiguous
        err_num = err_den = 0.0
        for b in range(w.B):
            for h in range(w.H):
                q, k, v = Q[b, h].float(), K[b, h].float(), V[b, h].float()
                sc = (q @ k.t().contiguous()) / math.sqrt(w.D)
                if w.causal:
                    sc = sc.masked_fill(torch.ones_like(sc, dtype=torch.bool).triu(1), float("-inf"))
                ref = torch.softmax(sc, dim=-1) @ v
                err_num += float(torch.linalg.vector_norm(out[b, h].float() - ref) ** 2)
                err_den += float(torch.linalg.vector_norm(ref) ** 2)
        row(wname, "flash_attn_fwd", ms, tms, math.sqrt(err_num / err_den), flops=w.flops,
            comparator="F.scaled_dot_product_attention")
        del Q, K, V, out

    print("| workload | path | ours, us | rate | of peak | torch comparator | torch, us | torch / ours | "
          "rel. Frobenius vs fp32 |")
    print("|---|---|---:|---:|---:|---|---:|---:|---:|")
    for r in rows:
        print("| %s | `%s` | %.2f | %.1f %s | %.3f | %s | %.2f | %.2f | %.2e |" % (
            r["workload"], r["path"], r["ours_us"], r["rate"], r["unit"], r["frac_of_peak"], r["torch"],
            r["torch_us"], r["torch_over_ours"], r["rel_fro_vs_fp32"]))
    print(json.dumps({"report": rows}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gemm_4096")
    ap.add_argument("--config", type=int, default=None, help="force a kernel config index")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="GEMM workloads: skip the other workloads measured under context.workloads")
    ap.add_argument("--rotate", type=int, default=None,
                    help="copies of B to rotate through (default: 3 for HBM-bound workloads, else 1)")
    ap.add_argument("--b-transposed", action="store_true",
                    help="GEMM workloads: B stored transposed, Bt[N][K], through gemm_f16_bt")
    ap.add_argument("--attn-kernel", choices=sorted(ATTN_KERNELS), default="auto",
                    help="attention workloads: force the block-serial or the pipelined kernel (D = 128)")
    ap.add_argument("--hbm-calibration", action="store_true",
                    help="run only the fp32 vector-add kernel on buffers of known size (the reference "
                         "point that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes)")
    ap.add_argument("--mfma-calibration", action="store_true",
                    help="run only the register-only MFMA loop (both MFMA shapes) and the shipped 4096^3 GEMM "
                         "back to back, with board power and clock: the practical MFMA ceiling under the power "
                         "limit")
    ap.add_argument("--report", action="store_true",
                    help="run every workload, ours beside the torch comparator, and print one table of latency, "
                         "rate, fraction of peak and error against a float32 reference (then the rows as JSON)")
    ap.add_argument("--clock-series", action="store_true",
                    help="run only the 4096^3 GEMM and the MLP shape back to back for 80 ms each after idle, and print "
                         "the time per launch of every ~1 ms chunk (how the power controller settles)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the GEMM runs on a single MI355X and the library has no "
              "multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch

    import dense_tiled_gemm_04_amd as g
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    g.load()
    if args.hbm_calibration:
        return hbm_calibration(g, torch)
    if args.mfma_calibration:
        return mfma_calibration(g, torch)
    if args.clock_series:
        return clock_series(g, torch)
    if args.report:
        return report(g, torch)
    if args.workload in workloads.SOFTMAX_WORKLOADS:
        return bench_softmax(args, g, torch, workloads.SOFTMAX_WORKLOADS[args.workload])
    if args.workload in workloads.ATTENTION_WORKLOADS:
        return bench_attention(args, g, torch, workloads.ATTENTION_WORKLOADS[args.workload])
    w = workloads.WORKLOADS[args.workload]
    A, B, bias, digest = gemm_workload_inputs(w)
    bt = args.b_transposed
    m = measure_gemm(g, torch, w, A, B, bias, args.steps, args.warmup, bt=bt, rotate=args.rotate,
                     config=args.config)
    if not m["finite"]:
        print("bench.py: non-finite values in C for %s" % w.name, file=sys.stderr)
        return 1
    ms = m["ms"]
    roof = roofline_of(m)
    tflops = w.flops / (ms * 1e-3) / 1e12
    gbs = w.algorithmic_bytes / (ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, A, B, bias)
    del A, B, bias

    head = context_line(m)
    context = {
        "regime": ("the %d timed launches follow %d untimed ones (the %d requested, extended to >= %.0f ms of "
                   "back-to-back work, %.1f ms here): after idle the power controller boosts, throttles and settles "
                   "within ~40 ms, so this is the settled rate; context.sustained is the same over >= 25 ms (median "
                   "of ~1 ms chunks)"
                   % (args.steps, m["warmup_launches"], args.warmup, WARMUP_MS, m["warmup_ms"])),
        "warmup_launches": m["warmup_launches"],
        "sustained": head["sustained"],
        "algorithmic_GBps": round(gbs, 1),
        "input_sha256": {w.name: digest},
        "status": {w.name + ("_bt" if bt else ""): head["status"]},
    }
    if "gemm_f16_time_median_ms" in head:
        context["gemm_f16_time_median_ms"] = head["gemm_f16_time_median_ms"]
    if "warm_unrotated" in head:
        context["warm_unrotated"] = head["warm_unrotated"]
    if "torch_GBps" in head:
        context["torch_GBps"] = head["torch_GBps"]
    context[("torch_linear_ms" if bt else "torch_matmul_ms")] = head.get("torch_ms")
    if "torch_ms" in m:
        context["torch_tflops"] = round(w.flops / (m["torch_ms"] * 1e-3) / 1e12, 3)
        context["interleaved"] = head["interleaved"]
    if not args.no_context and args.config is None:
        # the other headline workloads on the same clock, each in its own try (a failure is recorded, not fatal)
        context["workloads"] = {}
        for name in CONTEXT_WORKLOADS:
            if name == w.name:
                continue
            key = name + ("_bt" if bt else "")
            try:
                wc = workloads.WORKLOADS[name]
                Ac, Bc, bc, dg = gemm_workload_inputs(wc)
                context["input_sha256"][name] = dg
                mc = measure_gemm(g, torch, wc, Ac, Bc, bc, args.steps, args.warmup, bt=bt)
                del Ac, Bc, bc
                line = context_line(mc)
                context["workloads"][key] = line
                context["status"][key] = line["status"]
            except Exception as e:  # keep going, like the pages' section runner
                context["status"][key] = "fail: %s" % str(e).splitlines()[0][:200]

    out = {
        "metric": "fp16 GEMM TFLOPS (4096\u00b3; fused bias+GELU MLP) + % of MI355X MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "epilogue": w.epilogue,
                   "b_layout": "Bt[N][K]" if bt else "B[K][N]",
                   "inputs": "seeded numpy draws (%s), B copies rotated: %d" % (w.note, m["rotate"])},
        "roofline": roof,
        "cpu_baseline": cpu,
        "context": context,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
