#!/usr/bin/env python3
"""Benchmark of C = A * B^T (fp16 in, fp32 accumulate/out) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8192^3] [--dtype f16|bf16]
                    [--inputs uniform|hash_int|integer] [--no-cpu-baseline] [--no-extras]
                    [--sweeps S] [--page-shapes] [--shard-shapes] [--vendor]
                    [--calibrate-copy]

A step is one call of gemm_f16_f32_abt through the C ABI on synthetic
operands already resident in HBM (uniform [-1, 1] fp16, seeds 1 and 2). The
timed region is --steps back-to-back calls bracketed by device
synchronisation; `value` is 2*M*N*K * steps / elapsed in TFLOP/s. Each call is also bracketed by HIP
events on the launch stream: their mean, median and minimum are the kernel's
launch durations, from which `roofline.achieved` is computed against the fp16
MFMA peak (2.5 PFLOP/s dense).

Clock: the library's clock probe (gemm_f16_set_clock_probe) is on during the
timed calls: the first wave of workgroup 0 of every main-kernel launch adds
its shader-clock cycles and 100 MHz real-time ticks to two counters, so
`roofline.sclk_mhz` is the average shader clock while the timed kernels ran
and `roofline.frac_at_sclk` the fraction of the peak at that clock. The
board's own telemetry (amdsmi gpu_metrics: gfx clocks, socket power, time at
the package power limit) updates too slowly for a window of a few
milliseconds, so `sustained` runs the headline call back to back for about two
seconds after everything else and reports the probe clock, the per-call time
and the board's power and power-limit residency over that loop. The probe's
workgroup 0 runs on one XCD; the board reports each XCD's clock, and they
differ by several percent at the power limit. Every CU of the headline's plan
has the same work, so the XCD with the slowest clock finishes last:
`sustained.frac_at_slowest_xcd_clk` is the fraction of the peak at that
XCD's mean clock over the window.

`configs` (unless --no-extras; measured before the headline, so that the
headline's warm-up starts on a running GPU rather than an idle one, unless
--headline-first): the five workloads the way "SASS-Level Kernel
Generation for Blackwell" measures (section "How we measured"): every call
runs alone and the time of a call is its GPU time; the median over the last N
calls is reported, over four sweeps run in forward, reverse, forward and
reverse order, as the pages interleave their runs. A short
spin kernel is queued ahead of each timed call so that the call's events and
kernels reach the GPU together: the events then bracket the call's kernels
(and the gaps between them), not the host's launch latency. Beside it, the
same calls back to back (one pair of events around N calls) and the host time
to issue one call through the Python binding. Each config carries its own
roofline: MFMA for the compute-bound shapes, HBM for those below the ridge.
`pages_inputs`: the headline shape on the input kind the pages time on
(integers in [-3, 3] from a hash), which draws less power on this board.

`cpu_baseline` times the CPU reference (oracle/) on a bounded sample of the
same workload: whole rows of C, sized from a first timing to about 25 s (in
practice 10-20 s) on the host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("TFLOP/s and µs/call per M×N×K (fp16→fp32 A·Bᵀ); "
          "% of MI355X MFMA peak")
PEAK_TFLOPS = 2500.0         # MI355X dense fp16 MFMA (published)
PEAK_SCLK_MHZ = 2400.0       # the clock the published peak assumes
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E (published)
# The pages' own numbers (one B200, "SASS-Level Kernel Generation for Blackwell",
# section "The numbers"): midpoints of the ranges, in us per call. Context only.
PAGE_US = {"8192^3": (553.1 + 554.3) / 2, "1024^3": (4.64 + 4.67) / 2,
           "2048x2048x16384": (73.92 + 74.11) / 2, "1024x1024x65536": (76.93 + 77.22) / 2,
           "1536^3": 7.87, "2048^3": 14.46, "3072x1280x2048": 14.08, "4096x4096x1024": 26.11,
           "4096^3": (75.78 + 75.97) / 2, "8192x2048x4096": (75.84 + 75.97) / 2,
           "16384^3": (4132.8 + 4239.4) / 2}
# Timed calls per shape, as the pages time them ("How we measured").
CALLS = {"256^3": 400, "1024^3": 400, "2048x2048x16384": 200, "1024x1024x65536": 200,
         "8192^3": 40, "1536^3": 400, "2048^3": 400, "3072x1280x2048": 400,
         "4096x4096x1024": 300, "4096^3": 200, "8192x2048x4096": 200, "16384^3": 12,
         # one GPU's share of a workload split over 8 GPUs (not timed on the pages)
         "8192^3 M/8": 200, "2048x2048x16384 K/8": 400, "1024x1024x65536 K/8": 400}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_fp16_gemm_03_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def algorithmic(M, N, K):
    flops = 2.0 * M * N * K
    nbytes = 2.0 * (M * K + N * K) + 4.0 * M * N
    return flops, nbytes


def roofline_time(M, N, K):
    """(seconds at the roofline, bound) for one call of the shape."""
    f, b = algorithmic(M, N, K)
    t_mfma = f / (PEAK_TFLOPS * 1e12)
    t_hbm = b / (HBM_PEAK_GBS * 1e9)
    return (t_mfma, "mfma") if t_mfma >= t_hbm else (t_hbm, "hbm")


def make_device_operands(torch, shape, dev, dtype="f16", kind="uniform"):
    """Host operands (float16, or uint16 bfloat16 bits) and their device copies."""
    from dense_fp16_gemm_03_amd import inputs

    A, B = inputs.workload_operands(shape, kind, dtype)
    if dtype == "bf16":
        def dev_t(x):
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        def dev_t(x):
            return torch.from_numpy(x).to(dev)
    return A, B, dev_t(A), dev_t(B)


class ClockSampler:
    """Board telemetry sampled by a thread through amdsmi (in-process, no
    child): per-XCD gfx clocks, socket power, and the accumulated time at
    the package power limit (PPT) and energy. `window(t0, t1)` summarises
    the samples taken between two perf_counter() instants. Optional: if
    amdsmi is unavailable, every summary is None."""

    def __init__(self):
        self.samples = []  # (t, [gfx MHz per XCD], socket W, ppt_acc, acc_counter, energy)
        self.ok = False
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()  # one read to see that it works
            self.samples.clear()
            self.ok = True
        except Exception as e:  # noqa: BLE001 - telemetry is optional context
            log(f"[bench] no telemetry: {type(e).__name__}: {e}")

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, int) and 0 < c < 10000]

        def num(key):
            v = m.get(key)
            return v if isinstance(v, (int, float)) else None

        self.samples.append((time.perf_counter(), clks, num("current_socket_power"),
                             num("ppt_residency_acc"), num("accumulation_counter"),
                             num("energy_accumulator")))

    def _loop(self):
        while not self._stop.is_set():
            try:
                self._read()
            except Exception:  # noqa: BLE001
                return
            time.sleep(0.0005)

    def start(self):
        if self.ok and self._thread is None:
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join(timeout=5)
            self._thread = None

    def window(self, t0, t1):
        """Summary of the samples taken in [t0, t1] (None if there are none)."""
        inside = [s for s in self.samples if t0 <= s[0] <= t1 and s[1]]
        if not inside:
            return None
        per_xcd = np.array([s[1] for s in inside if len(s[1]) == len(inside[0][1])], float)
        out = {"samples": len(inside),
               "gfx_clk_mhz_mean": round(float(per_xcd.mean()), 1),
               "gfx_clk_mhz_per_xcd": [round(float(v), 1) for v in per_xcd.mean(axis=0)],
               "gfx_clk_mhz_min": round(float(per_xcd.min()), 1),
               "gfx_clk_mhz_max": round(float(per_xcd.max()), 1)}
        pw = [s[2] for s in inside if s[2] is not None]
        if pw:
            out["socket_power_w_mean"] = round(float(np.mean(pw)), 1)
            out["socket_power_w_max"] = float(max(pw))
        # time at the power limit: residency counter over the accumulation
        # counter, between the first and last sample of the window
        a, b = inside[0], inside[-1]
        if None not in (a[3], b[3], a[4], b[4]) and b[4] > a[4]:
            out["ppt_limited_frac"] = round((b[3] - a[3]) / (b[4] - a[4]), 3)
        out["source"] = "amdsmi gpu_metrics, sampled in-process during the calls"
        return out


class Probe:
    """The library's clock probe over a region of calls: counters on the
    device, zeroed in stream order before the region, read after it."""

    def __init__(self, torch, gemm, dev):
        self.torch, self.gemm = torch, gemm
        self.ctr = torch.zeros(2, dtype=torch.int64, device=dev)

    def __enter__(self):
        self.ctr.zero_()
        self.gemm.gemm_f16_set_clock_probe(self.ctr.data_ptr())
        return self

    def __exit__(self, *exc):
        self.gemm.gemm_f16_set_clock_probe(0)

    def mhz(self):
        """Average shader clock (MHz) of the probed launches (after a sync)."""
        self.torch.cuda.synchronize()
        cycles, ticks = (int(v) for v in self.ctr.tolist())
        return round(100.0 * cycles / ticks, 1) if ticks > 0 else None


def time_headline(torch, gemm, At, Bt, C, steps, warmup, probe):
    """Warm-up, then `steps` back-to-back calls bracketed by synchronisation,
    each also between HIP events on the launch stream; the clock probe is on
    for the timed calls only."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        gemm.gemm_abt(At, Bt, C, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    with probe:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s, e in ev:
            s.record(stream)
            gemm.gemm_abt(At, Bt, C, stream=stream)
            e.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    kernel_us = [s.elapsed_time(e) * 1e3 for s, e in ev]
    return t1 - t0, kernel_us, probe.mhz()


def sustained(torch, gemm, At, Bt, C, flops, probe, sampler, seconds=2.0):
    """The headline call back to back for about `seconds`: probe clock and
    per-call time over the whole loop, board telemetry (amdsmi) over its
    second half."""
    stream = torch.cuda.current_stream()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    calls = 0
    sampler.start()
    with probe:
        torch.cuda.synchronize()
        s.record(stream)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                gemm.gemm_abt(At, Bt, C, stream=stream)
            calls += 8
            torch.cuda.synchronize()
        e.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    sampler.stop()
    us = s.elapsed_time(e) * 1e3 / calls
    mhz = probe.mhz()
    out = {"calls": calls, "us_per_call": round(us, 3),
           "tflops": round(flops / (us * 1e-6) / 1e12, 2), "sclk_mhz": mhz,
           "board": sampler.window(t0 + (t1 - t0) / 2, t1)}
    if mhz:
        out["frac_at_sclk"] = frac_at_clock(flops, us, mhz)
    per_xcd = (out["board"] or {}).get("gfx_clk_mhz_per_xcd")
    if per_xcd:
        out["frac_at_slowest_xcd_clk"] = frac_at_clock(flops, us, min(per_xcd))
    return out


def frac_at_clock(flops, us, mhz):
    """Fraction of the MFMA peak at shader clock `mhz` reached by `flops`
    in `us` microseconds (the peak scales with the clock)."""
    return round(flops / (us * 1e-6) / 1e12 / (PEAK_TFLOPS * mhz / PEAK_SCLK_MHZ), 4)


class Spinner:
    """A spin kernel of a calibrated length (about `us` microseconds), queued
    ahead of a call timed alone so that the call's start event, kernels and
    end event are all in the queue before the GPU reaches them."""

    def __init__(self, torch, us=150.0):
        self.torch = torch
        self.cycles = 0
        self.us = None
        stream = torch.cuda.current_stream()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def took(cycles):
            torch.cuda._sleep(cycles)
            s.record(stream)
            torch.cuda._sleep(cycles)
            e.record(stream)
            e.synchronize()
            return s.elapsed_time(e) * 1e3

        cycles = 20000
        for _ in range(4):
            t = took(cycles)
            if t < 1.0:  # no measurable spin: grow by a bounded step
                cycles *= 10
            else:
                cycles = int(cycles * min(max(us / t, 0.1), 10.0))
            cycles = min(cycles, 50_000_000)
        t = took(cycles)
        if us / 3 <= t <= us * 3:
            self.cycles, self.us = cycles, round(t, 1)
        else:
            log(f"[bench] spin kernel not calibrated ({cycles} cycles took {t:.1f} us): "
                "calls alone are timed without it (their times include the launch latency)")

    def __call__(self):
        if self.cycles:
            self.torch.cuda._sleep(self.cycles)


def time_calls_alone(torch, fn, calls, warmup, spinner):
    """GPU time (us) of each of `calls` calls of fn(), every call alone."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    for _ in range(calls):
        spinner()
        s.record(stream)
        fn()
        e.record(stream)
        e.synchronize()
        out.append(s.elapsed_time(e) * 1e3)
    return out


def time_back_to_back(torch, fn, calls, warmup):
    """(GPU us per call over `calls` back-to-back calls between one pair of
    events, host us to issue one call)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record(stream)
    h0 = time.perf_counter()
    for _ in range(calls):
        fn()
    h1 = time.perf_counter()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) * 1e3 / calls, (h1 - h0) * 1e6 / calls


def measure_configs(torch, gemm, table, dev, dtype, sweeps, spinner, cache, probe):
    """Per-config lines: calls alone (median, min, max over sweeps, and the
    probe clock over them), back to back, host issue time, roofline
    fraction."""
    names = list(table)
    alone = {n: [] for n in names}
    clocks = {n: [] for n in names}
    for sweep in range(sweeps):
        order = names if sweep % 2 == 0 else names[::-1]
        for n in order:
            m, nn, k = table[n]
            if n not in cache:
                _, _, a, b = make_device_operands(torch, (m, nn, k), dev, dtype)
                c = torch.empty((m, nn), dtype=torch.float32, device=dev)
                cache[n] = (a, b, c)
            a, b, c = cache[n]
            for _ in range(20):
                gemm.gemm_abt(a, b, c)
            with probe:
                us = time_calls_alone(torch, lambda: gemm.gemm_abt(a, b, c), CALLS[n], 0,
                                      spinner)
            clocks[n].append(probe.mhz())
            alone[n].append(us)
            log(f"[bench] sweep {sweep} {n}: median {float(np.median(us)):.2f} us/call alone")
    out = []
    for n in names:
        m, nn, k = table[n]
        a, b, c = cache[n]
        b2b_us, host_us = time_back_to_back(torch, lambda: gemm.gemm_abt(a, b, c),
                                            CALLS[n], 50)
        f, by = algorithmic(m, nn, k)
        t_roof, bound = roofline_time(m, nn, k)
        meds = [float(np.median(x)) for x in alone[n]]
        allv = np.concatenate([np.asarray(x) for x in alone[n]])
        med = float(np.median(meds))
        entry = {"workload": n, "M": m, "N": nn, "K": k,
                 "us_per_call_alone": {"median": round(med, 3),
                                       "sweep_medians": [round(v, 3) for v in meds],
                                       "min": round(float(allv.min()), 3),
                                       "max": round(float(allv.max()), 3),
                                       "calls_per_sweep": CALLS[n], "sweeps": len(meds)},
                 "us_per_call_back_to_back": round(b2b_us, 3),
                 "host_us_per_call": round(host_us, 2),
                 "tflops": round(f / (med * 1e-6) / 1e12, 2),
                 "roofline": {"bound": bound, "t_roof_us": round(t_roof * 1e6, 3),
                              "frac": round(t_roof / (med * 1e-6), 4)},
                 "mfma_peak_frac": round(f / (med * 1e-6) / 1e12 / PEAK_TFLOPS, 4),
                 "plan": gemm.gemm_f16_f32_abt_describe(m, nn, k)}
        mhz = [c for c in clocks[n] if c]
        if mhz:
            entry["sclk_mhz"] = round(float(np.mean(mhz)), 1)
            if bound == "mfma":
                entry["frac_at_sclk"] = round(entry["mfma_peak_frac"] * PEAK_SCLK_MHZ
                                              / entry["sclk_mhz"], 4)
        if n in PAGE_US and dtype == "f16":
            entry["pages_b200_us"] = round(PAGE_US[n], 3)
        log(f"[bench] {n}: alone {med:.2f} us ({entry['roofline']['frac'] * 100:.1f}% of its "
            f"{bound} roofline), back to back {b2b_us:.2f} us, host {host_us:.2f} us/call")
        out.append(entry)
    return out


def cpu_baseline(A, B, M, N, K, budget_s=25.0):
    import oracle

    ref = oracle.gemm_abt_bf16 if A.dtype == np.uint16 else oracle.gemm_abt

    threads = oracle.default_threads()
    rows = max(1, threads)
    t0 = time.perf_counter()
    ref(A[:rows], B, threads=threads)
    t = time.perf_counter() - t0
    est = t / rows
    rows2 = int(min(M, max(rows, budget_s / max(est, 1e-9))))
    t0 = time.perf_counter()
    ref(A[:rows2], B, threads=threads)
    t = time.perf_counter() - t0
    flops = 2.0 * rows2 * N * K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{rows2 - 1} of C ({rows2}x{N}x{K}), {t:.1f} s, "
                      f"binary64 triple loop on {threads} threads"}


def _median_alone(torch, fn, calls, spinner, warmup=5):
    return float(np.median(time_calls_alone(torch, fn, calls, warmup, spinner)))


def load_vendor():
    import ctypes

    from dense_fp16_gemm_03_amd import build as b

    if not os.path.exists(b.VENDOR_LIBRARY):
        raise RuntimeError(f"{b.VENDOR_LIBRARY} is not built "
                           "(python -m dense_fp16_gemm_03_amd.build --vendor)")
    lib = ctypes.CDLL(b.VENDOR_LIBRARY)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.vendor_hipblaslt_prepare.argtypes = [i64] * 7
    lib.vendor_hipblaslt_prepare.restype = i64
    lib.vendor_hipblaslt_workspace.argtypes = [i64]
    lib.vendor_hipblaslt_workspace.restype = ctypes.c_size_t
    lib.vendor_hipblaslt_run.argtypes = [i64, p, p, p, p, ctypes.c_size_t, p]
    lib.vendor_hipblaslt_run.restype = ctypes.c_int
    return lib


def vendor_screen(torch, lib, A, B, C_ref, max_algorithms=64):
    """Runs every algorithm hipBLASLt's heuristic returns for C = A B^T (fp16
    in, fp32 out) on the device operands A, B and returns (count, workspace,
    exact): the indices whose C equals C_ref bit for bit. On integer-valued
    inputs, where every summation order gives the exact C, C_ref is this
    library's result, whose exactness on such inputs the GPU tests prove
    against the CPU reference (and the vendor test checks this screen
    against it directly)."""
    M, K = A.shape
    N = B.shape[0]
    count = lib.vendor_hipblaslt_prepare(M, N, K, K, K, N, max_algorithms)
    if count <= 0:
        return int(count), None, []
    ws_bytes = max(lib.vendor_hipblaslt_workspace(i) for i in range(count))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=A.device)
    stream = torch.cuda.current_stream().cuda_stream
    Cv = torch.empty((M, N), dtype=torch.float32, device=A.device)
    exact = []
    for i in range(count):
        Cv.fill_(float("nan"))
        st = lib.vendor_hipblaslt_run(i, A.data_ptr(), B.data_ptr(), Cv.data_ptr(),
                                      ws.data_ptr(), ws.numel(), stream)
        torch.cuda.synchronize()
        if st == 0 and torch.equal(Cv, C_ref):
            exact.append(i)
    return int(count), ws, exact


def vendor_arm(torch, gemm, names, dev, spinner):
    """hipBLASLt context arm ("How we measured" in "SASS-Level Kernel
    Generation for Blackwell"): every algorithm of the vendor heuristic is run
    on hash-integer inputs, where any summation order is exact, and kept only
    if its C is exact (vendor_screen); the fastest kept one is then timed
    against ours, calls alone, in the order ours, vendor, vendor, ours, on
    both uniform and hash-integer inputs. Context only, never the bench value."""
    from dense_fp16_gemm_03_amd import inputs

    lib = load_vendor()
    out = []
    for n in names:
        M, N, K = inputs.WORKLOADS[n]
        Ah, Bh = (torch.from_numpy(x).to(dev) for x in inputs.workload_operands((M, N, K),
                                                                                 "hash_int"))
        Ch = torch.empty((M, N), dtype=torch.float32, device=dev)
        gemm.gemm_abt(Ah, Bh, Ch)
        torch.cuda.synchronize()
        count, ws, exact = vendor_screen(torch, lib, Ah, Bh, Ch)
        if not exact:
            log(f"[vendor] {n}: {count} algorithms, none exact")
            out.append({"workload": n, "algorithms": count, "exact": 0})
            continue
        stream = torch.cuda.current_stream().cuda_stream
        Cv = torch.empty_like(Ch)

        def run_vendor(i, A_, B_):
            st = lib.vendor_hipblaslt_run(i, A_.data_ptr(), B_.data_ptr(), Cv.data_ptr(),
                                          ws.data_ptr(), ws.numel(), stream)
            if st != 0:
                raise RuntimeError(f"hipBLASLt algorithm {i} failed with status {st}")

        screen_calls = 10 if M * N * K >= 1 << 36 else 50
        times = [(_median_alone(torch, lambda: run_vendor(i, Ah, Bh), screen_calls, spinner), i)
                 for i in exact]
        best = min(times)[1]
        entry = {"workload": n, "M": M, "N": N, "K": K, "algorithms": count,
                 "exact": len(exact), "best_algorithm": best}
        for kind, (A_, B_) in (("uniform", make_device_operands(torch, (M, N, K), dev)[2:]),
                               ("hash_int", (Ah, Bh))):
            ours, theirs = [], []
            for who in ("ours", "vendor", "vendor", "ours"):
                if who == "ours":
                    ours.append(_median_alone(torch, lambda: gemm.gemm_abt(A_, B_, Ch),
                                              CALLS[n], spinner))
                else:
                    theirs.append(_median_alone(torch, lambda: run_vendor(best, A_, B_),
                                                CALLS[n], spinner))
            entry[kind] = {"ours_us": [round(min(ours), 3), round(max(ours), 3)],
                           "hipblaslt_us": [round(min(theirs), 3), round(max(theirs), 3)]}
            log(f"[vendor] {n} {kind}: ours {min(ours):.2f}-{max(ours):.2f} us, hipBLASLt "
                f"{min(theirs):.2f}-{max(theirs):.2f} us (algorithm {best} of {count}, "
                f"{len(exact)} exact)")
        out.append(entry)
        del Ah, Bh, Ch, Cv, ws
        torch.cuda.empty_cache()
    return out


def calibrate_copy(torch):
    """A plain copy of known size for scaling the HBM byte counters:
    1 GiB fp32 read + 1 GiB written per launch (torch's elementwise kernel)."""
    n = (1 << 30) // 4
    x = torch.rand(n, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(5):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                      "launches": 5}), flush=True)


def library_md5() -> str:
    from dense_fp16_gemm_03_amd import gemm

    with open(gemm.LIBRARY, "rb") as f:
        return hashlib.md5(f.read()).hexdigest()


def parse_shape(text):
    """(M, N, K) from 'MxNxK' with positive integers, else None."""
    parts = text.split("x")
    if len(parts) != 3 or not all(p.isdigit() and int(p) > 0 for p in parts):
        return None
    return tuple(int(p) for p in parts)


def traffic_for(workload):
    """HBM bytes per launch from committed rocprofv3 counters, if they match this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("source_hash") != source_hash():
        return None
    return entry.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--dtype", default="f16", choices=("f16", "bf16"),
                    help="operand type: binary16 (the workloads' type) or bfloat16")
    ap.add_argument("--inputs", default="uniform", choices=("uniform", "hash_int", "integer"),
                    help="input kind of the headline calls (the workloads are quoted on "
                         "uniform; the others are controls for the data-dependent clock)")
    ap.add_argument("--workload", default="8192^3",
                    help="one of the five workloads, one of the pages' other shapes, "
                         "or any MxNxK")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline calls (no configs table, no hash-integer "
                         "row); profiling runs use this so their traces hold one shape and "
                         "one input kind")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="skip the sustained loop with the board's telemetry")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB fp32 copy kernel (counter calibration)")
    ap.add_argument("--sweeps", type=int, default=4,
                    help="sweeps over the configs, alternately forward and reverse (the "
                         "pages' fwd, rev, fwd, rev)")
    ap.add_argument("--headline-first", action="store_true",
                    help="time the headline before the per-workload table (by default the "
                         "table runs first)")
    ap.add_argument("--page-shapes", action="store_true",
                    help="also time the other shapes of the pages' table in `configs`")
    ap.add_argument("--shard-shapes", action="store_true",
                    help="also time one GPU's share of each large workload split over 8 "
                         "GPUs (M/8 for 8192^3, K/8 for the long-K shapes) in `configs`")
    ap.add_argument("--vendor", action="store_true",
                    help="also time hipBLASLt's fastest exact algorithm on every workload "
                         "(context only)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from dense_fp16_gemm_03_amd import gemm, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    gemm.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    name = args.workload
    all_shapes = {**inputs.WORKLOADS, **inputs.PAGE_SHAPES, **inputs.SHARD_SHAPES}
    shape = all_shapes.get(name) or parse_shape(name)
    if shape is None:
        print(f"unknown workload {name!r}; known: {', '.join(all_shapes)}, or MxNxK",
              file=sys.stderr)
        sys.exit(2)
    M, N, K = shape
    flops, nbytes = algorithmic(M, N, K)
    log(f"[bench] workload {name}: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    A, B, At, Bt = make_device_operands(torch, (M, N, K), dev, args.dtype, args.inputs)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)

    probe = Probe(torch, gemm, dev)

    def run_configs():
        spinner = Spinner(torch)
        table = dict(inputs.WORKLOADS)
        if args.page_shapes:
            table.update(inputs.PAGE_SHAPES)
        if args.shard_shapes:
            table.update(inputs.SHARD_SHAPES)
        cache = {}
        if name in table and args.inputs == "uniform":
            cache[name] = (At, Bt, C)
        t0 = time.perf_counter()
        out = measure_configs(torch, gemm, table, dev, args.dtype, args.sweeps, spinner, cache,
                              probe)
        t1 = time.perf_counter()
        del cache
        torch.cuda.empty_cache()
        log(f"[bench] configs measured in {t1 - t0:.1f} s (spin ahead of each call alone: "
            f"{spinner.us} us)")
        return out

    # The per-workload table (the pages' method) runs before the headline
    # unless --headline-first: the headline's warm-up calls then start on a
    # GPU that has been running rather than idle (its clock right after idle
    # dips for the first tens of milliseconds of full load; the probe clock
    # of the timed calls is reported either way).
    configs, pages_inputs = [], None
    if not args.no_extras and not args.headline_first:
        configs = run_configs()
    elapsed, kernel_us, sclk = time_headline(torch, gemm, At, Bt, C, args.steps, args.warmup,
                                             probe)
    ms_per_step = elapsed / args.steps * 1e3
    value = flops * args.steps / elapsed / 1e12
    k_mean = float(np.mean(kernel_us))
    k_med = float(np.median(kernel_us))
    k_min = float(np.min(kernel_us))
    achieved = flops / (k_mean * 1e-6) / 1e12
    log(f"[bench] {args.steps} steps in {elapsed * 1e3:.2f} ms: {value:.1f} TFLOP/s; "
        f"kernel mean {k_mean:.2f} us, median {k_med:.2f}, min {k_min:.2f} "
        f"({achieved:.1f} TFLOP/s)")
    # committed counters are for the binary16 path on uniform inputs
    traffic = traffic_for(name) if (args.dtype == "f16" and args.inputs == "uniform") else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel_us": {"mean": round(k_mean, 3), "median": round(k_med, 3),
                              "min": round(k_min, 3), "calls": len(kernel_us)},
                "algorithmic_bytes": nbytes, "algorithmic_flops": flops}
    if sclk:
        roofline["sclk_mhz"] = sclk
        roofline["sclk_source"] = "clock probe over the timed launches (workgroup 0)"
        roofline["peak_at_sclk"] = round(PEAK_TFLOPS * sclk / PEAK_SCLK_MHZ, 1)
        roofline["frac_at_sclk"] = round(achieved / (PEAK_TFLOPS * sclk / PEAK_SCLK_MHZ), 4)
        log(f"[bench] shader clock during the timed calls: {sclk} MHz "
            f"({roofline['frac_at_sclk'] * 100:.1f}% of the peak at that clock)")

    if not args.no_extras:
        if args.headline_first:
            configs = run_configs()
        # The same workload on the input kind the pages time on (integers in
        # [-3, 3] from a hash of the index): context for the data-dependent
        # power draw, never the value.
        if args.dtype == "f16" and args.inputs == "uniform":
            a = torch.from_numpy(inputs.hash_int(M, K, 1)).to(dev)
            b = torch.from_numpy(inputs.hash_int(N, K, 2)).to(dev)
            el, kus, sclk_h = time_headline(torch, gemm, a, b, C, args.steps, args.warmup,
                                            probe)
            avg_us = float(np.mean(kus))
            pages_inputs = {"workload": name, "inputs": "hash_int [-3, 3]",
                            "kernel_us_mean": round(avg_us, 3),
                            "kernel_us_median": round(float(np.median(kus)), 3),
                            "tflops": round(flops / (avg_us * 1e-6) / 1e12, 2),
                            "mfma_peak_frac": round(flops / (avg_us * 1e-6) / 1e12
                                                    / PEAK_TFLOPS, 4),
                            "calls": args.steps, "sclk_mhz": sclk_h}
            if sclk_h:
                pages_inputs["frac_at_sclk"] = round(pages_inputs["mfma_peak_frac"]
                                                     * PEAK_SCLK_MHZ / sclk_h, 4)
            log(f"[bench] {name} on hash-integer inputs: {avg_us:.2f} us/call "
                f"({pages_inputs['mfma_peak_frac'] * 100:.1f}% of peak) at {sclk_h} MHz")
            del a, b
            torch.cuda.empty_cache()
    sus = None
    if not args.no_telemetry:
        sampler = ClockSampler()
        sus = sustained(torch, gemm, At, Bt, C, flops, probe, sampler)
        log(f"[bench] sustained: {sus}")

    vendor = None
    if args.vendor:
        vendor = vendor_arm(torch, gemm, list(inputs.WORKLOADS), dev, Spinner(torch))

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU reference on a sample ...")
        cpu = cpu_baseline(A, B, M, N, K)
        log(f"[bench] cpu: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")

    vs = None
    if name in PAGE_US and args.dtype == "f16" and args.inputs == "uniform":
        vs = round(value / (flops / (PAGE_US[name] * 1e-6) / 1e12), 4)  # pages: binary16
    data = {"uniform": f"synthetic: uniform[-1,1] {args.dtype}, seeds 1 (A) and 2 (B), "
                       "resident in HBM",
            "hash_int": "synthetic: integers in [-3,3] from a hash of the index (the pages' "
                        "input kind), resident in HBM",
            "integer": f"synthetic: integers in {{-2..2}} {args.dtype}, seeds 3 (A) and 4 (B), "
                       "resident in HBM"}[args.inputs]
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": vs, "dtype": args.dtype,
        "data": data,
        "config": {"workload": f"gemm_abt {M}x{N}x{K}", "M": M, "N": N, "K": K,
                   "accumulate": "f32", "output": "f32",
                   "plan": gemm.gemm_f16_f32_abt_describe(M, N, K),
                   "source_hash": source_hash(), "library_md5": library_md5()},
        "roofline": roofline, "cpu_baseline": cpu, "configs": configs,
        "pages_inputs": pages_inputs, "sustained": sus,
    }
    if vendor is not None:
        line["vendor_hipblaslt"] = vendor
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
