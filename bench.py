#!/usr/bin/env python3
"""Benchmark of C = A * B^T (fp16 in, fp32 accumulate/out) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8192^3] [--dtype f16|bf16]
                    [--no-cpu-baseline] [--no-extras] [--shapes] [--vendor] [--calibrate-copy]

A step is one call of gemm_f16_f32_abt through the C ABI on synthetic
operands already resident in HBM (uniform [-1, 1] fp16, seeds 1 and 2). The
timed region is K back-to-back calls bracketed by device synchronisation;
`value` is 2*M*N*K*K / elapsed in TFLOP/s. Each call is also bracketed by HIP
events on the launch stream: their mean is the kernel's average launch
duration, from which `roofline.achieved` is computed against the fp16 MFMA
peak (2.5 PFLOP/s dense).

At 8192^3 the line also carries `long_k`: the two long-K workloads, 200
back-to-back calls after 100 untimed ones, between one pair of HIP events
(their main and reduce kernels and the gaps between calls), as fractions of
peak beside the headline; and `pages_inputs`: 8192^3 again on the input kind
the pages time on (integers in [-3, 3] from a hash), which draws less power
on this board. `--no-extras` leaves both out. The default 30
warm-up calls of the headline, and the 100 here, let the board's clocks
settle: the first 20 or so calls of a new shape run several percent slower.

With --shapes, per-shape lines (`shapes`) time the five workloads the way "SASS-Level Kernel
Generation for Blackwell" measures (section "How we measured"): every call
runs alone (synchronised after each), the time of a call is its GPU time, and
the median over the last N calls is reported, over sweeps run in forward then
reverse order.

`cpu_baseline` times the CPU reference (oracle/) on a bounded sample of the
same workload: whole rows of C, sized from a first timing to about 25 s (in
practice 10-20 s) on the host's
cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("TFLOP/s and µs/call per M×N×K (fp16→fp32 A·Bᵀ); "
          "% of MI355X MFMA peak")
PEAK_TFLOPS = 2500.0         # MI355X dense fp16 MFMA (published)
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
         "4096x4096x1024": 300, "4096^3": 200, "8192x2048x4096": 200, "16384^3": 12}
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


def make_device_operands(torch, shape, dev, dtype="f16"):
    """Host operands (float16, or uint16 bfloat16 bits) and their device copies."""
    from dense_fp16_gemm_03_amd import inputs

    A, B = inputs.workload_operands(shape, "uniform", dtype)
    if dtype == "bf16":
        def dev_t(x):
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        def dev_t(x):
            return torch.from_numpy(x).to(dev)
    return A, B, dev_t(A), dev_t(B)


def time_throughput(torch, gemm, At, Bt, C, steps, warmup):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        gemm.gemm_abt(At, Bt, C, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        gemm.gemm_abt(At, Bt, C, stream=stream)
        e.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kernel_ms = [s.elapsed_time(e) for s, e in ev]
    return t1 - t0, kernel_ms


def time_loop(torch, gemm, At, Bt, C, calls, warmup):
    """Microseconds per call over `calls` back-to-back calls, from one pair of
    HIP events around the whole loop (no event between calls)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        gemm.gemm_abt(At, Bt, C, stream=stream)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record(stream)
    for _ in range(calls):
        gemm.gemm_abt(At, Bt, C, stream=stream)
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) * 1e3 / calls


def time_calls_alone(torch, gemm, At, Bt, C, calls, warmup=20):
    """Median GPU time of a call when every call runs alone."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        gemm.gemm_abt(At, Bt, C, stream=stream)
    torch.cuda.synchronize()
    out = []
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(calls):
        s.record(stream)
        gemm.gemm_abt(At, Bt, C, stream=stream)
        e.record(stream)
        e.synchronize()
        out.append(s.elapsed_time(e) * 1e3)
    out.sort()
    return out[len(out) // 2]


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


def _time_alone(torch, fn, calls, warmup=5):
    """Median GPU time (us) of fn() when every call runs alone."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    for _ in range(calls):
        s.record(stream)
        fn()
        e.record(stream)
        e.synchronize()
        out.append(s.elapsed_time(e) * 1e3)
    out.sort()
    return out[len(out) // 2]


def vendor_arm(torch, gemm, names, dev):
    """hipBLASLt context arm ("How we measured" in "SASS-Level Kernel
    Generation for Blackwell"): every algorithm of the vendor heuristic is run
    on hash-integer inputs, where any summation order is exact, and kept only
    if its C equals ours bit for bit; the fastest kept one is then timed
    against ours, calls alone, in the order ours, vendor, vendor, ours, on
    both uniform and hash-integer inputs. Context only, never the bench value."""
    import ctypes

    from dense_fp16_gemm_03_amd import build as b
    from dense_fp16_gemm_03_amd import inputs

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
    out = []
    for n in names:
        M, N, K = inputs.WORKLOADS[n]
        count = lib.vendor_hipblaslt_prepare(M, N, K, K, K, N, 64)
        if count <= 0:
            log(f"[vendor] {n}: heuristic returned {count}")
            out.append({"workload": n, "algorithms": int(count)})
            continue
        ws_bytes = max(lib.vendor_hipblaslt_workspace(i) for i in range(count))
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream().cuda_stream
        Ch = torch.empty((M, N), dtype=torch.float32, device=dev)
        Cv = torch.empty_like(Ch)
        Ah, Bh = (torch.from_numpy(x).to(dev) for x in inputs.workload_operands((M, N, K),
                                                                                 "hash_int"))
        gemm.gemm_abt(Ah, Bh, Ch)

        def run_vendor(i, A_, B_, C_):
            st = lib.vendor_hipblaslt_run(i, A_.data_ptr(), B_.data_ptr(), C_.data_ptr(),
                                          ws.data_ptr(), ws.numel(), stream)
            if st != 0:
                raise RuntimeError(f"hipBLASLt algorithm {i} failed with status {st}")

        screen_calls = 10 if M * N * K >= 1 << 36 else 50
        exact, times = 0, []
        for i in range(count):
            Cv.fill_(float("nan"))
            run_vendor(i, Ah, Bh, Cv)
            torch.cuda.synchronize()
            if not torch.equal(Cv, Ch):
                continue
            exact += 1
            times.append((_time_alone(torch, lambda: run_vendor(i, Ah, Bh, Cv), screen_calls), i))
        if not times:
            out.append({"workload": n, "algorithms": int(count), "exact": 0})
            continue
        best = min(times)[1]
        entry = {"workload": n, "M": M, "N": N, "K": K, "algorithms": int(count),
                 "exact": exact, "best_algorithm": best}
        for kind, (A_, B_) in (("uniform", make_device_operands(torch, (M, N, K), dev)[2:]),
                               ("hash_int", (Ah, Bh))):
            ours, theirs = [], []
            for who in ("ours", "vendor", "vendor", "ours"):
                if who == "ours":
                    ours.append(_time_alone(torch, lambda: gemm.gemm_abt(A_, B_, Ch), CALLS[n]))
                else:
                    theirs.append(_time_alone(torch, lambda: run_vendor(best, A_, B_, Cv),
                                              CALLS[n]))
            entry[kind] = {"ours_us": [round(min(ours), 3), round(max(ours), 3)],
                           "hipblaslt_us": [round(min(theirs), 3), round(max(theirs), 3)]}
            log(f"[vendor] {n} {kind}: ours {min(ours):.2f}-{max(ours):.2f} us, hipBLASLt "
                f"{min(theirs):.2f}-{max(theirs):.2f} us (algorithm {best} of {count}, "
                f"{exact} exact)")
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


def telemetry(torch, gemm, At, Bt, C, seconds=3.0):
    """Clock and power while the GEMM runs back to back: amd-smi (a child
    process) samples the board during a loop of calls. Context for reading the
    power-limited clock, outside the timed region; None if amd-smi fails."""
    import shutil
    import subprocess

    smi = shutil.which("amd-smi")
    if smi is None:
        return None
    stream = torch.cuda.current_stream()

    def burst():
        for _ in range(8):
            gemm.gemm_abt(At, Bt, C, stream=stream)
        torch.cuda.synchronize()

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:  # reach the loaded clock first
        burst()
    proc = subprocess.Popen([smi, "metric", "-g", "0", "--power", "--clock", "--json"],
                            stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    t0 = time.perf_counter()
    while proc.poll() is None and time.perf_counter() - t0 < seconds:
        burst()
    try:
        out, _ = proc.communicate(timeout=30)
        d = json.loads(out)
        gpu = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clocks = [v["clk"]["value"] for k, v in gpu["clock"].items()
                  if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
        power = gpu["power"]["socket_power"]["value"]
        return {"gfx_clk_mhz": clocks, "socket_power_w": power,
                "source": "amd-smi metric --power --clock, sampled during back-to-back calls"}
    except Exception:  # noqa: BLE001 - telemetry is optional context
        proc.kill()
        return None


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


def traffic_for(workload, kernel_avg_s):
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
    ap.add_argument("--workload", default="8192^3",
                    help="one of the five workloads, one of the pages' other shapes, "
                         "or any MxNxK")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", "--no-long-k", dest="no_extras", action="store_true",
                    help="at 8192^3, skip the extra rows (the two long-K workloads and the "
                         "hash-integer inputs); profiling runs use this so their traces hold "
                         "one shape and one input kind")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="skip the amd-smi clock/power sample after the timed region")
    ap.add_argument("--shapes", action="store_true",
                    help="also time the five workloads, each call alone")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB fp32 copy kernel (counter calibration)")
    ap.add_argument("--sweeps", type=int, default=4,
                    help="sweeps over the shapes, alternately forward and reverse")
    ap.add_argument("--page-shapes", action="store_true",
                    help="with --shapes, also time the other shapes of the pages' table")
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
    all_shapes = {**inputs.WORKLOADS, **inputs.PAGE_SHAPES}
    shape = all_shapes.get(name) or parse_shape(name)
    if shape is None:
        print(f"unknown workload {name!r}; known: {', '.join(all_shapes)}, or MxNxK",
              file=sys.stderr)
        sys.exit(2)
    M, N, K = shape
    flops, nbytes = algorithmic(M, N, K)
    log(f"[bench] workload {name}: {gemm.gemm_f16_f32_abt_describe(M, N, K)}")
    A, B, At, Bt = make_device_operands(torch, (M, N, K), dev, args.dtype)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)

    elapsed, kernel_ms = time_throughput(torch, gemm, At, Bt, C, args.steps, args.warmup)
    ms_per_step = elapsed / args.steps * 1e3
    value = flops * args.steps / elapsed / 1e12
    avg_kernel_s = sum(kernel_ms) / len(kernel_ms) / 1e3
    achieved = flops / avg_kernel_s / 1e12
    log(f"[bench] {args.steps} steps in {elapsed * 1e3:.2f} ms: {value:.1f} TFLOP/s; "
        f"kernel avg {avg_kernel_s * 1e6:.2f} us ({achieved:.1f} TFLOP/s)")
    # committed counters are for the binary16 path
    traffic = traffic_for(name, avg_kernel_s) if args.dtype == "f16" else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel_avg_us": round(avg_kernel_s * 1e6, 3),
                "algorithmic_bytes": nbytes, "algorithmic_flops": flops}

    shapes = []
    if args.shapes:
        table = dict(inputs.WORKLOADS)
        if args.page_shapes:
            table.update(inputs.PAGE_SHAPES)
        names = list(table)
        results = {n: [] for n in names}
        for sweep in range(args.sweeps):
            order = names if sweep % 2 == 0 else names[::-1]
            for n in order:
                m, nn, k = table[n]
                if n == name:
                    a, b = At, Bt
                    c = C
                else:
                    _, _, a, b = make_device_operands(torch, (m, nn, k), dev, args.dtype)
                    c = torch.empty((m, nn), dtype=torch.float32, device=dev)
                us = time_calls_alone(torch, gemm, a, b, c, CALLS[n])
                results[n].append(us)
                log(f"[bench] sweep {sweep} {n}: median {us:.2f} us/call")
                del a, b, c
                torch.cuda.empty_cache()
        for n in names:
            m, nn, k = table[n]
            f, by = algorithmic(m, nn, k)
            lo, hi = min(results[n]), max(results[n])
            mid = (lo + hi) / 2
            t_roof = max(f / (PEAK_TFLOPS * 1e12), by / (HBM_PEAK_GBS * 1e9))
            entry = {"workload": n, "M": m, "N": nn, "K": k, "us_per_call": [round(lo, 3),
                     round(hi, 3)], "tflops": round(f / (mid * 1e-6) / 1e12, 2),
                     "bound": "mfma" if f / by > PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
                     else "hbm",
                     "roofline_frac": round(t_roof / (mid * 1e-6), 4),
                     "mfma_peak_frac": round(f / (mid * 1e-6) / 1e12 / PEAK_TFLOPS, 4),
                     "calls": CALLS[n], "plan": gemm.gemm_f16_f32_abt_describe(m, nn, k)}
            if n in PAGE_US:
                entry["pages_b200_us"] = PAGE_US[n]
            shapes.append(entry)

    long_k = []
    pages_inputs = None
    if name == "8192^3" and not args.no_extras:
        # The two long-K workloads, back to back like the headline, so every
        # bench line carries their fraction of peak as well (not the value).
        for n in ("2048x2048x16384", "1024x1024x65536"):
            m, nn, k = inputs.WORKLOADS[n]
            _, _, a, b = make_device_operands(torch, (m, nn, k), dev, args.dtype)
            c = torch.empty((m, nn), dtype=torch.float32, device=dev)
            # the board's clocks settle over the first ~100 calls of a new shape
            avg_us = time_loop(torch, gemm, a, b, c, 200, 100)
            f, _ = algorithmic(m, nn, k)
            long_k.append({"workload": n, "us_per_call": round(avg_us, 3),
                           "tflops": round(f / (avg_us * 1e-6) / 1e12, 2),
                           "mfma_peak_frac": round(f / (avg_us * 1e-6) / 1e12 / PEAK_TFLOPS, 4),
                           "calls": 200, "plan": gemm.gemm_f16_f32_abt_describe(m, nn, k)})
            log(f"[bench] {n}: {avg_us:.2f} us/call back to back "
                f"({long_k[-1]['mfma_peak_frac'] * 100:.1f}% of peak)")
            del a, b, c
            torch.cuda.empty_cache()
        # The same workload on the input kind the pages time on (integers in
        # [-3, 3] from a hash of the index): context for the data-dependent
        # power draw, never the value.
        if args.dtype == "f16":
            a = torch.from_numpy(inputs.hash_int(M, K, 1)).to(dev)
            b = torch.from_numpy(inputs.hash_int(N, K, 2)).to(dev)
            avg_us = time_loop(torch, gemm, a, b, C, args.steps, args.warmup)
            pages_inputs = {"workload": name, "inputs": "hash_int [-3, 3]",
                            "us_per_call": round(avg_us, 3),
                            "tflops": round(flops / (avg_us * 1e-6) / 1e12, 2),
                            "mfma_peak_frac": round(flops / (avg_us * 1e-6) / 1e12 / PEAK_TFLOPS, 4),
                            "calls": args.steps}
            log(f"[bench] {name} on hash-integer inputs: {avg_us:.2f} us/call "
                f"({pages_inputs['mfma_peak_frac'] * 100:.1f}% of peak)")
            del a, b
            torch.cuda.empty_cache()

    vendor = None
    if args.vendor:
        vendor = vendor_arm(torch, gemm, list(inputs.WORKLOADS), dev)

    tele = None if args.no_telemetry else telemetry(torch, gemm, At, Bt, C)
    if tele is not None:
        log(f"[bench] telemetry: gfx clocks {tele['gfx_clk_mhz']} MHz, "
            f"socket power {tele['socket_power_w']} W")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU reference on a sample ...")
        cpu = cpu_baseline(A, B, M, N, K)
        log(f"[bench] cpu: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")

    vs = None
    if name in PAGE_US and args.dtype == "f16":  # the pages time binary16 only
        vs = round(value / (flops / (PAGE_US[name] * 1e-6) / 1e12), 4)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": vs, "dtype": args.dtype,
        "data": f"synthetic: uniform[-1,1] {args.dtype}, seeds 1 (A) and 2 (B), resident in HBM",
        "config": {"workload": f"gemm_abt {M}x{N}x{K}", "M": M, "N": N, "K": K,
                   "accumulate": "f32", "output": "f32",
                   "plan": gemm.gemm_f16_f32_abt_describe(M, N, K),
                   "source_hash": source_hash(), "library_md5": library_md5()},
        "roofline": roofline, "cpu_baseline": cpu, "shapes": shapes, "long_k": long_k,
        "pages_inputs": pages_inputs, "telemetry": tele,
    }
    if vendor is not None:
        line["vendor_hipblaslt"] = vendor
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
