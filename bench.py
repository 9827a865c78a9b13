#!/usr/bin/env python3
"""Throughput of C = ReLU(A.B) (fp16 in, fp32 accumulate, fp16 out) on one MI355X.

One "step" is one call of the library through the C ABI on the headline
workload, M = N = K = 4096, with A and B already resident in HBM
(``gemm_relu_f16``; ``gemm_relu_f16_ws`` with a workspace allocated up front
for a workload whose plan takes one).
Prints ONE JSON line (rank 0) with the metric, the roofline of the dominant
kernel measured live with HIP events on the launch stream, and the CPU oracle
timed on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--no-cpu-baseline]
                  [--no-workloads] [--workload NAME] [--reps R] [--workload-settle-ms MS]
                  [--no-oracle-table] [--copy-probe MIB] [--read-probe MIB]
                  [--vendor-reference] [--extra-shapes]

The JSON line also carries the HBM read ceiling measured by the library's
read probe, a per-workload table (every call variant timed after its own
clock settling, R >= 100 launches back to back and R event-bracketed ones)
and the oracle's timings per workload on one thread and on all cores.
``--copy-probe`` runs only a device-to-device copy of known size; it is what
the HBM-traffic counters are calibrated against.  ``--read-probe`` runs only
the read probe.  ``--vendor-reference`` only
times torch.mm + relu_ (the vendor BLAS) on the same workloads, for context;
``--extra-shapes`` times the library (and torch.mm + relu_) on shapes beyond
the workloads: mid-M, narrow small-M, long K, B given transposed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from dense_gemm_epilogue_tiled_amd import roofline  # noqa: E402  (host arithmetic only)

MFMA_F16_PEAK_TFLOPS = roofline.MI355X_MFMA_F16_TFLOPS
HBM_PEAK_GBS = roofline.MI355X_HBM_GBS

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")


def kernel_source_hash() -> str:
    """Hash of the kernel sources; counter-derived traffic is only reported
    while it matches the hash recorded when the counters were taken."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_epilogue_tiled_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def algorithmic(w):
    return roofline.algorithmic_flops(w.M, w.N, w.K), roofline.algorithmic_bytes(w.M, w.N, w.K)


def make_device_operands(torch, w, copies=1):
    """Seeded N(0,1) fp16 operands generated on the GPU (B scaled by K^-1/2
    where the workload says so). Same distribution as the CPU generator."""
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    A = torch.randn(w.M, w.K, generator=g, device="cuda", dtype=torch.float32).half()
    Bs = []
    for _ in range(copies):
        b = torch.randn(w.K, w.N, generator=g, device="cuda", dtype=torch.float32)
        if w.b_scaled:
            b.mul_(w.K ** -0.5)
        Bs.append(b.half())
    C = torch.empty(w.M, w.N, device="cuda", dtype=torch.float16)
    return A, Bs, C


def workspace_for(gr, torch, w, A, B, C):
    """The device workspace the library asks for on this problem (None if
    none), allocated once, outside any timed region, as a caller would."""
    st, size = gr.gemm_relu_f16_workspace_size(w.M, w.N, w.K, A.data_ptr(), w.K, B.data_ptr(), w.N,
                                               C.data_ptr(), w.N)
    if st != 0:
        raise gr.GemmReluError(st, "gemm_relu_f16_workspace_size")
    return torch.empty(size, dtype=torch.uint8, device="cuda") if size else None


def launcher(gr, torch, w, A, B, C, stream, ws=None):
    """One library call on the workload: gemm_relu_f16, or gemm_relu_f16_ws
    when the problem takes a workspace."""
    h = stream.cuda_stream
    a, b, c = A.data_ptr(), B.data_ptr(), C.data_ptr()
    M, N, K = w.M, w.N, w.K
    if ws is None:
        fn = gr.lib().gemm_relu_f16

        def run():
            st = fn(M, N, K, a, K, b, N, c, N, h)
            if st != 0:
                raise gr.GemmReluError(st)
    else:
        fn = gr.lib().gemm_relu_f16_ws
        wp, wb = ws.data_ptr(), ws.numel()

        def run():
            st = fn(M, N, K, a, K, b, N, c, N, wp, wb, h)
            if st != 0:
                raise gr.GemmReluError(st, "gemm_relu_f16_ws")
    return run


def plan_for(gr, w, A, B, C, ws):
    st, plan = gr.gemm_relu_f16_plan_ws(w.M, w.N, w.K, A.data_ptr(), w.K, B.data_ptr(), w.N, C.data_ptr(), w.N,
                                        0 if ws is None else ws.numel())
    assert st == 0
    return plan


def time_launches(torch, run, stream, reps):
    """Per-launch durations (ms) from HIP event pairs on the launch stream."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for s, e in evs:
        s.record(stream)
        run()
        e.record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in evs]


def cpu_baseline(w, max_seconds=20.0):
    """The oracle (as it stands) on the host cores, on whole rows of the
    workload's result: rows are added in chunks until about ``max_seconds``
    of work is done or the matrix is complete. Work per row is exactly
    2 N K FLOP, so the rate needs no extrapolation."""
    import numpy as np
    import oracle

    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    threads = max(1, threads)
    oracle.set_threads(threads)
    A, B = synth.operands(w)
    done, t_total, chunk = 0, 0.0, 64
    while done < w.M and t_total < max_seconds:
        rows = np.arange(done, min(w.M, done + chunk))
        t0 = time.perf_counter()
        oracle.gemm_relu_rows(A, B, rows)
        t_total += time.perf_counter() - t0
        done += rows.size
        chunk = min(chunk * 2, 1024)
    flops = 2.0 * done * w.N * w.K
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(flops / t_total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": "%d full rows of the %dx%dx%d result (%.1f GFLOP, %.2f s; C triple loop, fp32 "
                  "accumulation, OpenMP over rows; %s)" % (done, w.M, w.N, w.K, flops / 1e9, t_total, model),
    }


# rows of the result the oracle computes for the per-workload timings where
# the whole matrix would take too long: (all cores, one thread)
ORACLE_ROWS = {"square4096": (256, 16), "mlp8192x28672x8192": (64, 2), "ragged4099x3071x2050": (None, 128)}


def cpu_oracle_table():
    """The oracle (as it stands) per workload, on all host cores and on one
    thread: the whole matrix for the 1024^3 and small-M workloads (and the
    ragged one on all cores), R full rows elsewhere (work per row is exactly
    2 N K FLOP).  ``parity_check_s`` is the wall time of the oracle calls the
    workload's GPU parity test makes: the whole matrix, or 4096 sampled
    elements plus 8 full rows and 8 full columns."""
    import numpy as np
    import oracle

    allc = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        allc = min(allc, int(os.environ["OMP_NUM_THREADS"]))
    allc = max(1, allc)
    table = {}
    for name, w in synth.WORKLOADS.items():
        A, B = synth.operands(w)
        row = {}
        for label, threads, pick in (("all_cores", allc, 0), ("single_thread", 1, 1)):
            r = ORACLE_ROWS.get(name, (None, None))[pick]
            t0 = time.perf_counter()
            if r is None:
                oracle.gemm_relu_full(A, B, threads=threads)
                rows = w.M
            else:
                oracle.gemm_relu_rows(A, B, np.arange(r), threads=threads)
                rows = r
            dt = time.perf_counter() - t0
            flops = 2.0 * rows * w.N * w.K
            row[label] = {"threads": threads, "sample": "full matrix" if r is None else "%d rows" % r,
                          "seconds": round(dt, 3), "tflops": round(flops / dt / 1e12, 5),
                          # work per row is exactly 2 N K FLOP, so this is exact in work
                          "full_matrix_s": round(dt * w.M / rows, 3)}
        t0 = time.perf_counter()
        if w.check == "full":
            oracle.gemm_relu_full(A, B, threads=allc)
            what = "full matrix"
        else:
            ii, jj = synth.sample_indices(w.M, w.N, 4096, w.seed)
            oracle.gemm_relu_elems(A, B, ii, jj, threads=allc)
            oracle.gemm_relu_rows(A, B, np.linspace(0, w.M - 1, 8).astype(np.int64), threads=allc)
            oracle.gemm_relu_cols(A, B, np.linspace(0, w.N - 1, 8).astype(np.int64), threads=allc)
            what = "4096 elements + 8 rows + 8 columns"
        row["parity_check_s"] = round(time.perf_counter() - t0, 3)
        row["parity_check"] = what
        table[name] = row
        print("[oracle] %s %s" % (name, row), file=sys.stderr, flush=True)
        del A, B
    oracle.set_threads(allc)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    table["host"] = {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
                     "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"), "cpu_model": model,
                     "what": "the oracle as it stands, a reported baseline, not the optimisation target"}
    return table


def traffic_for(workload: str, src_hash: str):
    """HBM bytes per launch (fetched + written) from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                parts = line.split()
                if len(parts) == 4 and not line.startswith("#") and parts[0] == workload:
                    if parts[1] != src_hash:
                        return None
                    return int(parts[2]) + int(parts[3])
    except (OSError, ValueError):
        return None
    return None


def time_back_to_back(torch, runs, stream, reps):
    """Average launch time (ms) over ``reps`` back-to-back launches between one
    event pair on the launch stream, cycling through ``runs``."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        runs[i % len(runs)]()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure(torch, runs, stream, reps, settle_ms):
    """Settle the clock on the launches, then time them back to back (the
    figure the rates use) and one event pair per launch (median, min, p90)."""
    settle(torch, lambda: [r() for r in runs], settle_ms)
    avg = time_back_to_back(torch, runs, stream, reps)
    per = sorted(time_launches(torch, runs[i % len(runs)], stream, 1)[0] for i in range(reps))
    return {
        "avg_us": round(avg * 1e3, 2),
        "per_launch_median_us": round(statistics.median(per) * 1e3, 2),
        "per_launch_min_us": round(per[0] * 1e3, 2),
        "per_launch_p90_us": round(per[int(0.9 * (len(per) - 1))] * 1e3, 2),
    }


def rates(w, stats):
    flops, nbytes = algorithmic(w)
    t = stats["avg_us"] * 1e-6
    return {
        "tflops": round(flops / t / 1e12, 1),
        "gbs": round(nbytes / t / 1e9, 1),
        "frac_mfma": round(flops / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
        "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
    }


def forced_ws_launcher(gr, w, A, B, C, stream, ws, path):
    fn = gr.lib().gemm_relu_f16_forced_ws
    M, N, K = w.M, w.N, w.K
    a, b, c, h = A.data_ptr(), B.data_ptr(), C.data_ptr(), stream.cuda_stream
    wp, wb = ws.data_ptr(), ws.numel()

    def run():
        st = fn(M, N, K, a, K, b, N, c, N, wp, wb, h, path)
        if st != 0:
            raise gr.GemmReluError(st, "gemm_relu_f16_forced_ws")
    return run


def bench_workload(gr, torch, w, reps, settle_ms, read_ceiling=None):
    """Secondary measurement of one workload, per call variant: the plain call
    (gemm_relu_f16, in place), the call with a workspace (gemm_relu_f16_ws,
    with what the library asks for, or 1 MiB where it asks for none), and on
    the ragged workload the packed path forced.  Each variant: clock settled
    first, ``reps`` back-to-back launches between one event pair (the figure
    the rates use), and ``reps`` event-bracketed launches for the spread.
    The small-M workload rotates four copies of B (4 x 256 MiB, well above
    the 256 MB last-level cache) so every launch streams B from HBM."""
    cold = w.name.startswith("smallm")
    copies = 4 if cold else 1
    A, Bs, C = make_device_operands(torch, w, copies=copies)
    stream = torch.cuda.current_stream()
    ws = workspace_for(gr, torch, w, A, Bs[0], C)
    if ws is None:
        ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    variants = {"in_place": None, "workspace": ws}
    out = {"cache": "cold (4 rotating copies of B)" if cold else "warm", "reps": reps, "variants": {}}
    for name, wsv in variants.items():
        runs = [launcher(gr, torch, w, A, B, C, stream, wsv) for B in Bs]
        plan = plan_for(gr, w, A, Bs[0], C, wsv)
        st = measure(torch, runs, stream, reps, settle_ms)
        st.update(rates(w, st))
        st.update({"path": plan["path_name"], "workspace_bytes": plan["workspace"], "grid": plan["grid"],
                   "split_k": plan["split_k"]})
        out["variants"][name] = st
    if w.name.startswith("ragged"):
        big = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        runs = [forced_ws_launcher(gr, w, A, Bs[0], C, stream, big, gr.GR_PATH_TILE_PACKED)]
        st = measure(torch, runs, stream, reps, settle_ms)
        st.update(rates(w, st))
        st.update({"path": "tile_packed (forced)", "workspace_bytes": 64 << 20})
        out["variants"]["packed_forced"] = st
        del big
    # top-level figures: the fastest variant, named
    best = min(out["variants"], key=lambda k: out["variants"][k]["avg_us"])
    out["best_variant"] = best
    out.update({k: out["variants"][best][k] for k in ("avg_us", "tflops", "gbs", "frac_mfma", "frac_hbm", "path")})
    if cold and read_ceiling:
        out["frac_of_read_ceiling"] = round(out["gbs"] / read_ceiling["gbs"], 4)
    del A, Bs, C, ws, variants
    torch.cuda.empty_cache()
    if not cold:
        fl = bench_flushed(gr, torch, w, reps, settle_ms)
        out["flushed"] = fl
    torch.cuda.empty_cache()
    return out


def flush_pairs(w):
    """Operand pairs rotated for the flushed timing: enough that the pairs
    together hold at least 512 MiB, twice the 256 MB last-level cache."""
    pair = 2 * (w.M * w.K + w.K * w.N)
    return max(2, min(128, -(-(512 << 20) // pair)))


def bench_flushed(gr, torch, w, reps, settle_ms):
    """Launch times with A and B evicted from every cache: back-to-back
    launches, each on its own copy of both operands, rotating over
    flush_pairs(w) copies (with the workspace the library asks for, if any).
    No flush buffer is written (its write-back would land in the timed
    launch)."""
    n = flush_pairs(w)
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    pairs = []
    for _ in range(n):
        a = torch.randn(w.M, w.K, generator=g, device="cuda", dtype=torch.float32).half()
        b = torch.randn(w.K, w.N, generator=g, device="cuda", dtype=torch.float32)
        if w.b_scaled:
            b.mul_(w.K ** -0.5)
        pairs.append((a, b.half()))
    C = torch.empty(w.M, w.N, device="cuda", dtype=torch.float16)
    stream = torch.cuda.current_stream()
    ws = workspace_for(gr, torch, w, pairs[0][0], pairs[0][1], C)
    runs = [launcher(gr, torch, w, a, b, C, stream, ws) for a, b in pairs]
    st = measure(torch, runs, stream, reps, settle_ms)
    st.update(rates(w, st))
    st["pairs"] = n
    del pairs, runs, C, ws
    return st


def read_ceiling(gr, torch, nbytes=256 << 20, copies=4, reps=100, settle_ms=100.0):
    """The HBM read ceiling the small-M path is judged against: the library's
    read probe (gemm_relu_stream_read) on ``copies`` rotating buffers of
    ``nbytes`` each, back to back, in both of its read patterns; the ceiling
    is the faster one."""
    bufs = [torch.randint(0, 1 << 30, (nbytes // 4,), device="cuda", dtype=torch.int32) for _ in range(copies)]
    sink = torch.empty(256, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    fn = gr.lib().gemm_relu_stream_read

    def mk(b, pattern):
        def run():
            st = fn(b.data_ptr(), nbytes, pattern, sink.data_ptr(), h)
            if st != 0:
                raise gr.GemmReluError(st, "gemm_relu_stream_read")
        return run
    out = {"bytes_per_launch": nbytes, "rotating_buffers": copies, "patterns": {}}
    for name, pattern in (("contiguous", gr.GR_READ_CONTIGUOUS), ("row_pieces", gr.GR_READ_ROW_PIECES)):
        st = measure(torch, [mk(b, pattern) for b in bufs], stream, reps, settle_ms)
        gbs = nbytes / (st["avg_us"] * 1e-6) / 1e9
        out["patterns"][name] = {"avg_us": st["avg_us"], "per_launch_median_us": st["per_launch_median_us"],
                                 "gbs": round(gbs, 1)}
    del bufs, sink
    torch.cuda.empty_cache()
    best = max(out["patterns"], key=lambda k: out["patterns"][k]["gbs"])
    out.update({"pattern": best, "avg_us": out["patterns"][best]["avg_us"], "gbs": out["patterns"][best]["gbs"],
                "frac_of_peak": round(out["patterns"][best]["gbs"] / HBM_PEAK_GBS, 4),
                "what": "gemm_relu_stream_read: 256 workgroups x 512 threads, nontemporal 16-byte loads, 32 KiB "
                        "in flight per workgroup; contiguous 1/256 chunks, or 256-byte pieces of 32 KiB rows "
                        "(the small-M split's pattern)"})
    return out


def settle(torch, run, ms):
    """Untimed back-to-back launches for ``ms`` milliseconds of wall time.
    Under full load the shader clock moves for tens of milliseconds (at
    4096^3 the first launches take about 125 us, the ones after 40 ms about
    103 us, after 70 ms about 102 us), longer than a few warmup steps last, so
    the timed region would otherwise measure the ramp.  Returns the number of
    launches."""
    n = 0
    t_end = time.perf_counter() + ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(20):
            run()
        n += 20
        torch.cuda.synchronize()
    return n


def observed_sclk(torch, run, seconds=1.0):
    """The shader clock under this load: the kernel runs back-to-back for
    ``seconds`` (outside the timed region) while a thread reads the current
    level of /sys/class/drm/card*/device/pp_dpm_sclk (a smoothed average,
    which settles within a few tenths of a second); returns the median MHz of
    the last half of the samples of the card whose clock rose most, or None
    where the file cannot be read."""
    import glob
    import threading
    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not files:
        return None
    samples = {f: [] for f in files}
    done = threading.Event()

    def poll():
        while not done.is_set():
            for f in files:
                try:
                    with open(f) as fh:
                        for line in fh:
                            if "*" in line:
                                samples[f].append(int(line.split(":")[1].lower().split("mhz")[0]))
                except (OSError, ValueError, IndexError):
                    pass
            time.sleep(0.005)
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(50):
            run()
        torch.cuda.synchronize()
    done.set()
    th.join()
    best = None
    for vals in samples.values():
        if len(vals) >= 8:
            m = statistics.median(vals[len(vals) // 2:])
            best = m if best is None or m > best else best
    return best


def copy_probe(torch, mib, reps=20):
    """A device-to-device copy of ``mib`` MiB (torch's copy kernel): the
    STREAM-like copy rate (bytes read + written per second), and the kernel
    the HBM-traffic counters are calibrated against."""
    n = mib * 1024 * 1024 // 2
    src = torch.randn(n, device="cuda", dtype=torch.float32).half()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    avg = time_back_to_back(torch, [lambda: dst.copy_(src)], stream, reps)
    med = statistics.median(time_launches(torch, lambda: dst.copy_(src), stream, reps))
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": n * 2, "bytes_written": n * 2, "avg_us": round(avg * 1e3, 2),
            "per_launch_median_us": round(med * 1e3, 2), "gbs_rw": round(4.0 * n / (avg * 1e-3) / 1e9, 1),
            "frac_of_peak": round(4.0 * n / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def vendor_reference(torch, reps=30):
    """Context only: torch.mm (hipBLASLt) followed by an in-place ReLU on the
    same workloads, timed like the per-workload table (warm, HIP events).
    Not the product and not a target; printed as its own JSON line."""
    out = {}
    for name, w in synth.WORKLOADS.items():
        A, Bs, C = make_device_operands(torch, w)
        B = Bs[0]
        stream = torch.cuda.current_stream()

        def run():
            torch.relu_(torch.mm(A, B, out=C))
        for _ in range(5):
            run()
        torch.cuda.synchronize()
        times = sorted(time_launches(torch, run, stream, reps if w.M * w.N * w.K < 1e12 else 10))
        med = statistics.median(times)
        flops, _ = algorithmic(w)
        out[name] = {"median_us": round(med * 1e3, 2), "tflops": round(flops / (med * 1e-3) / 1e12, 1)}
        del A, Bs, B, C
        torch.cuda.empty_cache()
    print(json.dumps({"vendor_reference": out, "what": "torch.mm + torch.relu_ (hipBLASLt), warm, context only"}))


EXTRA_SHAPES = [
    # (label, M, N, K, layout) -- shapes beyond the workloads, for the paths they exercise
    ("mid-M", 64, 4096, 4096, "nn"),
    ("narrow small-M", 8, 4096, 8192, "nn"),
    ("long K, few tiles", 1024, 1024, 16384, "nn"),
    ("B transposed, square", 4096, 4096, 4096, "bt"),
    ("B transposed, small-M", 8, 16384, 8192, "bt"),
    ("B transposed, narrow small-M", 16, 4096, 4096, "bt"),
    ("bfloat16, square", 4096, 4096, 4096, "bf16"),
    ("bfloat16, square 1024", 1024, 1024, 1024, "bf16"),
    ("bfloat16, MLP projection", 8192, 28672, 8192, "bf16"),
    ("bfloat16, small-M", 8, 16384, 8192, "bf16"),
    ("bias + GELU, square", 4096, 4096, 4096, "epi:f16:gelu"),
    ("bias + GELU (tanh), MLP projection", 8192, 28672, 8192, "epi:f16:gelu_tanh"),
    ("bias + SiLU, bfloat16, MLP projection", 8192, 28672, 8192, "epi:bf16:silu"),
    ("bias + SiLU, small-M", 8, 16384, 8192, "epi:f16:silu"),
    ("linear layer (weight N x K), bfloat16, bias + GELU", 4096, 4096, 4096, "lin:bf16:gelu"),
    ("linear layer, bfloat16, bias + SiLU, MLP projection", 8192, 28672, 8192, "lin:bf16:silu"),
    ("linear layer, fp16, bias + GELU (tanh), small-M", 8, 16384, 8192, "lin:f16:gelu_tanh"),
    ("fp8 e4m3, square", 4096, 4096, 4096, "fp8"),
    ("fp8 e4m3, square 8192", 8192, 8192, 8192, "fp8"),
    ("fp8 e4m3, MLP projection", 8192, 28672, 8192, "fp8"),
    ("fp8 e4m3, mid-M", 128, 8192, 8192, "fp8"),
    ("fp8 e4m3, long K, few tiles", 1024, 1024, 8192, "fp8"),
    ("MX fp8 (E8M0 scale per 32 k), square", 4096, 4096, 4096, "mxfp8"),
    ("MX fp8, square 8192", 8192, 8192, 8192, "mxfp8"),
    ("MX fp8, MLP projection", 8192, 28672, 8192, "mxfp8"),
    ("MX fp4 (E2M1, E8M0 scale per 32 k), square", 4096, 4096, 4096, "mxfp4"),
    ("MX fp4, square 8192", 8192, 8192, 8192, "mxfp4"),
    ("MX fp4, MLP projection", 8192, 28672, 8192, "mxfp4"),
]


def extra_shapes(gr, torch, reps=30):
    """Context only: library calls on shapes beyond the workloads (without and
    with the workspace the library asks for; B given transposed through the
    _bt calls) next to torch.mm + relu_. Warm, HIP events per launch."""
    out = []
    stream = torch.cuda.current_stream()
    for label, M, N, K, layout in EXTRA_SHAPES:
        g = torch.Generator(device="cuda").manual_seed(M + N + K)
        dt = torch.bfloat16 if "bf16" in layout else torch.float16
        A = torch.randn(M, K, generator=g, device="cuda").to(dt)
        B = (torch.randn(K, N, generator=g, device="cuda") * K ** -0.5).to(dt)
        C = torch.empty(M, N, device="cuda", dtype=dt)
        row = {"shape": "%dx%dx%d" % (M, N, K), "what": label, "layout": layout}
        runs = {}
        if layout == "mxfp4":
            # random E2M1 pairs (every byte is two valid codes) and scales
            A4 = torch.randint(0, 256, (M, K // 2), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
            B4 = torch.randint(0, 256, (N, K // 2), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
            sa4 = torch.randint(124, 130, (M, K // 32), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
            sb4 = torch.randint(124, 130, (N, K // 32), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
            h = stream.cuda_stream

            def ours4():
                st = gr.gemm_mxfp4_bt(M, N, K, A4.data_ptr(), K // 2, sa4.data_ptr(), K // 32, B4.data_ptr(), K // 2,
                                      sb4.data_ptr(), K // 32, None, gr.GR_ACT_RELU, C.data_ptr(), N, gr.GR_FMT_F16, h)
                if st != gr.GR_OK:
                    raise gr.GemmReluError(st, "gemm_mxfp4_bt")
            runs["ours"] = ours4

            def vendor4():
                a, b = A4.view(torch.float4_e2m1fn_x2), B4.view(torch.float4_e2m1fn_x2)
                return torch.relu_(torch._scaled_mm(a, b.t(), scale_a=sa4.view(torch.float8_e8m0fnu),
                                                    scale_b=sb4.view(torch.float8_e8m0fnu), out_dtype=torch.float16))
            try:
                vendor4()
                runs["vendor"] = vendor4
            except Exception as e:  # the vendor MX fp4 path may be missing
                row["vendor_error"] = str(e)[:120]
        elif layout == "mxfp8":
            A8 = torch.randn(M, K, generator=g, device="cuda").to(torch.float8_e4m3fn)
            Bt8 = torch.randn(N, K, generator=g, device="cuda").to(torch.float8_e4m3fn)
            sa8 = torch.randint(124, 130, (M, K // 32), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
            sb8 = torch.randint(124, 130, (N, K // 32), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
            runs["ours"] = lambda: gr.gemm_mxfp8(A8, sa8, Bt8, sb8, act="relu", out=C, stream=stream)

            def vendor_mx():
                return torch.relu_(torch._scaled_mm(A8, Bt8.t(), scale_a=sa8.view(torch.float8_e8m0fnu),
                                                    scale_b=sb8.view(torch.float8_e8m0fnu), out_dtype=torch.float16))
            try:
                vendor_mx()
                runs["vendor"] = vendor_mx
            except Exception as e:  # the vendor MX path may be missing
                row["vendor_error"] = str(e)[:120]
        elif layout == "fp8":
            A8 = torch.randn(M, K, generator=g, device="cuda").to(torch.float8_e4m3fn)
            Bt8 = torch.randn(N, K, generator=g, device="cuda").to(torch.float8_e4m3fn)
            sa, sb = 1.0 / 64, 1.0 / 64
            runs["ours"] = lambda: gr.gemm_fp8(A8, Bt8, sa, sb, act="relu", out=C, stream=stream, workspace=None)
            st, size = gr.gemm_fp8_bt_workspace_size(M, N, K, A8.data_ptr(), K, Bt8.data_ptr(), K, C.data_ptr(), N)
            if size:
                ws8 = torch.empty(size, dtype=torch.uint8, device="cuda")
                runs["ours_ws"] = lambda: gr.gemm_fp8(A8, Bt8, sa, sb, act="relu", out=C, stream=stream, workspace=ws8)
                row["workspace_bytes"] = size
            ta = torch.tensor(sa, device="cuda")
            tb = torch.tensor(sb, device="cuda")

            def vendor():
                return torch.relu_(torch._scaled_mm(A8, Bt8.t(), scale_a=ta, scale_b=tb, out_dtype=torch.float16))
            try:
                vendor()
                runs["vendor"] = vendor
            except Exception as e:  # the vendor fp8 path may be missing
                row["vendor_error"] = str(e)[:120]
        elif layout.startswith("lin:"):
            act = layout.split(":")[2]
            W = B.t().contiguous()  # N x K
            bias = torch.randn(N, generator=g, device="cuda").to(dt)
            fn = {"gelu": torch.nn.functional.gelu, "silu": torch.nn.functional.silu,
                  "gelu_tanh": lambda x: torch.nn.functional.gelu(x, approximate="tanh")}[act]
            runs["ours"] = lambda: gr.linear(A, W, bias, act, C, stream)
            runs["vendor"] = lambda: fn(torch.nn.functional.linear(A, W, bias))
        elif layout.startswith("epi:"):
            act = layout.split(":")[2]
            bias = torch.randn(N, generator=g, device="cuda").to(dt)
            fn = {"gelu": torch.nn.functional.gelu, "silu": torch.nn.functional.silu,
                  "gelu_tanh": lambda x: torch.nn.functional.gelu(x, approximate="tanh")}[act]
            runs["ours"] = lambda: gr.gemm_bias_act(A, B, bias, act, C, stream)
            runs["vendor"] = lambda: fn(torch.addmm(bias, A, B, out=C))
        elif layout == "bf16":
            runs["ours"] = lambda: gr.gemm_relu(A, B, C, stream, workspace=None)
            runs["vendor"] = lambda: torch.relu_(torch.mm(A, B, out=C))
        elif layout == "bt":
            Bt = B.t().contiguous()
            runs["ours"] = lambda: gr.gemm_relu_bt(A, Bt, C, stream)
            runs["vendor"] = lambda: torch.relu_(torch.mm(A, Bt.t(), out=C))
        else:
            st, size = gr.gemm_relu_f16_workspace_size(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N)
            ws = torch.empty(size, dtype=torch.uint8, device="cuda") if size else None
            runs["ours"] = lambda: gr.gemm_relu(A, B, C, stream, workspace=None)
            if ws is not None:
                runs["ours_ws"] = lambda: gr.gemm_relu(A, B, C, stream, workspace=ws)
                row["workspace_bytes"] = size
            runs["vendor"] = lambda: torch.relu_(torch.mm(A, B, out=C))
        for name, run in runs.items():
            for _ in range(5):
                run()
            torch.cuda.synchronize()
            med_ms = statistics.median(time_launches(torch, run, stream, reps))
            row[name + "_us"] = round(med_ms * 1e3, 2)
            row[name + "_tflops"] = round(2.0 * M * N * K / (med_ms * 1e-3) / 1e12, 1)
        out.append(row)
        print("[extra] %s" % row, file=sys.stderr, flush=True)
        del A, B, C
        torch.cuda.empty_cache()
    print(json.dumps({"extra_shapes": out, "what": "library calls vs torch.mm + relu_, warm, context only"}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="untimed back-to-back launches for this long before the warmup steps: the shader "
                         "clock takes some 40-70 ms of full load to settle")
    ap.add_argument("--workload", default="square4096", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the secondary per-workload table")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB")
    ap.add_argument("--read-probe", type=int, default=0, metavar="MIB",
                    help="only time the library's HBM read probe on 4 rotating buffers of MIB MiB "
                         "(a multiple of 8)")
    ap.add_argument("--reps", type=int, default=100,
                    help="launches per variant in the per-workload table (back to back, and one event pair each)")
    ap.add_argument("--workload-settle-ms", type=float, default=100.0,
                    help="clock settling before each variant of the per-workload table")
    ap.add_argument("--no-oracle-table", action="store_true", help="skip the per-workload oracle timings")
    ap.add_argument("--no-sclk", action="store_true", help="skip the shader-clock reading (counter runs)")
    ap.add_argument("--rotate", type=int, default=1, metavar="COPIES",
                    help="the timed steps cycle through this many copies of B (4 x 256 MiB on the small-M "
                         "workload: every launch streams B from HBM)")
    ap.add_argument("--vendor-reference", action="store_true",
                    help="only time torch.mm + relu_ on the workloads (context, not the product)")
    ap.add_argument("--extra-shapes", action="store_true",
                    help="only time the library and torch.mm + relu_ on shapes beyond the workloads")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the product shards on N with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import dense_gemm_epilogue_tiled_amd as gr

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    gr.lib()  # fail loudly if the HIP library is missing

    if args.copy_probe:
        print(json.dumps(copy_probe(torch, args.copy_probe)))
        return
    if args.read_probe:
        print(json.dumps({"read_ceiling": read_ceiling(gr, torch, nbytes=args.read_probe << 20)}), flush=True)
        return
    if args.vendor_reference:
        vendor_reference(torch)
        return
    if args.extra_shapes:
        extra_shapes(gr, torch)
        return

    w = synth.WORKLOADS[args.workload]
    flops, nbytes = algorithmic(w)
    A, Bs, C = make_device_operands(torch, w, copies=max(1, args.rotate))
    stream = torch.cuda.current_stream()
    ws = workspace_for(gr, torch, w, A, Bs[0], C)
    runs = [launcher(gr, torch, w, A, B, C, stream, ws) for B in Bs]
    turn = [0]

    def run():
        runs[turn[0] % len(runs)]()
        turn[0] += 1
    plan = plan_for(gr, w, A, Bs[0], C, ws)

    settle_launches = settle(torch, run, args.settle_ms)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / args.steps

    value = flops * args.steps / wall / 1e12
    dominant_bound = "hbm" if flops / nbytes < MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
    src_hash = kernel_source_hash()
    if dominant_bound == "mfma":
        achieved = flops / (ev_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4)}
    else:
        achieved = nbytes / (ev_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic_for(args.workload, src_hash)
    roof["kernel_avg_us"] = round(ev_ms * 1e3, 2)
    sclk = None if args.no_sclk else observed_sclk(torch, run)
    if sclk and dominant_bound == "mfma":
        # the same achieved rate against the peak at the clock the chip held
        roof["observed_sclk_mhz"] = sclk
        peak_at_sclk = MFMA_F16_PEAK_TFLOPS * sclk / roofline.MI355X_PEAK_SCLK_MHZ
        roof["frac_at_observed_sclk"] = round(achieved / peak_at_sclk, 4)
    roof["algorithmic_flops"] = flops
    roof["algorithmic_bytes"] = nbytes
    del A, Bs, C, ws, run, runs
    torch.cuda.empty_cache()

    out = {
        "metric": "TFLOP/s fp16 GEMM+ReLU (fp32 acc) at 4096^3 on 1 GPU; % of MFMA/HBM roofline",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "settle_launches": settle_launches,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "layout": "row-major A(MxK) B(KxN) C(MxN)",
                   "b_copies_rotated": max(1, args.rotate),
                   "accumulate": "fp32", "path": plan["path_name"],
                   "tile": [plan["block_m"], plan["block_n"], plan["block_k"]], "grid": plan["grid"],
                   "threads": plan["threads"], "workspace_bytes": plan["workspace"],
                   "kernel_source_hash": src_hash},
        "roofline": roof,
    }

    if not args.no_workloads:
        ceiling = read_ceiling(gr, torch, settle_ms=args.workload_settle_ms)
        out["read_ceiling"] = ceiling
        out["copy_probe"] = copy_probe(torch, 1024)
        print("[bench] read ceiling %s" % (ceiling,), file=sys.stderr, flush=True)
        table = {}
        for name, wl in synth.WORKLOADS.items():
            table[name] = bench_workload(gr, torch, wl, max(args.reps, 1), args.workload_settle_ms, ceiling)
            print("[bench] %s %s" % (name, table[name]), file=sys.stderr, flush=True)
        out["workloads"] = table

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, max_seconds=15.0)
        if not args.no_oracle_table:
            out["cpu_oracle"] = cpu_oracle_table()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
