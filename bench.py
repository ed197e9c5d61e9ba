"""Benchmark of the quantised matmul hot path on one MI355X.

Headline: A8W8 8192 x 8192 x 8192 (int8 x int8 -> int32 -> fp32 scales ->
bf16), throughput in tera int8 ops per second, with inputs resident in HBM.
One step is one call of the operator on that batch.  The same run also times
the other rows of the path (decode-shaped A8W8 at M = 1, 4, 16 with
K = N = 8192 in GB/s, MatMulInteger, W8A32 and its gradient at M = 1 and 16
likewise, batched MatMulInteger 8 x 512 x 2048 x 2048, W8A32
4096^3, the two small parity shapes, A8W8 with an int32 accumulator input
at 8192^3 and at decode M = 16, MatMulInteger with per-row activation zero
points, the W8A32 input gradient at 4096^3, DynamicQuantizeLinear on the
[8, 512, 2048] fp32 activation and its chain into MatMulInteger, ConvInteger on
a 3x3 layer of 64 images) and reports them under "rows".
Decode and MatMulInteger rotate through enough distinct buffers (> 512 MiB)
that no call finds its inputs in the 256 MB Infinity Cache.

"ceilings" holds what this machine reaches on a streaming read of 1 GiB and
on an int8 matrix-core loop with random and with all-one operands (the
library's calibration kernels); each row also reports its fraction of the
matching measured ceiling beside the fraction of the spec peak.

After the GPU rows, the CPU oracle (plain loops, every host thread OpenMP
offers) runs once on each row's full workload; its time and rate go into the
row as "cpu_oracle" (the two small parity shapes also on one thread), and its
time on the whole 8192^3 headline workload is the top-level "cpu_baseline".
It is a reported baseline, not a target.

Prints one JSON line.  Options: --gpus N (only 1 is supported: the path
runs on one GPU), --steps K, --warmup W, --no-cpu-baseline, --only NAME.

HBM traffic of the headline kernel comes from hardware counters taken by
rocprofv3 (FETCH_SIZE, then WRITE_SIZE, each in its own run), scaled by what
the same counters read for a plain copy of known size (--copy-calibration
runs one).  --pmc-summary turns those four rocprofv3 databases into
profiles/traffic.json, stamped with a hash of the library sources; the
benchmark reports the traffic only while the sources still match.
"""
import argparse
import glob
import hashlib
import json
import os
import sqlite3
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # dense int8 matrix-core peak, tera-ops/s
PEAK_FP32_TFLOPS = 157.3     # dense fp32 matrix-core peak
PEAK_BF16_TFLOPS = 2500.0    # dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0        # HBM3E
COPY_BYTES = 256 << 20       # size of the calibration copy
CEIL_READ_BYTES = 1 << 30    # streaming-read ceiling: 1 GiB, four times the Infinity Cache
CEIL_MFMA_ROUNDS = 50        # matrix-core ceiling: 50 rounds = 215 G int8 ops per launch
CEIL_MFMA_F32_ROUNDS = 200   # fp32 matrix-core ceiling: 200 rounds = 53.7 G flops per launch
CEIL_MFMA_BF16_ROUNDS = 100  # bf16 matrix-core ceiling: 100 rounds = 215 G flops per launch
SPREAD_CALLS = 100           # single calls timed one by one for each row's median / p10 / p90
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


HEADLINE_SOURCES = ("int8_dma_impl.h", "int8_dma_256x256w8k128.hip", "device_common.h")


def source_hash(sources=HEADLINE_SOURCES):
    """sha256 over the sources a kernel is compiled from (default: the headline's)."""
    h = hashlib.sha256()
    for f in sorted(os.path.join(ROOT, "quantized_int8_gemm_amd", "csrc", n) for n in sources):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()


def _pmc_avg(db_dir, counter, match):
    """Average per dispatch of `counter` over kernels whose name contains `match`."""
    dbs = glob.glob(os.path.join(db_dir, "**", "*.db"), recursive=True)
    vals = []
    for db in dbs:
        c = sqlite3.connect(db)
        for name, v in c.execute("select kernel_name, value from counters_collection where counter_name = ?",
                                 (counter,)):
            if match in name:
                vals.append(float(v))
    if not vals:
        raise SystemExit(f"no {counter} samples for kernels matching {match!r} under {db_dir}")
    return sum(vals) / len(vals), len(vals)


def pmc_summary(args):
    """Write the traffic summary (profiles/traffic.json for the headline, or
    --traffic-out for another kernel) from four rocprofv3 --pmc runs."""
    fetch, nf = _pmc_avg(args.fetch_db, "FETCH_SIZE", args.kernel_match)
    write, nw = _pmc_avg(args.write_db, "WRITE_SIZE", args.kernel_match)
    cfetch, _ = _pmc_avg(args.copy_fetch_db, "FETCH_SIZE", "neg_kernel")
    cwrite, _ = _pmc_avg(args.copy_write_db, "WRITE_SIZE", "neg_kernel")
    f_scale = COPY_BYTES / (cfetch * 1024.0)
    w_scale = COPY_BYTES / (cwrite * 1024.0)
    traffic = fetch * 1024.0 * f_scale + write * 1024.0 * w_scale
    sources = tuple(args.sources.split(",")) if args.sources else HEADLINE_SOURCES
    out = {"kernel_match": args.kernel_match, "source_sha256": source_hash(sources), "sources": list(sources),
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "dispatches": [nf, nw],
           "copy_bytes": COPY_BYTES, "copy_fetch_kib": cfetch, "copy_write_kib": cwrite,
           "fetch_scale": f_scale, "write_scale": w_scale, "traffic_bytes_per_dispatch": traffic,
           "workload": args.workload}
    with open(args.traffic_out or TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def trace_summary(args):
    """Per-kernel statistics of a rocprofv3 kernel-trace csv (every dispatch)
    and, for the kernel named by --kernel-match, the mean over --window."""
    import csv
    durs = {}
    with open(args.trace_summary, newline="") as f:
        for r in csv.DictReader(f):
            durs.setdefault(r["Kernel_Name"], []).append(
                (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    out = {"kernels": []}
    for name, v in sorted(durs.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        ds = [d for _, d in v]
        out["kernels"].append({"kernel": name, "calls": len(ds), "total_us": sum(ds), "mean_us": sum(ds) / len(ds),
                               "min_us": min(ds), "max_us": max(ds)})
    hits = [k for k in durs if args.kernel_match in k]
    if hits and args.window:
        seq = [d for _, d in sorted(durs[hits[0]])]
        a, b = (int(x) if x else None for x in args.window.split(":"))
        w = seq[a:b]
        out["window"] = {"kernel": hits[0], "slice": args.window, "calls": len(w), "mean_us": sum(w) / len(w),
                         "min_us": min(w), "max_us": max(w)}
    print(json.dumps(out, indent=1))


def measured_traffic():
    """HBM bytes per launch from profiles/traffic.json, if the sources match."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except OSError:
        return None
    return t["traffic_bytes_per_dispatch"] if t.get("source_sha256") == source_hash() else None


def conv_workspace_bytes(q, N, C, H, W, M, kH, kW, pad=1):
    """Workspace of a stride-1 convolution padded by `pad` on every side."""
    import ctypes
    i64 = lambda *v: (ctypes.c_int64 * len(v))(*v)
    return int(q._binding.lib.conv_integer_workspace_bytes(N, C, H, W, M, kH, kW, 1, i64(pad, pad, pad, pad),
                                                           i64(1, 1), i64(1, 1)))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="time one row only (prefill, decode, mmi, acc, w8a32, dql, conv, small, ceilings)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--pmc-summary", action="store_true",
                    help="write profiles/traffic.json from rocprofv3 databases")
    ap.add_argument("--fetch-db")
    ap.add_argument("--write-db")
    ap.add_argument("--copy-fetch-db")
    ap.add_argument("--copy-write-db")
    ap.add_argument("--kernel-match", default="int8_dma_kernel<256, 256, 128, 64, 2, false, 1, 0, 0, 128, false>")
    ap.add_argument("--workload", default="a8w8_prefill_8192x8192x8192_bf16",
                    help="--pmc-summary: the workload the counters were taken on")
    ap.add_argument("--sources", default=None,
                    help="--pmc-summary: comma-separated csrc files of the kernel (default: the headline's)")
    ap.add_argument("--traffic-out", default=None,
                    help="--pmc-summary: output path (default profiles/traffic.json)")
    ap.add_argument("--trace-summary", default=None, metavar="KERNEL_TRACE_CSV",
                    help="summarise a rocprofv3 --kernel-trace csv: per-kernel dispatch statistics, and for "
                         "--kernel-match the mean over the dispatches in --window (a python slice of that "
                         "kernel's dispatches in start order)")
    ap.add_argument("--window", default=None,
                    help="--trace-summary: slice of the matching kernel's dispatches, e.g. -120:-100")
    return ap.parse_args()


SPIN_UP_S = 0.3


def progress(msg):
    """One line on stderr per finished step (stdout carries only the JSON line)."""
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def time_calls(fn, sets, steps, warmup, stream):
    """Average milliseconds per call over `steps` calls, cycling `sets`.

    Before the `warmup` calls the same call repeats, untimed, for SPIN_UP_S
    seconds: an idle GPU needs a few hundred milliseconds of load before its
    clocks settle, and a handful of 0.5 ms warm-up calls does not cover that
    (the first timed block then reads about 20% slow)."""
    import torch
    t_end = time.perf_counter() + SPIN_UP_S
    i = 0
    while time.perf_counter() < t_end:
        fn(sets[i % len(sets)])
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(sets[i % len(sets)])
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def _spread(vals_us):
    v = sorted(vals_us)
    pick = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    return {"n": len(v), "median_us": pick(0.5), "p10_us": pick(0.1), "p90_us": pick(0.9)}


def per_call_spread(fn, sets, n, stream):
    """Median, p10 and p90 of n single calls, each bracketed by its own HIP
    events on the launching stream (run after a row's timed block, so the
    calls find the clocks settled).  A call timed alone also carries its own
    launch gap, so for calls of a few tens of microseconds the median reads
    about 2 us above the back-to-back mean that "us" reports."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(sets[i % len(sets)])
        b.record(stream)
    torch.cuda.synchronize()
    return _spread([a.elapsed_time(b) * 1e3 for a, b in evs])


def time_graph(fn, sets, steps, replays, stream, spread=False):
    """Average milliseconds per call with `steps` calls captured in one HIP
    graph and the graph replayed `replays` times: the GPU's own time per call,
    without the per-call host work of an eager launch (which exceeds a
    15-microsecond kernel).  The calls must allocate nothing (pass out= and
    workspace=).  Spin-up and warm-up as in time_calls.  With spread=True it
    also returns the per-call spread over `replays` more replays, each timed
    on its own."""
    import torch
    t_end = time.perf_counter() + SPIN_UP_S
    i = 0
    while time.perf_counter() < t_end:
        fn(sets[i % len(sets)])
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(sets[i % len(sets)])
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(replays):
        g.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (replays * steps)
    if not spread:
        return ms
    # per-call time of each replay on its own (replay time / steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    for a, b in evs:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    return ms, _spread([a.elapsed_time(b) * 1e3 / steps for a, b in evs])


def cpu_oracle_rows(rows, si):
    """Time the CPU oracle (test infrastructure, plain loops on every host
    thread OpenMP offers) once on each measured row's full workload and
    attach the result to the row as "cpu_oracle"; the two small parity
    shapes are also timed on one thread.  Returns the top-level
    cpu_baseline: the whole 8192^3 A8W8 workload."""
    import oracle
    threads = oracle.threads()
    oracle.a8w8(*si.a8w8_inputs(4, 64, 64, seed=1))          # starts the thread pool

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def attach(name, dt, ops=None, nbytes=None, one_thread_s=None):
        progress(f"oracle {name}: {dt:.2f} s on {threads} threads")
        r = {"s": dt, "threads": threads}
        if ops is not None:
            r["TOPS"] = ops / dt / 1e12
            r["GOPS"] = ops / dt / 1e9
        if nbytes is not None:
            r["GB/s"] = nbytes / dt / 1e9
        if one_thread_s is not None:
            r["s_1thread"] = one_thread_s
            if ops is not None:
                r["GOPS_1thread"] = ops / one_thread_s / 1e9
        rows[name]["cpu_oracle"] = r

    def one_thread(fn):
        oracle.set_threads(1)
        try:
            return timed(fn)
        finally:
            oracle.set_threads(threads)

    baseline = None
    if "a8w8_prefill_8192_bf16" in rows:
        A, W, s_a, s_w = si.a8w8_inputs(8192, 8192, 8192, seed=505)
        dt = timed(lambda: oracle.a8w8(A, W, s_a, s_w))   # acc, fp32 and bf16 outputs in one pass
        ops = 2.0 * 8192 ** 3
        attach("a8w8_prefill_8192_bf16", dt, ops=ops)
        if "a8w8_prefill_8192_fp32" in rows:
            attach("a8w8_prefill_8192_fp32", dt, ops=ops)
        baseline = {"value": ops / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
                    "sample": f"the whole 8192x8192x8192 A8W8 workload, one oracle call ({dt:.1f} s)"}
        del A, W
    for m in (1, 4, 16, 64):
        name = f"a8w8_decode_m{m}_8192_bf16"
        if name in rows:
            A, W, s_a, s_w = si.a8w8_inputs(m, 8192, 8192, seed=404 + m)
            dt = timed(lambda: oracle.a8w8(A, W, s_a, s_w))
            attach(name, dt, ops=2.0 * m * 8192 * 8192,
                   nbytes=m * 8192 + 8192 * 8192 + 4 * m + 4 * 8192 + 2 * m * 8192)
    for m in (1, 4, 16):
        name = f"a8w8_decode_wnk_m{m}_8192_bf16"
        if name in rows:
            A, W, s_a, s_w = si.a8w8_inputs(m, 8192, 8192, seed=404 + m)
            Wt = np.ascontiguousarray(W.T)
            dt = timed(lambda: oracle.a8w8(A, Wt, s_a, s_w, b_trans=True))
            attach(name, dt, ops=2.0 * m * 8192 * 8192,
                   nbytes=m * 8192 + 8192 * 8192 + 4 * m + 4 * 8192 + 2 * m * 8192)
    for m in (1, 16):
        name = f"matmul_integer_decode_m{m}_8192"
        if name in rows:
            A, B, zb = si.matmul_integer_inputs(1, m, 8192, 8192, seed=450 + m)
            dt = timed(lambda: oracle.matmul_integer(A[0], B, 128, zb))
            attach(name, dt, ops=2.0 * m * 8192 * 8192, nbytes=m * 8192 + 8192 * 8192 + 8192 + 4 * m * 8192)
    mmi_ops = 2.0 * 8 * 512 * 2048 * 2048
    mmi_bytes = 8 * 512 * 2048 + 2048 * 2048 + 2048 + 4 * 8 * 512 * 2048
    if "matmul_integer_8x512x2048x2048" in rows:
        A, B, zb = si.matmul_integer_inputs(8, 512, 2048, 2048, seed=303)
        dt = timed(lambda: oracle.matmul_integer(A, B, 128, zb))
        attach("matmul_integer_8x512x2048x2048", dt, ops=mmi_ops, nbytes=mmi_bytes)
    if "a8w8_acc_prefill_8192_bf16" in rows:
        A, W, s_a, s_w = si.a8w8_inputs(8192, 8192, 8192, seed=505)
        acc = si.randint(si.rng(606), (8192, 8192), -2**20, 2**20, np.int32)
        dt = timed(lambda: oracle.a8w8_acc(acc, A, W, s_a, s_w))
        attach("a8w8_acc_prefill_8192_bf16", dt, ops=2.0 * 8192 ** 3)
        del A, W, acc
    if "a8w8_acc_decode_m16_8192_bf16" in rows:
        g = si.rng(606)
        si.randint(g, (8192, 8192), -2**20, 2**20, np.int32)   # the prefill row's draw comes first
        acc_m = si.randint(g, (16, 8192), -2**20, 2**20, np.int32)
        A, W, s_a, s_w = si.a8w8_inputs(16, 8192, 8192, seed=420)
        dt = timed(lambda: oracle.a8w8_acc(acc_m, A, W, s_a, s_w))
        attach("a8w8_acc_decode_m16_8192_bf16", dt, ops=2.0 * 16 * 8192 * 8192,
               nbytes=16 * 8192 + 8192 * 8192 + 4 * 16 + 4 * 8192 + 4 * 16 * 8192 + 2 * 16 * 8192)
    if "matmul_integer_row_zp_8x512x2048x2048" in rows:
        A, B, zb = si.matmul_integer_inputs(8, 512, 2048, 2048, seed=303)
        za = si.randint(si.rng(9), (512,), 0, 255, np.uint8)
        dt = timed(lambda: oracle.matmul_integer(A, B, za, zb))
        attach("matmul_integer_row_zp_8x512x2048x2048", dt, ops=mmi_ops)
    if "w8a32_4096" in rows:
        A, W = si.w8a32_inputs(4096, 4096, 4096, seed=506)
        dt = timed(lambda: oracle.w8a32(A, W, 0.01, -5))
        attach("w8a32_4096", dt, ops=2.0 * 4096 ** 3)
        if "w8a32_input_grad_4096" in rows:
            dC, _ = si.w8a32_inputs(4096, 4096, 4096, seed=507)
            dt = timed(lambda: oracle.w8a32_input_grad(dC, W, 0.01, -5))
            attach("w8a32_input_grad_4096", dt, ops=2.0 * 4096 ** 3)
    if "dynamic_quantize_linear_8x512x2048" in rows:
        x = si.dql_inputs((8, 512, 2048), seed=303)
        n = x.size
        dt = timed(lambda: oracle.dynamic_quantize_linear(x))
        attach("dynamic_quantize_linear_8x512x2048", dt, nbytes=4 * n + n + 4 + 1)
        if "dql_then_matmul_integer_8x512x2048x2048" in rows:
            _, B, zb = si.matmul_integer_inputs(1, 1, 2048, 2048, seed=303)

            def chain():
                y, _, zp = oracle.dynamic_quantize_linear(x)
                oracle.matmul_integer(y, B, int(zp), zb)
            attach("dql_then_matmul_integer_8x512x2048x2048", timed(chain), ops=mmi_ops)
    if "conv_integer_64x64x32x32_k3x3_m128" in rows:
        x, w, zw = si.conv_integer_inputs(64, 64, 32, 32, 128, 3, 3, seed=808)
        dt = timed(lambda: oracle.conv_integer(x, w, 128, zw, pads=(1, 1, 1, 1)))
        attach("conv_integer_64x64x32x32_k3x3_m128", dt, ops=2.0 * 64 * 128 * 32 * 32 * 64 * 9)
    if "a8w8_256x1024x1024_fp32" in rows:
        A, W, s_a, s_w = si.a8w8_inputs(256, 1024, 1024, seed=202)
        fn = lambda: oracle.a8w8(A, W, s_a, s_w)
        attach("a8w8_256x1024x1024_fp32", timed(fn), ops=2.0 * 256 * 1024 * 1024, one_thread_s=one_thread(fn))
    for m in (1, 16):
        name = f"w8a32_decode_m{m}_8192"
        if name in rows:
            A, W = si.w8a32_inputs(m, 8192, 8192, seed=520 + m)
            dC, _ = si.w8a32_inputs(m, 1, 8192, seed=530 + m)
            nbytes = 8192 * 8192 + 4 * m * 8192 * 2
            attach(name, timed(lambda: oracle.w8a32(A, W, 0.01, -5)), ops=2.0 * m * 8192 * 8192, nbytes=nbytes)
            gname = f"w8a32_input_grad_decode_m{m}_8192"
            if gname in rows:
                attach(gname, timed(lambda: oracle.w8a32_input_grad(dC, W, 0.01, -5)), ops=2.0 * m * 8192 * 8192,
                       nbytes=nbytes)
    if "w8a32_64x128x64" in rows:
        A, W = si.w8a32_inputs(64, 64, 128, seed=101)
        fn = lambda: oracle.w8a32(A, W, 0.02, 3)
        attach("w8a32_64x128x64", timed(fn), ops=2.0 * 64 * 64 * 128, one_thread_s=one_thread(fn))
    return baseline


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.trace_summary:
        trace_summary(args)
        return
    if args.copy_calibration:
        # an elementwise kernel that reads COPY_BYTES and writes COPY_BYTES
        import torch
        src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the kernels run on one GPU's share; see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_int8_gemm_amd as q
    import seeded_inputs as si

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    steps, warmup = args.steps, args.warmup
    rows = {}

    def to(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    def want(name):
        return args.only is None or args.only == name

    # ---- headline: A8W8 8192^3, bf16 out --------------------------------
    M = N = K = 8192
    A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=505)
    tA, tW, ta, tw = to(A), to(W), to(s_a), to(s_w)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    head_ms = None
    if want("prefill"):
        call = lambda s: q.qgemm_a8w8(tA, tW, ta, tw, out_dtype=torch.bfloat16, out=out)
        head_ms = time_calls(call, [None], steps, warmup, stream)
        kernel = q.last_kernel()
        ops = 2.0 * M * N * K
        tops = ops / (head_ms * 1e-3) / 1e12
        rows["a8w8_prefill_8192_bf16"] = {"kernel": kernel, "us": head_ms * 1e3, "TOPS": tops,
                                          "frac_int8_peak": tops / PEAK_INT8_TOPS,
                                          "per_call": per_call_spread(call, [None], SPREAD_CALLS, stream)}
        outf = torch.empty((M, N), dtype=torch.float32, device=dev)
        callf = lambda s: q.qgemm_a8w8(tA, tW, ta, tw, out=outf)
        ms = time_calls(callf, [None], steps, warmup, stream)
        rows["a8w8_prefill_8192_fp32"] = {"kernel": q.last_kernel(), "us": ms * 1e3, "TOPS": ops / (ms * 1e-3) / 1e12,
                                          "frac_int8_peak": ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS,
                                          "per_call": per_call_spread(callf, [None], SPREAD_CALLS, stream)}
        del outf
    del A, W

    progress(f"GPU rows so far: {sorted(rows)}")
    # ---- decode: M in {1, 4, 16}, K = N = 8192, bf16 out ---------------
    if want("decode"):
        # 9 rotating weight copies (576 MiB, beyond the 256 MB Infinity
        # Cache); timed as a replayed HIP graph of 36 calls (the GPU's time
        # per call) and as eager calls (bound by the host's per-call work)
        # and M = 64 (a batch of decode rows), past the decode kernel: the
        # tiled kernel with K split across workgroups
        for m in (1, 4, 16, 64):
            A, W, s_a, s_w = si.a8w8_inputs(m, 8192, 8192, seed=404 + m)
            base_w = to(W)
            sets = [(to(A), base_w if r == 0 else base_w.clone(), to(s_a), to(s_w),
                     torch.empty((m, 8192), dtype=torch.bfloat16, device=dev)) for r in range(9)]
            ws = torch.zeros(q.workspace_bytes(q.QG_OP_A8W8, 1, m, 8192, 8192), dtype=torch.uint8, device=dev)
            call = lambda s: q.qgemm_a8w8(s[0], s[1], s[2], s[3], out_dtype=torch.bfloat16, out=s[4], workspace=ws)
            ms_eager = time_calls(call, sets, max(steps * 5, 50), warmup * 2, stream)
            ms, spread = time_graph(call, sets, 36, max(steps // 2, 5), stream, spread=True)
            nbytes = m * 8192 + 8192 * 8192 + 4 * m + 4 * 8192 + 2 * m * 8192
            gbs = nbytes / (ms * 1e-3) / 1e9
            rows[f"a8w8_decode_m{m}_8192_bf16"] = {"kernel": q.last_kernel(), "us": ms * 1e3, "GB/s": gbs,
                                                   "frac_hbm_peak": gbs / PEAK_HBM_GBS, "timing": "hip_graph",
                                                   "us_eager": ms_eager * 1e3, "per_call": spread}
            del sets, base_w, ws
        # The same decode rows with the weight stored as [N,K] (b_trans, the
        # usual layout of a linear layer's weight): whole columns per
        # workgroup, no split-K exchange, no workspace
        for m in (1, 4, 16):
            A, W, s_a, s_w = si.a8w8_inputs(m, 8192, 8192, seed=404 + m)
            base_w = to(np.ascontiguousarray(W.T))
            sets = [(to(A), base_w if r == 0 else base_w.clone(), to(s_a), to(s_w),
                     torch.empty((m, 8192), dtype=torch.bfloat16, device=dev)) for r in range(9)]
            call = lambda s: q.qgemm_a8w8(s[0], s[1], s[2], s[3], out_dtype=torch.bfloat16, b_trans=True, out=s[4])
            ms, spread = time_graph(call, sets, 36, max(steps // 2, 5), stream, spread=True)
            nbytes = m * 8192 + 8192 * 8192 + 4 * m + 4 * 8192 + 2 * m * 8192
            gbs = nbytes / (ms * 1e-3) / 1e9
            rows[f"a8w8_decode_wnk_m{m}_8192_bf16"] = {"kernel": q.last_kernel(), "us": ms * 1e3, "GB/s": gbs,
                                                       "frac_hbm_peak": gbs / PEAK_HBM_GBS, "timing": "hip_graph",
                                                       "per_call": spread}
            del sets, base_w
        # MatMulInteger at decode shapes (uint8 activations with zero point
        # 128, int8 weight with per-column zero points), same rotation
        for m in (1, 16):
            A, B, zb = si.matmul_integer_inputs(1, m, 8192, 8192, seed=450 + m)
            base_b, tzb = to(B), to(zb)
            sets = [(to(A[0]), base_b if r == 0 else base_b.clone(),
                     torch.empty((m, 8192), dtype=torch.int32, device=dev)) for r in range(9)]
            ws = torch.zeros(q.workspace_bytes(q.QG_OP_MATMUL_INTEGER, 1, m, 8192, 8192), dtype=torch.uint8,
                             device=dev)
            call = lambda s: q.matmul_integer(s[0], s[1], 128, tzb, out=s[2], workspace=ws)
            ms, spread = time_graph(call, sets, 36, max(steps // 2, 5), stream, spread=True)
            nbytes = m * 8192 + 8192 * 8192 + 8192 + 4 * m * 8192
            gbs = nbytes / (ms * 1e-3) / 1e9
            rows[f"matmul_integer_decode_m{m}_8192"] = {"kernel": q.last_kernel(), "us": ms * 1e3, "GB/s": gbs,
                                                        "frac_hbm_peak": gbs / PEAK_HBM_GBS, "timing": "hip_graph",
                                                        "per_call": spread}
            del sets, base_b, ws

    progress(f"GPU rows so far: {sorted(rows)}")
    # ---- MatMulInteger 8 x 512 x 2048 x 2048, shared B -------------------
    if want("mmi"):
        A, B, zb = si.matmul_integer_inputs(8, 512, 2048, 2048, seed=303)
        tB, tzb = to(B), to(zb)
        sets = [(to(A), torch.empty((8, 512, 2048), dtype=torch.int32, device=dev)) for _ in range(13)]
        call = lambda s: q.matmul_integer(s[0], tB, 128, tzb, out=s[1])
        ms = time_calls(call, sets, max(steps * 5, 50), warmup * 2, stream)
        ops = 2.0 * 8 * 512 * 2048 * 2048
        nbytes = 8 * 512 * 2048 + 2048 * 2048 + 2048 + 4 * 8 * 512 * 2048
        rows["matmul_integer_8x512x2048x2048"] = {
            "kernel": q.last_kernel(), "us": ms * 1e3, "TOPS": ops / (ms * 1e-3) / 1e12,
            "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "frac_int8_peak": ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS,
            "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "per_call": per_call_spread(call, sets, SPREAD_CALLS, stream)}
        del sets

    progress(f"GPU rows so far: {sorted(rows)}")
    # ---- A8W8 with an int32 accumulator input; per-row MatMulInteger zp --
    if want("acc"):
        M = N = K = 8192
        A, W, s_a, s_w = si.a8w8_inputs(M, N, K, seed=505)
        tA, tW, ta, tw = to(A), to(W), to(s_a), to(s_w)
        del A, W
        g = si.rng(606)
        acc = torch.from_numpy(si.randint(g, (M, N), -2**20, 2**20, np.int32)).to(dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        calla = lambda s: q.qgemm_a8w8_acc(acc, tA, tW, ta, tw, out_dtype=torch.bfloat16, out=out)
        ms = time_calls(calla, [None], steps, warmup, stream)
        ops = 2.0 * M * N * K
        rows["a8w8_acc_prefill_8192_bf16"] = {"kernel": q.last_kernel(), "us": ms * 1e3,
                                              "TOPS": ops / (ms * 1e-3) / 1e12,
                                              "frac_int8_peak": ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS,
                                              "per_call": per_call_spread(calla, [None], SPREAD_CALLS, stream)}
        del acc, out, tA, tW
        m = 16
        A, W, s_a, s_w = si.a8w8_inputs(m, 8192, 8192, seed=404 + m)
        base_w = to(W)
        acc_m = torch.from_numpy(si.randint(g, (m, 8192), -2**20, 2**20, np.int32)).to(dev)
        sets = [(to(A), base_w if r == 0 else base_w.clone(), to(s_a), to(s_w),
                 torch.empty((m, 8192), dtype=torch.bfloat16, device=dev)) for r in range(9)]
        ws = torch.zeros(q.workspace_bytes(q.QG_OP_A8W8, 1, m, 8192, 8192), dtype=torch.uint8, device=dev)
        call = lambda s: q.qgemm_a8w8_acc(acc_m, s[0], s[1], s[2], s[3], out_dtype=torch.bfloat16, out=s[4],
                                          workspace=ws)
        ms, spread = time_graph(call, sets, 36, max(steps // 2, 5), stream, spread=True)
        nbytes = m * 8192 + 8192 * 8192 + 4 * m + 4 * 8192 + 4 * m * 8192 + 2 * m * 8192
        rows["a8w8_acc_decode_m16_8192_bf16"] = {"kernel": q.last_kernel(), "us": ms * 1e3,
                                                 "GB/s": nbytes / (ms * 1e-3) / 1e9,
                                                 "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                 "timing": "hip_graph", "per_call": spread}
        del sets, base_w, ws
        A, B, zb = si.matmul_integer_inputs(8, 512, 2048, 2048, seed=303)
        za = to(si.randint(g, (512,), 0, 255, np.uint8))
        tB, tzb = to(B), to(zb)
        sets = [(to(A), torch.empty((8, 512, 2048), dtype=torch.int32, device=dev)) for _ in range(13)]
        call = lambda s: q.matmul_integer(s[0], tB, za, tzb, out=s[1])
        ms = time_calls(call, sets, max(steps * 5, 50), warmup * 2, stream)
        ops = 2.0 * 8 * 512 * 2048 * 2048
        rows["matmul_integer_row_zp_8x512x2048x2048"] = {
            "kernel": q.last_kernel(), "us": ms * 1e3, "TOPS": ops / (ms * 1e-3) / 1e12,
            "frac_int8_peak": ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS,
            "per_call": per_call_spread(call, sets, SPREAD_CALLS, stream)}
        del sets

    progress(f"GPU rows so far: {sorted(rows)}")
    # ---- W8A32 4096^3 -----------------------------------------------------
    if want("w8a32"):
        A, W = si.w8a32_inputs(4096, 4096, 4096, seed=506)
        tA, tW = to(A), to(W)
        outc = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
        fl = 2.0 * 4096 ** 3

        def w8a32_row(call):
            ms = time_calls(call, [None], steps, warmup, stream)
            kern = q.last_kernel()
            r = {"kernel": kern, "us": ms * 1e3, "TFLOPS": fl / (ms * 1e-3) / 1e12,
                 "frac_fp32_peak": fl / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
                 "per_call": per_call_spread(call, [None], SPREAD_CALLS, stream)}
            if "bf16x3" in kern:
                # the exact three-way split: three bf16 products per algorithmic one
                r["matrix_cores"] = "bf16, fp32 operand split exactly in three"
                r["frac_bf16_peak_3x"] = 3 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
            else:
                r["matrix_cores"] = "fp32"
            return r

        callw = lambda s: q.qgemm_w8a32(tA, tW, 0.01, -5, out=outc)
        rows["w8a32_4096"] = w8a32_row(callw)
        # its input gradient: dA = dC @ ((W - zp) * scale)^T, same weight
        dC, _ = si.w8a32_inputs(4096, 4096, 4096, seed=507)
        tdC = to(dC)
        callg = lambda s: q.qgemm_w8a32_input_grad(tdC, tW, 0.01, -5, out=outc)
        rows["w8a32_input_grad_4096"] = w8a32_row(callg)
        # the same two calls on the fp32 matrix cores, for comparison
        prev = os.environ.get("QGEMM_W8A32")
        os.environ["QGEMM_W8A32"] = "fp32"
        try:
            rows["w8a32_4096_fp32_cores"] = w8a32_row(callw)
            rows["w8a32_input_grad_4096_fp32_cores"] = w8a32_row(callg)
        finally:
            if prev is None:
                os.environ.pop("QGEMM_W8A32", None)
            else:
                os.environ["QGEMM_W8A32"] = prev
        del A, W, tA, tW, outc, dC, tdC
        # decode-sized W8A32 and its gradient (M = 1, 16 at N = K = 8192),
        # graph-timed over 9 rotating weights like the int8 decode rows
        for m in (1, 16):
            A, W = si.w8a32_inputs(m, 8192, 8192, seed=520 + m)
            dC, _ = si.w8a32_inputs(m, 1, 8192, seed=530 + m)
            base_w = to(W)
            sets = [(to(A), base_w if r == 0 else base_w.clone(), to(dC),
                     torch.empty((m, 8192), dtype=torch.float32, device=dev)) for r in range(9)]
            nbytes = 8192 * 8192 + 4 * m * 8192 * 2
            for grad, name in ((False, f"w8a32_decode_m{m}_8192"), (True, f"w8a32_input_grad_decode_m{m}_8192")):
                ws = torch.zeros(max(q.workspace_bytes(q.QG_OP_W8A32_INPUT_GRAD if grad else q.QG_OP_W8A32,
                                                       1, m, 8192, 8192), 256), dtype=torch.uint8, device=dev)
                if grad:
                    call = lambda s: q.qgemm_w8a32_input_grad(s[2], s[1], 0.01, -5, out=s[3], workspace=ws)
                else:
                    call = lambda s: q.qgemm_w8a32(s[0], s[1], 0.01, -5, out=s[3], workspace=ws)
                ms, spread = time_graph(call, sets, 36, max(steps // 2, 5), stream, spread=True)
                gbs = nbytes / (ms * 1e-3) / 1e9
                rows[name] = {"kernel": q.last_kernel(), "us": ms * 1e3, "GB/s": gbs,
                              "frac_hbm_peak": gbs / PEAK_HBM_GBS, "timing": "hip_graph", "per_call": spread}
                del ws
            del sets, base_w

    progress(f"GPU rows so far: {sorted(rows)}")
    # ---- DynamicQuantizeLinear on [8, 512, 2048] fp32, and its chain ----
    if want("dql"):
        shape = (8, 512, 2048)
        n = 8 * 512 * 2048
        x = si.dql_inputs(shape, seed=303)
        sets = [(to(x), torch.empty(shape, dtype=torch.uint8, device=dev)) for _ in range(13)]
        call = lambda s: q.dynamic_quantize_linear(s[0], out=s[1])
        ms = time_calls(call, sets, max(steps * 5, 50), warmup * 2, stream)
        nbytes = 4 * n + n + 4 + 1          # read x, write y (the scalars)
        gbs = nbytes / (ms * 1e-3) / 1e9
        rows["dynamic_quantize_linear_8x512x2048"] = {"kernel": q.last_kernel(), "us": ms * 1e3, "GB/s": gbs,
                                                     "frac_hbm_peak": gbs / PEAK_HBM_GBS,
                                                     "per_call": per_call_spread(call, sets, SPREAD_CALLS, stream)}
        # fp32 activations -> uint8 + zero point (on the device) -> MatMulInteger
        _, B, zb = si.matmul_integer_inputs(1, 1, 2048, 2048, seed=303)
        tB, tzb = to(B), to(zb)
        sets = [(s[0], s[1], torch.empty((8, 512, 2048), dtype=torch.int32, device=dev)) for s in sets]

        def chain(s):
            y, _, zp = q.dynamic_quantize_linear(s[0], out=s[1])
            q.matmul_integer(y, tB, zp.reshape(1), tzb, out=s[2])
        ms = time_calls(chain, sets, max(steps * 5, 50), warmup * 2, stream)
        ops = 2.0 * 8 * 512 * 2048 * 2048
        rows["dql_then_matmul_integer_8x512x2048x2048"] = {"kernels": "dql + " + q.last_kernel(), "us": ms * 1e3,
                                                          "TOPS": ops / (ms * 1e-3) / 1e12,
                                                          "per_call": per_call_spread(chain, sets, SPREAD_CALLS, stream)}
        del sets, x

    progress(f"GPU rows so far: {sorted(rows)}")
    # ---- ConvInteger: a 3x3 tokenizer-sized layer -------------------------
    if want("conv"):
        N_, C_, H_, W_, M_ = 64, 64, 32, 32, 128
        x, w, zw = si.conv_integer_inputs(N_, C_, H_, W_, M_, 3, 3, seed=808)
        tw, tzw = to(w), to(zw)
        sets = [(to(x), torch.empty((N_, M_, H_, W_), dtype=torch.int32, device=dev)) for _ in range(13)]
        ws = torch.empty(conv_workspace_bytes(q, N_, C_, H_, W_, M_, 3, 3), dtype=torch.uint8, device=dev)
        call = lambda s: q.conv_integer(s[0], tw, 128, tzw, pads=(1, 1, 1, 1), out=s[1], workspace=ws)
        ms = time_calls(call, sets, max(steps * 5, 50), warmup * 2, stream)
        ops = 2.0 * N_ * M_ * H_ * W_ * C_ * 9
        nbytes = N_ * C_ * H_ * W_ + M_ * C_ * 9 + M_ + 4 * N_ * M_ * H_ * W_
        rows["conv_integer_64x64x32x32_k3x3_m128"] = {"kernels": q.last_kernel(), "us": ms * 1e3,
                                                     "TOPS": ops / (ms * 1e-3) / 1e12,
                                                     "GB/s": nbytes / (ms * 1e-3) / 1e9,
                                                     "frac_int8_peak": ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS,
                                                     "per_call": per_call_spread(call, sets, SPREAD_CALLS, stream)}
        del sets, ws

    progress(f"GPU rows so far: {sorted(rows)}")
    # ---- the small parity shapes (launch-latency bound) ------------------
    if want("small"):
        A, W, s_a, s_w = si.a8w8_inputs(256, 1024, 1024, seed=202)
        sA, sW, sa, sw = to(A), to(W), to(s_a), to(s_w)
        o = torch.empty((256, 1024), dtype=torch.float32, device=dev)
        call = lambda s: q.qgemm_a8w8(sA, sW, sa, sw, out=o)
        ms_eager = time_calls(call, [None], 100, 10, stream)
        ms, spread = time_graph(call, [None], 50, 10, stream, spread=True)
        rows["a8w8_256x1024x1024_fp32"] = {"kernel": q.last_kernel(), "us": ms * 1e3, "timing": "hip_graph",
                                           "us_eager": ms_eager * 1e3, "per_call": spread}
        A, W = si.w8a32_inputs(64, 64, 128, seed=101)
        wA, wW = to(A), to(W)
        o = torch.empty((64, 64), dtype=torch.float32, device=dev)
        call = lambda s: q.qgemm_w8a32(wA, wW, 0.02, 3, out=o)
        ms_eager = time_calls(call, [None], 100, 10, stream)
        ms, spread = time_graph(call, [None], 50, 10, stream, spread=True)
        rows["w8a32_64x128x64"] = {"kernel": q.last_kernel(), "us": ms * 1e3, "timing": "hip_graph",
                                   "us_eager": ms_eager * 1e3, "per_call": spread}

    progress(f"GPU rows so far: {sorted(rows)}")
    # ---- measured ceilings: streaming read, int8 matrix-core loop -------
    ceilings = None
    if args.only is None or args.only == "ceilings":
        buf = torch.randint(0, 256, (CEIL_READ_BYTES,), dtype=torch.uint8, device=dev)
        ms = time_calls(lambda s: q.calib_read(buf), [None], steps, warmup, stream)
        hbm = CEIL_READ_BYTES / (ms * 1e-3) / 1e9
        del buf
        g = si.rng(7)
        rnd = to(si.randint(g, (4096,), -128, 127, np.int8))
        ones = torch.ones(4096, dtype=torch.int8, device=dev)
        mf = {}
        for name, opnd, shape in (("random", rnd, "16x16x64"), ("ones", ones, "16x16x64"),
                                  ("random_32x32x32", rnd, "32x32x32")):
            nops = q.calib_mfma_i8(opnd, CEIL_MFMA_ROUNDS, shape=shape)
            ms = time_calls(lambda s, o=opnd, sh=shape: q.calib_mfma_i8(o, CEIL_MFMA_ROUNDS, shape=sh), [None],
                            steps, warmup, stream)
            mf[name] = nops / (ms * 1e-3) / 1e12
        # fp32 matrix-core loop (the W8A32 kernels' instruction), operands uniform in [-1, 1)
        f32ops = to(si.rng(8).uniform(-1.0, 1.0, size=1024).astype(np.float32))
        nfl = q.calib_mfma_f32(f32ops, CEIL_MFMA_F32_ROUNDS)
        ms = time_calls(lambda s: q.calib_mfma_f32(f32ops, CEIL_MFMA_F32_ROUNDS), [None], steps, warmup, stream)
        mf32 = nfl / (ms * 1e-3) / 1e12
        # bf16 matrix-core loop (the W8A32 split's instruction), operands uniform in [-1, 1)
        bfops = to(si.rng(9).uniform(-1.0, 1.0, size=2048).astype(np.float32)).to(torch.bfloat16)
        nbf = q.calib_mfma_bf16(bfops, CEIL_MFMA_BF16_ROUNDS)
        ms = time_calls(lambda s: q.calib_mfma_bf16(bfops, CEIL_MFMA_BF16_ROUNDS), [None], steps, warmup, stream)
        mbf = nbf / (ms * 1e-3) / 1e12
        ceilings = {"hbm_read_GBs": hbm, "mfma_i8_random_TOPS": mf["random"], "mfma_i8_ones_TOPS": mf["ones"],
                    "mfma_i8_32x32x32_random_TOPS": mf["random_32x32x32"],
                    "mfma_f32_random_TFLOPS": mf32, "mfma_bf16_random_TFLOPS": mbf,
                    "note": "streaming read of 1 GiB; int8 matrix-core loop (v_mfma_i32_16x16x64_i8, the GEMM "
                            "kernels' instruction) on random / all-one operands, and with v_mfma_i32_32x32x32_i8 "
                            "on the random operands; fp32 and bf16 matrix-core loops on operands uniform in [-1, 1)"}
        for name, r in rows.items():
            if "GB/s" in r and "frac_hbm_peak" in r and "_decode_" in name:
                r["frac_hbm_read_ceiling"] = r["GB/s"] / hbm
            if "TOPS" in r:
                r["frac_mfma_random_ceiling"] = r["TOPS"] / mf["random"]
            if "TFLOPS" in r and r.get("matrix_cores", "fp32") == "fp32":
                r["frac_mfma_f32_ceiling"] = r["TFLOPS"] / mf32
            if "frac_bf16_peak_3x" in r:
                r["frac_mfma_bf16_ceiling_3x"] = 3 * r["TFLOPS"] / mbf

    progress(f"GPU rows so far: {sorted(rows)}")
    # ---- CPU baseline: the oracle beside every row ------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_oracle_rows(rows, si)

    line = {
        "metric": "int8 GEMM TOPS and skinny-M GB/s; % of MI355X int8 MFMA / HBM peak",
        "value": rows.get("a8w8_prefill_8192_bf16", {}).get("TOPS"),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "a8w8_prefill_8192x8192x8192_bf16", "M": 8192, "N": 8192, "K": 8192,
                   "out_dtype": "bf16", "parallelism": "single_gpu"},
    }
    if head_ms is not None:
        tops = rows["a8w8_prefill_8192_bf16"]["TOPS"]
        line["roofline"] = {"kernel": rows["a8w8_prefill_8192_bf16"]["kernel"], "bound": "mfma",
                            "achieved": tops, "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                            "frac": tops / PEAK_INT8_TOPS, "traffic": measured_traffic()}
        if ceilings is not None:
            line["roofline"]["measured_ceiling"] = ceilings["mfma_i8_random_TOPS"]
            line["roofline"]["frac_measured_ceiling"] = tops / ceilings["mfma_i8_random_TOPS"]
    line["ceilings"] = ceilings
    line["cpu_baseline"] = cpu
    line["rows"] = rows
    print(json.dumps(line))


if __name__ == "__main__":
    main()
