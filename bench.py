#!/usr/bin/env python3
"""Benchmark of the QPN weight-streaming skinny GEMM on one MI355X.

Headline workload (one "step"): the NVFP4 skinny GEMM at the two decoder
shapes K=5120 -> N=17408 (gate/up-like) and K=17408 -> N=5120 (down-like),
each at M = 1, 4 and 8 activation rows: six qpn_gemm_nvfp4 calls through the
C ABI.  Weights are synthetic N(0, 0.02) packed on the GPU; every call reads a
different packed copy (>= 1 GiB of copies per shape) so the 256 MB Infinity
Cache cannot serve the weights.  Inputs are resident in HBM before timing.

The launches of the timed region are recorded once into a HIP graph (through
torch.cuda.CUDAGraph, on the stream the library launches on) and replayed, so
host launch overhead stays out of the measurement; the graph holds exactly
`--steps` steps.

value = algorithmic weight bytes of one step (codes + UE4M3 scales + the
4-byte tensor scale of each call) / wall time of one step, in GB/s (1e9 B/s).

breakdown: each headline call's launch time (median, p10 and p90 over 15
replays of a graph of 44 back-to-back launches), GB/s and % of 8 TB/s.
configs: the metric's other configurations, timed the same way in every run
and not part of `value`: NVFP4 2048x2048 at M=1; FP8 K=5120 -> N=6144 and
N=5120 at M = 1, 2, 4; one decoder layer at M=8 (QKV and O FP8, gate/up and
down NVFP4), each GEMM and the four back to back; the 151936-row NVFP4
lm_head with its fused argmax at M = 1 and 8.

roofline: the dominant kernel (largest share of the step).  Its average
launch duration is timed with HIP events around a graph of back-to-back
launches of that call (rotating copies) on the launch stream; achieved =
its algorithmic bytes per launch / that average.  traffic comes from the
committed rocprofv3 PMC summary when it matches the current kernel source.

cpu_baseline: the FP64 oracle (test infrastructure, C with OpenMP over rows)
computing complete headline steps (all six calls, every row) on every thread
for about eight seconds, then a bounded one-thread sample; with the host CPU
model.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--extra] [--no-cpu-baseline]
    python bench.py --traffic-workload | --contraction-ab | --prefill-workload   (profiling)
    python bench.py --summarize-traffic FETCH_CSV WRITE_CSV   (profiles/traffic.json from the PMC passes)
    python bench.py --summarize-sq AB_CSV AB_JSON HEAD_CSV BENCH_JSON   (SQ counter tables)
    python bench.py --summarize-trace KERNEL_TRACE_CSV   (per-kernel median / p10 / p90 durations)
    python bench.py --summarize-pmc COUNTER_CSV [MATCH]   (per-kernel counter averages)
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, decimal GB/s
ROTATE_BYTES = 1 << 30          # >= 1 GiB of distinct packed copies per shape
METRIC = "effective weight GB/s and % of HBM peak, NVFP4 & FP8 skinny GEMM at M=1/8"
BATCH = 44                      # launches per per-call timing graph (2 rotations)

HEADLINE = [  # (name, n, k, format)
    ("gate_up_K5120_N17408", 17408, 5120, "nvfp4"),
    ("down_K17408_N5120", 5120, 17408, "nvfp4"),
]
HEADLINE_M = (1, 4, 8)

# The other configurations of the metric, timed in every run and reported
# under "configs" (the headline value is the NVFP4 step above):
# the small NVFP4 GEMV, the FP8 skinny GEMMs, one decoder layer at M = 8 and
# the lm_head with its fused argmax.
CONFIGS = [
    ("cfg1_nvfp4_K2048_N2048", 2048, 2048, "nvfp4", (1,)),
    ("cfg3_fp8_K5120_N6144", 6144, 5120, "fp8", (1, 2, 4)),
    ("cfg3_fp8_K5120_N5120", 5120, 5120, "fp8", (1, 2, 4)),
]
LMHEAD = ("cfg5_lmhead_nvfp4_K5120_N151936", 151936, 5120)
# One decoder layer's four projections at M = 8, back to back: QKV and O in
# FP8, gate/up and down in NVFP4 (213,368,840 weight bytes per layer).  Each
# GEMM draws its weights with its own seed (0, 1, 2, 3 in this order).
LAYER = [("qkv_fp8_K5120_N7168", 7168, 5120, "fp8"), ("o_fp8_K5120_N5120", 5120, 5120, "fp8"),
         ("gateup_nvfp4_K5120_N34816", 34816, 5120, "nvfp4"),
         ("down_nvfp4_K17408_N5120", 5120, 17408, "nvfp4")]
EXTRA = [  # measured only with --extra
    ("fp8_K5120_N6144", 6144, 5120, "fp8", (8,)),
    ("fp8_K5120_N5120", 5120, 5120, "fp8", (8,)),
]
# The same layer with its FP8 projections converted to NVFP4 (all-FP4, the
# derived-checkpoint variant: 0.5625 instead of 1 byte per QKV/O weight).
LAYER_ALLFP4 = [("qkv_fp8>nvfp4_K5120_N7168", 7168, 5120, "fp8>nvfp4"),
                ("o_fp8>nvfp4_K5120_N5120", 5120, 5120, "fp8>nvfp4")] + LAYER[2:]
# The same layer's per-rank shards under 4-way tensor parallelism (column-
# parallel QKV and gate/up split N, row-parallel O and down split K), and the
# per-rank lm_head vocabulary shard, each on one GPU.
TP4 = [("tp4_qkv_fp8_K5120_N1792", 1792, 5120, "fp8"), ("tp4_o_fp8_K1280_N5120", 5120, 1280, "fp8"),
       ("tp4_gateup_nvfp4_K5120_N8704", 8704, 5120, "nvfp4"),
       ("tp4_down_nvfp4_K4352_N5120", 5120, 4352, "nvfp4")]
TP4_LMHEAD = ("tp4_lmhead_nvfp4_K5120_N37984", 37984, 5120, "nvfp4")
# Prefill-sized activation blocks through the tiled MFMA kernel.
PREFILL = [("prefill_gate_up_nvfp4_K5120_N17408", 17408, 5120, "nvfp4", (16, 32, 64, 128, 256)),
           ("prefill_down_nvfp4_K17408_N5120", 5120, 17408, "nvfp4", (16, 32, 64, 128, 256)),
           ("prefill_fp8_K5120_N6144", 6144, 5120, "fp8", (32, 64, 128, 256)),
           ("prefill_fp8_K5120_N5120", 5120, 5120, "fp8", (32, 64, 128, 256))]
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16 matrix peak


def algo_bytes(n, k, fmt):
    """Bytes the method must read once: codes + scales (+ 4-byte tensor scale)."""
    if fmt == "nvfp4":
        return n * k // 2 + n * k // 16 + 4
    return n * k + 4 * n


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("qpn_gemm.hip", "qpn_common.h"):
        with open(os.path.join(HERE, "fp8_quantized_skinny_qpn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Shape:
    def __init__(self, qpn, torch, name, n, k, fmt, ms, seed=0):
        from fp8_quantized_skinny_qpn_amd import synth
        self.name, self.n, self.k, self.fmt, self.ms = name, n, k, fmt, ms
        w = torch.from_numpy(synth.weights(n, k, seed=seed)).cuda()
        if fmt == "fp8>nvfp4":  # FP8 weights converted to NVFP4 (the derived checkpoint)
            pw = qpn.requant_fp8_to_nvfp4(qpn.pack_fp8(w))
            fmt = self.fmt = "nvfp4"
        else:
            pw = qpn.pack_nvfp4(w) if fmt == "nvfp4" else qpn.pack_fp8(w)
        del w
        self.copies = [pw] + [pw.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / pw.nbytes)) - 1)]
        self.x = torch.from_numpy(synth.activations(8, k, seed=seed)).cuda()
        self.y = {m: torch.empty((m, n), dtype=torch.float16, device="cuda") for m in ms}
        self.xm = {m: self.x[:m].contiguous() for m in ms}
        self.bytes = algo_bytes(n, k, fmt)
        op = qpn.OP_GEMM_NVFP4 if fmt == "nvfp4" else qpn.OP_GEMM_FP8
        # split-K workspace, zero-filled once (the library keeps it zeroed)
        self.ws = torch.zeros(max(256, max((qpn.workspace_bytes(op, m, n, k) for m in ms), default=0)),
                              dtype=torch.uint8, device="cuda")
        self.i = 0

    def next_copy(self):
        pw = self.copies[self.i]
        self.i = (self.i + 1) % len(self.copies)
        return pw


def one_step(qpn, shapes):
    """One pass: every (shape, M) call once, each on the next rotated copy."""
    for s in shapes:
        for m in s.ms:
            qpn.gemm(s.next_copy(), s.xm[m], out=s.y[m], ws=s.ws)


def capture(torch, fn):
    """Record the launches fn() makes into a graph (on torch's capture stream,
    which is the stream the library launches on)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps):
    """Per-replay times (s) of graph g, measured with HIP events on the stream
    the graph is replayed on."""
    out = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1) * 1e-3)
    return out


def time_call(qpn, torch, s, m, batch=BATCH, reps=15, plan=0):
    """Average launch time (s) of one (shape, M) call in each of `reps`
    replays of a graph of `batch` back-to-back launches (rotating copies)."""
    g = capture(torch, lambda: [qpn.gemm(s.next_copy(), s.xm[m], out=s.y[m], ws=s.ws, plan=plan)
                                for _ in range(batch)])
    g.replay()
    torch.cuda.synchronize()
    per = [t / batch for t in time_graph(torch, g, reps)]
    del g
    return per


def call_stats(per, nbytes):
    """Per-call figures from per-replay averages: median, p10 and p90 (over
    the replays), effective weight GB/s and % of 8 TB/s at the median."""
    med = float(np.median(per))
    return {"us": round(med * 1e6, 3),
            "us_p10": round(float(np.percentile(per, 10)) * 1e6, 3),
            "us_p90": round(float(np.percentile(per, 90)) * 1e6, 3),
            "GBps": round(nbytes / med / 1e9, 1),
            "pct_hbm_peak": round(100 * nbytes / med / 1e9 / HBM_PEAK_GBPS, 1),
            "weight_bytes": nbytes}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# rows of each headline weight the 1-thread oracle sample computes
CPU_1T_ROWS = 512


def cpu_baseline(min_seconds=8.0):
    """The FP64 oracle (test infrastructure, C, OpenMP over output rows):
    complete headline steps on every thread of this process, repeated until
    about min_seconds of wall time, then a bounded one-thread sample (the
    first CPU_1T_ROWS output rows of each of the six headline calls, scaled
    by their weight bytes)."""
    import oracle
    from fp8_quantized_skinny_qpn_amd import synth
    packed = []
    for name, n, k, _ in HEADLINE:
        w = synth.weights(n, k, seed=0)
        codes, scales, g = oracle.pack_nvfp4(w)
        del w
        packed.append((name, n, k, codes, scales, g, synth.activations(8, k, seed=0)))
    threads = oracle.threads()
    steps, total_t = 0, 0.0
    while total_t < min_seconds or steps == 0:
        for name, n, k, codes, scales, g, x8 in packed:
            for m in HEADLINE_M:
                t = time.perf_counter()
                oracle.gemm_nvfp4(codes, scales, g, x8[:m])
                total_t += time.perf_counter() - t
        steps += 1
    step_bytes = sum(algo_bytes(n, k, "nvfp4") for _, n, k, *_ in packed) * len(HEADLINE_M)
    # one thread, a row sample of every call
    oracle.set_threads(1)
    t1, b1 = 0.0, 0
    try:
        for name, n, k, codes, scales, g, x8 in packed:
            r = min(CPU_1T_ROWS, n)
            c, sc = np.ascontiguousarray(codes[:r]), np.ascontiguousarray(scales[:r])
            for m in HEADLINE_M:
                t = time.perf_counter()
                oracle.gemm_nvfp4(c, sc, g, x8[:m])
                t1 += time.perf_counter() - t
                b1 += r * k // 2 + r * k // 16
    finally:
        oracle.set_threads(threads)
    return {
        "value": round(step_bytes * steps / total_t / 1e9, 6),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{steps} complete headline step(s) (6 calls, every row) on the FP64 oracle "
                   f"(C, OpenMP over rows, {threads} threads), {total_t:.1f} s of wall time; "
                   f"packing untimed"),
        "value_1thread": round(b1 / t1 / 1e9, 6),
        "sample_1thread": (f"the first {CPU_1T_ROWS} output rows of each of the 6 headline calls "
                           f"on one thread, {t1:.1f} s, weight bytes of those rows"),
    }


def traffic_for(kernel_name):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None
    when it is absent or was taken on a different kernel source."""
    path = os.path.join(HERE, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(kernel_name)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def read_ceiling(qpn, torch):
    """Measured read ceiling: nontemporal 16-byte loads streaming a 2 GiB
    buffer (far larger than the 256 MB Infinity Cache)."""
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(2):
        qpn.debug_read_ceiling(buf, sink)
    g = capture(torch, lambda: qpn.debug_read_ceiling(buf, sink))
    ts = time_graph(torch, g, 7)
    del g, buf
    torch.cuda.empty_cache()
    return (2 << 30) / float(np.median(ts)) / 1e9


def read_ceiling_call(qpn, torch, nbytes):
    """Read ceiling at one call's size: the same streaming read over nbytes
    (rounded down to 16), on rotating regions of >= 1 GiB in all, timed like
    a GEMM call (average launch time in back-to-back graphs).  Returns
    (seconds per launch, bytes read)."""
    nb = nbytes // 256 * 256
    regions = max(2, math.ceil(ROTATE_BYTES / nb))
    buf = torch.empty(regions * nb, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    views = [buf[i * nb:(i + 1) * nb] for i in range(regions)]
    g = capture(torch, lambda: [qpn.debug_read_ceiling(views[i % regions], sink) for i in range(BATCH)])
    g.replay()
    torch.cuda.synchronize()
    per = [t / BATCH for t in time_graph(torch, g, 5)]
    del g, views, buf
    torch.cuda.empty_cache()
    return float(np.median(per)), nb


def traffic_workload(qpn, torch):
    """Workload for the rocprofv3 PMC passes (FETCH_SIZE, WRITE_SIZE), one per
    run: calibration kernels of known size (a 256 MiB streaming read and a
    256 MiB fill), then each headline call six times on rotating copies."""
    cal = 256 << 20
    buf = torch.empty(cal, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(3):
        qpn.debug_read_ceiling(buf, sink)
    for _ in range(3):
        buf.zero_()
    torch.cuda.synchronize()
    del buf
    for name, n, k, fmt in HEADLINE:
        s = Shape(qpn, torch, name, n, k, fmt, HEADLINE_M)
        for m in s.ms:
            for _ in range(6):
                qpn.gemm(s.next_copy(), s.xm[m], out=s.y[m], ws=s.ws)
            torch.cuda.synchronize()
            log(f"{name} M={m}: {qpn.kernel_name(fmt, m, n, k)}")
        del s
        torch.cuda.empty_cache()


def summarize_traffic(fetch_csv, write_csv):
    """Turn the two rocprofv3 PMC passes of --traffic-workload (FETCH_SIZE and
    WRITE_SIZE counter_collection CSVs) into per-launch HBM bytes: each
    counter is scaled by what it reads for the calibration kernel of known
    size (the 256 MiB streaming read for FETCH_SIZE, the 256 MiB fill for
    WRITE_SIZE), and the GEMM launches are assigned, in order, six to each
    headline call.  Writes profiles/traffic.json (tagged with the kernel
    source hash, so bench.py reports it only while the kernel is unchanged)
    and prints the markdown table of the traffic summary."""
    import csv
    cal = 256 << 20

    def rows(path, counter):
        out = []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]) * 1024))
        out.sort()
        return out

    def factor(rs, pick):
        vals = [v for _, name, v in rs if pick(name)]
        if not vals:
            raise SystemExit("calibration kernel not found")
        return cal / float(np.median(vals))

    fr, wr = rows(fetch_csv, "FETCH_SIZE"), rows(write_csv, "WRITE_SIZE")
    f_fac = factor(fr, lambda n: "read_ceiling_kernel" in n)
    w_fac = factor(wr, lambda n: "FillFunctor<unsigned char>" in n)
    calls = [f"{name}_M{m}" for name, _, _, _ in HEADLINE for m in HEADLINE_M]
    gf = [(name, v * f_fac) for _, name, v in fr if "skinny_gemm_kernel" in name]
    gw = [(name, v * w_fac) for _, name, v in wr if "skinny_gemm_kernel" in name]
    if len(gf) != 6 * len(calls) or len(gw) != 6 * len(calls):
        raise SystemExit(f"expected {6 * len(calls)} GEMM launches, got {len(gf)} / {len(gw)}")
    per_kernel = {}
    lines = ["| call | kernel | HBM read MB | HBM write MB | read / algorithmic |", "|---|---|---:|---:|---:|"]
    hsh = kernel_source_hash()
    for i, call in enumerate(calls):
        kname = gf[6 * i][0].split("(")[0].replace("void ", "")
        rd = float(np.mean([v for _, v in gf[6 * i:6 * i + 6]]))
        wt = float(np.mean([v for _, v in gw[6 * i:6 * i + 6]]))
        n, k = next((n, k) for name, n, k, _ in HEADLINE if call.startswith(name))
        ab = algo_bytes(n, k, "nvfp4")
        lines.append(f"| {call} | `{kname}` | {rd / 1e6:.3f} | {wt / 1e6:.3f} | {rd / ab:.3f} |")
        e = per_kernel.setdefault(kname, {"source_hash": hsh, "calls": [], "read_bytes": [], "write_bytes": []})
        e["calls"].append(call)
        e["read_bytes"].append(int(round(rd)))
        e["write_bytes"].append(int(round(wt)))
    for e in per_kernel.values():
        e["bytes_per_launch"] = int(round(np.mean(e["read_bytes"]) + np.mean(e["write_bytes"])))
    with open(os.path.join(HERE, "profiles", "traffic.json"), "w") as fh:
        json.dump(per_kernel, fh, indent=1)
        fh.write("\n")
    print(f"FETCH_SIZE factor {f_fac:.4f}, WRITE_SIZE factor {w_fac:.4f}")
    print("\n".join(lines))


def summarize_trace(trace_csv):
    """Launch durations from a rocprofv3 kernel-trace CSV per kernel and grid
    size (one call shape): count, mean, median, p10, p90, min and max in
    microseconds, as markdown lines, longest total time first."""
    import csv
    per = {}
    with open(trace_csv) as fh:
        for r in csv.DictReader(fh):
            name = (r["Kernel_Name"].replace("(anonymous namespace)", "{anon}")
                    .split("(")[0].replace("void ", ""))
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            per.setdefault((name, int(r["Grid_Size_X"])), []).append(dur)
    out = ["| kernel | grid threads | launches | mean us | median us | p10 us | p90 us | min us | max us |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for (name, grid), d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(d)
        out.append(f"| `{name}` | {grid} | {a.size} | {a.mean():.3f} | {np.median(a):.3f} | "
                   f"{np.percentile(a, 10):.3f} | {np.percentile(a, 90):.3f} | {a.min():.3f} | "
                   f"{a.max():.3f} |")
    return out


def summarize_pmc(counter_csv, match=""):
    """Per-kernel averages of every counter in a rocprofv3 PMC pass (one
    row per kernel name and grid size whose name contains `match`), as
    markdown lines."""
    import csv
    per, order = {}, []
    with open(counter_csv) as fh:
        for r in csv.DictReader(fh):
            name = (r["Kernel_Name"].replace("(anonymous namespace)", "{anon}")
                    .split("(")[0].replace("void ", ""))
            if match not in name:
                continue
            key = (name, int(r["Grid_Size"]))
            if key not in per:
                per[key] = {}
                order.append(key)
            per[key].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    counters = sorted({c for d in per.values() for c in d})
    out = ["| kernel | grid threads | " + " | ".join(counters) + " |",
           "|---|---:|" + "---:|" * len(counters)]
    for key in order:
        d = per[key]
        vals = [f"{np.mean(d[c]):,.0f}" if c in d else "" for c in counters]
        out.append(f"| `{key[0]}` | {key[1]} | " + " | ".join(vals) + " |")
    return out


def prefill_calls():
    """The (call, m) pairs of --prefill-workload, in launch order; each is
    launched six times in a row."""
    return [(name, n, k, m) for name, n, k, fmt, ms in PREFILL for m in ms]


def summarize_prefill(trace_csv, counter_csvs):
    """The --prefill-workload runs: one row per (call, m) with its kernel,
    median launch time and TFLOP/s from the kernel trace, and the average of
    each counter of the given PMC passes of the same workload.  The GEMM
    dispatches of each run are taken in dispatch order, six per call."""
    import csv

    def gemm_dispatches(path, kind):
        rows = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = (r["Kernel_Name"].replace("(anonymous namespace)", "{anon}")
                        .split("(")[0].replace("void ", ""))
                if "gemm_kernel" not in name:
                    continue
                d = rows.setdefault(int(r["Dispatch_Id"]), {"kernel": name})
                if kind == "trace":
                    d["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
                else:
                    d[r["Counter_Name"]] = float(r["Counter_Value"])
        return [rows[i] for i in sorted(rows)]

    calls = prefill_calls()
    trace = gemm_dispatches(trace_csv, "trace")
    if len(trace) != 6 * len(calls):
        raise SystemExit(f"{trace_csv}: {len(trace)} GEMM dispatches, expected {6 * len(calls)}")
    passes = [gemm_dispatches(c, "pmc") for c in counter_csvs]
    for c, rows in zip(counter_csvs, passes):
        if len(rows) != len(trace):
            raise SystemExit(f"{c}: {len(rows)} GEMM dispatches, expected {len(trace)}")
    counters = [sorted(k for k in rows[0] if k != "kernel") for rows in passes]
    head = ["call", "m", "kernel", "median us", "TFLOP/s"] + [c for cs in counters for c in cs]
    out = ["| " + " | ".join(head) + " |", "|---|---:|---|" + "---:|" * (len(head) - 3)]
    for i, (name, n, k, m) in enumerate(calls):
        block = trace[6 * i: 6 * i + 6]
        us = float(np.median([d["us"] for d in block]))
        vals = []
        for rows, cs in zip(passes, counters):
            b = rows[6 * i: 6 * i + 6]
            vals += [f"{np.mean([d.get(c, 0.0) for d in b]):,.0f}" for c in cs]
        out.append(f"| {name} | {m} | `{block[0]['kernel']}` | {us:.1f} | {2.0 * m * n * k / us / 1e6:.0f} | "
                   + " | ".join(vals) + " |")
    return out


SQ_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES")


def summarize_sq(counter_csv, rows):
    """Per-call SQ counter averages from a rocprofv3 PMC pass: the GEMM
    dispatches form one contiguous run per row of `rows` (call, kernel, us),
    in order; counters are averaged over a run's dispatches.  Busy fractions
    use the row's time at the 2.4 GHz engine clock: VALU busy =
    SQ_ACTIVE_INST_VALU / (256 CUs x cycles), MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles).  Returns markdown lines."""
    import csv
    per = {}
    with open(counter_csv) as fh:
        for r in csv.DictReader(fh):
            d = per.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    runs = []
    for did in sorted(per):
        d = per[did]
        if "skinny_gemm_kernel" not in d["kernel"]:
            continue
        if runs and runs[-1][0] == d["kernel"]:
            runs[-1][1].append(d)
        else:
            runs.append((d["kernel"], [d]))
    if len(runs) != len(rows):
        raise SystemExit(f"{len(runs)} GEMM dispatch runs for {len(rows)} calls")
    out = ["| call | contraction | kernel | us | VALU insts / launch | MFMA insts / launch | VALU busy % | MFMA busy % |",
           "|---|---|---|---:|---:|---:|---:|---:|"]
    for (kname, ds), row in zip(runs, rows):
        short = kname.split("(")[0].replace("void ", "")
        if short != row["kernel"]:
            raise SystemExit(f"dispatch run {short} does not match {row['kernel']}")
        avg = {c: float(np.mean([d.get(c, 0.0) for d in ds])) for c in SQ_COUNTERS}
        cycles = row["us"] * 1e-6 * 2.4e9
        out.append(f"| {row['call']} | {row.get('contraction', 'mfma')} | `{short}` | {row['us']:.2f} | "
                   f"{avg['SQ_INSTS_VALU']:,.0f} | {avg['SQ_INSTS_MFMA']:,.0f} | "
                   f"{100 * avg['SQ_ACTIVE_INST_VALU'] / (256 * cycles):.1f} | "
                   f"{100 * avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * cycles):.1f} |")
    return out


# The contraction A/B: plans 1 and 2 (MFMA) against plans 12 and 11, the same
# launch shapes contracting with VALU dot products instead.
CONTRACTION_AB = ((1, 1, 12), (8, 2, 11))  # (M, MFMA plan, VALU-dot plan)


def contraction_ab(qpn, torch):
    """Headline shapes at M = 1 and 8 through the MFMA plan and its VALU-dot
    twin: six launches each (for the PMC passes), then the time of each in
    back-to-back graphs.  Prints one JSON line."""
    rows = []
    for name, n, k, fmt in HEADLINE:
        s = Shape(qpn, torch, name, n, k, fmt, (1, 8))
        # room for every forced plan's K splits
        s.ws = torch.zeros(max(qpn.workspace_bytes(qpn.OP_GEMM_NVFP4, m, n, k, plan=p)
                               for m, a, b in CONTRACTION_AB for p in (a, b)) + 256,
                           dtype=torch.uint8, device="cuda")
        for m, p_mfma, p_vdot in CONTRACTION_AB:
            for plan in (p_mfma, p_vdot):
                for _ in range(6):
                    qpn.gemm(s.next_copy(), s.xm[m], out=s.y[m], ws=s.ws, plan=plan)
                torch.cuda.synchronize()
                med = float(np.median(time_call(qpn, torch, s, m, plan=plan)))
                kname = qpn.kernel_name(fmt, m, n, k, plan=plan)
                log(f"{name} M={m} plan {plan}: {med * 1e6:.2f} us  {kname}")
                rows.append({"call": f"{name}_M{m}", "plan": plan, "kernel": kname,
                             "contraction": "valu_dot" if plan == p_vdot else "mfma",
                             "us": round(med * 1e6, 3), "GBps": round(s.bytes / med / 1e9, 1)})
        del s
        torch.cuda.empty_cache()
    print(json.dumps({"contraction_ab": rows}), flush=True)


def prefill_workload(qpn, torch):
    """Workload for profiling the prefill kernel: each PREFILL call and block
    size six times on rotating copies."""
    from fp8_quantized_skinny_qpn_amd import synth
    for name, n, k, fmt, ms in PREFILL:
        sh = Shape(qpn, torch, name, n, k, fmt, ())
        xs = torch.from_numpy(synth.activations(256, k, seed=0, m_max=256)).cuda()
        for m in ms:
            xm = xs[:m].contiguous()
            ym = torch.empty((m, n), dtype=torch.float16, device="cuda")
            for _ in range(6):
                qpn.prefill(sh.next_copy(), xm, out=ym)
            torch.cuda.synchronize()
            log(f"{name} M={m}")
        del sh, xs
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--extra", action="store_true", help="also time the other configurations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from the two PMC passes of --traffic-workload")
    ap.add_argument("--summarize-sq", nargs=4, metavar=("AB_CSV", "AB_JSON", "HEAD_CSV", "BENCH_JSON"),
                    help="SQ counter tables from the PMC passes of --contraction-ab and "
                         "--traffic-workload and the JSON lines of --contraction-ab and bench.py")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="per-kernel duration statistics from a rocprofv3 kernel trace")
    ap.add_argument("--summarize-pmc", nargs="+", metavar=("COUNTER_CSV", "MATCH"),
                    help="per-kernel counter averages from a rocprofv3 PMC pass (optionally only "
                         "kernels whose name contains MATCH)")
    ap.add_argument("--summarize-prefill", nargs="+", metavar=("KERNEL_TRACE_CSV", "COUNTER_CSV"),
                    help="per-call table of the --prefill-workload runs: trace times and the "
                         "counters of any PMC passes of the same workload")
    ap.add_argument("--traffic-workload", action="store_true",
                    help="only run the workload of the PMC traffic passes (no JSON line)")
    ap.add_argument("--prefill-workload", action="store_true",
                    help="only run the prefill calls (for profiling; no JSON line)")
    ap.add_argument("--contraction-ab", action="store_true",
                    help="only time the headline calls with MFMA and with VALU-dot contraction")
    args = ap.parse_args()

    if args.summarize_traffic:  # host only: post-processes rocprofv3 output
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_pmc:  # host only: post-processes rocprofv3 output
        print("\n".join(summarize_pmc(*args.summarize_pmc[:2])))
        return
    if args.summarize_prefill:  # host only: post-processes rocprofv3 output
        print("\n".join(summarize_prefill(args.summarize_prefill[0], args.summarize_prefill[1:])))
        return
    if args.summarize_trace:  # host only: post-processes rocprofv3 output
        print("\n".join(summarize_trace(args.summarize_trace)))
        return
    if args.summarize_sq:  # host only: post-processes rocprofv3 output
        ab_csv, ab_json, head_csv, bench_json = args.summarize_sq
        ab = json.loads(open(ab_json).read().strip().splitlines()[-1])["contraction_ab"]
        bl = json.loads(open(bench_json).read().strip().splitlines()[-1])["breakdown"]
        head = [{"call": c, "kernel": v["kernel"], "us": v["us"]} for c, v in bl.items()]
        print("\n".join(["MFMA against VALU dot:"] + summarize_sq(ab_csv, ab) +
                        ["", "Headline calls:"] + summarize_sq(head_csv, head)))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}): the QPN skinny "
              "GEMM is measured on one MI355X; sharding across GPUs is a design note only.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from fp8_quantized_skinny_qpn_amd import qpn  # fails loudly when libqpn.so is missing
    if args.traffic_workload:
        traffic_workload(qpn, torch)
        return
    if args.contraction_ab:
        contraction_ab(qpn, torch)
        return
    if args.prefill_workload:
        prefill_workload(qpn, torch)
        return

    log("setting up headline shapes")
    shapes = [Shape(qpn, torch, name, n, k, fmt, HEADLINE_M) for name, n, k, fmt in HEADLINE]
    for _ in range(2):
        one_step(qpn, shapes)
    torch.cuda.synchronize()

    # warmup and timed graphs hold exactly W and K steps
    g_warm = capture(torch, lambda: [one_step(qpn, shapes) for _ in range(max(1, args.warmup))])
    g_timed = capture(torch, lambda: [one_step(qpn, shapes) for _ in range(args.steps)])
    if args.warmup > 0:
        g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_timed.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del g_warm, g_timed
    step_s = (t1 - t0) / args.steps
    step_bytes = sum(s.bytes * len(s.ms) for s in shapes)
    value = step_bytes / step_s / 1e9

    # per-call launch times of the headline calls
    breakdown, per_kernel = {}, {}
    for s in shapes:
        for m in s.ms:
            per = time_call(qpn, torch, s, m)
            kname = qpn.kernel_name(s.fmt, m, s.n, s.k, lmhead=False)
            breakdown[f"{s.name}_M{m}"] = {"kernel": kname, **call_stats(per, s.bytes),
                                           "rotated_copies": len(s.copies)}
            k = per_kernel.setdefault(kname, {"t": [], "bytes": s.bytes, "calls": []})
            k["t"] += per
            k["calls"].append(f"{s.name}_M{m}")
    dom = max(per_kernel, key=lambda kn: float(np.mean(per_kernel[kn]["t"])) * len(per_kernel[kn]["calls"]))
    dk = per_kernel[dom]
    avg_s = float(np.mean(dk["t"]))
    achieved = dk["bytes"] / avg_s / 1e9
    del shapes
    torch.cuda.empty_cache()

    configs = time_configs(qpn, torch)
    extra = time_extra(qpn, torch) if args.extra else {}

    ceiling = read_ceiling(qpn, torch)
    call_s, call_b = read_ceiling_call(qpn, torch, dk["bytes"])

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 1),
        "read_ceiling_GBps": round(ceiling, 1),
        "pct_read_ceiling": round(100 * value / ceiling, 1),
        "config": {
            "workload": "nvfp4_skinny_gemm K5120->N17408 and K17408->N5120, M in {1,4,8}",
            "calls_per_step": len(HEADLINE) * len(HEADLINE_M),
            "weights": "NVFP4 (E2M1 codes, UE4M3 per 16-K block, FP32 tensor scale) packed from N(0,0.02) fp32, seed 0",
            "activations": "fp16 N(0,1), seed 0",
            "step_weight_bytes": step_bytes,
            "timing": "HIP graph of exactly `steps` steps, replayed once between device synchronisations",
            "per_call_timing": (f"median, p10 and p90 over 15 replays of a graph of {BATCH} back-to-back "
                                "launches on rotating copies (>= 1 GiB per shape)"),
            "plans": {f"{name}_M{m}": qpn.gemm_plan(qpn.OP_GEMM_NVFP4, m, n, k).__dict__
                      for name, n, k, _ in HEADLINE for m in HEADLINE_M},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "calls": dk["calls"],
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_for(dom),
            "algorithmic_bytes_per_launch": dk["bytes"],
            "avg_launch_us": round(avg_s * 1e6, 3),
            "launches_timed": len(dk["t"]) * BATCH,
            # the same streaming read at this call's size: what any single
            # launch of this many bytes reaches on this GPU
            "read_ceiling_at_call_size": {"bytes": call_b, "us": round(call_s * 1e6, 3),
                                          "GBps": round(call_b / call_s / 1e9, 1),
                                          "frac_hbm_peak": round(call_b / call_s / 1e9 / HBM_PEAK_GBPS, 4)},
            "frac_of_read_ceiling_at_call_size": round(achieved / (call_b / call_s / 1e9), 4),
        },
        "cpu_baseline": cpu,
        "breakdown": breakdown,
        "configs": configs,
    }
    if extra:
        out["extra_configs"] = extra
    print(json.dumps(out), flush=True)


def time_configs(qpn, torch):
    """The other configurations of the metric, timed in every run: the small
    NVFP4 GEMV, the FP8 calls, one decoder layer at M = 8 (each GEMM and the
    four back to back) and the lm_head with its fused argmax at M = 1 and 8."""
    from fp8_quantized_skinny_qpn_amd import synth
    out = {}
    for name, n, k, fmt, ms in CONFIGS:
        log(f"config: {name}")
        sh = Shape(qpn, torch, name, n, k, fmt, ms)
        for m in ms:
            out[f"{name}_M{m}"] = {"kernel": qpn.kernel_name(fmt, m, n, k),
                                   **call_stats(time_call(qpn, torch, sh, m), sh.bytes)}
        del sh
        torch.cuda.empty_cache()
    # cfg4: the layer, each GEMM alone and the four back to back
    log("config: cfg4 layer at M=8")
    lshapes = [Shape(qpn, torch, name, n, k, fmt, (8,), seed=i)
               for i, (name, n, k, fmt) in enumerate(LAYER)]
    for sh in lshapes:
        out[f"cfg4_{sh.name}_M8"] = {"kernel": qpn.kernel_name(sh.fmt, 8, sh.n, sh.k),
                                     **call_stats(time_call(qpn, torch, sh, 8), sh.bytes)}
    out["cfg4_layer_M8"] = {"calls": [sh.name for sh in lshapes],
                            **call_stats(time_layer(qpn, torch, lshapes), sum(sh.bytes for sh in lshapes))}
    del lshapes
    torch.cuda.empty_cache()
    # cfg5: the lm_head with the fused argmax
    name, n, k = LMHEAD
    log(f"config: {name}")
    w = torch.from_numpy(synth.weights(n, k, seed=0)).cuda()
    pw = qpn.pack_nvfp4(w)
    del w
    torch.cuda.empty_cache()
    copies = [pw] + [pw.clone() for _ in range(2)]
    x8 = torch.from_numpy(synth.activations(8, k, seed=0)).cuda()
    b = algo_bytes(n, k, "nvfp4")
    for m in (1, 8):
        xm = x8[:m].contiguous()
        lg = torch.empty((m, n), dtype=torch.float16, device="cuda")
        am = torch.empty((m,), dtype=torch.int32, device="cuda")
        ws = torch.zeros(qpn.workspace_bytes(qpn.OP_LMHEAD_NVFP4, m, n, k), dtype=torch.uint8, device="cuda")
        qpn.lmhead_nvfp4(copies[0], xm, lg, am, ws)
        g = capture(torch, lambda: [qpn.lmhead_nvfp4(copies[i % 3], xm, lg, am, ws) for i in range(12)])
        per = [t / 12 for t in time_graph(torch, g, 15)]
        del g
        out[f"{name}_M{m}"] = {"kernels": [qpn.kernel_name("nvfp4", m, n, k, lmhead=True),
                                           "qpn::argmax_finalize_kernel"],
                               **call_stats(per, b)}
    del copies, pw
    torch.cuda.empty_cache()
    return out


def time_layer(qpn, torch, lshapes, reps=15):
    """Per-replay average time (s) of one layer: the GEMMs of lshapes back
    to back at M = 8, in graphs of BATCH // 4 layers on rotating copies."""
    g = capture(torch, lambda: [qpn.gemm(sh.next_copy(), sh.xm[8], out=sh.y[8], ws=sh.ws)
                                for _ in range(BATCH // 4) for sh in lshapes])
    g.replay()
    torch.cuda.synchronize()
    per = [t / (BATCH // 4) for t in time_graph(torch, g, reps)]
    del g
    return per


def time_extra(qpn, torch):
    """--extra: FP8 at M = 8, the lm_head without argmax and with the fused
    verification, the per-rank shard shapes under 4-way tensor parallelism,
    prefill-sized blocks and the all-FP4 layer."""
    from fp8_quantized_skinny_qpn_amd import synth
    extra = {}
    for name, n, k, fmt, ms in EXTRA:
        log(f"extra: {name}")
        sh = Shape(qpn, torch, name, n, k, fmt, ms)
        for m in ms:
            extra[f"{name}_M{m}"] = {"kernel": qpn.kernel_name(fmt, m, n, k),
                                     **call_stats(time_call(qpn, torch, sh, m), sh.bytes)}
        del sh
        torch.cuda.empty_cache()
    name, n, k = LMHEAD
    log(f"extra: {name}")
    w = torch.from_numpy(synth.weights(n, k, seed=0)).cuda()
    pw = qpn.pack_nvfp4(w)
    del w
    torch.cuda.empty_cache()
    copies = [pw] + [pw.clone() for _ in range(2)]
    x8 = torch.from_numpy(synth.activations(8, k, seed=0)).cuda()
    b = algo_bytes(n, k, "nvfp4")
    for m in (1, 8):
        xm = x8[:m].contiguous()
        lg = torch.empty((m, n), dtype=torch.float16, device="cuda")
        am = torch.empty((m,), dtype=torch.int32, device="cuda")
        ws = torch.zeros(qpn.workspace_bytes(qpn.OP_LMHEAD_NVFP4, m, n, k), dtype=torch.uint8, device="cuda")
        # the same weights through the plain GEMM (no argmax), for the argmax's share
        g = capture(torch, lambda: [qpn.gemm(copies[i % 3], xm, out=lg) for i in range(12)])
        per = [t / 12 for t in time_graph(torch, g, 5)]
        del g
        extra[f"{name}_gemm_only_M{m}"] = call_stats(per, b)
        # the lm_head of a k = m - 1 draft verify round, acceptance fused
        if m > 1:
            draft = torch.zeros((m - 1,), dtype=torch.int32, device="cuda")
            res = torch.empty((2,), dtype=torch.int32, device="cuda")
            qpn.lmhead_verify_nvfp4(copies[0], xm, draft, lg, am, res, ws)
            g = capture(torch, lambda: [qpn.lmhead_verify_nvfp4(copies[i % 3], xm, draft, lg, am, res, ws)
                                        for i in range(12)])
            per = [t / 12 for t in time_graph(torch, g, 5)]
            del g
            extra[f"{name}_verify_M{m}"] = call_stats(per, b)
    del copies, pw
    torch.cuda.empty_cache()
    # per-rank (TP=4) shard shapes, one call at a time
    for name, n, k, fmt in TP4 + [TP4_LMHEAD]:
        log(f"extra: {name}")
        sh = Shape(qpn, torch, name, n, k, fmt, (1, 8))
        for m in (1, 8):
            extra[f"{name}_M{m}"] = {"kernel": qpn.kernel_name(fmt, m, n, k),
                                     **call_stats(time_call(qpn, torch, sh, m, reps=5), sh.bytes)}
        del sh
        torch.cuda.empty_cache()
    # prefill-sized blocks: time, matrix-unit rate and weight rate
    for name, n, k, fmt, ms in PREFILL:
        log(f"extra: {name}")
        sh = Shape(qpn, torch, name, n, k, fmt, ())
        xs = torch.from_numpy(synth.activations(256, k, seed=0, m_max=256)).cuda()
        op = qpn.OP_PREFILL_NVFP4 if fmt == "nvfp4" else qpn.OP_PREFILL_FP8
        ws = torch.zeros(max(256, max(qpn.workspace_bytes(op, m, n, k) for m in ms)),
                         dtype=torch.uint8, device="cuda")
        for m in ms:
            xm = xs[:m].contiguous()
            ym = torch.empty((m, n), dtype=torch.float16, device="cuda")
            qpn.prefill(sh.next_copy(), xm, out=ym, ws=ws)
            g = capture(torch, lambda: [qpn.prefill(sh.next_copy(), xm, out=ym, ws=ws) for _ in range(16)])
            per = [t / 16 for t in time_graph(torch, g, 5)]
            del g
            med = float(np.median(per))
            tf = 2.0 * m * n * k / med / 1e12
            pl = qpn.gemm_plan(op, m, n, k)
            extra[f"{name}_M{m}"] = {**call_stats(per, sh.bytes), "TFLOPs": round(tf, 1),
                                     "pct_mfma_f16_peak": round(100 * tf / MFMA_F16_PEAK_TFLOPS, 1),
                                     "workgroups": pl.workgroups, "splits": pl.splits}
        del sh, xs, ws
        torch.cuda.empty_cache()
    # whole layers at M = 8: the all-FP4 variant and the per-rank shards
    for lname, layer in (("layer_allfp4_M8", LAYER_ALLFP4), ("tp4_layer_M8", TP4)):
        log(f"extra: {lname}")
        lshapes = [Shape(qpn, torch, name, n, k, fmt, (8,), seed=i)
                   for i, (name, n, k, fmt) in enumerate(layer)]
        extra[lname] = {"calls": [sh.name for sh in lshapes],
                        **call_stats(time_layer(qpn, torch, lshapes, reps=5), sum(sh.bytes for sh in lshapes))}
        del lshapes
        torch.cuda.empty_cache()
    return extra


if __name__ == "__main__":
    main()
