#!/usr/bin/env python3
"""Benchmark of the QPN weight-streaming skinny GEMM on one MI355X.

Headline workload (one "step"): the NVFP4 skinny GEMM at the two decoder
shapes K=5120 -> N=17408 (gate/up-like) and K=17408 -> N=5120 (down-like),
each at M = 1, 4 and 8 activation rows: six qpn_gemm_nvfp4 calls through the
C ABI.  Weights are synthetic N(0, 0.02) packed on the GPU; every call reads a
different packed copy (>= 1 GiB of copies per shape) so the 256 MB Infinity
Cache cannot serve the weights.  Inputs are resident in HBM before timing.

value = algorithmic weight bytes of one step (codes + UE4M3 scales + the
4-byte tensor scale of each call) / time of one step, in GB/s (1e9 B/s).
The roofline object reports the dominant kernel: its per-launch algorithmic
bytes over its average launch duration, timed live with HIP events on the
stream the kernels run on.  The CPU baseline times the FP64 oracle on a
bounded row sample of the same six calls.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--extra] [--no-cpu-baseline]
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

HEADLINE = [  # (name, n, k, format)
    ("gate_up_K5120_N17408", 17408, 5120, "nvfp4"),
    ("down_K17408_N5120", 5120, 17408, "nvfp4"),
]
HEADLINE_M = (1, 4, 8)

EXTRA = [  # measured only with --extra (the other configurations' timings)
    ("cfg1_K2048_N2048", 2048, 2048, "nvfp4", (1,)),
    ("fp8_K5120_N6144", 6144, 5120, "fp8", (1, 2, 4)),
    ("fp8_K5120_N5120", 5120, 5120, "fp8", (1, 2, 4)),
    ("layer_qkv_fp8_K5120_N7168", 7168, 5120, "fp8", (8,)),
    ("layer_o_fp8_K5120_N5120", 5120, 5120, "fp8", (8,)),
    ("layer_gateup_nvfp4_K5120_N34816", 34816, 5120, "nvfp4", (8,)),
    ("layer_down_nvfp4_K17408_N5120", 5120, 17408, "nvfp4", (8,)),
]
LMHEAD = ("lmhead_nvfp4_K5120_N151936", 151936, 5120)


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
        pw = qpn.pack_nvfp4(w) if fmt == "nvfp4" else qpn.pack_fp8(w)
        del w
        self.copies = [pw] + [pw.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / pw.nbytes)) - 1)]
        self.x = torch.from_numpy(synth.activations(8, k, seed=seed)).cuda()
        self.y = {m: torch.empty((m, n), dtype=torch.float16, device="cuda") for m in ms}
        self.xm = {m: self.x[:m].contiguous() for m in ms}
        self.bytes = algo_bytes(n, k, fmt)
        self.i = 0
        self.waves = None

    def next_copy(self):
        pw = self.copies[self.i]
        self.i = (self.i + 1) % len(self.copies)
        return pw


def run_step(qpn, shapes, events=None):
    """One pass: every (shape, M) call once, each on the next rotated copy."""
    for s in shapes:
        for m in s.ms:
            pw = s.next_copy()
            if events is not None:
                events[(s.name, m)][0].append(_record())
            qpn.gemm(pw, s.xm[m], out=s.y[m])
            if events is not None:
                events[(s.name, m)][1].append(_record())


_torch = None


def _record():
    e = _torch.cuda.Event(enable_timing=True)
    e.record()
    return e


def cpu_baseline(shapes, budget_s=12.0):
    """FP64 oracle on a bounded row sample of the same calls (CPU leg only)."""
    import oracle
    from fp8_quantized_skinny_qpn_amd import synth
    threads = oracle.threads()
    # calibrate rows per call so the whole sample takes about budget_s seconds
    total_t, total_b, sample = 0.0, 0, []
    rows_per_call = 64
    s0 = shapes[0]
    rows = np.arange(rows_per_call)
    w = synth.weight_rows(s0.n, s0.k, rows, seed=0)
    g = np.float32(1e-4)
    c, sc = oracle.pack_nvfp4_rows(w, g)
    x = synth.activations(8, s0.k, seed=0)
    t = time.perf_counter()
    oracle.gemm_nvfp4(c, sc, g, x)
    dt = time.perf_counter() - t
    per_mac = dt / (rows_per_call * s0.k * 8)
    macs_total = sum(s.k * m for s in shapes for m in s.ms)
    rows_per_call = int(max(16, min(4096, budget_s / (per_mac * macs_total))))
    for s in shapes:
        rows = np.arange(rows_per_call) * (s.n // rows_per_call)
        w = synth.weight_rows(s.n, s.k, rows, seed=0)
        g, _ = oracle.nvfp4_tensor_scale(w)  # scale of the sample; timing depends on bytes only
        c, sc = oracle.pack_nvfp4_rows(w, g)
        for m in s.ms:
            x = synth.activations(8, s.k, seed=0)[:m]
            t = time.perf_counter()
            oracle.gemm_nvfp4(c, sc, g, x)
            total_t += time.perf_counter() - t
            total_b += algo_bytes(rows_per_call, s.k, "nvfp4") - 4
    return {
        "value": round(total_b / total_t / 1e9, 6),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"FP64 oracle GEMM (qpn_oracle_gemm_nvfp4, OpenMP over rows) on {rows_per_call} "
                   f"evenly spaced rows of each of the 6 headline calls "
                   f"({', '.join(s.name for s in shapes)} x M={list(HEADLINE_M)}); "
                   f"{total_t:.1f} s of CPU time; GB/s over the sampled rows' weight bytes"),
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--extra", action="store_true", help="also time the other configurations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}): the QPN skinny "
              "GEMM is measured on one MI355X; sharding across GPUs is a design note only.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    global _torch
    _torch = torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from fp8_quantized_skinny_qpn_amd import qpn  # fails loudly when libqpn.so is missing

    log("setting up headline shapes")
    shapes = [Shape(qpn, torch, name, n, k, fmt, HEADLINE_M) for name, n, k, fmt in HEADLINE]
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        run_step(qpn, shapes)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides, with
    # an event pair around every launch
    events = {(s.name, m): ([], []) for s in shapes for m in s.ms}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(qpn, shapes, events)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    step_s = (t1 - t0) / args.steps
    step_bytes = sum(s.bytes * len(s.ms) for s in shapes)
    value = step_bytes / step_s / 1e9

    breakdown = {}
    per_kernel = {}
    for s in shapes:
        for m in s.ms:
            st, en = events[(s.name, m)]
            us = [a.elapsed_time(b) * 1e3 for a, b in zip(st, en)]
            med = float(np.median(us))
            kname = qpn.kernel_name(s.fmt, s.n, s.k, lmhead=False)
            breakdown[f"{s.name}_M{m}"] = {
                "kernel": kname, "us_median": round(med, 3),
                "us_p10": round(float(np.percentile(us, 10)), 3),
                "us_p90": round(float(np.percentile(us, 90)), 3),
                "GBps": round(s.bytes / med / 1e3, 1),
                "pct_hbm_peak": round(100 * s.bytes / med / 1e3 / HBM_PEAK_GBPS, 1),
                "weight_bytes": s.bytes, "rotated_copies": len(s.copies),
            }
            k = per_kernel.setdefault(kname, {"us": [], "bytes": s.bytes})
            k["us"] += us
    dom = max(per_kernel, key=lambda kn: sum(per_kernel[kn]["us"]))
    dk = per_kernel[dom]
    avg_us = float(np.mean(dk["us"]))
    achieved = dk["bytes"] / avg_us / 1e3
    traffic = traffic_for(dom)

    extra = {}
    if args.extra:
        for name, n, k, fmt, ms in EXTRA:
            log(f"extra: {name}")
            sh = Shape(qpn, torch, name, n, k, fmt, ms)
            ev = {(name, m): ([], []) for m in ms}
            for _ in range(5):
                run_step(qpn, [sh])
            for _ in range(50):
                run_step(qpn, [sh], ev)
            torch.cuda.synchronize()
            for m in ms:
                us = [a.elapsed_time(b) * 1e3 for a, b in zip(*ev[(name, m)])]
                med = float(np.median(us))
                extra[f"{name}_M{m}"] = {"us_median": round(med, 3), "GBps": round(sh.bytes / med / 1e3, 1),
                                         "pct_hbm_peak": round(100 * sh.bytes / med / 1e3 / HBM_PEAK_GBPS, 1)}
            del sh
            torch.cuda.empty_cache()
        from fp8_quantized_skinny_qpn_amd import synth
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
            ws = torch.empty(qpn.workspace_bytes(qpn.OP_LMHEAD_NVFP4, m, n, k), dtype=torch.uint8, device="cuda")
            us = []
            for it in range(40):
                e0 = _record()
                qpn.lmhead_nvfp4(copies[it % 3], xm, lg, am, ws)
                e1 = _record()
                if it >= 10:
                    us.append((e0, e1))
            torch.cuda.synchronize()
            t = [a.elapsed_time(bb) * 1e3 for a, bb in us]
            med = float(np.median(t))
            extra[f"{name}_M{m}"] = {"us_median": round(med, 3), "GBps": round(b / med / 1e3, 1),
                                     "pct_hbm_peak": round(100 * b / med / 1e3 / HBM_PEAK_GBPS, 1)}

    # measured read ceiling: the same nontemporal 16-byte loads streaming a
    # 2 GiB buffer (far larger than the 256 MB Infinity Cache)
    ceil_buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(2):
        qpn.debug_read_ceiling(ceil_buf, sink)
    ce = []
    for _ in range(5):
        e0 = _record()
        qpn.debug_read_ceiling(ceil_buf, sink)
        e1 = _record()
        ce.append((e0, e1))
    torch.cuda.synchronize()
    ceil_us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ce]))
    read_ceiling = ceil_buf.numel() / ceil_us / 1e3
    del ceil_buf
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(shapes)

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
        "read_ceiling_GBps": round(read_ceiling, 1),
        "pct_read_ceiling": round(100 * value / read_ceiling, 1),
        "config": {
            "workload": "nvfp4_skinny_gemm K5120->N17408 and K17408->N5120, M in {1,4,8}",
            "calls_per_step": len(shapes) * len(HEADLINE_M),
            "weights": "NVFP4 (E2M1 codes, UE4M3 per 16-K block, FP32 tensor scale) packed from N(0,0.02) fp32, seed 0",
            "activations": "fp16 N(0,1), seed 0",
            "step_weight_bytes": step_bytes,
            "rotated_copies_per_shape": [len(s.copies) for s in shapes],
            "waves_per_panel": {s.name: qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 8, s.n, s.k)[1] for s in shapes},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dk["bytes"],
            "avg_launch_us": round(avg_us, 3),
            "launches_timed": len(dk["us"]),
        },
        "cpu_baseline": cpu,
        "breakdown": breakdown,
    }
    if extra:
        out["extra_configs"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
