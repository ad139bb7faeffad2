#!/usr/bin/env python3
"""Benchmark of the fused add + RMSNorm + per-token FP8 path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--suite] [--no-cpu-baseline]

One step = one call of nq_fused_add_rmsnorm_quant_fp8 over one batch of
M=8192 tokens of hidden size 2816 (bf16 x and residual in HBM, fresh bf16
residual, e4m3 codes and fp32 per-token scales out): every stage of the hot
path -- load, residual add and write-back, both row reductions, normalize,
scale, quantize and pack -- runs inside that one kernel.  Inputs are seeded
synthetic activations (N(0,1) with 1% outlier channels x50), resident in HBM
before timing starts; steps rotate over enough buffer sets (4 x 161.5 MB)
that no step finds its data in the 256 MB last-level cache.

Prints ONE JSON line.  `value` is whole-job throughput in GB/s of
algorithmic bytes (inputs + residual write + fp8 output + scales, gamma
once; see fp4_quantization_amd/traffic.py) over the K timed steps;
`roofline.achieved` is the same bytes over the kernel's mean launch duration
measured with HIP events on the launch stream.  `--suite` also prints one
line per workload (all five) to stderr.  `--profile-mode` runs a short fixed
sequence meant to be wrapped by rocprofv3.  `--summarize` turns rocprofv3
output into the text summaries kept under profiles/.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused add+RMSNorm+FP8-quant GB/s & % HBM peak, M=8192 d=2816; µs/call M=1"
HBM_PEAK_GBPS = 8000.0
MAIN_KERNEL_SOURCES = ["fp4_quantization_amd/csrc/nq_rmsnorm_fp8.hip",
                       "fp4_quantization_amd/csrc/nq_device.hpp",
                       "fp4_quantization_amd/csrc/nq_rows.hpp"]
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "rmsnorm_fp8_m8192_d2816_hbm_counters.md")
LLC_BYTES = 256 << 20


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in MAIN_KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------- workloads --

class RmsFp8Case:
    """Rotating buffer sets of one fused add+RMSNorm+FP8 workload."""

    def __init__(self, torch, nq, M, d, seed=0, static=False, sets=None):
        from fp4_quantization_amd import workloads as W, traffic
        self.torch, self.nq, self.M, self.d = torch, nq, M, d
        w = W.rms_2816(M, seed) if d == 2816 else W.rms_small(seed, M)
        rd, wr = traffic.fused_add_rmsnorm_fp8(M, d, residual=True, static=static)
        self.bytes = rd + wr
        x = torch.from_numpy(w["x"]).view(torch.bfloat16).cuda()
        r = torch.from_numpy(w["residual"]).view(torch.bfloat16).cuda()
        self.g = torch.from_numpy(w["gamma"]).cuda()
        self.eps = w["eps"]
        self.ss = torch.tensor([0.05], dtype=torch.float32, device="cuda") if static else None
        n = sets or max(1, min(8, -(-2 * LLC_BYTES // max(self.bytes, 1))))
        self.sets = []
        for _ in range(n):
            self.sets.append(dict(x=x.clone(), r=r.clone(),
                                  ro=torch.empty_like(r), q=torch.empty(M, d, dtype=torch.uint8, device="cuda"),
                                  s=torch.empty(M, dtype=torch.float32, device="cuda")))
        self.label = f"fused add+RMSNorm+per-token FP8 (e4m3), M={M}, d={d}" + (", static scale" if static else "")

    def step(self, i, stream=None):
        b = self.sets[i % len(self.sets)]
        self.nq.nq_fused_add_rmsnorm_quant_fp8(b["x"], b["r"], b["ro"], self.g, self.eps, self.ss,
                                               b["q"], None if self.ss is not None else b["s"], stream=stream)


class GroupCase:
    def __init__(self, torch, nq, M, K=4096, ue8m0=False):
        from fp4_quantization_amd import workloads as W, traffic
        self.torch, self.nq = torch, nq
        w = W.group_t3(M, K)
        self.bytes = traffic.total(traffic.group_fp8(M, K))
        x = torch.from_numpy(w["x"]).view(torch.bfloat16).cuda()
        n = max(1, min(8, -(-2 * LLC_BYTES // self.bytes)))
        self.sets = [dict(x=x.clone(), q=torch.empty(M, K, dtype=torch.uint8, device="cuda"),
                          s=torch.empty(M * K // 128, dtype=torch.float32, device="cuda")) for _ in range(n)]
        self.mode = nq.NQ_SCALE_UE8M0 if ue8m0 else nq.NQ_SCALE_FP32
        self.label = f"per-token-group FP8, group 128, {'UE8M0' if ue8m0 else 'fp32'} scales, M={M}, K={K}"

    def step(self, i, stream=None):
        b = self.sets[i % len(self.sets)]
        self.nq.nq_per_token_group_quant_fp8(b["x"], b["q"], b["s"], 128, self.mode, stream=stream)


class LayerNormCase:
    def __init__(self, torch, nq, M=16384, d=4096):
        from fp4_quantization_amd import workloads as W, traffic
        self.torch, self.nq = torch, nq
        w = W.layernorm_rows(M, d)
        self.bytes = traffic.total(traffic.layernorm_fp8(M, d))
        x = torch.from_numpy(w["x"]).view(torch.bfloat16).cuda()
        self.g = torch.from_numpy(w["gamma"]).cuda()
        self.b = torch.from_numpy(w["beta"]).cuda()
        self.sc = torch.tensor([w["scale"]], dtype=torch.float32, device="cuda")
        self.eps = w["eps"]
        n = max(1, min(8, -(-2 * LLC_BYTES // self.bytes)))
        self.sets = [dict(x=x.clone(), q=torch.empty(M, d, dtype=torch.uint8, device="cuda")) for _ in range(n)]
        self.label = f"LayerNorm + static FP8 (scale tensor 0.05), M={M}, d={d}"

    def step(self, i, stream=None):
        b = self.sets[i % len(self.sets)]
        self.nq.nq_layernorm_quant_fp8(b["x"], self.g, self.b, self.eps, self.sc, b["q"], stream=stream)


class Nvfp4Case:
    def __init__(self, torch, nq, M, sliced=False):
        from fp4_quantization_amd import workloads as W, traffic
        self.torch, self.nq = torch, nq
        w = W.nvfp4_slice(M) if sliced else W.nvfp4_7168(M)
        d = w["d"]
        self.bytes = traffic.total(traffic.rmsnorm_nvfp4(M, d, residual=not sliced))
        x = torch.from_numpy(w["x"]).view(torch.bfloat16).cuda()
        r = None if sliced else torch.from_numpy(w["residual"]).view(torch.bfloat16).cuda()
        self.g = torch.from_numpy(w["gamma"]).cuda()
        self.gs = torch.tensor([W.NVFP4_NOMINAL_GLOBAL_SCALE], dtype=torch.float32, device="cuda")
        self.eps, self.d = w["eps"], d
        n = max(1, min(8, -(-2 * LLC_BYTES // self.bytes)))
        self.sets = []
        for _ in range(n):
            self.sets.append(dict(x=x.clone(), r=None if r is None else r.clone(),
                                  ro=None if r is None else torch.empty_like(r),
                                  q=torch.empty(M, d // 2, dtype=torch.uint8, device="cuda"),
                                  sf=torch.empty(M, d // 16, dtype=torch.uint8, device="cuda")))
        self.label = (f"RMSNorm + NVFP4 on a 1536-of-2112 column slice, M={M}" if sliced
                      else f"residual-add + RMSNorm + NVFP4, M={M}, d=7168")

    def step(self, i, stream=None):
        b = self.sets[i % len(self.sets)]
        self.nq.nq_rmsnorm_quant_nvfp4(b["x"][:, :self.d], b["r"], b["ro"], self.g, self.eps, self.gs,
                                       b["q"], b["sf"], stream=stream)


class CopyCase:
    """The 128-bit copy kernel over the same byte count: a same-box ceiling."""

    def __init__(self, torch, nq, nbytes):
        self.torch, self.nq = torch, nq
        n = nbytes // 2 // 16 * 16
        sets = max(1, min(8, -(-2 * LLC_BYTES // (2 * n))))
        self.sets = [(torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255),
                      torch.empty(n, dtype=torch.uint8, device="cuda")) for _ in range(sets)]
        self.bytes = 2 * n
        self.label = f"128-bit copy, {n} bytes read + {n} written"

    def step(self, i, stream=None):
        s, d = self.sets[i % len(self.sets)]
        self.nq.nq_diag_copy(s, d, stream=stream)


# ---------------------------------------------------------------- timing --

def time_eager(torch, case, steps, warmup):
    """Wall time of `steps` back-to-back calls, and each launch's own
    duration from an event pair around it, all on the current stream."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        case.step(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        starts[i].record(stream)
        case.step(warmup + i)
        ends[i].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t0.elapsed_time(t1)
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    return total_ms, per, wall


def time_graph(torch, case, calls=20, replays=50):
    """Per-call time of `calls` launches captured in one graph (launch gaps
    removed), median over replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            case.step(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            case.step(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    del g
    return float(np.median(times)) / calls


# ----------------------------------------------------------- cpu baseline --

def cpu_baseline(budget_s=12.0):
    """The oracle (plain single-threaded C) on a bounded sample of the same
    workload: as many rows of M=8192, d=2816 as fit in about budget_s
    seconds, scaled to GB/s of the same algorithmic bytes."""
    import oracle
    from fp4_quantization_amd import workloads as W, traffic
    w = W.rms_2816(8192, 0)
    oracle.lib()
    rows, elapsed, batch = 0, 0.0, 16
    t0 = time.perf_counter()
    while elapsed < budget_s and rows < 8192:
        lo, hi = rows, min(8192, rows + batch)
        oracle.fused_add_rmsnorm_quant_fp8(w["x"][lo:hi], w["residual"][lo:hi], w["gamma"], w["eps"])
        rows = hi
        elapsed = time.perf_counter() - t0
        batch = min(batch * 2, 512)
    rd, wr = traffic.fused_add_rmsnorm_fp8(rows, 2816)
    return {"value": round((rd + wr) / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of 8192 rows of the M=8192, d=2816 workload (seed 0), {elapsed:.1f} s, "
                      f"single-threaded, host {platform.processor() or platform.machine()}, "
                      f"{os.cpu_count()} cores visible"}


# ------------------------------------------------------- counter traffic --

def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None when it is missing or was taken on different kernel sources."""
    if not os.path.exists(COUNTER_SUMMARY):
        return None
    txt = open(COUNTER_SUMMARY).read()
    try:
        src = txt.split("kernel_source_hash:")[1].split()[0]
        val = float(txt.split("hbm_bytes_per_launch:")[1].split()[0])
    except (IndexError, ValueError):
        return None
    return val if src == kernel_source_hash() else None


# ------------------------------------------------------------------ main --

def run_suite(torch, nq, steps, warmup):
    cases = [
        ("rms_small", lambda: RmsFp8Case(torch, nq, 64, 256)),
        ("rms_2816_m1", lambda: RmsFp8Case(torch, nq, 1, 2816, sets=64)),
        ("rms_2816_m16", lambda: RmsFp8Case(torch, nq, 16, 2816, sets=64)),
        ("rms_2816_m256", lambda: RmsFp8Case(torch, nq, 256, 2816)),
        ("rms_2816_m8192", lambda: RmsFp8Case(torch, nq, 8192, 2816)),
        ("rms_2816_m8192_static", lambda: RmsFp8Case(torch, nq, 8192, 2816, static=True)),
        ("group_m32768_fp32", lambda: GroupCase(torch, nq, 32768)),
        ("group_m32768_ue8m0", lambda: GroupCase(torch, nq, 32768, ue8m0=True)),
        ("group_m1", lambda: GroupCase(torch, nq, 1)),
        ("layernorm_m16384", lambda: LayerNormCase(torch, nq)),
        ("nvfp4_7168_m1", lambda: Nvfp4Case(torch, nq, 1)),
        ("nvfp4_7168_m64", lambda: Nvfp4Case(torch, nq, 64)),
        ("nvfp4_7168_m8192", lambda: Nvfp4Case(torch, nq, 8192)),
        ("nvfp4_slice_m1", lambda: Nvfp4Case(torch, nq, 1, sliced=True)),
        ("nvfp4_slice_m64", lambda: Nvfp4Case(torch, nq, 64, sliced=True)),
        ("nvfp4_slice_m8192", lambda: Nvfp4Case(torch, nq, 8192, sliced=True)),
        ("copy_161MB", lambda: CopyCase(torch, nq, 161_524_736)),
    ]
    for name, make in cases:
        case = make()
        total_ms, per, _ = time_eager(torch, case, steps, warmup)
        us_graph = time_graph(torch, case) * 1e3
        line = {"workload": name, "label": case.label, "bytes_per_call": case.bytes,
                "us_per_call_graph": round(us_graph, 3),
                "us_per_launch_events": round(float(per.mean()) * 1e3, 3),
                "GBps_graph": round(case.bytes / (us_graph * 1e-6) / 1e9, 1),
                "pct_hbm_peak_graph": round(100 * case.bytes / (us_graph * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1)}
        log(json.dumps(line))
        del case
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--suite", action="store_true", help="also time all five workloads (stderr)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-mode", action="store_true",
                    help="short fixed run for rocprofv3: copy reference + main kernel steps")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path is row-parallel and would shard rows across GPUs with no communication, "
              "but no multi-GPU run is part of it.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from fp4_quantization_amd import nq

    if args.profile_mode:
        # 10 copies of exactly 64 MiB read + 64 MiB written, then 20 main steps
        src = torch.empty(64 << 20, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(10):
            nq.nq_diag_copy(src, dst)
        case = RmsFp8Case(torch, nq, 8192, 2816)
        for i in range(20):
            case.step(i)
        torch.cuda.synchronize()
        log("profile-mode done")
        return

    case = RmsFp8Case(torch, nq, 8192, 2816)
    total_ms, per, wall = time_eager(torch, case, args.steps, args.warmup)
    ms_per_step = total_ms / args.steps
    value = case.bytes / (ms_per_step * 1e-3) / 1e9
    kernel_ms = float(per.mean())
    achieved = case.bytes / (kernel_ms * 1e-3) / 1e9
    log(f"main: {args.steps} steps, {total_ms:.3f} ms on the stream ({wall * 1e3:.1f} ms wall), "
        f"{ms_per_step * 1e3:.2f} us/step, kernel mean {kernel_ms * 1e3:.2f} us")
    del case
    torch.cuda.empty_cache()

    m1 = RmsFp8Case(torch, nq, 1, 2816, sets=64)
    m1_us = time_graph(torch, m1, calls=100) * 1e3
    _, m1_per, _ = time_eager(torch, m1, 200, 20)
    del m1

    if args.suite:
        run_suite(torch, nq, min(args.steps, 50), min(args.warmup, 5))

    traffic_bytes = read_traffic()
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fused residual-add + RMSNorm + per-token dynamic e4m3 quant, "
                               "M=8192 tokens, d=2816, bf16 x/residual N(0,1) with 28 outlier channels x50",
                   "M": 8192, "d": 2816, "bytes_per_step": case_bytes_8192(),
                   "buffer_sets": 4, "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "m1_us_per_call": round(m1_us, 3),
        "m1_us_per_launch_events": round(float(m1_per.mean()) * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_bytes},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


def case_bytes_8192():
    from fp4_quantization_amd import traffic
    return traffic.total(traffic.fused_add_rmsnorm_fp8(8192, 2816))


if __name__ == "__main__":
    main()
