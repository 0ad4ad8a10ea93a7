#!/usr/bin/env python3
"""Benchmark of the normalization-prologue GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the hot path on one batch of synthetic input that is
already resident in device memory. The headline workload is RMSNorm + MatMul
+ SiLU on x[512, 14336] and W[49152, 14336] in fp16 (the fused norm + GEMM +
SiLU configuration the metric is quoted on). W is rotated over device copies
so that timed calls stream it from HBM instead of the 256 MB last-level cache.

The same process also measures the other workloads of the path, before the
headline one, and reports them under "workloads" in the same JSON line:
LayerNorm + Linear + bias (x[64,256] latency and x[1024,8192]), the fused
FFN (x[512,14336], 49152 -> 14336) and the decode GEMM x[M,8192] .
W[28672,8192] in bf16 for M = 1, 8, 32. Each is timed the same way, with
max(W, 100) warmup and max(K, 20) timed steps.

Timing: K steps back to back between two HIP events recorded on the stream
the kernels are launched on; `value` and `roofline.achieved` are algorithmic
FLOPs (or bytes) per step over that time per step. One step of a normalizing
call with M > 32 is two launches (row statistics, then the main kernel),
which the per-step time includes.

Prints ONE JSON line with the throughput, the roofline object of the
dominant kernel and the fp64 CPU oracle timed on a bounded sample of the
headline workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused norm+GEMM+SiLU TFLOP/s & % MFMA peak; decode GB/s & % HBM peak"
PEAK_MFMA_F16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense fp16/bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0           # HBM3E, 8 TB/s
LLC_BYTES = 256 << 20           # Infinity Cache (MALL)
HEADLINE = "rms_matmul_silu_512x14336"
# ":folded" = the same workload with gamma / beta folded into the weights
# (inference mode), the folding itself done once before the timed region
EXTRAS = ("ffn_silu_512x14336x49152", "ln_linear_bias_1024x8192", "decode_rms_gemm_m1",
          "decode_rms_gemm_m8", "decode_rms_gemm_m32", "ln_linear_bias_64x256",
          "rms_matmul_silu_512x14336:folded", "ln_linear_bias_1024x8192:folded",
          "attn_out_rmsnorm_512x8192")


def workload(name: str):
    import synth
    if name not in synth.WORKLOADS:
        raise SystemExit(f"unknown workload {name!r}; choose from {sorted(synth.WORKLOADS)}")
    return synth.WORKLOADS[name](seed=0)


def kernel_sources_sha() -> str:
    """Short hash of the HIP/C sources, to tell whether recorded counters
    still describe the kernels being run."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "norm_gemm_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload_name: str):
    """HBM bytes per step measured with rocprofv3 (FETCH_SIZE and WRITE_SIZE,
    scaled by a copy-kernel calibration), or None when no record exists for
    this workload (its name, plus ":folded" for the folded variant) or the
    kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path, encoding="utf-8") as f:
            rec = json.load(f).get(workload_name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sources_sha256_16") != kernel_sources_sha():
        return None
    return int(rec["traffic_bytes_per_launch"])


def upload(bits, dtype, device):
    """uint16 bit patterns -> fp16/bf16 device tensor with the same bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == 0 else torch.bfloat16).to(device)


def algorithmic(case):
    """FLOPs (2 per multiply-add of every GEMM) and bytes (each input and the
    output read or written once; the FFN's intermediate h is not counted)."""
    M, K, N = case.M, case.K, case.N
    nbytes = sum(int(a.size) * 2 for a in case.arrays.values() if a is not None)
    if case.kind == "ffn":
        F = case.F
        return 2 * M * K * F + 2 * M * F * N, nbytes + M * N * 2
    if case.kind == "gated_ffn":
        F = case.F
        return 2 * M * K * 2 * F + 2 * M * F * N, nbytes + M * N * 2
    return 2 * M * N * K, nbytes + M * N * 2


def launches_per_step(case) -> int:
    """Kernel launches of one step (aligned shapes, workspace with room for
    the split-K partials): a statistics pass before a normalizing GEMM with
    M > 32; the FFN's second GEMM split over K (its partial sum is a second
    launch) when its 128 x 256 tiles leave CUs idle; the gated GEMM's split
    last round (one more launch for its sum)."""
    if case.kind == "gemm_norm":
        return 2
    first = 1 + (1 if case.norm and case.M > 32 else 0)
    if case.kind not in ("ffn", "gated_ffn"):
        return first
    import ctypes
    import torch
    import norm_gemm_amd as ng
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    lib = ng.lib
    if case.kind == "gated_ffn" and case.M > 32:
        # the gated GEMM's last round in K halves adds the sum of their partials
        lib.ng_gated_split_tiles.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_int]
        first += 1 if lib.ng_gated_split_tiles(case.M, case.F, case.K, cus) > 0 else 0
    lib.ng_skip_slice_plan.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_void_p,
                                                              ctypes.c_void_p]
    tiles = -(-case.M // 128) * -(-case.N // 256)
    split = case.M > 32 and ((2 * tiles <= cus and -(-case.F // 64) >= 4) or
                             lib.ng_skip_slice_plan(case.M, case.N, case.F, cus, None, None))
    return first + (2 if split else 1)


def measure(name: str, steps: int, warmup: int):
    """Time `steps` back-to-back steps of workload `name` after `warmup`
    untimed ones; returns (case, result dict)."""
    import torch
    import norm_gemm_amd as ng

    base_name, _, mode = name.partition(":")
    folded = mode == "folded"
    case = workload(base_name)
    dev = torch.device("cuda:0")
    A = case.arrays
    flops, nbytes = algorithmic(case)
    is_ffn = case.kind in ("ffn", "gated_ffn")
    ffn_call = ng.fused_gated_ffn if case.kind == "gated_ffn" else ng.fused_ffn
    ws_size = (ng.fused_gated_ffn_workspace_size if case.kind == "gated_ffn"
               else ng.fused_ffn_workspace_size)
    wkeys = ("W1", "W2") if is_ffn else ("W",)
    wbytes = sum(A[k].size * 2 for k in wkeys)
    copies = max(2, math.ceil(1.5 * LLC_BYTES / wbytes) + 1)
    up = {k: upload(v, case.dtype, dev) for k, v in A.items() if v is not None and k not in wkeys}
    base = {k: upload(A[k], case.dtype, dev) for k in wkeys}
    wsets = [{k: (base[k] if c == 0 else base[k].clone()) for k in wkeys} for c in range(copies)]
    if folded:
        for w in wsets:
            w["W"], w["c1"], w["c2"] = ng.norm_gemm_fold_weights(
                w["W"], up.get("gamma"), up.get("beta"), up.get("bias"))
        torch.cuda.synchronize()
    get = up.get
    out = torch.empty(case.M, case.N, dtype=up["x"].dtype, device=dev)
    ws = None
    if is_ffn:
        # the plain FFN's workspace also holds the two fp32 partial sums of y
        # that the second GEMM's split K writes (the gated FFN's holds them)
        extra = 8 * case.M * case.N if case.kind == "ffn" else 0
        ws = torch.empty(ws_size(case.M, case.F, up["x"].dtype) + extra, dtype=torch.uint8,
                         device=dev)
    elif case.kind == "gemm_norm":
        ws = torch.empty(2 * ng.fused_gemm_norm_workspace_size(case.M, case.N),
                         dtype=torch.uint8, device=dev)

    def step(i):
        w = wsets[i % copies]
        if is_ffn:
            ffn_call(get("x"), w["W1"], w["W2"], get("gamma"), get("beta"), get("b1"),
                     get("b2"), eps=case.eps, norm=case.norm, act=case.act,
                     workspace=ws, out=out)
        elif case.kind == "gemm_norm":
            ng.fused_gemm_norm(get("x"), w["W"], get("bias"), get("gamma"), get("beta"),
                               eps=case.eps, norm=case.norm, workspace=ws, out=out)
        elif folded:
            ng.fused_norm_gemm_folded(get("x"), w["W"], w["c1"], w["c2"], eps=case.eps,
                                      norm=case.norm, act=case.act, out=out)
        else:
            ng.fused_norm_gemm(get("x"), w["W"], get("gamma"), get("beta"), get("bias"),
                               eps=case.eps, norm=case.norm, act=case.act, out=out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # K steps back to back between two events on the launch stream (per-step
    # events would add their own gaps).
    stream = torch.cuda.current_stream(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / steps

    decode = case.M <= 32
    if decode:
        value = nbytes / (ms_per_step * 1e-3) / 1e9
        unit, bound, peak, runit = "GB/s", "hbm", PEAK_HBM_GBS, "GB/s"
    else:
        value = flops / (ms_per_step * 1e-3) / 1e12
        unit, bound, peak, runit = "TFLOP/s", "mfma", PEAK_MFMA_F16_TFLOPS, "TFLOP/s"
    res = {
        "workload": case.name + (" (gamma/beta folded into the weights)" if folded else ""),
        "value": round(value, 2),
        "unit": unit,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "steps": steps,
        "warmup": warmup,
        "launches_per_step": launches_per_step(case),
        "roofline": {"bound": bound, "achieved": round(value, 1), "peak": peak, "unit": runit,
                     "frac": round(value / peak, 4),
                     "traffic": recorded_traffic(case.name + (":folded" if folded else ""))},
        "host_wall_s": round(wall, 4),
        "weight_copies": copies,
    }
    del wsets, base, up, out, ws
    torch.cuda.empty_cache()
    return case, res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(case, seconds: float):
    """The fp64 oracle as it stands, on whole output rows of the workload,
    doubling the row count until about `seconds` of wall time are spent."""
    import oracle
    done_rows = 0
    spent = 0.0
    batch = 1
    row = 0
    while spent < seconds and row < case.M:
        rows = list(range(row, min(case.M, row + batch)))
        t0 = time.perf_counter()
        oracle.run_case(case, rows=rows)
        spent += time.perf_counter() - t0
        done_rows += len(rows)
        row += len(rows)
        batch *= 2
    flops, nbytes = algorithmic(case)
    frac = done_rows / case.M
    if case.M <= 32:
        # the oracle streams all of W for every row, so its rate is reported
        # as the workload's algorithmic bytes scaled by the rows completed
        value, unit = nbytes * frac / spent / 1e9, "GB/s"
    else:
        value, unit = flops * frac / spent / 1e12, "TFLOP/s"
    return {"value": round(value, 6), "unit": unit, "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{done_rows} of {case.M} output rows (all {case.N} columns) of "
                      f"{case.name}, {spent:.1f} s, fp64",
            "cpu_model": cpu_model(), "compile_flags": " ".join(oracle.COMPILE_FLAGS)}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The GPU clock ramps up over tens of milliseconds of sustained load.
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true",
                    help="measure only --workload (no other workloads; e.g. under a profiler)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (e.g. under a profiler)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: this build has no multi-GPU path "
              f"(got --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    torch.cuda.set_device(0)

    extras = []
    if not args.only:
        for name in EXTRAS:
            if name == args.workload:
                continue
            _, r = measure(name, max(args.steps, 20), max(args.warmup, 100))
            extras.append(r)
            print(f"# {name}: {r['value']} {r['unit']} ({r['us_per_step']} us/step)",
                  file=sys.stderr, flush=True)

    case, main_res = measure(args.workload, args.steps, args.warmup)
    cpu = None if args.no_cpu_baseline else cpu_baseline(case, args.cpu_seconds)
    A = case.arrays
    is_ffn = case.kind in ("ffn", "gated_ffn")
    line = {
        "metric": METRIC,
        "value": main_res["value"],
        "unit": main_res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if case.dtype == 0 else "bf16",
        "data": "synthetic (seeded PCG64 normals; W rotated over %d device copies)"
                % main_res["weight_copies"],
        "config": {"workload": main_res["workload"], "M": case.M, "K": case.K, "N": case.N,
                   **({"F": case.F} if is_ffn else {}),
                   "norm": ["none", "layernorm", "rmsnorm"][case.norm],
                   "act": ["none", "silu", "relu", "gelu"][case.act],
                   "gated": case.kind == "gated_ffn",
                   "bias": (A.get("bias") is not None) or (A.get("b1") is not None),
                   "eps": case.eps, "launches_per_step": main_res["launches_per_step"]},
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "timing": {"us_per_step": main_res["us_per_step"], "host_wall_s": main_res["host_wall_s"],
                   "region": "K back-to-back steps between two events on the launch stream"},
        "workloads": extras,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
