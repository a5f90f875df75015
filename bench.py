#!/usr/bin/env python3
"""Benchmark of the gfx950 GEMM library on one MI355X.

One step = one call of the library on one batch of seeded synthetic operands
already resident in HBM: planning, the macro-tile (or skinny / GEMV) kernel
and, when the plan splits K, the reduction.  Prints ONE JSON line.

Headline workload: fp16 in / fp32 accumulate / fp16 out, M = N = K = 8192,
row-major A and B (no transpose), entries N(0,1)/sqrt(K) from seed 1;
reported in TFLOP/s (2MNK per step) against the dense fp16 matrix-core peak.
Secondary lines in the same JSON object: the memory-bound 8192 x 128 x 8192
product and the 1 x 8192 x 8192 GEMV, in GB/s of algorithmic bytes
(A, B and C once each) against HBM bandwidth; their inputs rotate over copies
totalling >= 512 MiB so the 256 MB Infinity Cache cannot serve them.

The CPU baseline is the float64 oracle, timed on a bounded sample of the
headline workload's output rows on this host.
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
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s + % MFMA peak (fp16 8192³); GB/s + % HBM peak (8192×128×8192)"
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["tiled_gemm_02_amd/csrc/kernels/common.hpp",
                  "tiled_gemm_02_amd/csrc/kernels/mfma_gemm.hpp",
                  "tiled_gemm_02_amd/csrc/kernels/mfma_gemm3.hpp",
                  "tiled_gemm_02_amd/csrc/kernels/mfma_pingpong.hpp",
                  "tiled_gemm_02_amd/csrc/kernels/instances.inc",
                  "tiled_gemm_02_amd/csrc/kernels/gemv.hpp",
                  "tiled_gemm_02_amd/csrc/kernels/skinny.hpp",
                  "tiled_gemm_02_amd/csrc/kernels/aux_kernels.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        path = os.path.join(ROOT, rel)
        if os.path.exists(path):
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current kernels."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = data.get(workload)
    if not ent or ent.get("kernel_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def dev_tensor(arr, dtype_code, device):
    import numpy as np
    import torch
    from gemm_inputs import BF16
    a = np.ascontiguousarray(arr)
    if dtype_code == BF16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def prepare(name: str, device, rotate: bool):
    import torch
    from gemm_inputs import DTYPE_NAMES, ELEM_BYTES, WORKLOADS, make_problem
    w = dict(WORKLOADS[name])
    epi = w.pop("epilogue", None)
    slope = w.pop("slope", 0.01)
    p = make_problem(**w)
    A = dev_tensor(p.A, p.dtype, device)
    B = dev_tensor(p.B, p.dtype, device)
    s = ELEM_BYTES[p.dtype]
    alg_bytes = s * (p.M * p.K + p.K * p.N + p.M * p.N)
    copies = 1
    if rotate:
        copies = max(1, math.ceil(ROTATE_BYTES / max(1, s * (p.M * p.K + p.K * p.N))))
    As = [A] + [A.clone() for _ in range(copies - 1)]
    Bs = [B] + [B.clone() for _ in range(copies - 1)]
    C = torch.empty((p.M, p.N), dtype=A.dtype, device=device)
    return dict(p=p, As=As, Bs=Bs, C=C, epi=epi, slope=slope, copies=copies, alg_bytes=alg_bytes,
                flops=2.0 * p.M * p.N * p.K, dtype=DTYPE_NAMES[p.dtype])


def time_workload(name: str, steps: int, warmup: int, device, rotate: bool):
    import torch
    import tiled_gemm_02_amd as tg
    d = prepare(name, device, rotate)
    p = d["p"]
    epi = (tg.TG_EPI_LEAKY_RELU, d["slope"]) if d["epi"] else None
    stream = torch.cuda.current_stream(device)
    # split-K partials: one workspace for the whole run, as a caller that
    # cares about throughput passes it (without it the library makes a
    # stream-ordered allocation per call)
    plan0 = tg.plan_for(d["As"][0], d["Bs"][0], trans_a=p.trans_a, trans_b=p.trans_b)
    ws = None
    if plan0["workspace_bytes"] > 0:
        ws = torch.empty(int(plan0["workspace_bytes"]), dtype=torch.uint8, device=device)

    def step(i):
        j = i % d["copies"]
        tg.gemm(d["As"][j], d["Bs"][j], trans_a=p.trans_a, trans_b=p.trans_b, epilogue=epi,
                out=d["C"], workspace=ws, stream=stream.cuda_stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize(device)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize(device)
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    total_ms = evs[0].elapsed_time(evs[-1])
    plan = tg.plan_for(d["As"][0], d["Bs"][0], trans_a=p.trans_a, trans_b=p.trans_b)
    per_sorted = sorted(per)
    return dict(name=name, p=p, d=d, ms_per_step=total_ms / steps,
                ms_median=per_sorted[len(per_sorted) // 2], ms_min=per_sorted[0], wall_s=wall,
                plan=plan)


def cpu_baseline(name: str, target_s: float):
    """The oracle on a bounded sample of output rows of the workload, on the host cores."""
    import numpy as np
    import oracle
    from gemm_inputs import WORKLOADS, make_problem
    w = dict(WORKLOADS[name])
    epi = w.pop("epilogue", None)
    slope = w.pop("slope", 0.01)
    p = make_problem(**w)
    A64 = oracle.to_f64(p.A, p.dtype)
    B64 = oracle.to_f64(p.B, p.dtype)
    threads = oracle.default_threads()

    def run(rows):
        I = np.repeat(np.arange(rows, dtype=np.int64), p.N)
        J = np.tile(np.arange(p.N, dtype=np.int64), rows)
        t0 = time.perf_counter()
        oracle.gemm_points(p.M, p.N, p.K, A64, p.lda, p.trans_a, B64, p.ldb, p.trans_b, I, J,
                           dtype=p.dtype, epi=1 if epi else 0, slope=slope, threads=threads)
        return time.perf_counter() - t0

    t1 = run(1)
    rows = int(max(1, min(p.M, target_s / max(t1, 1e-6))))
    t = run(rows)
    macs = rows * p.N * p.K
    return {"value": 2.0 * macs / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} full output rows ({rows}x{p.N} elements, {macs / 1e9:.1f} G multiply-adds) "
                      f"of the {p.M}x{p.N}x{p.K} {name} workload, fp64 triple loop, {t:.1f} s"}


def roofline_entry(r, bound):
    d = r["d"]
    avg_s = r["ms_per_step"] / 1e3
    traffic = measured_traffic(r["name"])
    if bound == "mfma":
        achieved = d["flops"] / avg_s / 1e12
        peak = PEAK_TFLOPS[d["dtype"]]
        unit = "TFLOP/s"
    else:
        achieved = d["alg_bytes"] / avg_s / 1e9
        peak = PEAK_HBM_GBS
        unit = "GB/s"
    return {"bound": "hbm" if bound == "hbm" else "mfma", "achieved": round(achieved, 2),
            "peak": peak, "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="f16_8192")
    ap.add_argument("--secondary", default="f16_skinny_8192x128x8192,f16_gemv_1x8192x8192",
                    help="comma-separated memory-bound workloads reported alongside ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(a product shards by rows of A with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_gemm_02_amd as tg
    from gemm_inputs import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tg.load()
    device = torch.device("cuda:0")
    log("device", torch.cuda.get_device_name(0), "cus", tg.tg_device_cus())

    w = WORKLOADS[args.workload]
    mem_bound = w["N"] <= 256 or w["M"] == 1
    log("timing", args.workload)
    r = time_workload(args.workload, args.steps, args.warmup, device, rotate=mem_bound)
    d = r["d"]
    if mem_bound:
        value, unit = d["alg_bytes"] / (r["ms_per_step"] / 1e3) / 1e9, "GB/s"
    else:
        value, unit = d["flops"] / (r["ms_per_step"] / 1e3) / 1e12, "TFLOP/s"
    p = r["p"]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": d["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "M": p.M, "N": p.N, "K": p.K,
                   "layout": ["NN", "TN", "NT", "TT"][p.trans], "epilogue": d["epi"] or "none",
                   "seed": p.desc["seed"], "dist": p.desc["dist"], "plan": {
                       k: r["plan"][k] for k in ("path_name", "tile_m", "tile_n", "split_k",
                                                  "tiles", "waves", "occupancy")}},
        "ms_median": round(r["ms_median"], 5),
        "roofline": roofline_entry(r, "hbm" if mem_bound else "mfma"),
    }
    sec = []
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        log("timing", name)
        rs = time_workload(name, max(args.steps, 50), args.warmup, device, rotate=True)
        ent = roofline_entry(rs, "hbm")
        sec.append({"workload": name, "value": ent["achieved"], "unit": "GB/s",
                    "ms_per_step": round(rs["ms_per_step"], 5),
                    "plan": {k: rs["plan"][k] for k in ("path_name", "tile_m", "tile_n", "split_k",
                                                         "workgroups")},
                    "roofline": ent, "rotated_copies": rs["d"]["copies"]})
        del rs
        torch.cuda.empty_cache()
    if sec:
        out["secondary"] = sec
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
