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

Every timed workload first runs untimed steps back to back for a quarter
second ("settle"), then its warm-up steps, then the timed steps: the engine
clock ramps up from idle over tens of milliseconds of load, and a workload of
a few milliseconds in all would otherwise be timed on the ramp.

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
# The pages' own arithmetic-intensity figures ("Matrix Multiplication
# Background User's Guide", section 2), quoted with the hardware they are
# stated for, beside this chip's ridge point (dense matrix peak / HBM rate).
PAGES_CONTEXT = {
    "v100_fp16_tensor_core_ops_per_byte": 138.9,
    "ai_8192x128x8192_fp16_flop_per_byte": 124.1,
    "ai_8192x8192x8192_fp16_flop_per_byte": 2730,
    "ai_gemv_flop_per_byte": "< 1",
    "hardware_of_those_figures": "NVIDIA V100 (the guide's example)",
}


def ridge(dtype_name: str) -> float:
    """FLOP per byte at which the dense matrix peak and HBM bandwidth meet on MI355X."""
    return PEAK_TFLOPS[dtype_name] * 1e12 / (PEAK_HBM_GBS * 1e9)


def bound_of(M: int, N: int, K: int, dtype_code: int) -> str:
    """'hbm' when the algorithmic arithmetic intensity 2MNK / s(MK + KN + MN)
    is below the chip's ridge for that type, else 'mfma' (the guide's
    section 2 test, with MI355X's figures)."""
    from gemm_inputs import DTYPE_NAMES, ELEM_BYTES
    s = ELEM_BYTES[dtype_code]
    ai = 2.0 * M * N * K / (s * (M * K + K * N + M * N))
    return "hbm" if ai < ridge(DTYPE_NAMES[dtype_code]) else "mfma"


def host_cpu() -> dict:
    """CPUs this process may run on, the machine's logical CPU count and the CPU model."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"usable_cpus": usable, "nproc": os.cpu_count(), "cpu_model": model}
ROTATE_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
_K = "tiled_gemm_02_amd/csrc/kernels/"
# The sources each kernel family's code comes from: its counters are void once
# any of them changes.
# instances.inc: the instantiations and launch shapes (e.g. the ring depth); the
# instance units (inst_*.hip): which tiles exist; plan.{h,cpp}: which kernel, tile
# and split a workload gets (the softmax launch shape included)
_PLAN = ["tiled_gemm_02_amd/csrc/plan.h", "tiled_gemm_02_amd/csrc/plan.cpp"]
_INST = [_K + "inst_f16.hip", _K + "inst_bf16.hip", _K + "inst_f32.hip"]
KERNEL_SOURCES = {
    "mfma": [_K + "common.hpp", _K + "instances.inc", _K + "mfma_gemm.hpp", _K + "mfma_gemm3.hpp",
             _K + "mfma_pingpong.hpp"] + _INST + _PLAN,
    "skinny": [_K + "common.hpp", _K + "instances.inc", _K + "skinny.hpp"] + _INST + _PLAN,
    "gemv": [_K + "common.hpp", _K + "instances.inc", _K + "gemv.hpp"] + _INST + _PLAN,
    "softmax": [_K + "common.hpp", _K + "instances.inc", _K + "softmax.hpp"] + _INST + _PLAN,
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_family(workload: str) -> str:
    if workload.startswith("softmax_"):
        return "softmax"
    if "skinny" in workload:
        return "skinny"
    if "gemv" in workload:
        return "gemv"
    return "mfma"


def kernel_source_hash(family: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
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
    if not ent or ent.get("kernel_hash") != kernel_source_hash(kernel_family(workload)):
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


SETTLE_S = 0.25   # untimed GPU-busy seconds before a workload's warm-up steps


def settle(step, device, seconds: float = SETTLE_S) -> int:
    """Run untimed steps back to back until `seconds` of wall time have passed.

    The engine clock ramps up from its idle level over tens of milliseconds of
    load: after host-side input preparation (seconds of numpy) a workload whose
    warm-up plus timed steps add up to a few milliseconds would otherwise be
    timed at the ramp's start.  Returns the number of steps run."""
    import torch
    t0 = time.perf_counter()
    n, chunk = 0, 1
    while True:
        for _ in range(chunk):
            step(n)
            n += 1
        torch.cuda.synchronize(device)
        if time.perf_counter() - t0 >= seconds:
            return n
        chunk = min(chunk * 2, 256)


def time_back_to_back(call, stream, reps: int) -> float:
    """Mean milliseconds of `reps` calls issued back to back between two
    events on the launch stream."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def prepare(name: str, device, rotate: bool):
    import torch
    from gemm_inputs import DTYPE_NAMES, ELEM_BYTES, WORKLOADS, make_problem
    w = dict(WORKLOADS[name])
    epi = w.pop("epilogue", None)
    slope = w.pop("slope", 0.01)
    alpha = w.pop("alpha", 1.0)
    beta = w.pop("beta", 0.0)
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
    if beta != 0.0:
        from gemm_inputs import make_c_old
        C = dev_tensor(make_c_old(p.M, p.N, p.dtype, p.desc["seed"]), p.dtype, device)
        alg_bytes += s * p.M * p.N   # the old C is read
    else:
        C = torch.empty((p.M, p.N), dtype=A.dtype, device=device)
    return dict(p=p, As=As, Bs=Bs, C=C, epi=epi, slope=slope, alpha=alpha, beta=beta,
                copies=copies, alg_bytes=alg_bytes,
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
                out=d["C"], alpha=d["alpha"], beta=d["beta"], workspace=ws, stream=stream.cuda_stream)

    n_settle = settle(step, device)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize(device)
    # the timed steps run back to back between two events: an event after
    # every step would add a queue marker to each microsecond-scale step
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize(device)
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    # per-step times (median, minimum) from a second, separately timed pass
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize(device)
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    plan = tg.plan_for(d["As"][0], d["Bs"][0], trans_a=p.trans_a, trans_b=p.trans_b)
    per_sorted = sorted(per)
    return dict(name=name, p=p, d=d, ms_per_step=total_ms / steps,
                ms_median=per_sorted[len(per_sorted) // 2], ms_min=per_sorted[0], wall_s=wall,
                plan=plan, settle_steps=n_settle)


def prepare_softmax(name: str, device):
    import torch
    from gemm_inputs import DTYPE_NAMES, ELEM_BYTES, SOFTMAX_WORKLOADS, make_softmax_input
    w = SOFTMAX_WORKLOADS[name]
    p = make_softmax_input(w["M"], w["N"], w["dtype"], w["dist"], w["seed"])
    X = dev_tensor(p.X, p.dtype, device)
    s = ELEM_BYTES[p.dtype]
    copies = max(1, math.ceil(ROTATE_BYTES / (s * p.M * p.N)))
    Xs = [X] + [X.clone() for _ in range(copies - 1)]
    Y = torch.empty_like(X)
    return dict(p=p, Xs=Xs, Y=Y, copies=copies, alg_bytes=2 * s * p.M * p.N,
                dtype=DTYPE_NAMES[p.dtype])


def time_softmax(name: str, steps: int, warmup: int, device):
    """One step = tg_softmax over the whole M x N input (rotated over copies
    whose total passes the last-level cache), timed with HIP events on the
    launch stream."""
    import torch
    import tiled_gemm_02_amd as tg
    d = prepare_softmax(name, device)
    p = d["p"]
    stream = torch.cuda.current_stream(device)

    def step(i):
        tg.softmax(d["Xs"][i % d["copies"]], out=d["Y"], stream=stream.cuda_stream)

    n_settle = settle(step, device)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize(device)
    total_ms = e0.elapsed_time(e1)
    q, c = tg.softmax_shape(p.N, p.dtype)
    return dict(name=name, p=p, d=d, ms_per_step=total_ms / steps, shape=(q, c), settle_steps=n_settle)


def cpu_baseline(name: str, target_s: float):
    """The oracle on a bounded sample of output rows of the workload, on the host cores."""
    import numpy as np
    import oracle
    from gemm_inputs import WORKLOADS, make_problem
    w = dict(WORKLOADS[name])
    epi = w.pop("epilogue", None)
    slope = w.pop("slope", 0.01)
    alpha = w.pop("alpha", 1.0)
    beta = w.pop("beta", 0.0)
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
    hc = host_cpu()
    return {"value": 2.0 * macs / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host_usable_cpus": hc["usable_cpus"], "host_nproc": hc["nproc"], "cpu_model": hc["cpu_model"],
            "sample": f"{rows} full output rows ({rows}x{p.N} elements, {macs / 1e9:.1f} G multiply-adds) "
                      f"of the {p.M}x{p.N}x{p.K} {name} workload, fp64 triple loop on {threads} threads, "
                      f"{t:.1f} s"}


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


# ---------------------------------------------------------------- HBM traffic counters
#
# roofline.traffic comes from two rocprofv3 counter passes per workload
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) over `bench.py --traffic-kernel
# NAME`, each scaled by what the same counter reads for a plain 256 MiB device
# copy (`--traffic-kernel copy`).  `--traffic-summarize DIR` turns the counter
# files into TRAFFIC_FILE, tagged with a hash of the kernel sources so that a
# changed kernel reports null until it is measured again.

TRAFFIC_WORKLOADS = ["f16_8192", "f16_skinny_8192x128x8192", "f16_gemv_1x8192x8192",
                     "softmax_f32_4096x32768", "softmax_f16_4096x32768", "f16_4096_nt", "f32_8192_nt",
                     "bf16_leaky_8192", "bf16_leaky_6912x2048x4096", "f32_256"]
COPY_BYTES = 256 << 20
DOMINANT = {"mfma": "mfma_", "skinny": "skinny_kernel", "softmax": "softmax_rows_kernel"}
# GEMV: gemv_cols / gemv_rows


def traffic_kernel(name: str, launches: int = 6):
    """Run one workload's kernels (or the calibration copy) for a counter pass."""
    import torch
    device = torch.device("cuda:0")
    if name == "copy":
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        for _ in range(launches):
            dst.copy_(src)
        torch.cuda.synchronize(device)
        return
    if name.startswith("softmax_"):
        time_softmax(name, launches, 1, device)
        return
    from gemm_inputs import WORKLOADS
    w = WORKLOADS[name]
    time_workload(name, launches, 1, device, rotate=bound_of(w["M"], w["N"], w["K"], w["dtype"]) == "hbm")


def _counter_avg(csv_path: str, sub: str, counter: str):
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if sub in r["Kernel_Name"] and r["Counter_Name"] == counter:
            d = int(r["Dispatch_Id"])
            per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    ids = sorted(per)[1:] if len(per) > 1 else sorted(per)   # the first dispatch runs cold
    return (sum(per[i] for i in ids) / len(ids), len(ids)) if ids else (None, 0)


def traffic_summarize(root: str):
    import glob
    import tiled_gemm_02_amd as tg
    from gemm_inputs import ELEM_BYTES, SOFTMAX_WORKLOADS, WORKLOADS

    def find(tag):
        f = glob.glob(os.path.join(root, tag, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter file under {root}/{tag}")
        return f[0]

    cf, _ = _counter_avg(find("copy_fetch"), "copy", "FETCH_SIZE")
    cw, _ = _counter_avg(find("copy_write"), "copy", "WRITE_SIZE")
    k_fetch = COPY_BYTES / (cf * 1024.0)
    k_write = COPY_BYTES / (cw * 1024.0)
    out = {"_calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                            "fetch_factor": k_fetch, "write_factor": k_write}}
    lines = ["# HBM traffic per launch of each workload's dominant kernel", "",
             "Counters: rocprofv3 `FETCH_SIZE` and `WRITE_SIZE` (KiB per dispatch, first dispatch",
             "dropped), one pass each, scaled by the reading of the same counter for a plain",
             f"{COPY_BYTES >> 20} MiB device copy (factors {k_fetch:.3f} fetch, {k_write:.3f} write).", "",
             "Commands (repository root, one MI355X; NAME is each workload below, and `copy`):", "",
             "```",
             f"rocprofv3 --pmc FETCH_SIZE -d {root}/NAME_fetch -o run --output-format csv -- python3 bench.py --traffic-kernel NAME",
             f"rocprofv3 --pmc WRITE_SIZE -d {root}/NAME_write -o run --output-format csv -- python3 bench.py --traffic-kernel NAME",
             f"python3 bench.py --traffic-summarize {root}",
             "```", "",
             "| Workload | Kernel | Fetch (MiB) | Write (MiB) | Total (MiB) | Algorithmic (MiB) | Ratio |",
             "|---|---|---|---|---|---|---|"]
    for name in TRAFFIC_WORKLOADS:
        fam = kernel_family(name)
        if fam == "softmax":
            w = SOFTMAX_WORKLOADS[name]
            sub = DOMINANT["softmax"] if w["N"] <= 32768 else "softmax_long_kernel"
            alg = 2 * ELEM_BYTES[w["dtype"]] * w["M"] * w["N"]
        else:
            w = WORKLOADS[name]
            plan = tg.tg_plan_model(w["M"], w["N"], w["K"], w["dtype"], w["trans"], num_cus=256)
            if plan["path_name"] == "gemv":
                sub = "gemv_rows" if plan["tile_m"] == 4 else "gemv_cols"
            else:
                sub = DOMINANT[plan["path_name"]]
            alg = ELEM_BYTES[w["dtype"]] * (w["M"] * w["K"] + w["K"] * w["N"] + w["M"] * w["N"])
        f, nf = _counter_avg(find(name + "_fetch"), sub, "FETCH_SIZE")
        wr, nw = _counter_avg(find(name + "_write"), sub, "WRITE_SIZE")
        if f is None or wr is None:
            raise SystemExit(f"no {sub} dispatches for {name}")
        fb, wb = f * 1024.0 * k_fetch, wr * 1024.0 * k_write
        out[name] = {"kernel": sub, "kernel_hash": kernel_source_hash(fam), "fetch_bytes": fb,
                     "write_bytes": wb, "bytes_per_launch": fb + wb, "alg_bytes": alg,
                     "dispatches": [nf, nw]}
        lines.append(f"| {name} | `{sub}` | {fb / 2**20:.1f} | {wb / 2**20:.1f} | {(fb + wb) / 2**20:.1f} | "
                     f"{alg / 2**20:.1f} | {(fb + wb) / alg:.3f} |")
    lines += ["", "Kernel source hashes: " + ", ".join(f"{f} `{kernel_source_hash(f)}`" for f in KERNEL_SOURCES), ""]
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    open(os.path.join(ROOT, "profiles", "traffic_summary.md"), "w").write("\n".join(lines))
    print("\n".join(lines))


# ---------------------------------------------------------------- kernel-time summary
#
# `rocprofv3 --kernel-trace --stats -d DIR -o run --output-format csv -- python3 bench.py ...`
# with the bench's own JSON line saved as DIR/bench.json; `--kernel-stats-summarize DIR OUT`
# groups the library's dispatches by (kernel, workgroup grid), which tells the workloads
# apart even where two of them run the same kernel, and sets each line's step time beside
# its dominant kernel's average from the same run.

def _dominant_match(line, name, wgx, wgy):
    """Whether a dispatch of `name` on a (wgx, wgy) workgroup grid is the dominant kernel of
    the bench line `line` (headline or secondary dict)."""
    plan = line.get("plan") or line.get("config", {}).get("plan") or {}
    cfg = line.get("config", {})
    dt = {"f16": "F16", "bf16": "BF16", "f32": "F32"}.get(cfg.get("dtype") or line.get("dtype"), "")
    wl = line.get("workload") or cfg.get("workload", "")
    if wl.startswith("softmax_"):
        return "softmax_rows_kernel" in name and f"<tg::{dt}," in name
    path = plan.get("path_name")
    if path == "mfma":
        return (name.startswith("void tg::mfma_") and f"<tg::{dt}," in name and wgx == plan.get("tiles")
                and wgy == max(1, plan.get("split_k", 1)))
    if path == "skinny":
        return "skinny_kernel" in name and f"<tg::{dt}," in name and wgx == plan.get("tiles") and \
            wgy == max(1, plan.get("split_k", 1))
    if path == "gemv":
        return "gemv_" in name and "reduce" not in name and f"<tg::{dt}," in name
    return False


def kernel_stats_summarize(root: str, out_path: str):
    import csv
    import glob
    trace = glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True)
    if not trace:
        raise SystemExit(f"no kernel_trace.csv under {root}")
    line = json.loads(open(os.path.join(root, "bench.json")).read().strip().splitlines()[-1])
    groups = {}
    for r in csv.DictReader(open(trace[0])):
        name = r["Kernel_Name"]
        if "tg::" not in name:
            continue
        wgx = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        wgy = int(r["Grid_Size_Y"]) // max(1, int(r["Workgroup_Size_Y"]))
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((name, wgx, wgy), []).append(us)
    total = sum(sum(v) for v in groups.values())
    lines = [line] + [dict(sc) for sc in line.get("secondary", [])]
    out = ["# Kernel time summary of the default benchmark command", "",
           "Command (repository root, one MI355X; the bench's own JSON line from the same run goes",
           "to bench.json):", "", "```",
           f"rocprofv3 --kernel-trace --stats -d {root} -o run --output-format csv -- "
           f"python3 bench.py {line.get('bench_args', '')}".rstrip() + f" > {root}/bench.json",
           f"python3 bench.py --kernel-stats-summarize {root} {out_path}", "```", "",
           "Dispatches are grouped by kernel and workgroup grid (x tiles, y K splits), which tells",
           "the workloads apart where two of them run the same kernel.  Each line's step time is",
           "the bench's own HIP-event figure from the profiled run (kernel tracing serialises the",
           "launches, so profiled steps run somewhat longer than unprofiled ones); a step holds the",
           "dominant kernel and, where the plan splits K, the reduction, so the kernel average must",
           "not exceed it.  Calls / Avg / Min / Max cover the launches of the timed pass only (the",
           "settle and warm-up launches before it, the first of them cold, and the per-step pass",
           "after it are left out); the table of all kernels below counts every launch.", "",
           "| Bench line | Step (us) | Dominant kernel | Grid | Calls | Avg (us) | Min (us) | Max (us) | Avg <= step |",
           "|---|---|---|---|---|---|---|---|---|"]
    for ln in lines:
        wl = ln.get("workload") or ln.get("config", {}).get("workload")
        if wl is None or wl.startswith("sweep"):
            continue
        step_us = ln["ms_per_step"] * 1e3
        hit = [(k, v) for k, v in groups.items() if _dominant_match(ln, *k)]
        if not hit:
            out.append(f"| {wl} | {step_us:.1f} | (no matching dispatch) | | | | | | |")
            continue
        (name, gx, gy), v = max(hit, key=lambda kv: len(kv[1]))
        # the launches of the timed pass: the timed pass and the per-step pass,
        # `steps` each, come last in the group (the settle and warm-up
        # launches come first, the coldest among them)
        n_timed = ln.get("steps") or max(int(line.get("steps", 50)), 50)
        v = v[-2 * n_timed:-n_timed]
        avg = sum(v) / len(v)
        short = name.replace("void tg::", "").split("(")[0]
        out.append(f"| {wl} | {step_us:.1f} | `{short}` | {gx} x {gy} | {len(v)} | {avg:.1f} | {min(v):.1f} | "
                   f"{max(v):.1f} | {'yes' if avg <= step_us else 'NO'} |")
    out += ["", "All library kernels of the run:", "",
            "| Kernel | Grid | Calls | Avg (us) | Min (us) | Max (us) | Share |", "|---|---|---|---|---|---|---|"]
    for (name, gx, gy), v in sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:40]:
        short = name.replace("void tg::", "").split("(")[0]
        out.append(f"| `{short}` | {gx} x {gy} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} | "
                   f"{100 * sum(v) / total:.1f}% |")
    out.append("")
    open(out_path, "w").write("\n".join(out))
    print("\n".join(out))


# ---------------------------------------------------------------- quantization sweep

def tile_label(pl: dict) -> str:
    """Macro tile of a plan, marked when two K groups share each workgroup."""
    t = f"{pl['tile_m']}x{pl['tile_n']}"
    return t + " x2K" if pl.get("k_groups", 1) == 2 else t


def sweep_summary(device, step: int = 64, reps: int = 20) -> dict:
    """The tile/wave-quantization sweep at a coarse step for the benchmark line:
    fp16 M = 2304, K = 4096, N = 1536 .. 6144 every `step` columns, the
    planner's plan, inputs N(0,1)/sqrt(K) from a seeded device generator (B is
    the first N columns of one 4096 x 6144 draw, made contiguous).  Each point
    is the mean of `reps` calls issued back to back between two events, after
    untimed calls that keep the GPU busy (a quarter second before the first
    point, 20 ms before each later one), with one persistent workspace;
    reported as TFLOP/s over the points."""
    import torch
    import tiled_gemm_02_amd as tg
    from gemm_inputs import sweep_ns
    M, K = 2304, 4096
    g = torch.Generator(device=device).manual_seed(0)
    A = (torch.randn((M, K), generator=g, device=device) / math.sqrt(K)).half()
    Bfull = (torch.randn((K, 6144), generator=g, device=device) / math.sqrt(K)).half()
    stream = torch.cuda.current_stream(device)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=device)
    pts = []
    first = True
    for N in sweep_ns(step=step):
        B = Bfull[:, :N].contiguous()
        C = torch.empty((M, N), dtype=torch.float16, device=device)

        def call(_i=0):
            tg.gemm(A, B, out=C, workspace=ws, stream=stream.cuda_stream)
        settle(call, device, SETTLE_S if first else 0.02)
        first = False
        ms = time_back_to_back(call, stream, reps)
        pl = tg.tg_gemm_plan(M, N, K, tg.TG_F16, tg.TG_NN)
        pts.append((N, 2.0 * M * N * K / ms / 1e9, pl))
    tf = sorted(v for _, v, _ in pts)
    low = sorted(v for n, v, _ in pts if n <= 1792)
    mean = sum(tf) / len(tf)
    peak = PEAK_TFLOPS["f16"]
    return {"workload": "sweep_2304xNx4096_f16", "unit": "TFLOP/s", "points": len(pts), "step": step,
            "n_range": [pts[0][0], pts[-1][0]],
            "value": round(mean, 2), "mean": round(mean, 2), "median": round(tf[len(tf) // 2], 2),
            "min": round(tf[0], 2), "max": round(tf[-1], 2),
            "median_n_le_1792": round(low[len(low) // 2], 2) if low else None,
            "per_point": [[n, round(v, 1), tile_label(pl), pl["split_k"], pl["tiles"]]
                          for n, v, pl in pts],
            "roofline": {"bound": "mfma", "achieved": round(mean, 2), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(mean / peak, 4), "traffic": None}}


def sweep(out_path: str, step: int, reps: int = 20, tune: bool = False):
    """fp16 M=2304, K=4096, N = 1536 .. 6144: the planner's tile against a fixed 256 x 256 one.

    Inputs are N(0,1)/sqrt(K), seeded; each point is the mean of `reps` calls issued back to
    back between two HIP events on the launch stream, after untimed calls that keep the GPU
    busy (a quarter second before the first point, 20 ms before each later one)."""
    import torch
    import tiled_gemm_02_amd as tg
    from gemm_inputs import F16, NN, sweep_ns
    device = torch.device("cuda:0")
    M, K = 2304, 4096
    g = torch.Generator(device=device).manual_seed(4)
    A = (torch.randn((M, K), generator=g, device=device) / math.sqrt(K)).half()
    Bfull = (torch.randn((K, 6144), generator=g, device=device) / math.sqrt(K)).half()
    Cfull = torch.empty((M, 6144), dtype=torch.float16, device=device)
    stream = torch.cuda.current_stream(device)
    fixed = dict(path=tg.TG_PATH_MFMA, tile_m=256, tile_n=256, split_k=1)
    tg.tune_cache_clear()   # the planner column is the heuristic, not a recorded winner

    # split-K partials go to one persistent workspace (as in the timed bench)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=device)

    first = [True]

    def timed(B, C, opts):
        def call(_i=0):
            tg.gemm(A, B, out=C, options=opts, workspace=ws, stream=stream.cuda_stream)
        settle(call, device, SETTLE_S if first[0] else 0.02)
        first[0] = False
        return time_back_to_back(call, stream, reps)

    rows = []
    tuned = []   # (N, planner TFLOP/s, best TFLOP/s, best options)
    for N in sweep_ns(step=step):
        B = Bfull[:, :N].contiguous()
        C = Cfull[:, :N]
        pl = tg.tg_gemm_plan(M, N, K, F16, NN)
        ms = timed(B, C, None)
        ms_f = timed(B, C, fixed)
        fl = 2.0 * M * N * K
        rows.append((N, tile_label(pl), "", pl["split_k"], pl["tiles"], pl["waves"],
                     fl / ms / 1e9, fl / ms_f / 1e9, pl["pred_eff"]))
        msg = (f"N={N} plan {tile_label(pl)} tiles {pl['tiles']} waves {pl['waves']}: "
               f"{rows[-1][6]:.0f} TFLOP/s (fixed 256x256: {rows[-1][7]:.0f})")
        if tune:
            best, _ = tg.autotune(A, B, out=C, workspace=ws, reps=3)
            ms_b = timed(B, C, None if best["path"] == tg.TG_PATH_AUTO else best)
            tuned.append((N, fl / ms / 1e9, fl / ms_b / 1e9, best))
            msg += f" (autotuned {tile_label(best)} s{best['split_k']}: {fl / ms_b / 1e9:.0f})"
        log(msg)
    better = sum(1 for r in rows if r[6] >= r[7] * 0.98)
    mean_p = sum(r[6] for r in rows) / len(rows)
    mean_f = sum(r[7] for r in rows) / len(rows)
    lines = ["# Tile/wave-quantization sweep: fp16 M=2304, K=4096, N = 1536 .. 6144", "",
             "Command (repository root, one MI355X):", "", "```",
             f"python3 bench.py --sweep {out_path} --sweep-step {step}", "```", "",
             f"{len(rows)} points, step {step}.  Mean TFLOP/s: planner {mean_p:.0f}, fixed 256x256 "
             f"{mean_f:.0f}; the planner is within 2 % of or above the fixed tile at {better} of "
             f"{len(rows)} points.", "",
             "Bands of equal plan (tile, waves of 256 CUs; x2K: two K groups per workgroup, summed in LDS); "
             "TFLOP/s min / median / max within the band:", "",
             "| N range | Tile | Split | Tiles | Waves | Planner TFLOP/s | Fixed 256x256 TFLOP/s |",
             "|---|---|---|---|---|---|---|"]
    i = 0
    while i < len(rows):
        j = i
        while j + 1 < len(rows) and rows[j + 1][1:4] == rows[i][1:4] and rows[j + 1][5] == rows[i][5]:
            j += 1
        band = rows[i:j + 1]
        def mmm(k):
            v = sorted(r[k] for r in band)
            return f"{v[0]:.0f} / {v[len(v) // 2]:.0f} / {v[-1]:.0f}"
        lines.append(f"| {band[0][0]}-{band[-1][0]} | {band[0][1]} | {band[0][3]} | "
                     f"{band[0][4]}-{band[-1][4]} | {band[0][5]} | {mmm(6)} | {mmm(7)} |")
        i = j + 1
    lines.append("")
    if tuned:
        ratio = sorted(t[1] / t[2] for t in tuned)
        within = sum(1 for r in ratio if r >= 0.95)
        lines += ["## The planner against benchmark mode", "",
                  f"At each point `tg_autotune` timed every candidate (planner's choice, every tile "
                  f"x split 1-8, skinny); the winner and the planner were then timed again the "
                  f"same way.  Planner / best TFLOP/s: median {ratio[len(ratio) // 2]:.3f}, "
                  f"minimum {ratio[0]:.3f}; within 5 % at {within} of {len(tuned)} points.", "",
                  "| N | Planner TFLOP/s | Best TFLOP/s | Best plan |", "|---|---|---|---|"]
        for (N, tp, tb, b) in tuned:
            if tp / tb < 0.95:
                plan = "planner's" if b["path"] == tg.TG_PATH_AUTO else (
                    f"{tile_label(b)} split {b['split_k']}" if b["path"] == tg.TG_PATH_MFMA
                    else f"skinny split {b['split_k']}")
                lines.append(f"| {N} | {tp:.0f} | {tb:.0f} | {plan} |")
        lines += ["", "(rows listed: points where the planner is more than 5 % below the best)", ""]
    open(out_path, "w").write("\n".join(lines))
    print("\n".join(lines))


def planner_check(out_path: str, reps: int = 10):
    """How close the planner's pick is to the fastest plan the library offers, over
    assorted fp16 products: M, N from 1024 to 8192 with K = 1024, 4096 and 8192 (NN)
    and four NT shapes.  At each shape the planner's plan and every macro tile (one K
    group, and the K-group forms) at K splits 1, 2 and 4 are timed back to back
    (`reps` calls between two events, after untimed calls that keep the GPU busy:
    a quarter second before the first timing, 20 ms before each later one), with one
    persistent workspace; plans needing more workspace are skipped."""
    import torch
    import tiled_gemm_02_amd as tg
    device = torch.device("cuda:0")
    stream = torch.cuda.current_stream(device)
    g = torch.Generator(device=device).manual_seed(6)
    ws_bytes = 256 << 20
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    tg.tune_cache_clear()
    tiles = [(256, 256, 1), (192, 256, 1), (256, 128, 1), (128, 128, 1), (128, 128, 2), (128, 64, 1),
             (64, 64, 1), (64, 64, 4)]
    cands = [None] + [dict(path=tg.TG_PATH_MFMA, tile_m=bm, tile_n=bn, k_groups=kg, split_k=sp)
                      for bm, bn, kg in tiles for sp in (1, 2, 4)]
    shapes = [(M, N, K, tg.TG_NN) for (M, N) in [(1024, 1024), (1024, 3072), (2048, 2048), (3072, 2048),
                                                  (3072, 3072), (4096, 2048), (4096, 4096), (6144, 4096),
                                                  (5120, 5120), (8192, 4096), (1536, 6144), (2560, 2560)]
              for K in (1024, 4096, 8192)]
    shapes += [(4096, 4096, 4096, tg.TG_NT), (2304, 2048, 4096, tg.TG_NT), (3072, 3072, 2048, tg.TG_NT),
               (2048, 2048, 8192, tg.TG_NT)]
    first = [True]
    rows = []
    for M, N, K, tr in shapes:
        A = (torch.randn((M, K), generator=g, device=device) / math.sqrt(K)).half()
        B = (torch.randn((N, K) if tr == tg.TG_NT else (K, N), generator=g, device=device) / math.sqrt(K)).half()
        C = torch.empty((M, N), dtype=torch.float16, device=device)
        times = []
        for o in cands:
            try:
                pl = tg.tg_gemm_plan(M, N, K, tg.TG_F16, tr, options=o)
            except tg.TgError:
                continue
            if pl["workspace_bytes"] > ws_bytes:
                continue

            def call(_i=0):
                tg.gemm(A, B, trans_b=tr == tg.TG_NT, out=C, options=o, workspace=ws, stream=stream.cuda_stream)
            settle(call, device, SETTLE_S if first[0] else 0.02)
            first[0] = False
            times.append((time_back_to_back(call, stream, reps), o is None, pl))
        # the planner's plan is also among the forced candidates (unless it splits K
        # another way): its time is the best of those timings, since the first
        # timing of a shape comes straight after the previous shape's
        pp = [t for t in times if t[1]][0][2]
        same = [t for t in times if (t[2]["tile_m"], t[2]["tile_n"], t[2]["split_k"], t[2]["k_groups"]) ==
                (pp["tile_m"], pp["tile_n"], pp["split_k"], pp["k_groups"])]
        planner = min(same, key=lambda t: t[0])
        best = min(times, key=lambda t: t[0])
        rows.append((M, N, K, tr, planner, best, planner[0] / best[0]))
        log(f"{M}x{N}x{K} {'NT' if tr == tg.TG_NT else 'NN'}: planner {tile_label(planner[2])} "
            f"s{planner[2]['split_k']} {planner[0] * 1e3:.1f} us, best {tile_label(best[2])} "
            f"s{best[2]['split_k']} {best[0] * 1e3:.1f} us")
        del A, B, C
    ratios = sorted(r[6] for r in rows)
    mean = sum(ratios) / len(ratios)
    behind = sum(1 for q in ratios if q > 1.05)
    lines = ["# The planner's pick against every plan, fp16 products", "",
             "Command (repository root, one MI355X):", "", "```",
             f"python3 bench.py --planner-check {out_path}", "```", "",
             f"{len(rows)} shapes.  Planner time / best time: mean {mean:.4f}, median "
             f"{ratios[len(ratios) // 2]:.4f}, worst {ratios[-1]:.3f}; more than 5 % behind at {behind}.", "",
             "| M | N | K | Layout | Planner plan | us | Best plan | us | Planner / best |",
             "|---|---|---|---|---|---|---|---|---|"]
    for M, N, K, tr, pl, b, q in rows:
        lines.append(f"| {M} | {N} | {K} | {'NT' if tr == tg.TG_NT else 'NN'} | {tile_label(pl[2])} split "
                     f"{pl[2]['split_k']} | {pl[0] * 1e3:.1f} | {tile_label(b[2])} split {b[2]['split_k']} | "
                     f"{b[0] * 1e3:.1f} | {q:.3f} |")
    lines.append("")
    open(out_path, "w").write("\n".join(lines))
    print("\n".join(lines))


def align_sweep(out_path: str, reps: int = 20):
    """fp16 NN products of about 4096^3 with one size off the 16-byte grid: K = 4096 + d
    (rows of A off the grid) and M = N = 4096 + d (ragged tiles and rows of B and C off
    the grid) for d = 0 .. 16 (the alignment effect of "Matrix Multiplication Background
    User's Guide", section 2.2, Figure 2).  Aligned sizes take the LDS-DMA kernels directly, the
    others aligned copies (staged in float32 when M or N is off the grid).  Each point is the
    mean of `reps` calls issued back to back after untimed calls that keep the GPU busy."""
    import torch
    import tiled_gemm_02_amd as tg
    device = torch.device("cuda:0")
    stream = torch.cuda.current_stream(device)
    g = torch.Generator(device=device).manual_seed(6)
    lines = ["# Alignment sweep: fp16 NN, one size off the 16-byte grid", "",
             "Command (repository root, one MI355X):", "", "```",
             f"python3 bench.py --align-sweep {out_path}", "```", "",
             "Loads: vector = 128-bit loads of the caller's operands, copied = aligned",
             "zero-padded copies first (padded in M and N too where those are off the grid;",
             "the kernel then stores only the M x N corner).", "",
             "| M | N | K | Path | Tile | Split | Loads | us | TFLOP/s |",
             "|---|---|---|---|---|---|---|---|---|"]
    shapes = [(4096, 4096, 4096 + d) for d in range(17)] + \
             [(4096 + d, 4096 + d, 4096) for d in range(1, 17)]
    for M, N, K in shapes:
        A = (torch.randn((M, K), generator=g, device=device) / math.sqrt(K)).half()
        B = (torch.randn((K, N), generator=g, device=device) / math.sqrt(K)).half()
        C = torch.empty((M, N), dtype=torch.float16, device=device)
        pl = tg.plan_for(A, B)

        def call(_i=0):
            tg.gemm(A, B, out=C, stream=stream.cuda_stream)
        settle(call, device, SETTLE_S if M == N == K == 4096 else 0.02)
        ms = time_back_to_back(call, stream, reps)
        tf = 2.0 * M * N * K / ms / 1e9
        loads = {0: "element-wise", 1: "vector", 2: "copied", 3: "copied as NT"}[pl["vector_io"]]
        # plan_for assumes packed operands; the real call sees the same strides here
        lines.append(f"| {M} | {N} | {K} | {pl['path_name']} | {tile_label(pl)} | "
                     f"{pl['split_k']} | {loads} | {ms * 1e3:.0f} | {tf:.0f} |")
        log(lines[-1])
    lines.append("")
    open(out_path, "w").write("\n".join(lines))
    print("\n".join(lines))


def stream_k_compare(out_path: str, reps: int = 20):
    """Stream-K against whole-tile plans: the planner's choice, forced stream-K
    (split_k = TG_SPLIT_STREAM_K) and forced 256 x 256 tiles without a split, on
    the M = 2304, K = 4096 quantization shapes that leave CUs idle, the bf16
    6912 x 2048 x 4096 shape, and small-M/N, large-K products.  Each point is the
    mean of `reps` calls issued back to back between two events, after untimed
    calls that keep the GPU busy, with a 256 MiB caller workspace; inputs
    N(0, 1)/64 from a seeded device generator."""
    import torch
    import tiled_gemm_02_amd as tg
    device = torch.device("cuda:0")
    stream = torch.cuda.current_stream(device)
    g = torch.Generator(device=device).manual_seed(1)
    ws = torch.empty(256 << 20, dtype=torch.uint8, device=device)
    tg.tune_cache_clear()

    first = [True]

    def timed(A, B, C, opts):
        def call(_i=0):
            tg.gemm(A, B, out=C, options=opts, workspace=ws, stream=stream.cuda_stream)
        settle(call, device, SETTLE_S if first[0] else 0.05)
        first[0] = False
        return time_back_to_back(call, stream, reps)

    lines = ["# Stream-K against whole-tile plans (one MI355X)", "",
             "Command (repository root, one MI355X):", "", "```",
             f"python3 bench.py --stream-k-compare {out_path}", "```", "",
             "Each point: mean of calls issued back to back after untimed busy calls, 256 MiB caller workspace;",
             "TFLOP/s = 2MNK / time.", "",
             "| Shape | dtype | Planner's plan | Planner TFLOP/s | Stream-K TFLOP/s (us) | 256x256, no split |",
             "|---|---|---|---|---|---|"]
    shapes = [(2304, n, 4096, torch.float16) for n in (2048, 3072, 3592, 4096, 4608, 5120, 5632)] + \
             [(6912, 2048, 4096, torch.bfloat16), (1024, 1024, 4096, torch.float16),
              (512, 512, 16384, torch.float16), (256, 256, 65536, torch.float16)]
    for M, N, K, dt in shapes:
        A = (torch.randn((M, K), generator=g, device=device) / 64).to(dt)
        B = (torch.randn((K, N), generator=g, device=device) / 64).to(dt)
        C = torch.empty((M, N), dtype=dt, device=device)
        fl = 2.0 * M * N * K
        pl = tg.plan_for(A, B)
        t_p = timed(A, B, C, None)
        t_sk = timed(A, B, C, dict(split_k=tg.TG_SPLIT_STREAM_K))
        t_dp = timed(A, B, C, dict(tile_m=256, tile_n=256, split_k=1))
        name = "bf16" if dt == torch.bfloat16 else "fp16"
        lines.append(f"| {M}x{N}x{K} | {name} | {tile_label(pl)} split {pl['split_k']} | "
                     f"{fl / t_p / 1e9:.0f} | {fl / t_sk / 1e9:.0f} ({t_sk * 1e3:.1f}) | {fl / t_dp / 1e9:.0f} |")
        log(lines[-1])
        del A, B, C
    lines.append("")
    open(out_path, "w").write("\n".join(lines))
    print("\n".join(lines))


def softmax_sweep(out_path: str, reps: int = 20):
    """Row softmax at M = 4096 over row lengths N = 256 .. 32768 and beyond (the
    shape of the Triton page's A100 figure, "OpenAI open-sources Triton",
    programming-model section), float32 and float16, in GB/s of one read and
    one write of X.  torch.softmax on the same tensors is timed beside it as
    context.  Inputs N(0, 1) from a seeded device generator; each point is the
    median of `reps` timed calls after two warm-up calls, alternating between
    enough input copies to exceed the last-level cache."""
    import torch
    import tiled_gemm_02_amd as tg
    device = torch.device("cuda:0")
    stream = torch.cuda.current_stream(device)
    g = torch.Generator(device=device).manual_seed(8)
    M = 4096
    lines = ["# Row softmax sweep, M = 4096", "",
             "Command (repository root, one MI355X):", "", "```",
             f"python3 bench.py --softmax-sweep {out_path}", "```", "",
             "GB/s = 2 M N (element bytes) / time: one read of X and one write of Y. Shape = waves",
             "per row x 16-byte chunks per lane of the register-resident kernel (0x0: two-pass",
             "kernel, which reads X twice). torch.softmax(dim=1) on the same tensors and a plain",
             "device copy of X into Y (the same bytes moved, no arithmetic) are context.", "",
             "| dtype | N | shape | us | GB/s | % of 8 TB/s | torch us | torch GB/s | copy GB/s |",
             "|---|---|---|---|---|---|---|---|---|"]

    def timed(fn, xs):
        for i in range(2):
            fn(xs[i % len(xs)])
        ts = []
        for i in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(xs[i % len(xs)])
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    for dt, tdt in [("f32", torch.float32), ("f16", torch.float16)]:
        for N in [256, 512, 1024, 2048, 4096, 8192, 12288, 16384, 24576, 32768, 65536]:
            es = torch.tensor([], dtype=tdt).element_size()
            copies = max(2, math.ceil(ROTATE_BYTES / (M * N * es)))
            xs = [torch.randn((M, N), generator=g, device=device).to(tdt) for _ in range(copies)]
            Y = torch.empty_like(xs[0])
            ms = timed(lambda x: tg.softmax(x, out=Y, stream=stream.cuda_stream), xs)
            mt = timed(lambda x: torch.softmax(x, dim=1), xs)
            mc = timed(lambda x: Y.copy_(x), xs)
            gbs, gbt = 2 * M * N * es / ms / 1e6, 2 * M * N * es / mt / 1e6
            gbc = 2 * M * N * es / mc / 1e6
            q, c = tg.softmax_shape(N, tg.TG_F32 if dt == "f32" else tg.TG_F16)
            lines.append(f"| {dt} | {N} | {q}x{c} | {ms * 1e3:.1f} | {gbs:.0f} | {gbs / PEAK_HBM_GBS * 100:.1f} | "
                         f"{mt * 1e3:.1f} | {gbt:.0f} | {gbc:.0f} |")
            log(lines[-1])
            del xs, Y
            torch.cuda.empty_cache()
    lines.append("")
    open(out_path, "w").write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="f16_8192")
    ap.add_argument("--secondary", default="f16_skinny_8192x128x8192,f16_gemv_1x8192x8192,"
                    "f16_4096_nt,bf16_leaky_8192,bf16_leaky_6912x2048x4096,f32_256,sweep,"
                    "softmax_f32_4096x32768,softmax_f16_4096x32768,f32_8192_nt",
                    help="comma-separated workloads reported alongside ('' for none); 'sweep' is "
                         "the M=2304, K=4096 N-sweep at step 64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--sweep", default=None,
                    help="run the M=2304, K=4096 N-sweep, write its summary to this file, then exit")
    ap.add_argument("--sweep-step", type=int, default=8)
    ap.add_argument("--sweep-tune", action="store_true",
                    help="with --sweep: also time tg_autotune's best plan at every point")
    ap.add_argument("--planner-check", default=None,
                    help="time the planner's pick against every plan on assorted fp16 products, "
                         "write the table to this file, then exit")
    ap.add_argument("--align-sweep", default=None,
                    help="run the K-alignment sweep, write its summary to this file, then exit")
    ap.add_argument("--stream-k-compare", default=None,
                    help="time stream-K against whole-tile plans, write the table to this file, then exit")
    ap.add_argument("--softmax-sweep", default=None,
                    help="run the M=4096 row-softmax sweep over N, write its summary to this file, then exit")
    ap.add_argument("--traffic-kernel", default=None,
                    help="run one workload (or 'copy') for a rocprofv3 counter pass, then exit")
    ap.add_argument("--traffic-summarize", default=None,
                    help="turn counter passes under this folder into the traffic table, then exit")
    ap.add_argument("--kernel-stats-summarize", nargs=2, default=None, metavar=("DIR", "OUT"),
                    help="turn a rocprofv3 kernel trace of a bench run (with its JSON line in DIR/bench.json) "
                         "into the kernel-time table OUT, then exit")
    args = ap.parse_args()
    if args.traffic_summarize:
        traffic_summarize(args.traffic_summarize)
        return
    if args.kernel_stats_summarize:
        kernel_stats_summarize(*args.kernel_stats_summarize)
        return

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
    if args.traffic_kernel:
        traffic_kernel(args.traffic_kernel)
        return
    if args.sweep:
        sweep(args.sweep, args.sweep_step, tune=args.sweep_tune)
        return
    if args.align_sweep:
        align_sweep(args.align_sweep)
        return
    if args.planner_check:
        planner_check(args.planner_check)
        return
    if args.softmax_sweep:
        softmax_sweep(args.softmax_sweep)
        return
    if args.stream_k_compare:
        stream_k_compare(args.stream_k_compare)
        return
    log("device", torch.cuda.get_device_name(0), "cus", tg.tg_device_cus())

    w = WORKLOADS[args.workload]
    mem_bound = bound_of(w["M"], w["N"], w["K"], w["dtype"]) == "hbm"
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
        "settle": {"seconds": SETTLE_S, "steps": r["settle_steps"]},
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": d["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "M": p.M, "N": p.N, "K": p.K,
                   "layout": ["NN", "TN", "NT", "TT"][p.trans], "epilogue": d["epi"] or "none",
                   "alpha": d["alpha"], "beta": d["beta"],
                   "seed": p.desc["seed"], "dist": p.desc["dist"], "plan": {
                       k: r["plan"][k] for k in ("path_name", "tile_m", "tile_n", "split_k", "k_groups",
                                                  "tiles", "waves", "occupancy")}},
        "bench_args": " ".join(sys.argv[1:]),
        "ms_median": round(r["ms_median"], 5),
        "roofline": roofline_entry(r, "hbm" if mem_bound else "mfma"),
        "context": dict(PAGES_CONTEXT, mi355x_ridge_fp16_flop_per_byte=round(ridge("f16"), 1),
                        mi355x_ridge_fp32_flop_per_byte=round(ridge("f32"), 1),
                        workload_ai_flop_per_byte=round(r["plan"]["arith_intensity"], 1)),
    }
    sec = []
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        log("timing", name)
        if name == "sweep":
            sec.append(sweep_summary(device))
            torch.cuda.empty_cache()
            continue
        if name.startswith("softmax_"):
            rs = time_softmax(name, max(args.steps, 50), args.warmup, device)
            ent = roofline_entry(rs, "hbm")
            p = rs["p"]
            sec.append({"workload": name, "value": ent["achieved"], "unit": "GB/s",
                        "ms_per_step": round(rs["ms_per_step"], 5),
                        "steps": max(args.steps, 50), "warmup": args.warmup, "settle_steps": rs["settle_steps"],
                        "config": {"M": p.M, "N": p.N, "dtype": rs["d"]["dtype"],
                                   "waves_per_row": rs["shape"][0], "chunks_per_lane": rs["shape"][1]},
                        "roofline": ent, "rotated_copies": rs["d"]["copies"]})
            del rs
            torch.cuda.empty_cache()
            continue
        ws = WORKLOADS[name]
        sec_mem = bound_of(ws["M"], ws["N"], ws["K"], ws["dtype"]) == "hbm"
        rs = time_workload(name, max(args.steps, 50), args.warmup, device, rotate=sec_mem)
        ent = roofline_entry(rs, "hbm" if sec_mem else "mfma")
        p = rs["p"]
        sec.append({"workload": name, "value": ent["achieved"], "unit": ent["unit"],
                    "ms_per_step": round(rs["ms_per_step"], 5),
                    "us_per_step": round(rs["ms_per_step"] * 1e3, 2),
                    "steps": max(args.steps, 50), "warmup": args.warmup, "settle_steps": rs["settle_steps"],
                    "config": {"M": p.M, "N": p.N, "K": p.K, "dtype": rs["d"]["dtype"],
                               "layout": ["NN", "TN", "NT", "TT"][p.trans],
                               "epilogue": rs["d"]["epi"] or "none",
                               "ai_flop_per_byte": round(rs["plan"]["arith_intensity"], 1)},
                    "plan": {k: rs["plan"][k] for k in ("path_name", "tile_m", "tile_n", "split_k",
                                                         "k_groups", "tiles", "workgroups", "waves")},
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
