"""Capture and concurrency (run with -m gpu): the library's calls recorded into
a HIP graph (through torch.cuda.CUDAGraph) replay to the eager results bit for
bit, and calls from several host threads on their own streams are independent.

Every kernel here is deterministic (fixed summation orders), so a replay or a
concurrent call must reproduce the eager output exactly.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest

from gemm_inputs import BF16, F16, F32, NN, NT, make_problem, make_softmax_input
from tests.gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_graph_capture_replays_match_eager():
    import torch
    import tiled_gemm_02_amd as tg
    _say("case graph capture")
    dev = torch.device("cuda:0")
    # a whole-tile product, a split-K product (reduction kernel), a stream-K
    # product (fix-up kernel), 192 x 256 tiles, 128 x 128 tiles with two K
    # groups (alone, and with a K split), 64 x 64 tiles with four (16-bit, with
    # a K split) and float32 32 x 32 tiles with four, a float32 NN product through
    # its transposing copy, skinny and GEMV split-K products (reduction
    # kernels) and a row softmax, all with one caller workspace
    probs = [(make_problem(1024, 1024, 1024, F16, NN, "normal", seed=71), None),
             (make_problem(1024, 128, 4096, F16, NN, "normal", seed=77),
              dict(path=tg.TG_PATH_SKINNY, split_k=4)),
             (make_problem(1, 2048, 8192, F16, NN, "normal", seed=78), dict(path=tg.TG_PATH_GEMV, split_k=16)),
             (make_problem(256, 256, 8192, F16, NT, "normal", seed=72), dict(split_k=8)),
             (make_problem(1024, 1024, 4096, F16, NN, "normal", seed=73),
              dict(split_k=tg.TG_SPLIT_STREAM_K)),
             (make_problem(768, 1024, 1024, F16, NN, "normal", seed=75), dict(tile_m=192, tile_n=256)),
             (make_problem(2304, 1536, 1024, F16, NN, "normal", seed=79), dict(k_groups=2)),
             (make_problem(520, 392, 4104, BF16, NT, "normal", seed=80), dict(k_groups=2, split_k=3)),
             (make_problem(256, 256, 8192, F16, NN, "normal", seed=81),
              dict(tile_m=64, tile_n=64, k_groups=4, split_k=4)),
             (make_problem(256, 256, 256, F32, NN, "normal", seed=82), dict(tile_m=32, tile_n=32, k_groups=4)),
             (make_problem(1024, 1024, 1024, F32, NN, "normal", seed=76), dict(tile_m=256, tile_n=256))]
    assert tg.tg_gemm_plan(1024, 1024, 1024, tg.TG_F32, tg.TG_NN,
                           options=dict(tile_m=256, tile_n=256))["vector_io"] == 3
    ins = [(to_device(p.A, p.dtype), to_device(p.B, p.dtype), o, p) for p, o in probs]
    sp = make_softmax_input(300, 4000, F16, "normal", seed=74)
    X = to_device(sp.X, sp.dtype)
    ws = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    outs = [torch.empty((p.M, p.N), dtype=A.dtype, device=dev) for A, _, _, p in ins]
    Y = torch.empty_like(X)

    def work(stream):
        for (A, B, o, p), C in zip(ins, outs):
            tg.gemm(A, B, trans_b=p.trans_b, out=C, options=o, workspace=ws, stream=stream)
        tg.softmax(X, out=Y, stream=stream)

    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        work(s.cuda_stream)           # eager, also warms the library's caches
    s.synchronize()
    eager = [c.clone() for c in outs] + [Y.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        work(s.cuda_stream)
    A1, B1, o1, p1 = ins[1]
    C1 = torch.empty_like(outs[1])
    for rep in range(3):
        for t in outs + [Y]:
            t.fill_(float("nan"))     # eager work between replays
        # an eager call on the same workspace leaves its own partials there
        tg.gemm(A1, B1, out=C1, options=o1, workspace=ws, stream=s.cuda_stream)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (e, t) in enumerate(zip(eager, outs + [Y])):
            bits = torch.int32 if e.dtype == torch.float32 else torch.int16
            assert torch.equal(e.view(bits), t.view(bits)), (rep, i)


def test_calls_from_several_threads():
    import torch
    import tiled_gemm_02_amd as tg
    _say("case threads")
    dev = torch.device("cuda:0")
    probs = [make_problem(512 + 64 * i, 768, 1024 + 256 * i, F16, NN, "normal", seed=80 + i)
             for i in range(4)]
    # and a float32 NN product through its transposing copy (workspace per call)
    probs.append(make_problem(1024, 1024, 1024, F32, NN, "normal", seed=85))
    opts = [None] * 4 + [dict(tile_m=256, tile_n=256)]
    devs = [(to_device(p.A, p.dtype), to_device(p.B, p.dtype)) for p in probs]
    ref = []
    for (A, B), o in zip(devs, opts):
        ref.append(tg.gemm(A, B, options=o))
    torch.cuda.synchronize()
    outs = [torch.empty_like(r) for r in ref]
    errors = []

    def run(i):
        try:
            s = torch.cuda.Stream(device=dev)
            A, B = devs[i]
            for _ in range(20):
                tg.gemm(A, B, out=outs[i], options=opts[i], stream=s.cuda_stream)
            s.synchronize()
        except Exception as e:   # reported below
            errors.append((i, repr(e)))

    th = [threading.Thread(target=run, args=(i,)) for i in range(len(probs))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    for r, o in zip(ref, outs):
        bits = torch.int32 if r.dtype == torch.float32 else torch.int16
        assert torch.equal(r.view(bits), o.view(bits))
