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

from gemm_inputs import F16, NN, NT, make_problem, make_softmax_input
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
    # product (fix-up kernel) and a row softmax, all with caller workspace
    probs = [(make_problem(1024, 1024, 1024, F16, NN, "normal", seed=71), None),
             (make_problem(256, 256, 8192, F16, NT, "normal", seed=72), dict(split_k=8)),
             (make_problem(1024, 1024, 4096, F16, NN, "normal", seed=73),
              dict(split_k=tg.TG_SPLIT_STREAM_K))]
    ins = [(to_device(p.A, p.dtype), to_device(p.B, p.dtype), o, p) for p, o in probs]
    sp = make_softmax_input(300, 4000, F16, "normal", seed=74)
    X = to_device(sp.X, sp.dtype)
    ws = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    outs = [torch.empty((p.M, p.N), dtype=torch.float16, device=dev) for _, _, _, p in ins]
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
    for rep in range(3):
        for t in outs + [Y]:
            t.fill_(float("nan"))     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (e, t) in enumerate(zip(eager, outs + [Y])):
            assert torch.equal(e.view(torch.int16), t.view(torch.int16)), (rep, i)


def test_calls_from_several_threads():
    import torch
    import tiled_gemm_02_amd as tg
    _say("case threads")
    dev = torch.device("cuda:0")
    probs = [make_problem(512 + 64 * i, 768, 1024 + 256 * i, F16, NN, "normal", seed=80 + i)
             for i in range(4)]
    devs = [(to_device(p.A, p.dtype), to_device(p.B, p.dtype)) for p in probs]
    ref = []
    for (A, B) in devs:
        ref.append(tg.gemm(A, B))
    torch.cuda.synchronize()
    outs = [torch.empty_like(r) for r in ref]
    errors = []

    def run(i):
        try:
            s = torch.cuda.Stream(device=dev)
            A, B = devs[i]
            for _ in range(20):
                tg.gemm(A, B, out=outs[i], stream=s.cuda_stream)
            s.synchronize()
        except Exception as e:   # reported below
            errors.append((i, repr(e)))

    th = [threading.Thread(target=run, args=(i,)) for i in range(4)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    for r, o in zip(ref, outs):
        assert torch.equal(r.view(torch.int16), o.view(torch.int16))
