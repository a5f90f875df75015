"""tg_gemm_noalloc, the entry point that allocates nothing: its output
against tg_gemm_ex's (the entry point it varies) on the same operands and
plan, and against the float64 oracle, on two calls in a row (the second
smaller, so it reuses scratch the first left behind).  The plans below need
workspace -- K-split partials, aligned copies, stream-K pieces -- which here
comes from the library's static scratch.  Run with -m gpu."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
from gemm_inputs import BF16, F16, NN, NT, make_problem
from tests.gpu_helpers import EPI_CODES, from_device, to_device, torch_dtype

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def _say(*a):
    print(*a, flush=True)


def _both(p, epilogue=None, options=None):
    """(C from tg_gemm_noalloc, C from tg_gemm_ex with a workspace of its own), float64."""
    import torch
    import tiled_gemm_02_amd as tg
    A = to_device(p.A, p.dtype)
    B = to_device(p.B, p.dtype)
    outs = []
    stream = torch.cuda.current_stream().cuda_stream
    epi = None if epilogue is None else (tg.TG_EPI_LEAKY_RELU, 0.01)
    for which in ("noalloc", "ex"):
        C = torch.full((p.M, p.N), float("nan"), dtype=torch_dtype(p.dtype), device="cuda:0")
        if which == "noalloc":
            rc = tg.tg_gemm_noalloc(p.M, p.N, p.K, A.data_ptr(), p.lda, B.data_ptr(), p.ldb,
                                    C.data_ptr(), p.N, p.dtype, p.trans, epi, options, stream)
        else:
            need = tg.tg_workspace_size(p.M, p.N, p.K, p.dtype, p.trans, options)
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda:0")
            rc = tg.tg_gemm_ex(p.M, p.N, p.K, A.data_ptr(), p.lda, B.data_ptr(), p.ldb,
                               C.data_ptr(), p.N, p.dtype, p.trans, epi, options,
                               ws.data_ptr(), ws.numel(), stream)
        assert rc == tg.TG_OK, (which, tg.tg_last_error())
        torch.cuda.synchronize()
        outs.append(from_device(C, p.dtype))
    return outs


def _oracle_ok(p, got, epilogue=None):
    ref, absab = oracle.gemm_full(p.M, p.N, p.K, p.A, p.lda, p.trans_a, p.B, p.ldb, p.trans_b,
                                  dtype=p.dtype, epi=EPI_CODES[epilogue], slope=0.01)
    r = oracle.check(got, ref, absab, p.dtype)
    assert r["ok"], r


# (first call, second smaller call): shapes, dtype, layout, options, epilogue
PAIRS = [
    # skinny path, K split four ways: float32 partials in the scratch
    (((4096, 128, 4096), F16, NN, None, None), ((1024, 128, 2048), F16, NN, None, "leaky_relu")),
    # macro tiles with a forced K split, then a smaller split
    (((520, 776, 4104), BF16, NT, {"split_k": 4}, "leaky_relu"), ((264, 264, 1032), BF16, NT, {"split_k": 3}, None)),
    # operands off the 16-byte grid (aligned copies in the scratch), then a smaller one
    (((1031, 1029, 1027), F16, NN, None, None), ((777, 1003, 1001), F16, NT, None, None)),
    # stream-K pieces (64 workgroups: 32 MiB), then whole tiles split two ways
    (((256, 512, 1024), F16, NN, {"split_k": -1}, None), ((256, 256, 512), F16, NN, {"split_k": 2}, None)),
    # K groups inside the workgroups with a K split across them: two groups, then four
    (((520, 392, 4104), BF16, NT, {"k_groups": 2, "split_k": 3}, None),
     ((264, 264, 1032), F16, NN, {"tile_m": 64, "tile_n": 64, "k_groups": 4, "split_k": 2}, "leaky_relu")),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "x".join(map(str, p[0][0])))
def test_noalloc_matches_tg_gemm_ex(pair):
    import tiled_gemm_02_amd as tg
    for (shape, dtype, trans, opts, epi) in pair:
        M, N, K = shape
        _say("case noalloc", shape, dtype, trans, opts, epi)
        p = make_problem(M, N, K, dtype, trans, "normal", seed=51)
        need = tg.tg_workspace_size(M, N, K, dtype, trans, opts)
        assert 0 < need <= SCRATCH, need   # the call really uses the scratch
        got, ref_ex = _both(p, epi, opts)
        # the same plan and kernels on the same operands: the same bits
        np.testing.assert_array_equal(got, ref_ex)
        _oracle_ok(p, got, epi)


def test_noalloc_refuses_forced_plans_beyond_the_scratch():
    import torch
    import tiled_gemm_02_amd as tg
    M, N, K = 4096, 4096, 8192
    opts = {"split_k": 8}
    assert tg.tg_workspace_size(M, N, K, tg.TG_F16, NN, opts) > SCRATCH
    A = torch.zeros((M, K), dtype=torch.float16, device="cuda:0")
    B = torch.zeros((K, N), dtype=torch.float16, device="cuda:0")
    C = torch.zeros((M, N), dtype=torch.float16, device="cuda:0")
    rc = tg.tg_gemm_noalloc(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N, tg.TG_F16,
                            NN, None, opts, torch.cuda.current_stream().cuda_stream)
    assert rc == tg.TG_ERR_ARG
    assert "scratch" in tg.tg_last_error() and str(SCRATCH) in tg.tg_last_error()
    # unforced, a product whose planned aligned copies (75 MB) exceed the
    # scratch runs without them (element-wise loads), checked at sampled outputs
    from gemm_inputs import sample_points
    M, N, K = 5000, 4104, 4100
    assert tg.tg_workspace_size(M, N, K, tg.TG_F16, NN) > SCRATCH
    p = make_problem(M, N, K, F16, NN, "normal", seed=52)
    A = to_device(p.A, F16)
    B = to_device(p.B, F16)
    C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda:0")
    rc = tg.tg_gemm_noalloc(M, N, K, A.data_ptr(), p.lda, B.data_ptr(), p.ldb, C.data_ptr(), N,
                            F16, NN, None, None, torch.cuda.current_stream().cuda_stream)
    assert rc == tg.TG_OK, tg.tg_last_error()
    torch.cuda.synchronize()
    got = from_device(C, F16)
    assert np.isfinite(got).all()
    I, J = sample_points(M, N, 4096, 52)
    ref, absab = oracle.gemm_points(M, N, K, p.A, p.lda, p.trans_a, p.B, p.ldb, p.trans_b, I, J,
                                    dtype=F16, epi=0, slope=0.01)
    r = oracle.check(got[I, J], ref, absab, F16)
    assert r["ok"], r
