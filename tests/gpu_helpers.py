"""Helpers for GPU parity tests: move seeded problems to the device, run the
library, compare with the float64 oracle (full or at sampled positions)."""
from __future__ import annotations

import numpy as np

import oracle
from gemm_inputs import BF16, F16, F32, Problem, make_c_old, sample_points

EPI_CODES = {None: 0, "none": 0, "leaky_relu": 1}


def torch_dtype(d):
    import torch
    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[d]


def to_device(arr: np.ndarray, d, device="cuda:0"):
    import torch
    a = np.ascontiguousarray(arr)
    if d == BF16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def from_device(t, d) -> np.ndarray:
    """Device tensor -> float64 numpy (exact widening)."""
    import torch
    c = t.detach().cpu().contiguous()
    if d == BF16:
        bits = c.view(torch.int16).numpy().view(np.uint16)
        return oracle.to_f64(bits, BF16)
    return c.numpy().astype(np.float64)


def run_gpu(p: Problem, epilogue=None, slope=0.01, options=None, out_pad: int = 0, workspace=None,
            alpha=1.0, beta=0.0, c_old=None):
    """Run tg_gemm_ex on the problem; returns the float64 copy of C (M x N).

    C starts as NaN (so an unwritten element, or an old C read with beta = 0,
    shows), or as ``c_old`` (stored values) when given."""
    import torch
    import tiled_gemm_02_amd as tg
    A = to_device(p.A, p.dtype)
    B = to_device(p.B, p.dtype)
    epi = None if epilogue in (None, "none") else (tg.TG_EPI_LEAKY_RELU, slope)
    if out_pad:
        Cw = torch.full((p.M, p.N + out_pad), float("nan"), dtype=torch_dtype(p.dtype), device="cuda:0")
        C = Cw[:, :p.N]
    else:
        C = torch.full((p.M, p.N), float("nan"), dtype=torch_dtype(p.dtype), device="cuda:0")
    if c_old is not None:
        C.copy_(to_device(c_old, p.dtype))
    # the stored arrays may be padded: pass views of the logical width with the stored ld
    Av = A[:, : (p.M if p.trans_a else p.K)] if A.shape[1] else A
    Bv = B[:, : (p.K if p.trans_b else p.N)] if B.shape[1] else B
    tg.gemm(Av, Bv, trans_a=p.trans_a, trans_b=p.trans_b, epilogue=epi, out=C, options=options,
            workspace=workspace, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    got = from_device(C, p.dtype)
    if out_pad:
        tail = from_device(Cw[:, p.N:], p.dtype)
        assert np.all(np.isnan(tail)), "the kernel wrote outside C's columns"
    return got


def oracle_full(p: Problem, epilogue=None, slope=0.01):
    epi = EPI_CODES[epilogue]
    return oracle.gemm_full(p.M, p.N, p.K, p.A, p.lda, p.trans_a, p.B, p.ldb, p.trans_b,
                            dtype=p.dtype, epi=epi, slope=slope)


def check_full(p: Problem, epilogue=None, slope=0.01, options=None, out_pad=0, workspace=None):
    got = run_gpu(p, epilogue, slope, options, out_pad, workspace)
    ref, absab = oracle_full(p, epilogue, slope)
    r = oracle.check(got, ref, absab, p.dtype)
    return r, got, ref


def check_scaled(p: Problem, alpha: float, beta: float, epilogue=None, slope=0.01, options=None,
                 c_seed=0, workspace=None):
    """C = epi(alpha A.B + beta C_old) against the oracle; C_old is a seeded draw."""
    c_old = make_c_old(p.M, p.N, p.dtype, c_seed)
    got = run_gpu(p, epilogue, slope, options, workspace=workspace, alpha=alpha, beta=beta,
                  c_old=c_old)
    acc, absab = oracle_full(p, None)
    ref, scale = oracle.scaled(acc, absab, alpha, beta, oracle.to_f64(c_old, p.dtype),
                               EPI_CODES[epilogue], slope)
    r = oracle.check(got, ref, scale, p.dtype)
    return r, got, ref


def check_sampled(p: Problem, epilogue=None, slope=0.01, options=None, n=4096, seed=0):
    got = run_gpu(p, epilogue, slope, options)
    I, J = sample_points(p.M, p.N, n, seed)
    ref, absab = oracle.gemm_points(p.M, p.N, p.K, p.A, p.lda, p.trans_a, p.B, p.ldb, p.trans_b,
                                    I, J, dtype=p.dtype, epi=EPI_CODES[epilogue], slope=slope)
    r = oracle.check(got[I, J], ref, absab, p.dtype)
    assert np.isfinite(got).all(), "non-finite output (an element was not written)"
    return r
