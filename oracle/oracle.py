"""Python driver for the float64 reference GEMM.  TEST INFRASTRUCTURE ONLY.

Calls the triple loop in ``oracle.c`` (the definition of the product in BLAS
naming, "Matrix Multiplication Background User's Guide", section 2) through
ctypes, on operands widened exactly to float64, and states the tolerance a
GPU result is held to.

Tolerance (per output element, with (|A||B|)_ij = sum_k |A(i,k)| |B(k,j)| in
float64 and C_ref the float64 value after the epilogue):

    |C - C_ref| <= 1e-4 * (|A||B|)_ij + 1e-6 + r_out * |C_ref|

With alpha and beta (scaled()), (|A||B|)_ij becomes |alpha| (|A||B|)_ij +
|beta C_old|: the float32 accumulation error scales with alpha, and forming
alpha * sum + beta * C_old in float32 adds two roundings, far below 1e-4 of
that sum of magnitudes.

r_out is 0 for a float32 output, 1e-3 for float16 and 2^-8 for bfloat16.  The
first two terms bound float32 accumulation in any order; the third is the
rounding of the stored output.  1e-3 would be below bfloat16's own unit
roundoff (2^-8), so a perfectly rounded bfloat16 result could fail it; the
relative term is therefore max(1e-3, u_out).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
EPI_NONE, EPI_LEAKY_RELU = 0, 1

F32, F16, BF16 = 0, 1, 2
OUT_REL = {F32: 0.0, F16: 1e-3, BF16: max(1e-3, 2.0 ** -8)}
ACC_REL = 1e-4
ABS_FLOOR = 1e-6

_lib = None


def default_threads() -> int:
    """Host threads the oracle runs on: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = int(os.environ.get("ORACLE_THREADS", "16"))
    return max(1, min(n, cap))


def load():
    """Load liboracle.so, building it with the host compiler when missing or stale."""
    global _lib
    if _lib is not None:
        return _lib
    from . import build as _build
    path = _build.build(force=False)
    lib = ctypes.CDLL(path)
    i64, dp, ip = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)
    lib.oracle_gemm_full.argtypes = [i64, i64, i64, dp, i64, ctypes.c_int, dp, i64, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_double, dp, dp, i64, ctypes.c_int, ip]
    lib.oracle_gemm_full.restype = ctypes.c_int
    lib.oracle_gemm_points.argtypes = [i64, i64, i64, dp, i64, ctypes.c_int, dp, i64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_double, i64, ip, ip, dp, dp,
                                       ctypes.c_int, ip]
    lib.oracle_gemm_points.restype = ctypes.c_int
    lib.oracle_plant_fault.argtypes = [ctypes.c_int]
    lib.oracle_plant_fault.restype = None
    _lib = lib
    return lib


def plant_fault(kind: int) -> None:
    """Tests only: plant a known mistake in the triple loop (0 removes it)."""
    load().oracle_plant_fault(int(kind))


def to_f64(stored: np.ndarray, dtype: int) -> np.ndarray:
    """Exact widening of stored operand values to float64 (bfloat16 given as uint16 bits)."""
    if dtype == BF16:
        b = np.ascontiguousarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32).astype(np.float64)
    return np.ascontiguousarray(stored).astype(np.float64)


def _dp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _prep(A, B, dtype):
    A64 = np.ascontiguousarray(A if A.dtype == np.float64 else to_f64(A, dtype), dtype=np.float64)
    B64 = np.ascontiguousarray(B if B.dtype == np.float64 else to_f64(B, dtype), dtype=np.float64)
    if A64.size == 0:
        A64 = np.zeros(1)
    if B64.size == 0:
        B64 = np.zeros(1)
    return A64, B64


def gemm_full(M, N, K, A, lda, trans_a, B, ldb, trans_b, dtype=F32, epi=EPI_NONE, slope=0.0,
              threads=None, want_macs=False):
    """Whole product.  A and B are the stored arrays (storage type or float64).

    Returns (C_ref, absAB) as M x N float64 arrays, plus the multiply-add count
    when ``want_macs``.
    """
    lib = load()
    A64, B64 = _prep(A, B, dtype)
    C = np.zeros((max(M, 1), max(N, 1)), dtype=np.float64)
    absC = np.zeros_like(C)
    macs = np.zeros(1, dtype=np.int64)
    rc = lib.oracle_gemm_full(M, N, K, _dp(A64), lda, int(bool(trans_a)), _dp(B64), ldb,
                              int(bool(trans_b)), int(epi), float(slope), _dp(C), _dp(absC),
                              max(N, 1), int(threads or default_threads()), _ip(macs))
    if rc != 0:
        raise ValueError(f"oracle_gemm_full rejected its arguments (rc={rc})")
    C, absC = C[:M, :N], absC[:M, :N]
    return (C, absC, int(macs[0])) if want_macs else (C, absC)


def gemm_points(M, N, K, A, lda, trans_a, B, ldb, trans_b, I, J, dtype=F32, epi=EPI_NONE,
                slope=0.0, threads=None, want_macs=False):
    """Selected elements C[I[p], J[p]]; returns (values, absAB) float64 vectors."""
    lib = load()
    A64, B64 = _prep(A, B, dtype)
    I = np.ascontiguousarray(I, dtype=np.int64)
    J = np.ascontiguousarray(J, dtype=np.int64)
    n = int(I.size)
    out = np.zeros(max(n, 1), dtype=np.float64)
    absout = np.zeros_like(out)
    macs = np.zeros(1, dtype=np.int64)
    rc = lib.oracle_gemm_points(M, N, K, _dp(A64), lda, int(bool(trans_a)), _dp(B64), ldb,
                                int(bool(trans_b)), int(epi), float(slope), n,
                                _ip(I if n else np.zeros(1, np.int64)),
                                _ip(J if n else np.zeros(1, np.int64)), _dp(out), _dp(absout),
                                int(threads or default_threads()), _ip(macs))
    if rc != 0:
        raise ValueError(f"oracle_gemm_points rejected its arguments (rc={rc})")
    out, absout = out[:n], absout[:n]
    return (out, absout, int(macs[0])) if want_macs else (out, absout)


def scaled(acc: np.ndarray, absab: np.ndarray, alpha: float, beta: float, c_old=None,
           epi: int = EPI_NONE, slope: float = 0.0):
    """The full BLAS statement C = epi(alpha * (A.B) + beta * C_old), in float64.

    ``acc`` and ``absab`` are the plain product and (|A||B|) from gemm_full or
    gemm_points (called with EPI_NONE); ``c_old`` is the old C widened to
    float64, not used when ``beta`` is 0; with ``alpha`` 0 the product is not
    used either (BLAS: A and B are not referenced).  Returns (C_ref, scale) where scale =
    |alpha| (|A||B|)_ij + |beta C_old| replaces (|A||B|)_ij in tolerance().
    """
    acc = np.asarray(acc, dtype=np.float64)
    if alpha == 0.0:
        # BLAS: with alpha = 0, A and B are not referenced (a NaN there is no term)
        x = np.zeros_like(acc)
        scale = np.zeros_like(acc)
    else:
        x = alpha * acc
        scale = abs(alpha) * np.asarray(absab, dtype=np.float64)
    if beta != 0.0:
        c = np.asarray(c_old, dtype=np.float64)
        x = x + beta * c
        scale = scale + abs(beta) * np.abs(c)
    if epi == EPI_LEAKY_RELU:
        x = np.where(x >= 0.0, x, slope * x)
    return x, scale


def tolerance(ref: np.ndarray, absab: np.ndarray, out_dtype: int) -> np.ndarray:
    """Per-element bound on |C - C_ref| (module docstring)."""
    return ACC_REL * absab + ABS_FLOOR + OUT_REL[out_dtype] * np.abs(ref)


def check(got: np.ndarray, ref: np.ndarray, absab: np.ndarray, out_dtype: int) -> dict:
    """Compare float64-widened GPU output with the reference; returns a summary dict."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    tol = tolerance(ref, absab, out_dtype)
    ratio = np.where(np.isnan(err), np.inf, err / tol)
    bad = ~(err <= tol)  # NaN counts as a failure
    return dict(n=int(ref.size), fails=int(bad.sum()),
                max_err=float(np.where(np.isnan(err), np.inf, err).max()) if err.size else 0.0,
                max_ratio=float(ratio.max()) if ratio.size else 0.0,
                ok=bool(not bad.any()))
