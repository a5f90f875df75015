"""Float64 reference row softmax.  TEST INFRASTRUCTURE ONLY.

What it computes (the fused-softmax example of "OpenAI open-sources Triton",
the Chinese news article's programming-model section, and its A100 figure at
M = 4096): every row x of an M x N matrix X is normalised on its own,

    y_j = exp(x_j - m) / sum_k exp(x_k - m),   m = max_k x_k,

the numerically stable form in which the row maximum is subtracted before
exponentiating.  Readings of the page:

  * The fused listing pads columns past N with -inf before the maximum and
    the sum; exp(-inf - m) = 0, so padding is the same as leaving the column
    out.  The oracle has no padding; -inf entries of X itself behave the same
    way (they get y = 0).
  * The TorchScript listing on the same page exponentiates x instead of
    x - m.  In exact arithmetic the quotient is the same, but it overflows
    for entries above about 709 (float64) or 88 (float32); the fused listing's
    form is the one followed here.
  * Rows where the definition has no finite value give NaN, as its
    arithmetic does: an all -inf row (m = -inf, so x - m = -inf - (-inf)),
    a row holding +inf (inf - inf), a row holding NaN.

The definition is written out with numpy float64 primitives (maximum, exp,
sum, divide) along axis 1 and nothing else; X arrives already widened exactly
from its storage type.

Tolerance of a float32 implementation (per element, derived from its
arithmetic; z = x - m in float64):

    |y - y_ref| <= |y_ref| * (u_out + 2^-24 * (2 |z| + n_seq + 2 ceil(log2 N) + 8)) + a_out

  * 2 |z| 2^-24: the float32 subtraction x - m and the scaling by log2(e)
    before a base-2 exponential each perturb the exponent by at most
    |z| 2^-24, which moves exp(z) by the same relative amount;
  * n_seq 2^-24 + 2 ceil(log2 N) 2^-24: a sum of positive terms in float32
    with at most n_seq sequential additions per partial sum and a pairwise
    tree over the partial sums; n_seq = max(64, ceil(N / 4096)) covers both
    GPU forms (row kept in registers: at most 64 values per lane; rows too
    long for that: N / 4096 values per accumulator);
  * 8 * 2^-24: the exponential (a few ulp), the reciprocal of the sum and the
    final multiply;
  * u_out: rounding to the stored output (0 for float32, 2^-11 float16,
    2^-8 bfloat16);
  * a_out: outputs below the smallest normal number may be flushed or
    rounded coarsely (2^-126 for float32 and bfloat16 outputs, 2^-24, one
    subnormal step, for float16).

NaN is a value here: the check requires NaN at exactly the reference's NaN
positions and nowhere else.
"""
from __future__ import annotations

import math

import numpy as np

F32, F16, BF16 = 0, 1, 2
U_OUT = {F32: 0.0, F16: 2.0 ** -11, BF16: 2.0 ** -8}
A_OUT = {F32: 2.0 ** -126, F16: 2.0 ** -24, BF16: 2.0 ** -126}

# Tests only: a planted mistake (0 = none).  1: exponentiate x instead of
# x - m; 2: normalise columns instead of rows; 3: skip the division by the sum.
_fault = 0


def plant_fault(kind: int) -> None:
    """Tests only: plant a known mistake in softmax_rows (0 removes it)."""
    global _fault
    _fault = int(kind)


def softmax_rows(X: np.ndarray):
    """Row softmax of a float64 matrix.  Returns (Y, Z) with Z = X - rowmax(X)."""
    X = np.asarray(X, dtype=np.float64)
    if X.ndim != 2:
        raise ValueError("X must be 2-D (M x N)")
    M, N = X.shape
    if M == 0 or N == 0:
        return np.zeros((M, N)), np.zeros((M, N))
    axis = 0 if _fault == 2 else 1
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        m = np.max(X, axis=axis, keepdims=True)       # NaN propagates, as the definition does
        Z = X - m
        E = np.exp(X if _fault == 1 else Z)
        S = np.sum(E, axis=axis, keepdims=True)
        Y = E if _fault == 3 else E / S
    return Y, Z


def tolerance(y_ref: np.ndarray, z: np.ndarray, N: int, out_dtype: int) -> np.ndarray:
    """Per-element bound on |y - y_ref| (module docstring)."""
    n_seq = max(64, -(-N // 4096))
    logn = math.ceil(math.log2(N)) if N > 1 else 0
    with np.errstate(invalid="ignore"):
        zz = np.where(np.isfinite(z), np.abs(z), 0.0)
        rel = U_OUT[out_dtype] + 2.0 ** -24 * (2.0 * zz + n_seq + 2 * logn + 8)
        return np.abs(y_ref) * rel + A_OUT[out_dtype]


def check(got: np.ndarray, y_ref: np.ndarray, z: np.ndarray, N: int, out_dtype: int) -> dict:
    """Compare float64-widened GPU output with the reference; returns a summary dict."""
    got = np.asarray(got, dtype=np.float64)
    ref_nan = np.isnan(y_ref)
    got_nan = np.isnan(got)
    nan_mismatch = int(np.count_nonzero(ref_nan != got_nan))
    with np.errstate(invalid="ignore"):
        err = np.where(ref_nan | got_nan, 0.0, np.abs(got - y_ref))
        tol = tolerance(np.where(ref_nan, 0.0, y_ref), z, N, out_dtype)
        ratio = np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0))
    bad = ~(err <= tol)
    fails = int(np.count_nonzero(bad)) + nan_mismatch
    return dict(n=int(y_ref.size), fails=fails, nan_mismatch=nan_mismatch,
                max_err=float(err.max()) if err.size else 0.0,
                max_ratio=float(ratio.max()) if ratio.size else 0.0,
                ok=fails == 0)
