"""Seeded synthetic GEMM operands.

This module only *draws* inputs: random matrices, their rounding to the storage
type, their layout in memory (plain or stored-transposed), integer-valued test
operands and the output positions a sampled check looks at.  It holds none of
the matrix-multiply arithmetic and is imported by the GPU tests, the benchmark
and the oracle's tests alike, so both sides of a parity check consume the very
same bits.

Conventions (BLAS naming, as in "Matrix Multiplication Background User's
Guide", section 2): A is M x K, B is K x N, C is M x N, all row-major.  A
"transposed" operand is stored as the row-major array of its transpose:
A^T (K x M) with lda >= M, B^T (N x K) with ldb >= K; this is what the
Triton matmul tutorial's ``Y.T.contiguous()`` produces ("Learning Triton One
Kernel at a Time: Matrix Multiplication", section on memory coalescing).

Recipe:
  * draw in float64 from ``numpy.random.default_rng(seed)``: A first (logical
    M x K, row by row), then B (logical K x N, row by row);
  * "uniform": i.i.d. U[-1, 1); "normal": i.i.d. N(0, 1) / sqrt(K);
  * round to the storage type: float32 and float16 with numpy's
    round-to-nearest-even conversion; bfloat16 by rounding to float32 first and
    then to-nearest-even on the float32 bit pattern (kept as uint16 bits);
  * lay the logical matrix out as stored (a contiguous copy of the transpose
    for a transposed operand).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Storage-type codes, shared with the C ABI's dtype enumeration.
F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
DTYPE_CODES = {v: k for k, v in DTYPE_NAMES.items()}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}

# trans bit field: bit0 = A stored transposed, bit1 = B stored transposed.
NN, TN, NT, TT = 0, 1, 2, 3


def dtype_code(d) -> int:
    if isinstance(d, str):
        return DTYPE_CODES[d]
    return int(d)


def bf16_bits_from_f32(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, returned as uint16 bits.

    The top 16 bits of the float32 pattern are kept; the discarded low half is
    compared against the half-way point 0x8000, ties going to the even result.
    Inputs here are finite (no NaN handling is needed for drawn operands).
    """
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = u + np.uint64(0x7FFF) + lsb
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def round_to(x64: np.ndarray, dtype) -> np.ndarray:
    """Round float64 values to the storage type.

    Returns float32 / float16 arrays, or uint16 bit patterns for bfloat16.
    """
    d = dtype_code(dtype)
    if d == F32:
        return np.asarray(x64, dtype=np.float64).astype(np.float32)
    if d == F16:
        return np.asarray(x64, dtype=np.float64).astype(np.float16)
    if d == BF16:
        return bf16_bits_from_f32(np.asarray(x64, dtype=np.float64).astype(np.float32))
    raise ValueError(f"unknown dtype {dtype}")


def stored_to_f64(arr: np.ndarray, dtype) -> np.ndarray:
    """Exact widening of stored values (float32 / float16 / bf16 bits) to float64."""
    d = dtype_code(dtype)
    if d == BF16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr).astype(np.float64)


def draw_logical(M: int, N: int, K: int, dist: str, seed: int):
    """Draw the logical float64 operands A (M x K) and B (K x N)."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        A = rng.uniform(-1.0, 1.0, size=(M, K))
        B = rng.uniform(-1.0, 1.0, size=(K, N))
    elif dist == "normal":
        s = 1.0 / math.sqrt(K) if K > 0 else 1.0
        A = rng.standard_normal(size=(M, K)) * s
        B = rng.standard_normal(size=(K, N)) * s
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return A, B


@dataclass
class Problem:
    """One GEMM instance: stored operands plus the metadata the ABI needs."""
    M: int
    N: int
    K: int
    dtype: int
    trans: int
    A: np.ndarray          # stored array (row-major), storage type
    B: np.ndarray
    lda: int
    ldb: int
    desc: dict = field(default_factory=dict)

    @property
    def trans_a(self) -> bool:
        return bool(self.trans & 1)

    @property
    def trans_b(self) -> bool:
        return bool(self.trans & 2)


def _store(logical: np.ndarray, transposed: bool, ld_pad: int) -> tuple[np.ndarray, int]:
    """Row-major storage of ``logical`` (or of its transpose), rows padded by ld_pad."""
    m = logical.T if transposed else logical
    rows, cols = m.shape
    ld = max(1, cols + ld_pad)
    out = np.zeros((rows, ld), dtype=m.dtype)
    out[:, :cols] = m
    return out, ld


def layout(Alog: np.ndarray, Blog: np.ndarray, trans: int, ld_pad: int = 0):
    """Lay rounded logical operands out as stored; returns (A, lda, B, ldb)."""
    A, lda = _store(Alog, bool(trans & 1), ld_pad)
    B, ldb = _store(Blog, bool(trans & 2), ld_pad)
    return A, lda, B, ldb


def make_problem(M: int, N: int, K: int, dtype, trans: int = NN, dist: str = "uniform",
                 seed: int = 0, ld_pad: int = 0) -> Problem:
    """Seeded problem in the recipe of the module docstring."""
    d = dtype_code(dtype)
    A64, B64 = draw_logical(M, N, K, dist, seed)
    Ar, Br = round_to(A64, d), round_to(B64, d)
    A, lda, B, ldb = layout(Ar, Br, trans, ld_pad)
    return Problem(M, N, K, d, trans, A, B, lda, ldb,
                   dict(dist=dist, seed=seed, ld_pad=ld_pad))


def make_c_old(M: int, N: int, dtype, seed: int) -> np.ndarray:
    """Seeded old C for alpha/beta runs: i.i.d. U[-1, 1) from default_rng([seed, 7]),
    rounded to the storage type (bfloat16 as uint16 bits), M x N row-major."""
    d = dtype_code(dtype)
    x = np.random.default_rng([seed, 7]).uniform(-1.0, 1.0, size=(M, N))
    return round_to(x, d)


def make_int_problem(M: int, N: int, K: int, dtype, trans: int, lo: int, hi: int,
                     seed: int = 0) -> Problem:
    """Integer-valued operands drawn uniformly from {lo..hi} (inclusive).

    Small integers are exact in every storage type; with |C| small enough all
    partial sums are exact in float32 and the product is reproduced bit for bit.
    """
    rng = np.random.default_rng(seed)
    A64 = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float64)
    B64 = rng.integers(lo, hi + 1, size=(K, N)).astype(np.float64)
    d = dtype_code(dtype)
    A, lda, B, ldb = layout(round_to(A64, d), round_to(B64, d), trans)
    return Problem(M, N, K, d, trans, A, B, lda, ldb, dict(dist=f"int[{lo},{hi}]", seed=seed))


def sample_points(M: int, N: int, n: int, seed: int, tile_m: int = 256, tile_n: int = 256):
    """Output positions for a sampled check.

    ``n`` distinct positions drawn without replacement from
    ``default_rng([seed, n])``, plus the four corners and the first/last row
    and column around every ``tile_m`` x ``tile_n`` boundary that falls on a
    sampled row or column.  Returns (I, J) int64 arrays.
    """
    rng = np.random.default_rng([seed, n])
    total = M * N
    k = min(n, total)
    flat = rng.choice(total, size=k, replace=False)
    I = list((flat // N).astype(np.int64))
    J = list((flat % N).astype(np.int64))
    edge_r = {0, M - 1} | {r for b in range(tile_m, M, tile_m) for r in (b - 1, b)}
    edge_c = {0, N - 1} | {c for b in range(tile_n, N, tile_n) for c in (b - 1, b)}
    extra = {(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)}
    sr = sorted(edge_r)
    sc = sorted(edge_c)
    # a sparse grid of boundary rows x boundary columns, capped so it stays small
    for r in sr[:: max(1, len(sr) // 16)]:
        for c in sc[:: max(1, len(sc) // 16)]:
            extra.add((r, c))
    have = set(zip(I, J))
    for p in sorted(extra):
        if p not in have:
            I.append(p[0])
            J.append(p[1])
    return np.asarray(I, dtype=np.int64), np.asarray(J, dtype=np.int64)


# Named workloads, with the shapes, distributions and seeds they are measured on.
WORKLOADS = {
    "f32_256": dict(M=256, N=256, K=256, dtype=F32, trans=NN, dist="uniform", seed=0),
    "f16_4096_nt": dict(M=4096, N=4096, K=4096, dtype=F16, trans=NT, dist="normal", seed=0),
    "f16_skinny_8192x128x8192": dict(M=8192, N=128, K=8192, dtype=F16, trans=NN, dist="uniform", seed=0),
    "f16_gemv_1x8192x8192": dict(M=1, N=8192, K=8192, dtype=F16, trans=NN, dist="uniform", seed=0),
    "f16_8192": dict(M=8192, N=8192, K=8192, dtype=F16, trans=NN, dist="normal", seed=1),
    "bf16_leaky_8192": dict(M=8192, N=8192, K=8192, dtype=BF16, trans=NN, dist="normal", seed=1,
                            epilogue="leaky_relu", slope=0.01),
    "bf16_leaky_6912x2048x4096": dict(M=6912, N=2048, K=4096, dtype=BF16, trans=NN, dist="normal",
                                      seed=1, epilogue="leaky_relu", slope=0.01),
    # float32 at the headline size: NT (the 256 x 256 kernel directly) and NN
    # (through the transposing copy of B)
    "f32_8192_nt": dict(M=8192, N=8192, K=8192, dtype=F32, trans=NT, dist="normal", seed=1),
    "f32_8192": dict(M=8192, N=8192, K=8192, dtype=F32, trans=NN, dist="normal", seed=1),
    # the full BLAS statement C = alpha A.B + beta C_old (C_old from make_c_old, seed 1)
    "f16_8192_alpha_beta": dict(M=8192, N=8192, K=8192, dtype=F16, trans=NN, dist="normal", seed=1,
                                alpha=0.5, beta=1.0),
    # points of the M = 2304, K = 4096 sweep on the four-wave kernel's tiles (two K
    # groups on 128 x 128, 128 x 64, 128 x 128), for counter passes
    "f16_2304x1536x4096": dict(M=2304, N=1536, K=4096, dtype=F16, trans=NN, dist="normal", seed=1),
    "f16_2304x2560x4096": dict(M=2304, N=2560, K=4096, dtype=F16, trans=NN, dist="normal", seed=1),
    "f16_2304x3072x4096": dict(M=2304, N=3072, K=4096, dtype=F16, trans=NN, dist="normal", seed=1),
}


# ---------------------------------------------------------------- row softmax inputs
#
# Recipe: X (M x N, row-major, rows ld = N + ld_pad elements apart) drawn in
# float64 from default_rng([seed, 11]); "normal": i.i.d. N(0, 1), the input of
# the fused-softmax example on the Triton news page ("OpenAI open-sources
# Triton", programming-model section, a 583 x 931 matrix from torch.normal);
# "wide": N(0, 1) * 30, so that most exponentials of a row fall far below the
# row maximum (and below the float32 and float16 normal ranges); "specials":
# "normal" with a few rows overwritten by the degenerate cases the definition
# has - a constant row, a row with some -inf entries, an all -inf row, a row
# with a +inf entry, a row with a NaN entry, and a row of huge equal-magnitude
# values (+-1e4) - at seeded row positions (see softmax_special_rows).  Rounded
# to the storage type as the GEMM operands are.

SPECIAL_ROWS = ("constant", "some_neg_inf", "all_neg_inf", "pos_inf", "nan", "huge")


@dataclass
class SoftmaxProblem:
    """One row-softmax instance: stored X (M x ldx) plus the metadata the ABI needs."""
    M: int
    N: int
    dtype: int
    X: np.ndarray          # stored array, storage type (bfloat16 as uint16 bits)
    ldx: int
    desc: dict = field(default_factory=dict)


def softmax_special_rows(M: int, seed: int) -> dict:
    """Row index of each special case (distinct rows, seeded), for M >= len(SPECIAL_ROWS)."""
    rng = np.random.default_rng([seed, 12])
    rows = rng.choice(M, size=len(SPECIAL_ROWS), replace=False)
    return {name: int(r) for name, r in zip(SPECIAL_ROWS, rows)}


def draw_softmax_logical(M: int, N: int, dist: str, seed: int) -> np.ndarray:
    """Draw the logical float64 X (M x N) of the recipe above."""
    rng = np.random.default_rng([seed, 11])
    X = rng.standard_normal(size=(M, N))
    if dist == "wide":
        X *= 30.0
    elif dist == "specials":
        if M >= len(SPECIAL_ROWS) and N > 0:
            sp = softmax_special_rows(M, seed)
            X[sp["constant"], :] = 0.75
            cols = rng.choice(N, size=max(1, N // 3), replace=False)
            X[sp["some_neg_inf"], cols] = -np.inf
            if N > 1:
                X[sp["some_neg_inf"], 0] = 0.5      # keep one finite entry
            X[sp["all_neg_inf"], :] = -np.inf
            X[sp["pos_inf"], int(rng.integers(N))] = np.inf
            X[sp["nan"], int(rng.integers(N))] = np.nan
            X[sp["huge"], :] = np.where(rng.uniform(size=N) < 0.5, -1e4, 1e4)
    elif dist != "normal":
        raise ValueError(f"unknown distribution {dist!r}")
    return X


def make_softmax_input(M: int, N: int, dtype, dist: str = "normal", seed: int = 0,
                       ld_pad: int = 0) -> SoftmaxProblem:
    """Seeded row-softmax input in the recipe above."""
    d = dtype_code(dtype)
    X64 = draw_softmax_logical(M, N, dist, seed)
    Xr = round_to(X64, d)
    X, ldx = _store(Xr, False, ld_pad)
    return SoftmaxProblem(M, N, d, X, ldx, dict(dist=dist, seed=seed, ld_pad=ld_pad))


# Row-softmax workloads: the Triton page's example shape and its figure's row count
# (M = 4096) at the largest row it keeps on chip (about 32K columns).
SOFTMAX_WORKLOADS = {
    "softmax_f32_583x931": dict(M=583, N=931, dtype=F32, dist="normal", seed=0),
    "softmax_f32_4096x32768": dict(M=4096, N=32768, dtype=F32, dist="normal", seed=0),
    "softmax_f16_4096x32768": dict(M=4096, N=32768, dtype=F16, dist="normal", seed=0),
}


def sweep_ns(start: int = 1536, stop: int = 6144, step: int = 8):
    """N values of the tile/wave-quantization sweep at M=2304, K=4096."""
    return list(range(start, stop + 1, step))
