"""Pins for the float64 reference GEMM (CPU only).

Each test ties the oracle to something other than itself: a closed form, the
worked block decomposition of the Triton matmul tutorial, exact rational
arithmetic with the standard floating-point error bound, identity and
permutation products, a library matrix product, and planted mistakes that at
least one pin must catch.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gemm_inputs import BF16, F16, F32, NN, NT, TN, TT, layout, make_problem, round_to

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_tiled_fixture():
    X, Y, cur = [], [], None
    meta = {}
    with open(os.path.join(GOLDEN, "tiled_4x6_6x4.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line in ("X", "Y"):
                cur = X if line == "X" else Y
                continue
            parts = line.split()
            if parts[0] in ("shape", "dot_split", "block"):
                meta[parts[0] + ("_" + parts[1] if parts[0] == "shape" else "")] = parts[1:]
                continue
            cur.append([float(v) for v in parts])
    return np.array(X), np.array(Y), meta


def full(Alog, Blog, trans=NN, epi=0, slope=0.0, ld_pad=0, threads=2, want_macs=False):
    M, K = Alog.shape
    N = Blog.shape[1]
    A, lda, B, ldb = layout(Alog, Blog, trans, ld_pad)
    return oracle.gemm_full(M, N, K, A, lda, trans & 1, B, ldb, trans & 2, dtype=F32,
                            epi=epi, slope=slope, threads=threads, want_macs=want_macs)


# ---------------------------------------------------------------- worked example

def test_tiled_example_closed_form():
    X, Y, meta = _read_tiled_fixture()
    assert X.shape == (4, 6) and Y.shape == (6, 4)
    Z, _ = full(X, Y)
    for i in range(4):
        for j in range(4):
            assert Z[i, j] == 15 * i - 6 * i * j + 55 - 15 * j


def test_tiled_example_split_dot():
    """Z[0,0] equals the sum of two length-3 partial dot products."""
    X, Y, meta = _read_tiled_fixture()
    s = int(meta["dot_split"][0])
    Z, _ = full(X, Y)
    part = [sum(X[0, k] * Y[k, 0] for k in range(lo, lo + s)) for lo in range(0, 6, s)]
    assert len(part) == 2
    assert Z[0, 0] == part[0] + part[1]


def test_tiled_example_blocks():
    """Every 2x2 block of Z is the sum over three 2-wide contraction blocks."""
    X, Y, meta = _read_tiled_fixture()
    bm, bn, bk = (int(v) for v in meta["block"])
    Z, _ = full(X, Y)
    for bi in range(0, 4, bm):
        for bj in range(0, 4, bn):
            acc = np.zeros((bm, bn))
            nblocks = 0
            for bkk in range(0, 6, bk):
                xb = X[bi:bi + bm, bkk:bkk + bk]
                yb = Y[bkk:bkk + bk, bj:bj + bn]
                for r in range(bm):
                    for c in range(bn):
                        acc[r, c] += sum(xb[r, t] * yb[t, c] for t in range(bk))
                nblocks += 1
            assert nblocks == 3
            np.testing.assert_array_equal(Z[bi:bi + bm, bj:bj + bn], acc)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("trans", [NN, TN, NT, TT])
def test_rank_one_closed_form(trans):
    """A[i][k] = (i+1)(k+1), B[k][j] = (k+2)(j+3) - an asymmetric rank-one-per-k product."""
    M, N, K = 5, 7, 9
    A = np.array([[(i + 1) * (k + 1) for k in range(K)] for i in range(M)], float)
    B = np.array([[(k + 2) * (j + 3) for j in range(N)] for k in range(K)], float)
    S = sum((k + 1) * (k + 2) for k in range(K))
    Z, absab = full(A, B, trans)
    for i in range(M):
        for j in range(N):
            assert Z[i, j] == (i + 1) * (j + 3) * S
            assert absab[i, j] == Z[i, j]  # non-negative operands


def test_identity_and_permutation():
    rng = np.random.default_rng(7)
    M, K, N = 13, 11, 9
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    Z, _ = full(A, np.eye(K))
    np.testing.assert_array_equal(Z, A)
    Z, _ = full(np.eye(K), B)
    np.testing.assert_array_equal(Z, B)
    perm = rng.permutation(K)
    P = np.zeros((K, K))
    P[perm, np.arange(K)] = 1.0      # (A P)[:, j] = A[:, perm[j]]
    Z, _ = full(A, P)
    np.testing.assert_array_equal(Z, A[:, perm])
    Z, _ = full(P.T, B)              # (P^T B)[i, :] = B[perm[i], :]
    np.testing.assert_array_equal(Z, B[perm, :])


def test_trans_flags_bitwise_identical():
    rng = np.random.default_rng(3)
    A = rng.uniform(-1, 1, (17, 23))
    B = rng.uniform(-1, 1, (23, 19))
    base, babs = full(A, B, NN)
    for t in (TN, NT, TT):
        z, zabs = full(A, B, t)
        np.testing.assert_array_equal(z, base)
        np.testing.assert_array_equal(zabs, babs)
    z, _ = full(A, B, NN, ld_pad=5)
    np.testing.assert_array_equal(z, base)


def _fp64_bound(K, absab):
    u = 2.0 ** -53
    g = K * u / (1 - K * u)
    return g * absab


def test_exact_rational_within_error_bound():
    """|oracle - exact| <= gamma_K * (|A||B|), exact sum in rational arithmetic."""
    rng = np.random.default_rng(11)
    M, N, K = 6, 5, 37
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    Z, absab = full(A, B)
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(A[i, k]) * Fraction(B[k, j]) for k in range(K))
            err = abs(Fraction(Z[i, j]) - exact)
            assert err <= Fraction(_fp64_bound(K, absab[i, j]))
    # with dyadic operands of few bits the result is exact
    A2 = np.round(A * 8) / 8
    B2 = np.round(B * 8) / 8
    Z2, _ = full(A2, B2)
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(A2[i, k]) * Fraction(B2[k, j]) for k in range(K))
            assert Fraction(Z2[i, j]) == exact


def test_agrees_with_library_product():
    """numpy's BLAS product (another summation order) within 2 gamma_K."""
    rng = np.random.default_rng(5)
    A = rng.standard_normal((40, 70))
    B = rng.standard_normal((70, 30))
    Z, absab = full(A, B)
    lib = A @ B
    assert np.all(np.abs(Z - lib) <= 2 * _fp64_bound(70, absab) + 1e-300)


def test_mac_count_and_flops():
    """The product performs M*N*K multiply-adds, i.e. 2*M*N*K floating-point operations."""
    for (M, N, K) in [(3, 4, 5), (16, 1, 33), (1, 9, 2)]:
        A = np.ones((M, K))
        B = np.ones((K, N))
        Z, _, macs = full(A, B, want_macs=True)
        assert macs == M * N * K
        assert 2 * macs == 2 * M * N * K
        assert np.all(Z == K)


def test_points_match_full_bitwise():
    rng = np.random.default_rng(9)
    M, N, K = 21, 18, 25
    A = rng.uniform(-1, 1, (M, K))
    B = rng.uniform(-1, 1, (K, N))
    for trans in (NN, NT, TN, TT):
        Ast, lda, Bst, ldb = layout(A, B, trans, ld_pad=3)
        Z, absab = oracle.gemm_full(M, N, K, Ast, lda, trans & 1, Bst, ldb, trans & 2)
        I = rng.integers(0, M, 50)
        J = rng.integers(0, N, 50)
        v, av = oracle.gemm_points(M, N, K, Ast, lda, trans & 1, Bst, ldb, trans & 2, I, J)
        np.testing.assert_array_equal(v, Z[I, J])
        np.testing.assert_array_equal(av, absab[I, J])


def test_degenerate_shapes():
    Z, _ = full(np.zeros((4, 0)), np.zeros((0, 3)))
    assert Z.shape == (4, 3) and np.all(Z == 0)
    Z, _ = full(np.zeros((0, 5)), np.zeros((5, 3)))
    assert Z.shape == (0, 3)
    Z, _ = full(np.zeros((2, 5)), np.zeros((5, 0)))
    assert Z.shape == (2, 0)
    with pytest.raises(ValueError):
        oracle.gemm_full(2, 2, 2, np.zeros(4), 1, 0, np.zeros(4), 2, 0)  # lda < K


def test_leaky_relu_epilogue():
    """With A = I the product is B, so the epilogue acts element by element."""
    B = np.array([[-100.0, 0.0, 3.5], [-0.25, 2.0, -1e-3]])
    Z, _ = full(np.eye(2), B, epi=oracle.EPI_LEAKY_RELU, slope=0.01)
    expect = np.where(B >= 0, B, 0.01 * B)
    np.testing.assert_allclose(Z, expect, rtol=1e-15, atol=0)
    assert Z[0, 0] == pytest.approx(-1.0, rel=1e-15)
    assert Z[0, 1] == 0.0 and Z[0, 2] == 3.5


def test_integer_products_exact():
    rng = np.random.default_rng(2)
    A = rng.integers(-2, 3, (33, 512)).astype(float)
    B = rng.integers(-2, 3, (512, 31)).astype(float)
    Z, _ = full(A, B, threads=4)
    ref = A.astype(np.int64) @ B.astype(np.int64)
    np.testing.assert_array_equal(Z, ref.astype(float))


# ---------------------------------------------------------------- alpha and beta

def _brute(Alog, Blog):
    """Exact integer product by Python loops (independent of the oracle's C loop)."""
    M, K = Alog.shape
    N = Blog.shape[1]
    return np.array([[sum(int(Alog[i, k]) * int(Blog[k, j]) for k in range(K)) for j in range(N)]
                     for i in range(M)], dtype=float)


def test_scaled_beta_cancels_the_product():
    """C_old = A.B (by brute force) and beta = -1: alpha = 1 gives exactly 0,
    alpha = 3 gives exactly 2 A.B -- a dropped term, a wrong sign or the wrong
    operand scaled all break one of them."""
    rng = np.random.default_rng(21)
    A = rng.integers(-3, 4, (5, 7)).astype(float)
    B = rng.integers(-3, 4, (7, 6)).astype(float)
    P = _brute(A, B)
    acc, absab = full(A, B)
    Z, _ = oracle.scaled(acc, absab, 1.0, -1.0, P)
    np.testing.assert_array_equal(Z, np.zeros_like(P))
    Z, _ = oracle.scaled(acc, absab, 3.0, -1.0, P)
    np.testing.assert_array_equal(Z, 2.0 * P)


def test_scaled_alpha_zero_and_homogeneity():
    rng = np.random.default_rng(22)
    A = rng.integers(-3, 4, (4, 9)).astype(float)
    B = rng.integers(-3, 4, (9, 5)).astype(float)
    Cold = rng.integers(-5, 6, (4, 5)).astype(float)
    acc, absab = full(A, B)
    # alpha = 0: only the old C remains, scaled; the product is not referenced
    Z, _ = oracle.scaled(acc, absab, 0.0, 0.5, Cold)
    np.testing.assert_array_equal(Z, Cold / 2)
    Z, _ = oracle.scaled(np.full_like(acc, np.nan), absab, 0.0, 0.5, Cold)
    np.testing.assert_array_equal(Z, Cold / 2)
    # beta = 0: the product scales linearly and the old C is not used (NaN is harmless)
    Z1, _ = oracle.scaled(acc, absab, 1.0, 0.0, np.full_like(Cold, np.nan))
    Z4, _ = oracle.scaled(acc, absab, -4.0, 0.0, np.full_like(Cold, np.nan))
    np.testing.assert_array_equal(Z1, _brute(A, B))
    np.testing.assert_array_equal(Z4, -4.0 * Z1)


def test_scaled_epilogue_acts_after_the_sum():
    """With A = I: alpha B + beta C_old goes negative where alpha B alone does
    not, and the rectifier must see the sum."""
    B = np.array([[1.0, 2.0, -1.0]])
    Cold = np.array([[-3.0, -1.0, 4.0]])
    acc, absab = full(np.eye(1), B)
    Z, _ = oracle.scaled(acc, absab, 1.0, 1.0, Cold, oracle.EPI_LEAKY_RELU, 0.5)
    np.testing.assert_array_equal(Z, np.array([[-1.0, 1.0, 3.0]]))


def test_scaled_tolerance_scale_by_brute_force():
    rng = np.random.default_rng(23)
    A = rng.integers(-3, 4, (3, 8)).astype(float)
    B = rng.integers(-3, 4, (8, 4)).astype(float)
    Cold = rng.integers(-5, 6, (3, 4)).astype(float)
    acc, absab = full(A, B)
    _, scale = oracle.scaled(acc, absab, -2.0, 0.25, Cold)
    expect = 2.0 * _brute(np.abs(A), np.abs(B)) + 0.25 * np.abs(Cold)
    np.testing.assert_array_equal(scale, expect)


# ---------------------------------------------------------------- tolerance

def test_tolerance_admits_correctly_rounded_outputs():
    rng = np.random.default_rng(4)
    M, N, K = 32, 48, 512
    A = rng.standard_normal((M, K)) / np.sqrt(K)
    B = rng.standard_normal((K, N)) / np.sqrt(K)
    Z, absab = full(A, B)
    for d in (F16, BF16, F32):
        stored = round_to(Z, d)
        got = oracle.to_f64(stored, d)
        r = oracle.check(got, Z, absab, d)
        assert r["ok"], (d, r)
    # a result off by one part in a hundred fails
    r = oracle.check(Z * 1.01, Z, absab, F16)
    assert not r["ok"]
    r = oracle.check(np.full_like(Z, np.nan), Z, absab, F32)
    assert not r["ok"]


def test_tolerance_admits_float32_accumulation():
    """Sequential float32 accumulation of a 4096-deep product stays inside the bound."""
    rng = np.random.default_rng(6)
    K = 4096
    a = round_to(rng.standard_normal((8, K)) / 64, F32).astype(np.float64)
    b = round_to(rng.standard_normal((K, 8)) / 64, F32).astype(np.float64)
    Z, absab = full(a, b)
    acc = np.zeros((8, 8), dtype=np.float32)
    for k in range(K):
        acc = (acc + np.outer(a[:, k], b[k, :]).astype(np.float32)).astype(np.float32)
    r = oracle.check(acc.astype(np.float64), Z, absab, F32)
    assert r["ok"], r


# ---------------------------------------------------------------- planted mistakes

def _pins_pass() -> bool:
    tests = [test_tiled_example_closed_form, test_tiled_example_split_dot, test_tiled_example_blocks,
             test_identity_and_permutation, test_exact_rational_within_error_bound,
             test_leaky_relu_epilogue, test_mac_count_and_flops]
    try:
        for t in tests:
            t()
        test_rank_one_closed_form(NN)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("fault", [1, 2, 3, 4])
def test_planted_mistake_is_caught(fault):
    assert _pins_pass()
    oracle.plant_fault(fault)
    try:
        assert not _pins_pass(), f"planted fault {fault} went unnoticed"
    finally:
        oracle.plant_fault(0)
    assert _pins_pass()


def test_sampled_large_shape_runs():
    p = make_problem(300, 200, 257, F16, NT, "normal", seed=0)
    I = np.array([0, 299, 150, 17])
    J = np.array([0, 199, 100, 3])
    v, av = oracle.gemm_points(p.M, p.N, p.K, p.A, p.lda, p.trans_a, p.B, p.ldb, p.trans_b, I, J,
                               dtype=F16)
    A64 = oracle.to_f64(p.A, F16)
    B64 = oracle.to_f64(p.B, F16)
    for t in range(4):
        exact = sum(Fraction(A64[I[t], k]) * Fraction(B64[J[t], k]) for k in range(p.K))
        assert abs(Fraction(v[t]) - exact) <= Fraction(_fp64_bound(p.K, av[t]))
