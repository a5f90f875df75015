"""Seeded input generator: rounding, layout, determinism, sampling (CPU only)."""
import numpy as np

from gemm_inputs import (BF16, F16, F32, NN, NT, TN, TT, bf16_bits_from_f32, bf16_bits_to_f32,
                         make_int_problem, make_problem, round_to, sample_points, stored_to_f64)


def test_bf16_round_to_nearest_even_ties():
    # spacing of bfloat16 at 1.0 is 2^-7
    x = np.array([1.0 + 2.0 ** -8,            # tie between 1 and 1+2^-7 -> even (1.0)
                  1.0 + 3 * 2.0 ** -8,        # tie between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
                  1.0 + 2.0 ** -8 + 2.0 ** -20,  # just above the tie -> up
                  -(1.0 + 2.0 ** -8),         # sign is symmetric
                  3.0, 0.0, -0.0], dtype=np.float32)
    got = bf16_bits_to_f32(bf16_bits_from_f32(x)).astype(np.float64)
    expect = [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -1.0, 3.0, 0.0, -0.0]
    np.testing.assert_array_equal(got, expect)
    assert bf16_bits_from_f32(np.array([-0.0], np.float32))[0] == 0x8000


def test_bf16_rounding_error_bound():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(10000).astype(np.float32)
    r = bf16_bits_to_f32(bf16_bits_from_f32(x)).astype(np.float64)
    rel = np.abs(r - x) / np.abs(x)
    assert rel.max() <= 2.0 ** -8


def test_f16_matches_ieee_conversion():
    x = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65504.0, 6e-8])
    got = round_to(x, F16).astype(np.float64)
    np.testing.assert_array_equal(got, [1.0, 1.0 + 2.0 ** -9, 65504.0, 2.0 ** -24 * 1.0])


def test_problem_is_deterministic_and_laid_out():
    p1 = make_problem(33, 17, 29, F16, NN, "normal", seed=3)
    p2 = make_problem(33, 17, 29, F16, NN, "normal", seed=3)
    np.testing.assert_array_equal(p1.A, p2.A)
    np.testing.assert_array_equal(p1.B, p2.B)
    for t in (TN, NT, TT):
        q = make_problem(33, 17, 29, F16, t, "normal", seed=3)
        a = q.A.T if q.trans_a else q.A
        b = q.B.T if q.trans_b else q.B
        np.testing.assert_array_equal(a, p1.A)
        np.testing.assert_array_equal(b, p1.B)
    assert p1.lda == 29 and p1.ldb == 17
    q = make_problem(33, 17, 29, F32, TT, "uniform", seed=0, ld_pad=3)
    assert q.A.shape == (29, 36) and q.lda == 36 and q.ldb == 32
    assert np.all(q.A[:, 33:] == 0)


def test_distributions():
    p = make_problem(256, 256, 4096, F32, NN, "normal", seed=0)
    a = stored_to_f64(p.A, F32)
    assert abs(a.std() * 64 - 1.0) < 0.01
    p = make_problem(64, 64, 64, BF16, NN, "uniform", seed=0)
    a = stored_to_f64(p.A, BF16)
    assert a.min() >= -1.0 and a.max() <= 1.0 and p.A.dtype == np.uint16


def test_int_problem_exact_values():
    p = make_int_problem(8, 8, 16, BF16, NN, -1, 1, seed=0)
    a = stored_to_f64(p.A, BF16)
    assert set(np.unique(a)) <= {-1.0, 0.0, 1.0}


def test_sample_points_distinct_in_range():
    I, J = sample_points(1000, 700, 4096, seed=0)
    assert len(set(zip(I.tolist(), J.tolist()))) == len(I)
    assert I.min() >= 0 and I.max() < 1000 and J.min() >= 0 and J.max() < 700
    assert (0, 0) in set(zip(I.tolist(), J.tolist()))
    assert (999, 699) in set(zip(I.tolist(), J.tolist()))
    I2, J2 = sample_points(1000, 700, 4096, seed=0)
    np.testing.assert_array_equal(I, I2)
    I3, J3 = sample_points(3, 4, 4096, seed=0)
    assert len(I3) == 12
