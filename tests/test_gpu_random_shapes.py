"""Seeded random products against the float64 oracle (run with -m gpu).

Fixed lists of cases drawn from two seeds: sizes from 1 to 700 in every
dimension (aligned and not, so the vector, padded-copy and element-wise loads
all occur), every storage type and layout, padded leading dimensions, the
LeakyReLU epilogue, alpha / beta, and forced K splits or tiles where the
operands allow them; and 16-bit narrow, few-row and ragged products; and tiles with K groups (16-bit 128 x 128 with two,
float32 64 x 64 with four and 128 x 128 with two).  Every
output element is compared with the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

from gemm_inputs import BF16, F16, F32, NN, NT, TN, TT, make_problem
from tests.gpu_helpers import check_full, check_scaled

pytestmark = pytest.mark.gpu


def _cases(n=200, seed=2024):
    rng = np.random.default_rng(seed)

    def pick(xs):
        return xs[int(rng.integers(0, len(xs)))]

    def dim(lo=1, hi=700):
        # half the draws on the 16-byte grid of every type, half anywhere
        if rng.random() < 0.5:
            return int(rng.integers(max(1, lo // 8), hi // 8 + 1)) * 8
        return int(rng.integers(lo, hi + 1))

    out = []
    for i in range(n):
        kind = rng.random()
        dtype = pick([F32, F16, BF16])
        trans = pick([NN, NT, TN, TT])
        pad = pick([0, 0, 3, 6])
        opt = None
        if kind < 0.4:                       # anything
            M, N, K = dim(), dim(), dim()
            if rng.random() < 0.25 and K >= 64:
                opt = dict(split_k=int(rng.integers(2, 5)))
        elif kind < 0.55:                    # narrow outputs (skinny path when 16-bit)
            dtype, trans, pad = pick([F16, BF16]), pick([NN, NT]), 0
            M, N, K = int(rng.integers(32, 257)) * 8, int(rng.integers(1, 17)) * 8, int(rng.integers(8, 129)) * 8
        elif kind < 0.7:                     # GEMV forms
            M, N, K = (1, dim(1, 2000), dim(1, 1500)) if rng.random() < 0.5 else (dim(1, 2000), 1, dim(1, 1500))
        elif kind < 0.8:                     # large enough for the aligned copies
            M, N, K = dim(1000, 1100), dim(1000, 1100), dim(1000, 1100)
        else:                                # aligned operands, forced tiles
            pad = 0
            M, N, K = int(rng.integers(1, 80)) * 8, int(rng.integers(1, 80)) * 8, int(rng.integers(1, 80)) * 8
            if dtype == F32:
                tiles = [(128, 128), (64, 64)] + ([(256, 256)] if trans == NT else [])
            else:
                tiles = [(256, 256), (256, 128), (128, 128), (128, 64), (64, 64)] + \
                        ([(192, 256)] if not (trans & 1) else [])
            tm, tn = pick(tiles)
            opt = dict(tile_m=tm, tile_n=tn, split_k=int(rng.integers(1, 4)))
        epi = "leaky_relu" if rng.random() < 0.3 else None
        scaled = rng.random() < 0.3
        out.append((i, M, N, K, dtype, trans, pad, epi, scaled, opt))
    return out


CASES = _cases()


def _cases_narrow_and_ragged(n=80, seed=2025):
    """16-bit products the planner reads in place or copies one operand of:
    narrow outputs (N from 2 to 130, the skinny kernel, B copied alone when its
    rows are off the grid), a few rows (M from 2 to 16) beside a large B, and
    ragged M and N with K on the grid (the LDS-DMA kernels clamping rows), in
    every layout."""
    rng = np.random.default_rng(seed)

    def pick(xs):
        return xs[int(rng.integers(0, len(xs)))]

    out = []
    for i in range(n):
        kind = rng.random()
        dtype = pick([F16, BF16])
        trans = pick([NN, NT, TN, TT])
        K = int(rng.integers(1, 257)) * 8
        if kind < 0.4:
            M, N = int(rng.integers(128, 3001)), int(rng.integers(2, 131))
        elif kind < 0.7:
            M, N = int(rng.integers(2, 17)), int(rng.integers(128, 3001))
        else:
            M, N = int(rng.integers(100, 1101)), int(rng.integers(100, 1101))
        epi = "leaky_relu" if rng.random() < 0.3 else None
        scaled = rng.random() < 0.3
        out.append((200 + i, M, N, K, dtype, trans, 0, epi, scaled, None))
    return out


CASES += _cases_narrow_and_ragged()


def _cases_two_k_groups(n=40, seed=2026):
    """16-bit 128 x 128 tiles with two K groups per workgroup: every layout,
    M and N from 8 to 700 (ragged where the layout reads them in place), K
    from 8 to 3000 on the 16-byte grid (either group's tail, or group 1 one
    whole stage short), outer K splits 1 to 3."""
    rng = np.random.default_rng(seed)

    def pick(xs):
        return xs[int(rng.integers(0, len(xs)))]

    out = []
    for i in range(n):
        dtype = pick([F16, BF16])
        trans = pick([NN, NT, TN, TT])
        M = int(rng.integers(8, 701)) if not (trans & 1) else int(rng.integers(1, 88)) * 8
        N = int(rng.integers(8, 701)) if (trans & 2) else int(rng.integers(1, 88)) * 8
        K = int(rng.integers(1, 376)) * 8
        split = int(rng.integers(1, 4)) if K >= 384 else 1
        epi = "leaky_relu" if rng.random() < 0.3 else None
        scaled = rng.random() < 0.3
        out.append((300 + i, M, N, K, dtype, trans, 0, epi, scaled,
                    dict(tile_m=128, tile_n=128, split_k=split, k_groups=2)))
    return out


CASES += _cases_two_k_groups()


def _cases_f32_k_groups(n=24, seed=2027):
    """float32 on the register-staged kernel with K groups (64 x 64 with four,
    128 x 128 with two): every layout, M, N and K on the 16-byte grid from 4 to
    1200 (K down to one step, so some groups get no K), outer K splits 1 to 3."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        trans = [NN, NT, TN, TT][int(rng.integers(0, 4))]
        tile, kg = [(64, 4), (128, 2)][int(rng.integers(0, 2))]
        M, N, K = (int(rng.integers(1, 301)) * 4 for _ in range(3))
        split = int(rng.integers(1, 4)) if K >= 256 else 1
        epi = "leaky_relu" if rng.random() < 0.3 else None
        scaled = rng.random() < 0.3
        out.append((400 + i, M, N, K, F32, trans, 0, epi, scaled,
                    dict(tile_m=tile, tile_n=tile, split_k=split, k_groups=kg)))
    return out


CASES += _cases_f32_k_groups()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-d{c[4]}-t{c[5]}")
def test_random_product(case):
    i, M, N, K, dtype, trans, pad, epi, scaled, opt = case
    print("case random", case, flush=True)
    p = make_problem(M, N, K, dtype, trans, "normal", seed=1000 + i, ld_pad=pad)
    if scaled:
        r, _, _ = check_scaled(p, 0.75, -1.25, epilogue=epi, options=opt, c_seed=i)
    else:
        r, _, _ = check_full(p, epilogue=epi, options=opt)
    assert r["ok"], (case, r)
