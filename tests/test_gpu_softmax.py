"""GPU parity of the row softmax (tg_softmax) against the float64 oracle (run with -m gpu).

Tolerance (from oracle.softmax): |y - y_ref| <= |y_ref| (u_out + 2^-24 (2|z| + n_seq +
2 ceil(log2 N) + 8)) + a_out, NaN exactly where the reference has NaN.  Shapes cover the
register-resident kernel at every launch shape (one wave per row up to 16 waves per row),
ragged row tails, rows-per-block tails, the two-pass long-row kernel, unaligned rows,
in-place calls, degenerate rows, and the full 4096 x 32768 workloads at sampled rows.
"""
from __future__ import annotations

import numpy as np
import pytest

import gemm_inputs as gi
from gemm_inputs import BF16, F16, F32, SOFTMAX_WORKLOADS, make_softmax_input
from oracle import softmax as osm
from tests.gpu_helpers import from_device, to_device, torch_dtype

pytestmark = pytest.mark.gpu

DTYPES = [F32, F16, BF16]


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    import tiled_gemm_02_amd as tg
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tg.load()
    yield


def _device_input(p, offset: int = 0):
    """X on the device as an M x N view with row stride ldx; `offset` extra leading
    elements move the view off the 16-byte grid."""
    import torch
    flat = np.ascontiguousarray(p.X).reshape(-1)
    if offset:
        flat = np.concatenate([np.zeros(offset, dtype=flat.dtype), flat])
    t = to_device(flat, p.dtype)
    return torch.as_strided(t, (p.M, p.N), (p.ldx, 1), offset)


def _run(p, offset=0, out_pad=0, in_place=False):
    import torch
    import tiled_gemm_02_amd as tg
    X = _device_input(p, offset)
    if in_place:
        Y = X
    elif out_pad:
        Y = torch.full((p.M, p.N + out_pad), float("nan"), dtype=torch_dtype(p.dtype), device="cuda:0")[:, :p.N]
    else:
        Y = None
    Y = tg.softmax(X, out=Y)
    torch.cuda.synchronize()
    return from_device(Y, p.dtype), X


def _check(p, got, rows=None):
    x = gi.stored_to_f64(p.X, p.dtype)[:, :p.N]
    if rows is not None:
        x, got = x[rows], got[rows]
    y, z = osm.softmax_rows(x)
    r = osm.check(got, y, z, p.N, p.dtype)
    return r


N_CASES = [1, 2, 3, 7, 63, 64, 65, 255, 256, 257, 931, 1024, 1025, 2049, 4095, 4097, 8200,
           16383, 16385, 32768, 32769, 70001]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("N", N_CASES)
def test_rows_of_every_length(dtype, N):
    M = max(1, min(37, 2_000_000 // N))
    _say("case softmax", dtype, M, N)
    p = make_softmax_input(M, N, dtype, "normal", seed=N)
    got, _ = _run(p)
    r = _check(p, got)
    assert r["ok"], (dtype, M, N, r)


def test_page_example_583x931():
    """The Triton page's example: 583 x 931 float32 entries from N(0, 1)."""
    w = SOFTMAX_WORKLOADS["softmax_f32_583x931"]
    p = make_softmax_input(w["M"], w["N"], w["dtype"], w["dist"], w["seed"])
    got, _ = _run(p)
    r = _check(p, got)
    assert r["ok"], r
    assert np.allclose(got.sum(axis=1), 1.0, atol=1e-5)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("N", [5, 200, 931, 3000, 20000, 40000])
@pytest.mark.parametrize("dist", ["wide", "specials"])
def test_wide_and_degenerate_rows(dtype, N, dist):
    M = 23
    _say("case softmax", dist, dtype, M, N)
    p = make_softmax_input(M, N, dtype, dist, seed=7)
    got, _ = _run(p)
    r = _check(p, got)
    assert r["ok"], (dist, dtype, N, r)
    if dist == "specials":
        sp = gi.softmax_special_rows(M, 7)
        for name in ("all_neg_inf", "pos_inf", "nan"):
            assert np.isnan(got[sp[name]]).all(), name
        assert np.allclose(got[sp["constant"]], 1.0 / N, rtol=2.0 ** -7)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("N", [100, 1024, 5000, 32768, 33000])
def test_unaligned_rows_and_strides(dtype, N):
    """Rows off the 16-byte grid (odd leading dimension, base pointer one element in)
    and an output with its own leading dimension: the element-wise load path."""
    M = 13
    _say("case softmax unaligned", dtype, M, N)
    p = make_softmax_input(M, N, dtype, "normal", seed=3, ld_pad=3)
    got, _ = _run(p, offset=1, out_pad=5)
    r = _check(p, got)
    assert r["ok"], (dtype, N, r)
    p = make_softmax_input(M, N, dtype, "normal", seed=4, ld_pad=8)
    got, _ = _run(p, out_pad=8)
    r = _check(p, got)
    assert r["ok"], (dtype, N, r)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("N", [931, 32768, 50000])
def test_in_place(dtype, N):
    M = 9
    _say("case softmax in place", dtype, M, N)
    p = make_softmax_input(M, N, dtype, "normal", seed=5, ld_pad=2)
    got, X = _run(p, in_place=True)
    r = _check(p, got)
    assert r["ok"], (dtype, N, r)
    # the padding between rows is untouched
    import torch
    full = torch.as_strided(X, (M, p.ldx), (p.ldx, 1))
    pad = from_device(full, p.dtype)[:, N:]
    assert np.array_equal(pad, gi.stored_to_f64(p.X, p.dtype)[:, N:])


def test_long_rows():
    """Rows of a million elements: the two-pass kernel over many steps per thread."""
    for dtype, (M, N) in [(F32, (2, 1 << 20)), (F16, (3, (1 << 20) + 5)), (BF16, (1, 777_777))]:
        _say("case softmax long", dtype, M, N)
        p = make_softmax_input(M, N, dtype, "wide", seed=11)
        got, _ = _run(p)
        r = _check(p, got)
        assert r["ok"], (dtype, M, N, r)


@pytest.mark.parametrize("name", ["softmax_f32_4096x32768", "softmax_f16_4096x32768"])
def test_full_workload_sampled_rows(name):
    """The benchmarked workloads at full size, in the benchmark's launch
    configuration, checked at 48 seeded rows plus the first and last."""
    w = SOFTMAX_WORKLOADS[name]
    _say("case softmax full", name)
    p = make_softmax_input(w["M"], w["N"], w["dtype"], w["dist"], w["seed"])
    got, _ = _run(p)
    rows = np.unique(np.concatenate([[0, p.M - 1],
                                     np.random.default_rng(9).choice(p.M, 48, replace=False)]))
    r = _check(p, got, rows)
    assert r["ok"], (name, r)
    # every row sums to one within the float32 bound
    assert np.allclose(got.sum(axis=1), 1.0, atol=5e-3 if w["dtype"] != F32 else 1e-4)
