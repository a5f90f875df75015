"""Pins of the float64 row-softmax oracle (CPU only).

Each pin is a value fixed by the mathematics, not by the oracle: closed forms
(logs of small integers give rational results), the logistic function for
two-entry rows, constant rows, overflow-free huge entries, -inf entries,
scipy's independent softmax, and the degenerate rows whose value the
definition leaves undefined.  Every planted mistake (exponentiating x instead
of x - max, normalising columns, skipping the division) must fail one of
them.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import gemm_inputs as gi
from oracle import softmax as osm

LN2, LN3 = math.log(2.0), math.log(3.0)


def _pins():
    """Run every pin; returns a list of failure descriptions (empty = all pass)."""
    bad = []

    def close(name, got, want, rel=1e-14):
        got = np.asarray(got, dtype=np.float64)
        want = np.asarray(want, dtype=np.float64)
        if got.shape != want.shape or not np.allclose(got, want, rtol=rel, atol=0.0, equal_nan=True):
            bad.append(f"{name}: got {got!r}, want {want!r}")

    # exp(0) : exp(ln 2) : exp(ln 3) = 1 : 2 : 3
    y, _ = osm.softmax_rows([[0.0, LN2, LN3]])
    close("ln-ratios", y, [[1 / 6, 1 / 3, 1 / 2]])
    # a 2 x 2 matrix whose row and column normalisations differ
    y, _ = osm.softmax_rows([[0.0, LN3], [LN2, 0.0]])
    close("rows-not-columns", y, [[1 / 4, 3 / 4], [2 / 3, 1 / 3]])
    # two entries: the logistic function 1 / (1 + e^(b - a)) and its mirror
    for a, b in [(0.3, -1.7), (5.0, 5.0), (-20.0, 3.0), (12.5, -0.25)]:
        y, _ = osm.softmax_rows([[a, b]])
        close(f"logistic({a},{b})", y,
              [[1.0 / (1.0 + math.exp(b - a)), 1.0 / (1.0 + math.exp(a - b))]], rel=1e-12)
    # constant rows: 1 / N whatever the constant
    for c, n in [(0.0, 7), (-3.5, 64), (700.0, 5)]:
        y, _ = osm.softmax_rows(np.full((2, n), c))
        close(f"constant({c},{n})", y, np.full((2, n), 1.0 / n))
    # entries far beyond exp's range: e^0 / (2 + e^-1) for the two maxima
    y, _ = osm.softmax_rows([[1000.0, 999.0, 1000.0]])
    d = 2.0 + math.exp(-1.0)
    close("huge", y, [[1 / d, math.exp(-1.0) / d, 1 / d]])
    # -inf entries get exactly 0; the rest renormalise
    y, _ = osm.softmax_rows([[0.0, -np.inf, LN3]])
    close("neg-inf", y, [[1 / 4, 0.0, 3 / 4]])
    # one column: 1
    y, _ = osm.softmax_rows([[-2.0], [40.0]])
    close("one-column", y, [[1.0], [1.0]])
    # undefined rows are NaN: all -inf, +inf present, NaN present
    y, _ = osm.softmax_rows([[-np.inf, -np.inf], [np.inf, 0.0], [np.nan, 1.0]])
    if not np.isnan(y).all():
        bad.append(f"undefined rows: {y!r}")
    # z = x - max: 0 at the maximum, <= 0 elsewhere
    x = np.array([[1.5, -2.0, 4.0, 4.0]])
    _, z = osm.softmax_rows(x)
    close("z", z, [[-2.5, -6.0, 0.0, 0.0]])
    # an independent library routine on seeded, non-square inputs with a wide range
    from scipy.special import softmax as sp_softmax
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 33)) * 40.0
    y, _ = osm.softmax_rows(x)
    close("scipy", y, sp_softmax(x, axis=1), rel=1e-12)
    return bad


def test_oracle_pins():
    assert _pins() == []


@pytest.mark.parametrize("fault", [1, 2, 3])
def test_planted_mistakes_fail_a_pin(fault):
    osm.plant_fault(fault)
    try:
        assert _pins() != [], f"planted mistake {fault} passed every pin"
    finally:
        osm.plant_fault(0)


def test_rows_sum_to_one_and_are_independent():
    p = gi.make_softmax_input(19, 131, gi.F32, "wide", seed=2)
    x = gi.stored_to_f64(p.X, p.dtype)[:, :p.N]
    y, _ = osm.softmax_rows(x)
    assert np.allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert (y >= 0).all() and (y <= 1).all()
    # row i alone gives the same row
    for i in (0, 7, 18):
        yi, _ = osm.softmax_rows(x[i:i + 1])
        assert np.array_equal(yi[0], y[i])
    # adding a constant to one row changes nothing (to rounding)
    x2 = x.copy()
    x2[3] += 17.0
    y2, _ = osm.softmax_rows(x2)
    assert np.allclose(y2, y, rtol=1e-12, atol=1e-300)


def test_special_rows():
    p = gi.make_softmax_input(40, 24, gi.F32, "specials", seed=4)
    x = gi.stored_to_f64(p.X, p.dtype)[:, :p.N]
    y, _ = osm.softmax_rows(x)
    sp = gi.softmax_special_rows(40, 4)
    assert np.allclose(y[sp["constant"]], 1.0 / 24, rtol=1e-15)
    ninf = np.isneginf(x[sp["some_neg_inf"]])
    assert ninf.any() and (y[sp["some_neg_inf"]][ninf] == 0).all()
    assert np.isclose(y[sp["some_neg_inf"]].sum(), 1.0)
    for name in ("all_neg_inf", "pos_inf", "nan"):
        assert np.isnan(y[sp[name]]).all(), name
    top = x[sp["huge"]] == x[sp["huge"]].max()
    assert np.allclose(y[sp["huge"]][top], 1.0 / top.sum()) and (y[sp["huge"]][~top] == 0).all()
    others = [i for i in range(40) if i not in sp.values()]
    assert np.isfinite(y[others]).all()


def test_tolerance_accepts_rounding_and_rejects_real_errors():
    p = gi.make_softmax_input(8, 2000, gi.F32, "normal", seed=3)
    x = gi.stored_to_f64(p.X, p.dtype)[:, :p.N]
    y, z = osm.softmax_rows(x)
    # the reference rounded to each output type passes
    assert osm.check(y.astype(np.float32), y, z, p.N, gi.F32)["ok"]
    assert osm.check(y.astype(np.float16), y, z, p.N, gi.F16)["ok"]
    b = gi.stored_to_f64(gi.round_to(y, gi.BF16), gi.BF16)
    assert osm.check(b, y, z, p.N, gi.BF16)["ok"]
    # a relative error of 2^-12 fails for float32 outputs; a dropped max (all
    # outputs scaled by e^m) or a NaN in the wrong place fails everywhere
    assert not osm.check(y * (1 + 2.0 ** -12), y, z, p.N, gi.F32)["ok"]
    assert not osm.check(y * math.e, y, z, p.N, gi.F16)["ok"]
    g = y.copy()
    g[2, 5] = np.nan
    r = osm.check(g, y, z, p.N, gi.F32)
    assert not r["ok"] and r["nan_mismatch"] == 1


def test_empty_shapes():
    y, z = osm.softmax_rows(np.zeros((0, 5)))
    assert y.shape == (0, 5)
    y, z = osm.softmax_rows(np.zeros((3, 0)))
    assert y.shape == (3, 0)
