"""Row softmax boundary and host logic (CPU only): the launch-shape choice,
argument checking and quick returns of tg_softmax, without launching anything."""
from __future__ import annotations

import pytest
import torch

import tiled_gemm_02_amd as tg

F32, F16, BF16 = tg.TG_F32, tg.TG_F16, tg.TG_BF16


@pytest.mark.parametrize("dtype,E", [(F32, 4), (F16, 8), (BF16, 8)])
def test_shape_is_the_smallest_that_holds_the_row(dtype, E):
    caps = []
    for N in [0, 1, 7, 255, 256, 257, 931, 1024, 1025, 4096, 8191, 16384, 16385, 32768]:
        q, c = tg.softmax_shape(N, dtype)
        cap = q * 64 * c * E
        assert q in (1, 2, 4, 8, 16) and c * E <= 32, (N, q, c)
        assert cap >= N, (N, q, c)
        caps.append((N, cap))
        # no smaller capacity in the table holds it: halving either factor is too small
        if N > 256:
            assert cap // 2 < N, (N, q, c)
    # rows past 32768 take the two-pass kernel
    for N in [32769, 65536, 1 << 20]:
        assert tg.softmax_shape(N, dtype) == (0, 0)


def test_shape_rejects_bad_input():
    with pytest.raises(tg.TgError):
        tg.softmax_shape(10, 9)
    with pytest.raises(tg.TgError):
        tg.softmax_shape(-1, F32)


def test_argument_errors():
    # unknown dtype, negative sizes, short leading dimensions, NULL pointers
    assert tg.tg_softmax(4, 4, 16, 4, 64, 4, 7) == tg.TG_ERR_ARG
    assert tg.tg_softmax(-1, 4, 16, 4, 64, 4, F32) == tg.TG_ERR_ARG
    assert tg.tg_softmax(4, -4, 16, 4, 64, 4, F32) == tg.TG_ERR_ARG
    assert tg.tg_softmax(4, 8, 16, 7, 4096, 8, F32) == tg.TG_ERR_ARG
    assert "ldx" in tg.tg_last_error()
    assert tg.tg_softmax(4, 8, 16, 8, 4096, 7, F32) == tg.TG_ERR_ARG
    assert tg.tg_softmax(4, 8, None, 8, 4096, 8, F32) == tg.TG_ERR_NULL
    assert tg.tg_softmax(4, 8, 16, 8, None, 8, F32) == tg.TG_ERR_NULL
    assert tg.tg_softmax(1 << 31, 8, 16, 8, 4096, 8, F32) == tg.TG_ERR_ARG
    # Y overlapping X other than exactly in place
    base = 1 << 20
    assert tg.tg_softmax(4, 8, base, 8, base + 4, 8, F32) == tg.TG_ERR_ARG
    assert "overlap" in tg.tg_last_error()
    assert tg.tg_softmax(4, 8, base, 8, base, 16, F32) == tg.TG_ERR_ARG
    # disjoint, or the same rows in place, pass the checks (and then need a device)
    rc = tg.tg_softmax(4, 8, base, 8, base + 4 * 8 * 4, 8, F32)
    assert rc in (tg.TG_OK, tg.TG_ERR_DEVICE)
    rc = tg.tg_softmax(4, 8, base, 8, base, 8, F32)
    assert rc in (tg.TG_OK, tg.TG_ERR_DEVICE)


def test_quick_returns_need_no_device():
    assert tg.tg_softmax(0, 8, None, 8, None, 8, F16) == tg.TG_OK
    assert tg.tg_softmax(5, 0, None, 1, None, 1, BF16) == tg.TG_OK
    assert tg.tg_last_error() == ""


def test_no_device_is_reported():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert tg.tg_softmax(4, 8, 1 << 20, 8, 1 << 24, 8, F32) == tg.TG_ERR_DEVICE
