"""The Python binding refuses, on the host, operands whose pointers would take
a kernel outside its memory: host tensors, and views whose rows overlap (a
row stride below the row width).  Nothing here reaches a kernel (CPU only)."""
from __future__ import annotations

import pytest
import torch

import tiled_gemm_02_amd as tg


def test_ld_of_plain_and_strided_views():
    a = torch.zeros((6, 10), dtype=torch.float16)
    assert tg._ld(a) == 10
    assert tg._ld(a[:, :4]) == 10          # a slice of a wider matrix: ld > width
    assert tg._ld(a[:1]) == 10             # one row: any ld >= the width
    assert tg._ld(torch.zeros((0, 5))) == 5


@pytest.mark.parametrize("make", [
    lambda: torch.zeros(8, dtype=torch.float16).expand(4, 8),           # stride (0, 1)
    lambda: torch.zeros(16, dtype=torch.float16).as_strided((4, 8), (2, 1)),   # rows overlap
])
def test_ld_refuses_overlapping_rows(make):
    with pytest.raises(ValueError, match="overlap"):
        tg._ld(make())


def test_ld_refuses_column_major():
    with pytest.raises(ValueError, match="row-major"):
        tg._ld(torch.zeros((8, 6), dtype=torch.float16).t())


def test_host_tensors_are_refused_before_any_call():
    A = torch.zeros((16, 16), dtype=torch.float16)
    B = torch.zeros((16, 16), dtype=torch.float16)
    with pytest.raises(TypeError, match="CUDA"):
        tg.gemm(A, B)
    with pytest.raises(TypeError, match="CUDA"):
        tg.softmax(A)
    with pytest.raises(TypeError, match="CUDA"):
        tg.autotune(A, B)
    with pytest.raises(TypeError, match="CUDA"):
        tg.set_workspace(torch.zeros(256, dtype=torch.uint8))
