"""GPU parity for 16-bit operands whose rows lie more than 2^22 elements apart
(the BLAS statement's leading dimensions, "Matrix Multiplication Background
User's Guide", sections 1-2).  The LDS-DMA kernels address a tile's rows with
32-bit byte offsets, so such operands are read through zero-padded aligned
copies (products of a GFLOP or more, with workspace) or by the element-wise
64 x 64 kernel.  The device operands are strided views into buffers with the
wide leading dimension; the oracle is fed the compact logical operands.
"""
from __future__ import annotations

import numpy as np
import pytest

from gemm_inputs import BF16, F16, NN, NT, TN, TT, make_problem
from tests.gpu_helpers import EPI_CODES, from_device, torch_dtype
import oracle

pytestmark = pytest.mark.gpu

WIDE = (1 << 22) + 8   # elements between rows: above the LDS-DMA kernels' 2^22


def _say(*a):
    print(*a, flush=True)


def _wide(arr: np.ndarray, d, ld: int):
    """Device view of the stored operand `arr` (rows x cols) whose rows lie
    `ld` elements apart (ld - cols elements of NaN between them)."""
    import torch
    from tests.gpu_helpers import to_device
    rows, cols = arr.shape
    buf = torch.full((rows, ld), float("nan"), dtype=torch_dtype(d), device="cuda:0")
    buf[:, :cols].copy_(to_device(arr, d))
    return buf[:, :cols]


def _run(p, wide_a: bool, wide_b: bool, epilogue=None, options=None, workspace=None):
    import torch
    import tiled_gemm_02_amd as tg
    A = _wide(p.A, p.dtype, WIDE) if wide_a else _wide(p.A, p.dtype, p.A.shape[1])
    B = _wide(p.B, p.dtype, WIDE) if wide_b else _wide(p.B, p.dtype, p.B.shape[1])
    assert (A.stride(0) == WIDE) == wide_a and (B.stride(0) == WIDE) == wide_b
    C = torch.full((p.M, p.N), float("nan"), dtype=torch_dtype(p.dtype), device="cuda:0")
    epi = None if epilogue is None else (tg.TG_EPI_LEAKY_RELU, 0.01)
    tg.gemm(A, B, trans_a=p.trans_a, trans_b=p.trans_b, epilogue=epi, out=C, options=options,
            workspace=workspace)
    torch.cuda.synchronize()
    got = from_device(C, p.dtype)
    del A, B, C
    torch.cuda.empty_cache()
    return got


def _check(p, got, epilogue=None):
    ref, absab = oracle.gemm_full(p.M, p.N, p.K, p.A, p.lda, p.trans_a, p.B, p.ldb, p.trans_b,
                                  dtype=p.dtype, epi=EPI_CODES[epilogue], slope=0.01)
    r = oracle.check(got, ref, absab, p.dtype)
    assert r["ok"], r


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("trans", [NN, TN, NT, TT])
def test_wide_rows_small_product(dtype, trans):
    """Below a GFLOP: the element-wise kernel reads both wide operands in
    place; a ragged M/N edge (72 x 136 against 64 x 64 tiles), a K tail
    (200), unsplit and split in two with the leaky rectifier."""
    import tiled_gemm_02_amd as tg
    _say("case wide ld small", dtype, trans)
    p = make_problem(72, 136, 200, dtype, trans, "normal", seed=41)
    got = _run(p, True, True)
    _check(p, got)
    got = _run(p, True, True, epilogue="leaky_relu",
               options=dict(path=tg.TG_PATH_MFMA, tile_m=64, tile_n=64, split_k=2))
    _check(p, got, epilogue="leaky_relu")


@pytest.mark.parametrize("dtype,trans", [(F16, NT), (BF16, NN)])
def test_wide_rows_copied(dtype, trans):
    """About a GFLOP with A's rows 2^22 + 8 apart: A and B are copied into
    aligned buffers and the LDS-DMA kernels run on the copies (ragged N, K
    not a multiple of 64); without room for the copies the element-wise kernel
    runs instead.  Both compared in full against the oracle."""
    import torch
    import tiled_gemm_02_amd as tg
    _say("case wide ld copied", dtype, trans)
    M, N, K = 520, 1032, 1000
    p = make_problem(M, N, K, dtype, trans, "normal", seed=42)
    need = 2 * (M * K + K * 1040) + 4096
    ws = torch.empty(8 * need, dtype=torch.uint8, device="cuda:0")
    got = _run(p, True, False, workspace=ws)
    _check(p, got)
    got = _run(p, True, False, epilogue="leaky_relu", options=dict(split_k=2), workspace=ws)
    _check(p, got, epilogue="leaky_relu")
    small = torch.empty(256, dtype=torch.uint8, device="cuda:0")
    got = _run(p, True, False, workspace=small)
    _check(p, got)
