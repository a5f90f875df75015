"""GPU parity: the HIP library against the float64 oracle (run with -m gpu).

Tolerance (from the oracle): |C - C_ref| <= 1e-4 (|A||B|)_ij + 1e-6 + r_out |C_ref|,
r_out = 0 (f32), 1e-3 (f16), 2^-8 (bf16).  Integer-valued operands whose
partial sums are exact in float32 must match bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

from gemm_inputs import (BF16, F16, F32, NN, NT, TN, TT, WORKLOADS, make_int_problem, make_problem,
                         layout, round_to)
from tests.gpu_helpers import check_full, check_sampled, check_scaled, run_gpu, to_device

pytestmark = pytest.mark.gpu

DTYPES = [F32, F16, BF16]
TRANS = [NN, TN, NT, TT]


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    import tiled_gemm_02_amd as tg
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tg.load()
    _say("device", torch.cuda.get_device_name(0), "cus", tg.tg_device_cus())
    yield


# ---------------------------------------------------------------- small shapes, full compare

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("trans", TRANS)
@pytest.mark.parametrize("shape", [(64, 64, 64), (128, 96, 200), (200, 136, 72), (264, 520, 136)])
def test_aligned_shapes(dtype, trans, shape):
    M, N, K = shape
    _say("case", dtype, trans, shape)
    p = make_problem(M, N, K, dtype, trans, "uniform", seed=3)
    r, _, _ = check_full(p)
    assert r["ok"], r


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("trans", TRANS)
@pytest.mark.parametrize("shape", [(1, 7, 31), (7, 1, 33), (33, 31, 7), (31, 33, 1), (255, 257, 33),
                                   (257, 255, 31), (65, 130, 257)])
def test_ragged_shapes(dtype, trans, shape):
    M, N, K = shape
    _say("case", dtype, trans, shape)
    p = make_problem(M, N, K, dtype, trans, "normal", seed=5)
    r, _, _ = check_full(p)
    assert r["ok"], r


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("trans", TRANS)
def test_padded_leading_dims(dtype, trans):
    _say("case ld_pad", dtype, trans)
    p = make_problem(136, 72, 96, dtype, trans, "uniform", seed=1, ld_pad=8)
    r, _, _ = check_full(p, out_pad=8)
    assert r["ok"], r
    p = make_problem(100, 60, 90, dtype, trans, "uniform", seed=1, ld_pad=3)
    r, _, _ = check_full(p, out_pad=5)
    assert r["ok"], r


# ---------------------------------------------------------------- exactness pins on the GPU

@pytest.mark.parametrize("trans", TRANS)
@pytest.mark.parametrize("dtype,lo,hi,K", [(F16, -2, 2, 512), (BF16, -1, 1, 256), (F32, -4, 4, 1024)])
def test_integer_products_bitwise(trans, dtype, lo, hi, K):
    _say("case int", dtype, trans, K)
    p = make_int_problem(136, 200, K, dtype, trans, lo, hi, seed=2)
    r, got, ref = check_full(p)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("dtype", DTYPES)
def test_identity_and_permutation_bitwise(dtype):
    rng = np.random.default_rng(0)
    M, K = 96, 128
    A = round_to(rng.uniform(-1, 1, (M, K)), dtype)
    from gemm_inputs import Problem, stored_to_f64
    A64 = stored_to_f64(A, dtype)
    I = round_to(np.eye(K), dtype)
    p = Problem(M, K, K, dtype, NN, A, I, K, K)
    got = run_gpu(p)
    np.testing.assert_array_equal(got, A64)
    perm = rng.permutation(K)
    P = np.zeros((K, K))
    P[perm, np.arange(K)] = 1.0
    p = Problem(M, K, K, dtype, NN, A, round_to(P, dtype), K, K)
    got = run_gpu(p)
    np.testing.assert_array_equal(got, A64[:, perm])


# ---------------------------------------------------------------- degenerate and edge cases

@pytest.mark.parametrize("dtype", DTYPES)
def test_k_zero_writes_zero(dtype):
    import torch
    import tiled_gemm_02_amd as tg
    from tests.gpu_helpers import torch_dtype
    A = torch.empty((5, 0), dtype=torch_dtype(dtype), device="cuda:0")
    B = torch.empty((0, 7), dtype=torch_dtype(dtype), device="cuda:0")
    C = torch.full((5, 7), 3.0, dtype=torch_dtype(dtype), device="cuda:0")
    tg.gemm(A, B, out=C, epilogue=(tg.TG_EPI_LEAKY_RELU, 0.01))
    torch.cuda.synchronize()
    assert torch.all(C == 0)


def test_empty_outputs_are_noops():
    import torch
    import tiled_gemm_02_amd as tg
    A = torch.ones((0, 8), dtype=torch.float16, device="cuda:0")
    B = torch.ones((8, 4), dtype=torch.float16, device="cuda:0")
    C = tg.gemm(A, B)
    assert C.shape == (0, 4)
    assert tg.tg_gemm(4, 0, 8, 1, 8, 1, 0 + 1, 1, 1, tg.TG_F16, 0) == tg.TG_OK


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("trans", TRANS)
def test_leaky_relu_epilogue(dtype, trans):
    _say("case leaky", dtype, trans)
    p = make_problem(200, 264, 128, dtype, trans, "normal", seed=4)
    r, got, ref = check_full(p, epilogue="leaky_relu", slope=0.01)
    assert r["ok"], r
    assert (ref < 0).any() and (ref > 0).any()


# ---------------------------------------------------------------- forced plans

def _tiles(dtype, trans):
    if dtype == F32:   # the float32 256 x 256 kernel takes K-contiguous A and B only
        return ([(256, 256)] if trans == NT else []) + [(128, 128), (64, 64)]
    return [(256, 256), (192, 256), (256, 128), (128, 128), (128, 64), (64, 64)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("trans", [NN, NT])
def test_every_tile(dtype, trans):
    for tm, tn in _tiles(dtype, trans):
        _say("case tile", dtype, trans, tm, tn)
        p = make_problem(296, 280, 136, dtype, trans, "normal", seed=6)
        r, _, _ = check_full(p, options=dict(tile_m=tm, tile_n=tn, split_k=1))
        assert r["ok"], (tm, tn, r)
    # element-wise loads exist for 64 x 64 only; other forced tiles are refused
    import tiled_gemm_02_amd as tg
    p = make_problem(300, 281, 137, dtype, trans, "normal", seed=6)
    r, _, _ = check_full(p, options=dict(tile_m=64, tile_n=64, split_k=1))
    assert r["ok"], r
    with pytest.raises(tg.TgError):
        run_gpu(p, options=dict(tile_m=128, tile_n=128))
    if dtype == F32 and trans != NT:
        p = make_problem(296, 280, 136, dtype, trans, "normal", seed=6)
        with pytest.raises(tg.TgError):
            run_gpu(p, options=dict(tile_m=256, tile_n=256))


# 16-bit 192 x 256 tiles (the ping-pong kernel with 96 x 64 per wave, A
# K-contiguous): ragged edges, K tails, splits, alpha / beta with the
# epilogue; stored-transposed A is refused
TILE192_CASES = [
    (400, 520, 1000, F16, NN, 1, None, 1.0, 0.0),
    (200, 304, 72, BF16, NT, 1, None, 1.0, 0.0),
    (584, 264, 1032, F16, NT, 3, None, 1.0, 0.0),
    (384, 512, 512, BF16, NN, 2, "leaky_relu", 0.5, -1.0),
]


@pytest.mark.parametrize("case", TILE192_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-d{c[3]}-t{c[4]}-s{c[5]}")
def test_tile_192x256(case):
    import tiled_gemm_02_amd as tg
    M, N, K, dtype, trans, split, epi, alpha, beta = case
    _say("case tile 192", case)
    p = make_problem(M, N, K, dtype, trans, "normal", seed=31)
    opts = dict(tile_m=192, tile_n=256, split_k=split)
    if alpha == 1.0 and beta == 0.0:
        r, _, _ = check_full(p, epilogue=epi, options=opts)
    else:
        r, _, _ = check_scaled(p, alpha, beta, epilogue=epi, options=opts)
    assert r["ok"], (case, r)
    q = make_problem(M, N, K, dtype, TN, "normal", seed=31)
    with pytest.raises(tg.TgError):
        run_gpu(q, options=opts)


def test_tile_192x256_is_planned_and_sampled():
    """2304 x 4096 x 4096: 192 tiles of 192 x 256 against 144 of 256 x 256."""
    import tiled_gemm_02_amd as tg
    pl = tg.tg_gemm_plan(2304, 4096, 4096, tg.TG_F16, tg.TG_NN)
    assert (pl["tile_m"], pl["tile_n"], pl["tiles"]) == (192, 256, 192), pl
    p = make_problem(2304, 4096, 4096, F16, NN, "normal", seed=0)
    _say("case tile 192 sampled")
    r = check_sampled(p)
    assert r["ok"], r


# 16-bit 128 x 128 tiles with two K groups per workgroup (eight waves, each
# group over its part of the workgroup's K range, group 1's sums added to group
# 0's in LDS): every layout, ragged M (A plain) and N (B transposed), K tails in
# either group, a group 1 one whole stage short (K = 136: 72 and 64, so group 1
# runs an all-zero tail stage; K = 8: group 1 has no K at all), outer K splits
# (the last split's halves uneven), alpha / beta (old C: the direct stores) and
# the epilogue on the LDS-staged stores
KG2_CASES = [
    (296, 280, 136, F16, NN, 1, None, 1.0, 0.0),
    (300, 264, 200, BF16, NT, 1, None, 1.0, 0.0),
    (264, 300, 1032, F16, NT, 1, None, 1.0, 0.0),
    (392, 520, 72, BF16, TN, 1, None, 1.0, 0.0),
    (256, 256, 8, F16, TT, 1, None, 1.0, 0.0),
    (520, 392, 4104, F16, NN, 3, None, 1.0, 0.0),
    (136, 1000, 2056, BF16, TT, 2, None, 1.0, 0.0),
    (296, 280, 264, F16, NT, 1, "leaky_relu", 1.0, 0.0),
    (384, 512, 512, BF16, NN, 1, "leaky_relu", 0.5, -1.0),
    (200, 136, 1000, F16, TN, 1, None, -1.25, 0.75),
    (384, 512, 520, BF16, NT, 2, "leaky_relu", 0.5, -1.0),
]


@pytest.mark.parametrize("case", KG2_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-d{c[3]}-t{c[4]}-s{c[5]}")
def test_two_k_groups(case):
    import tiled_gemm_02_amd as tg
    M, N, K, dtype, trans, split, epi, alpha, beta = case
    _say("case two K groups", case)
    p = make_problem(M, N, K, dtype, trans, "normal", seed=41)
    opts = dict(tile_m=128, tile_n=128, split_k=split, k_groups=2)
    pl = tg.tg_gemm_plan(M, N, K, dtype, trans, options=opts)
    assert pl["k_groups"] == 2 and pl["split_k"] == split, pl
    if alpha == 1.0 and beta == 0.0:
        r, _, _ = check_full(p, epilogue=epi, options=opts)
    else:
        r, _, _ = check_scaled(p, alpha, beta, epilogue=epi, options=opts)
    assert r["ok"], (case, r)


# 16-bit 64 x 64 tiles with four K groups (sixteen waves): the workgroup's
# 64-deep stages dealt out in runs, a K tail as group 0's last stage, groups one
# stage short (K = 136: 3 stages over 4 groups; K = 8: groups 1-3 with no K),
# every layout, outer splits, alpha / beta and the epilogue
KG4_CASES = [
    (136, 200, 264, F16, NN, 1, None, 1.0, 0.0),
    (200, 136, 8, BF16, NT, 1, None, 1.0, 0.0),
    (96, 64, 136, F16, TN, 1, "leaky_relu", 1.0, 0.0),
    (264, 520, 1032, BF16, TT, 1, None, 0.5, -1.0),
    (520, 264, 4104, F16, NT, 3, None, 1.0, 0.0),
    (128, 128, 520, BF16, NN, 1, "leaky_relu", -1.25, 0.75),
]


@pytest.mark.parametrize("case", KG4_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-d{c[3]}-t{c[4]}-s{c[5]}")
def test_four_k_groups(case):
    import tiled_gemm_02_amd as tg
    M, N, K, dtype, trans, split, epi, alpha, beta = case
    _say("case four K groups", case)
    p = make_problem(M, N, K, dtype, trans, "normal", seed=44)
    opts = dict(tile_m=64, tile_n=64, split_k=split, k_groups=4)
    pl = tg.tg_gemm_plan(M, N, K, dtype, trans, options=opts)
    assert pl["k_groups"] == 4 and pl["split_k"] == split, pl
    if alpha == 1.0 and beta == 0.0:
        r, _, _ = check_full(p, epilogue=epi, options=opts)
    else:
        r, _, _ = check_scaled(p, alpha, beta, epilogue=epi, options=opts)
    assert r["ok"], (case, r)


def test_two_k_groups_refused_where_no_kernel_exists():
    """Four groups on 16-bit 128 x 128 tiles, two on the float32 256 x 256 tile,
    16-bit 256 x 256 tiles, the GEMV path and operands off the 16-byte grid have
    no K-group kernel: the call fails; k_groups = 3 is an argument error."""
    import tiled_gemm_02_amd as tg
    for dtype, shape, opts in [(F16, (256, 256, 256), dict(tile_m=128, tile_n=128, k_groups=4)),
                               (F32, (256, 256, 256), dict(tile_m=256, tile_n=256, k_groups=2)),
                               (F16, (256, 256, 256), dict(tile_m=256, tile_n=256, k_groups=2)),
                               (F16, (1, 256, 256), dict(path=tg.TG_PATH_GEMV, k_groups=2)),
                               (F16, (300, 282, 130), dict(k_groups=2))]:
        _say("case two K groups refused", dtype, shape, opts)
        p = make_problem(*shape, dtype, NN, "normal", seed=42)
        with pytest.raises(tg.TgError):
            run_gpu(p, options=opts)
    p = make_problem(256, 256, 256, F16, NN, "normal", seed=42)
    with pytest.raises(tg.TgError):
        run_gpu(p, options=dict(k_groups=3))


def test_two_k_groups_planned_and_sampled():
    """2304 x 1536 x 4096 (216 tiles of 128 x 128 for 256 CUs): the planner
    puts each tile on one eight-wave workgroup whose two K groups share the K
    loop, with no workspace; 4096 sampled outputs against the oracle, and the
    same product with the planner's former choice (K split two ways through
    float32 partials) agrees to the tolerance."""
    import tiled_gemm_02_amd as tg
    pl = tg.tg_gemm_plan(2304, 1536, 4096, tg.TG_F16, tg.TG_NN)
    assert (pl["tile_m"], pl["tile_n"], pl["k_groups"], pl["split_k"]) == (128, 128, 2, 1), pl
    assert pl["workspace_bytes"] == 0, pl
    p = make_problem(2304, 1536, 4096, F16, NN, "normal", seed=0)
    _say("case two K groups sampled")
    r = check_sampled(p)
    assert r["ok"], r
    r = check_sampled(p, options=dict(tile_m=128, tile_n=128, split_k=2, k_groups=1))
    assert r["ok"], r


# float32 on the register-staged kernel with K groups (64 x 64 and 32 x 32 with
# four, 128 x 128 with two; each group over consecutive 32-deep K steps, a group past
# the end of K loading zeros): every layout, ragged K, groups with no K, K splits,
# alpha / beta and the epilogue
F32_KG_CASES = [
    (256, 256, 256, NN, 64, 4, 1, None, 1.0, 0.0),
    (200, 136, 72, NT, 64, 4, 1, None, 1.0, 0.0),      # 3 steps over 4 groups
    (96, 160, 8, TN, 64, 4, 1, None, 1.0, 0.0),        # one step, three empty groups
    (264, 520, 1000, TT, 64, 4, 2, "leaky_relu", 0.5, -1.0),
    (520, 264, 1028, NN, 128, 2, 1, None, 1.0, 0.0),
    (264, 520, 100, NT, 128, 2, 1, "leaky_relu", 1.0, 0.0),
    (128, 128, 4, TN, 128, 2, 1, None, -1.25, 0.75),   # K = 4: group 1 empty
    (520, 264, 2000, TT, 128, 2, 3, None, 1.0, 0.0),
    (256, 256, 256, NN, 32, 4, 1, None, 1.0, 0.0),
    (36, 44, 1000, NT, 32, 4, 1, "leaky_relu", 0.5, -1.0),
    (200, 136, 72, TN, 32, 4, 1, None, 1.0, 0.0),       # 3 steps over 4 groups
    (264, 520, 1028, TT, 32, 4, 2, None, -1.25, 0.75),
]


@pytest.mark.parametrize("case", F32_KG_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-t{c[3]}-{c[4]}k{c[5]}s{c[6]}")
def test_f32_k_groups(case):
    import tiled_gemm_02_amd as tg
    M, N, K, trans, tile, kg, split, epi, alpha, beta = case
    _say("case f32 K groups", case)
    p = make_problem(M, N, K, F32, trans, "normal", seed=43)
    opts = dict(tile_m=tile, tile_n=tile, split_k=split, k_groups=kg)
    pl = tg.tg_gemm_plan(M, N, K, F32, trans, options=opts)
    assert pl["k_groups"] == kg and pl["split_k"] == split and pl["vector_io"] == 1, pl
    if alpha == 1.0 and beta == 0.0:
        r, _, _ = check_full(p, epilogue=epi, options=opts)
    else:
        r, _, _ = check_scaled(p, alpha, beta, epilogue=epi, options=opts)
    assert r["ok"], (case, r)


# float32 on the 256 x 256 ping-pong kernel: ragged M and N edges, a K tail
# (K % 16 != 0: the partial stage goes through registers), K splits, the
# epilogue and alpha / beta
F32_PP_CASES = [
    (300, 520, 1000, 1, None, 1.0, 0.0),
    (256, 256, 16, 1, None, 1.0, 0.0),
    (520, 264, 4, 1, None, 1.0, 0.0),
    (516, 772, 1204, 3, None, 1.0, 0.0),
    (264, 300, 2000, 2, "leaky_relu", 0.5, -1.5),
]


@pytest.mark.parametrize("case", F32_PP_CASES, ids=lambda c: "x".join(map(str, c[:4])))
def test_f32_pingpong(case):
    M, N, K, split, epi, alpha, beta = case
    _say("case f32 pingpong", case)
    p = make_problem(M, N, K, F32, NT, "normal", seed=21)
    opts = dict(tile_m=256, tile_n=256, split_k=split)
    if alpha == 1.0 and beta == 0.0:
        r, _, _ = check_full(p, epilogue=epi, options=opts)
    else:
        r, _, _ = check_scaled(p, alpha, beta, epilogue=epi, options=opts)
    assert r["ok"], (case, r)


# float32 in the other layouts through K-contiguous copies (vector_io 3): the
# operands stored M/N-contiguous are transposed into the workspace, the NT
# product runs on the 256 x 256 kernel; unaligned sizes copy and pad both
F32_NT_COPY_CASES = [
    (520, 1000, 1028, NN, 1.0, 0.0, None),
    (520, 1000, 1028, TN, 1.0, 0.0, None),
    (520, 1000, 1028, TT, 1.0, 0.0, None),
    (517, 1001, 1027, NN, 1.0, 0.0, None),
    (517, 1001, 1027, TT, 1.0, 0.0, None),
    (600, 904, 1100, TN, -0.5, 2.0, "leaky_relu"),
]


@pytest.mark.parametrize("case", F32_NT_COPY_CASES,
                         ids=lambda c: "x".join(map(str, c[:3])) + f"-t{c[3]}")
def test_f32_nt_copies(case):
    import tiled_gemm_02_amd as tg
    M, N, K, trans, alpha, beta, epi = case
    _say("case f32 nt copies", case)
    opts = dict(tile_m=256, tile_n=256, split_k=1)
    pl = tg.tg_gemm_plan(M, N, K, tg.TG_F32, trans, options=opts)
    assert pl["vector_io"] == 3 and pl["tile_m"] == 256, pl
    p = make_problem(M, N, K, F32, trans, "normal", seed=23)
    if alpha == 1.0 and beta == 0.0:
        r, _, _ = check_full(p, epilogue=epi, options=opts)
    else:
        r, _, _ = check_scaled(p, alpha, beta, epilogue=epi, options=opts)
    assert r["ok"], (case, r)


def test_f32_pingpong_is_planned_and_sampled():
    """A large float32 NT product plans the 256 x 256 tile; sampled outputs
    against the oracle."""
    import tiled_gemm_02_amd as tg
    for trans, vio in [(NT, 1), (NN, 3)]:
        p = make_problem(4096, 4096, 4096, F32, trans, "normal", seed=0)
        pl = tg.tg_gemm_plan(p.M, p.N, p.K, tg.TG_F32, trans)
        assert (pl["tile_m"], pl["tile_n"], pl["vector_io"]) == (256, 256, vio), pl
        _say("case f32 4096 sampled", trans)
        r = check_sampled(p)
        assert r["ok"], r


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("split", [2, 3, 5])
def test_split_k(dtype, split):
    _say("case split", dtype, split)
    p = make_problem(136, 96, 1000 if dtype != F32 else 1000, dtype, NN, "normal", seed=7)
    for epi in (None, "leaky_relu"):
        r, _, _ = check_full(p, epilogue=epi, options=dict(split_k=split))
        assert r["ok"], (split, epi, r)


def test_split_k_caller_workspace():
    import torch
    import tiled_gemm_02_amd as tg
    p = make_problem(128, 128, 2048, F16, NN, "normal", seed=8)
    need = tg.tg_workspace_size(128, 128, 2048, F16, NN, dict(split_k=4))
    assert need == 4 * 128 * 128 * 4
    ws = torch.empty(need // 4, dtype=torch.float32, device="cuda:0")
    r, _, _ = check_full(p, options=dict(split_k=4), workspace=ws)
    assert r["ok"], r
    small = torch.empty(16, dtype=torch.float32, device="cuda:0")
    with pytest.raises(tg.TgError):
        run_gpu(p, options=dict(split_k=4), workspace=small)
    r, _, _ = check_full(p, workspace=small)  # planner's choice falls back to no split
    assert r["ok"], r


def test_thread_default_workspace():
    """tg_set_workspace: calls without a workspace of their own use the
    thread's default; one too small for a forced split is an error, an
    unforced plan falls back; cleared, the library allocates again."""
    import torch
    import tiled_gemm_02_amd as tg
    _say("case default workspace")
    p = make_problem(256, 256, 8192, F16, NT, "normal", seed=91)
    need = tg.tg_workspace_size(256, 256, 8192, tg.TG_F16, tg.TG_NT, dict(split_k=8))
    assert need == 8 * 256 * 256 * 4
    assert tg.tg_workspace_bytes(256, 256, 8192, tg.TG_F16, tg.TG_NT) == \
        tg.tg_workspace_size(256, 256, 8192, tg.TG_F16, tg.TG_NT)
    buf = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    try:
        tg.set_workspace(buf)
        r, _, _ = check_full(p, options=dict(split_k=8))
        assert r["ok"], r
        tg.set_workspace(buf[:1024])
        with pytest.raises(tg.TgError):
            run_gpu(p, options=dict(split_k=8))
        r, _, _ = check_full(p)
        assert r["ok"], r
    finally:
        tg.set_workspace(None)
    r, _, _ = check_full(p, options=dict(split_k=8))
    assert r["ok"], r


@pytest.mark.parametrize("case", ["gemv", "skinny"])
def test_split_partials_ignore_stale_workspace(case):
    """K-split partials are fully rewritten by every call: arbitrary bytes left
    in a reused workspace must not change the result."""
    import torch
    import tiled_gemm_02_amd as tg
    if case == "gemv":
        M, N, K, opts = 1, 4096, 8192, None
    else:
        M, N, K, opts = 1024, 128, 4096, dict(path=tg.TG_PATH_SKINNY, split_k=4)
    p = make_problem(M, N, K, F16, NN, "uniform", seed=12)
    pl = tg.tg_gemm_plan(M, N, K, F16, NN, opts)
    assert pl["split_k"] > 1
    g = torch.Generator(device="cuda:0").manual_seed(5)
    ws = torch.randint(0, 256, (pl["workspace_bytes"],), dtype=torch.uint8, device="cuda:0", generator=g)
    for fill in (None, 0xFF, None):
        if fill is not None:
            ws.fill_(fill)
        r, _, _ = check_full(p, options=opts, workspace=ws)
        assert r["ok"], (case, fill, r)


@pytest.mark.parametrize("case", ["gemv", "gemv_generic", "skinny", "skinny_ragged"])
def test_split_reduction_many_splits(case):
    """Split-K products of the skinny and GEMV kernels at a few splits and at
    more than 255 (a K range of one stage or a few rows per split): the fixed-
    order reduction matches the oracle on a workspace of arbitrary bytes, and
    a repeated call on the same workspace is bit-identical."""
    import torch
    import tiled_gemm_02_amd as tg
    if case == "gemv":            # 16-byte rows: the vector kernel
        M, N, K, splits, opts = 1, 512, 8192, (16, 512), dict(path=tg.TG_PATH_GEMV)
    elif case == "gemv_generic":  # odd n: the element-wise kernel
        M, N, K, splits, opts = 1, 509, 4100, (12, 300), dict(path=tg.TG_PATH_GEMV)
    elif case == "skinny":
        M, N, K, splits, opts = 256, 128, 16448, (4, 257), dict(path=tg.TG_PATH_SKINNY)
    else:                         # a ragged row block, columns past N in the tile
        M, N, K, splits, opts = 200, 72, 16456, (3, 258), dict(path=tg.TG_PATH_SKINNY)
    p = make_problem(M, N, K, F16, NN, "uniform", seed=13)
    g = torch.Generator(device="cuda:0").manual_seed(6)
    for s in splits:
        o = dict(opts, split_k=s)
        pl = tg.tg_gemm_plan(M, N, K, F16, NN, o)
        _say("case split reduction", case, s, pl["split_k"], pl["workspace_bytes"])
        assert pl["path"] == opts["path"] and pl["split_k"] > 1
        assert (pl["split_k"] > 255) == (s > 255)
        ws = torch.randint(0, 256, (pl["workspace_bytes"],), dtype=torch.uint8, device="cuda:0", generator=g)
        r, got, _ = check_full(p, options=o, workspace=ws)
        assert r["ok"], (case, s, r)
        again = run_gpu(p, options=o, workspace=ws)
        assert np.array_equal(got, again), (case, s)


# ---------------------------------------------------------------- skinny path

@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("trans", [NN, NT])
@pytest.mark.parametrize("shape", [(128, 128, 256), (200, 64, 264), (1000, 120, 1000), (136, 8, 512),
                                   (584, 72, 1096), (4096, 128, 2048)])
def test_skinny(dtype, trans, shape):
    import tiled_gemm_02_amd as tg
    M, N, K = shape
    _say("case skinny", dtype, trans, shape)
    p = make_problem(M, N, K, dtype, trans, "uniform", seed=11)
    opts = dict(path=tg.TG_PATH_SKINNY)
    assert tg.tg_gemm_plan(M, N, K, dtype, trans, opts)["path"] == tg.TG_PATH_SKINNY
    r, _, _ = check_full(p, options=opts)
    assert r["ok"], r
    for split in (1, 3):
        r, _, _ = check_full(p, epilogue="leaky_relu", options=dict(path=tg.TG_PATH_SKINNY, split_k=split))
        assert r["ok"], (split, r)


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("trans", [NN, NT])
@pytest.mark.parametrize("shape", [(300, 2, 1024), (1000, 3, 2048), (256, 5, 520), (640, 7, 4096),
                                   (777, 12, 1032), (2000, 20, 1024), (400, 100, 512)])
def test_skinny_narrow_outputs(dtype, trans, shape):
    """Narrow products with N off the 16-byte grid (2 <= N <= 128, N % 8 != 0)
    take the skinny kernel: stored N x K, B is read in place; stored K x N with
    ldb = N, B alone is first copied into an aligned zero-padded buffer
    (vector_io 4) and A is read in place.  Ragged M, a forced split, the
    epilogue and alpha / beta through both forms."""
    import tiled_gemm_02_amd as tg
    M, N, K = shape
    _say("case skinny narrow", dtype, trans, shape)
    p = make_problem(M, N, K, dtype, trans, "uniform", seed=14)
    pl = tg.tg_gemm_plan(M, N, K, dtype, trans)
    assert pl["path"] == tg.TG_PATH_SKINNY and pl["vector_io"] == (1 if trans == NT else 4), pl
    r, _, _ = check_full(p)
    assert r["ok"], r
    r, _, _ = check_full(p, epilogue="leaky_relu", options=dict(path=tg.TG_PATH_SKINNY, split_k=3))
    assert r["ok"], r
    r, _, _ = check_scaled(p, 0.5, -1.0, epilogue="leaky_relu")
    assert r["ok"], r


def test_skinny_narrow_workload_size():
    """8192 x 4 x 8192 (B K x N with ldb = 4, copied) and 8192 x 12 x 8192 NT,
    the full matrix against the oracle."""
    import tiled_gemm_02_amd as tg
    for N, trans in ((4, NN), (12, NT)):
        p = make_problem(8192, N, 8192, F16, trans, "normal", seed=15)
        pl = tg.tg_gemm_plan(8192, N, 8192, F16, trans)
        assert pl["path"] == tg.TG_PATH_SKINNY, pl
        _say("case skinny narrow 8192", N, trans)
        r, _, _ = check_full(p)
        assert r["ok"], (N, trans, r)


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("trans", [NN, NT])
@pytest.mark.parametrize("shape", [(128, 128, 256), (200, 64, 264), (1000, 120, 1000), (136, 8, 512),
                                   (584, 72, 1096), (4160, 128, 2048)])
def test_skinny_tall_row_blocks(dtype, trans, shape):
    """The 128-row block form (tile_m = 128): ragged last blocks (M not a
    multiple of 128), every split, both B layouts, both output widths."""
    import tiled_gemm_02_amd as tg
    M, N, K = shape
    _say("case skinny rb128", dtype, trans, shape)
    p = make_problem(M, N, K, dtype, trans, "uniform", seed=12)
    for split in (1, 2, 4):
        opts = dict(path=tg.TG_PATH_SKINNY, tile_m=128, split_k=split)
        pl = tg.tg_gemm_plan(M, N, K, dtype, trans, opts)
        assert pl["path"] == tg.TG_PATH_SKINNY and pl["tile_m"] == 128
        r, _, _ = check_full(p, epilogue="leaky_relu" if split == 2 else None, options=opts)
        assert r["ok"], (split, r)


def test_skinny_integer_bitwise():
    import tiled_gemm_02_amd as tg
    p = make_int_problem(640, 128, 512, F16, NN, -2, 2, seed=3)
    r, got, ref = check_full(p, options=dict(path=tg.TG_PATH_SKINNY))
    np.testing.assert_array_equal(got, ref)


def test_skinny_is_chosen_for_the_narrow_workload():
    import tiled_gemm_02_amd as tg
    assert tg.tg_gemm_plan(8192, 128, 8192, F16, NN)["path"] == tg.TG_PATH_SKINNY


# ---------------------------------------------------------------- GEMV path

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("trans", TRANS)
@pytest.mark.parametrize("shape", [(1, 1024, 512), (1, 520, 33), (1000, 1, 512), (77, 1, 1031),
                                   (1, 1, 300)])
def test_gemv(dtype, trans, shape):
    import tiled_gemm_02_amd as tg
    M, N, K = shape
    _say("case gemv", dtype, trans, shape)
    p = make_problem(M, N, K, dtype, trans, "uniform", seed=9)
    assert tg.tg_gemm_plan(M, N, K, dtype, trans)["path"] == tg.TG_PATH_GEMV
    r, _, _ = check_full(p)
    assert r["ok"], r
    r, _, _ = check_full(p, epilogue="leaky_relu")
    assert r["ok"], r


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("lanes", [8, 16, 32, 64])
@pytest.mark.parametrize("split", [1, 3, 16])
def test_gemv_strip_widths_and_splits(dtype, lanes, split):
    """Every strip width of the vector cols kernel, with and without K splits
    (the partial-sum reduction), on a ragged K and a column count that leaves a
    partial last strip."""
    import tiled_gemm_02_amd as tg
    E = 4 if dtype == F32 else 8
    N = lanes * E * 5 + 2 * E
    _say("case gemv strips", dtype, lanes, split, N)
    p = make_problem(1, N, 1037, dtype, NN, "uniform", seed=12)
    opts = dict(path=tg.TG_PATH_GEMV, tile_n=lanes * E, split_k=split)
    pl = tg.tg_gemm_plan(1, N, 1037, dtype, NN, opts)
    assert pl["tile_n"] == lanes * E and pl["split_k"] == split and pl["vector_io"] == 1, pl
    r, _, _ = check_full(p, options=opts)
    assert r["ok"], r
    r, _, _ = check_full(p, epilogue="leaky_relu", options=opts)
    assert r["ok"], r


@pytest.mark.parametrize("dtype", DTYPES)
def test_gemv_ragged_lengths_on_aligned_rows(dtype):
    """Output lengths and K off the 16-byte grid with row strides on it (padded
    views): the vector cols kernel reads the chunk that straddles column n
    element by element (every strip width, with and without splits), the
    vector rows kernel reads the K tail element by element."""
    import tiled_gemm_02_amd as tg
    E = 4 if dtype == F32 else 8
    # M, N, K, trans, ld_pad (puts the padded leading dimensions on the grid), options
    cases = [(1, 4097, 1000, NN, 7, None), (1, 1001, 2048, NN, 7, None), (301, 1, 777, TT, 3, None),
             (1, 523, 1037, NN, 5, dict(path=tg.TG_PATH_GEMV, tile_n=8 * E, split_k=3)),
             (1, 523, 1037, NN, 5, dict(path=tg.TG_PATH_GEMV, tile_n=64 * E, split_k=1)),
             (1, 700, 1003, NT, 5, None), (500, 1, 1029, NT, 3, None)]
    for M, N, K, trans, pad, opts in cases:
        _say("case gemv ragged", dtype, M, N, K, trans, pad, opts)
        p = make_problem(M, N, K, dtype, trans, "uniform", seed=16, ld_pad=pad)
        assert p.lda % 8 == 0 or M == 1, p.lda
        r, _, _ = check_full(p, options=opts)
        assert r["ok"], (M, N, K, trans, r)
        r, _, _ = check_scaled(p, 0.5, -1.0, epilogue="leaky_relu", options=opts, c_seed=10)
        assert r["ok"], (M, N, K, trans, r)


def test_gemv_strided():
    p = make_problem(1, 600, 256, F16, NN, "uniform", seed=10, ld_pad=8)
    r, _, _ = check_full(p, out_pad=0)
    assert r["ok"], r
    p = make_problem(300, 1, 256, F16, TT, "uniform", seed=10, ld_pad=4)
    r, _, _ = check_full(p)
    assert r["ok"], r


# ---------------------------------------------------------------- the measured workloads

@pytest.mark.parametrize("name", ["f32_256", "f16_skinny_8192x128x8192", "f16_gemv_1x8192x8192"])
def test_workload_full(name):
    w = dict(WORKLOADS[name])
    _say("workload full", name)
    epi = w.pop("epilogue", None)
    slope = w.pop("slope", 0.01)
    p = make_problem(**w)
    r, _, _ = check_full(p, epilogue=epi, slope=slope)
    assert r["ok"], r


@pytest.mark.parametrize("name", ["f16_4096_nt", "f16_8192", "bf16_leaky_8192",
                                  "bf16_leaky_6912x2048x4096", "f32_8192_nt", "f32_8192"])
def test_workload_sampled(name):
    w = dict(WORKLOADS[name])
    _say("workload sampled", name)
    epi = w.pop("epilogue", None)
    slope = w.pop("slope", 0.01)
    p = make_problem(**w)
    r = check_sampled(p, epilogue=epi, slope=slope)
    assert r["ok"], r


@pytest.mark.parametrize("N", [1536, 1544, 3584, 3592, 6144])
def test_sweep_shapes_sampled(N):
    _say("sweep", N)
    p = make_problem(2304, N, 4096, F16, NN, "normal", seed=0)
    r = check_sampled(p)
    assert r["ok"], r
    r = check_sampled(p, options=dict(tile_m=256, tile_n=128, split_k=1))
    assert r["ok"], r


# ---------------------------------------------------------------- alpha and beta
#
# C = epi(alpha A.B + beta C_old) through every path that writes C: the macro
# tiles (ping-pong, four-wave and register-staged kernels), split-K and its
# reduction, the skinny stream, both GEMV forms, unaligned operands, K = 0 and
# alpha = 0.  C_old is a seeded draw; with beta = 0 C starts as NaN and must
# not be read.

SCALED = [
    # M, N, K, dtype, trans, ld_pad, options, alpha, beta, epilogue
    (512, 512, 256, F16, NN, 0, dict(tile_m=256, tile_n=256, split_k=1), 0.5, -1.25, None),
    (512, 512, 200, BF16, NT, 0, dict(tile_m=256, tile_n=256, split_k=1), 2.0, 0.5, "leaky_relu"),
    (520, 296, 264, F16, TT, 0, dict(tile_m=128, tile_n=128, split_k=1), -1.0, 1.0, "leaky_relu"),
    (304, 280, 520, BF16, TN, 0, dict(tile_m=256, tile_n=128, split_k=1), 1.5, 0.0, None),
    (200, 136, 1000, F16, NN, 0, dict(split_k=3), 1.0, 1.0, None),
    (200, 136, 1000, F32, NT, 0, dict(split_k=2), 0.75, -0.5, "leaky_relu"),
    (130, 70, 90, F32, TT, 0, None, -1.0, 2.0, "leaky_relu"),
    (100, 90, 70, F16, NN, 1, None, 2.0, 0.5, None),
    (1000, 120, 1000, BF16, NN, 0, dict(path=2, split_k=1), 0.25, -0.5, "leaky_relu"),
    (1000, 120, 1000, F16, NT, 0, dict(path=2, split_k=2), 1.5, 1.0, None),
    (1, 1000, 777, F16, NN, 0, None, 2.0, 1.0, None),
    (1, 520, 33, F32, NN, 0, None, -1.0, 0.5, "leaky_relu"),
    (777, 1, 1031, BF16, NN, 0, None, -0.5, 1.0, "leaky_relu"),
    (77, 1, 1031, F16, TN, 0, None, 3.0, -2.0, None),
    (64, 64, 0, F16, NN, 0, None, 3.0, 0.5, "leaky_relu"),
    (64, 48, 0, BF16, NN, 0, None, 1.0, 0.0, None),
]


@pytest.mark.parametrize("case", SCALED, ids=lambda c: "x".join(map(str, c[:3])) + f"-d{c[3]}-t{c[4]}")
def test_alpha_beta(case):
    import tiled_gemm_02_amd as tg
    M, N, K, dtype, trans, ld_pad, opts, alpha, beta, epi = case
    _say("case alpha/beta", case)
    p = make_problem(M, N, K, dtype, trans, "uniform", seed=31, ld_pad=ld_pad)
    if opts and opts.get("path") == 2:
        opts = dict(opts, path=tg.TG_PATH_SKINNY)
    r, got, _ = check_scaled(p, alpha, beta, epilogue=epi, options=opts, c_seed=3)
    assert r["ok"], (case, r)
    assert np.isfinite(got).all()


def test_alpha_zero_does_not_read_operands():
    """BLAS: with alpha = 0, A and B are not referenced (NaN there is harmless)."""
    p = make_problem(256, 192, 128, F16, NN, "uniform", seed=32)
    p.A[...] = np.float16(np.nan)
    p.B[...] = np.float16(np.nan)
    r, got, _ = check_scaled(p, 0.0, -1.5, epilogue="leaky_relu", c_seed=4)
    assert r["ok"], r
    assert np.isfinite(got).all()


def test_beta_needs_the_old_c():
    import torch
    import tiled_gemm_02_amd as tg
    A = torch.zeros((8, 8), dtype=torch.float16, device="cuda:0")
    with pytest.raises(ValueError):
        tg.gemm(A, A, beta=1.0)
    # unknown flag bits are an argument error
    C = torch.zeros((8, 8), dtype=torch.float16, device="cuda:0")
    bad = tg.Epilogue(0, 0.0, 2, 1.0, 0.0)
    with pytest.raises(tg.TgError):
        tg.gemm(A, A, out=C, epilogue=bad)


# ---------------------------------------------------------------- benchmark mode

@pytest.mark.parametrize("shape", [(2304, 2048, 4096, NN), (1024, 128, 2048, NN), (520, 296, 264, NT)])
def test_autotune_choice_is_valid_and_correct(shape):
    """tg_autotune returns options tg_gemm_ex accepts, no slower than the
    planner's own choice on the same timing, and the product under them
    matches the oracle."""
    import torch
    import tiled_gemm_02_amd as tg
    M, N, K, trans = shape
    _say("case autotune", shape)
    p = make_problem(M, N, K, F16, trans, "normal", seed=41)
    A = to_device(p.A, p.dtype)
    B = to_device(p.B, p.dtype)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda:0")
    opts, us = tg.autotune(A, B, trans_a=p.trans_a, trans_b=p.trans_b, workspace=ws, reps=3)
    assert us > 0
    assert opts["path"] in (tg.TG_PATH_AUTO, tg.TG_PATH_MFMA, tg.TG_PATH_SKINNY)
    r, _, _ = check_full(p, options=None if opts["path"] == tg.TG_PATH_AUTO else opts, workspace=ws)
    assert r["ok"], (opts, r)
    tg.tune_cache_clear()


def test_autotune_winner_is_cached_and_used():
    """tg_autotune records its winner per problem; calls without options then
    plan with it (tg_gemm_plan shows the same tile and split), still match the
    oracle, and run with too small a workspace; clearing the cache restores
    the heuristic."""
    import torch
    import tiled_gemm_02_amd as tg
    M, N, K = 1536, 2048, 4096
    _say("case autotune cache", (M, N, K))
    tg.tune_cache_clear()
    assert tg.tune_cache_size() == 0
    p = make_problem(M, N, K, F16, NN, "normal", seed=43)
    A = to_device(p.A, p.dtype)
    B = to_device(p.B, p.dtype)
    heuristic = tg.plan_for(A, B)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda:0")
    opts, _ = tg.autotune(A, B, workspace=ws, reps=2)
    assert tg.tune_cache_size() == 1
    want = heuristic if opts["path"] == tg.TG_PATH_AUTO else tg.plan_for(A, B, options=opts)
    got = tg.plan_for(A, B)
    for k in ("path", "tile_m", "tile_n", "split_k"):
        assert got[k] == want[k], (k, got, want, opts)
    # the cached plan runs without options, with or without room for a split
    r, _, _ = check_full(p)
    assert r["ok"], r
    small = torch.empty(4096, dtype=torch.uint8, device="cuda:0")
    r, _, _ = check_full(p, workspace=small)
    assert r["ok"], r
    # the same sizes with another leading dimension are another problem
    p2 = make_problem(M, N, K, F16, NN, "normal", seed=44, ld_pad=8)
    r, _, _ = check_full(p2)
    assert r["ok"], r
    assert tg.tune_cache_size() == 1
    tg.tune_cache_clear()
    assert tg.tune_cache_size() == 0
    again = tg.plan_for(A, B)
    for k in ("path", "tile_m", "tile_n", "split_k"):
        assert again[k] == heuristic[k]


# ---------------------------------------------------------------- stream-K
#
# One workgroup per CU takes an equal run of all tiles' 32-deep K stages; tiles
# split between workgroups are summed in K order by the fix-up kernel.  Cases:
# 16 pieces per tile, a K tail stage with one stage per workgroup, ragged
# tiles, every layout, two stages in all, and a K tail with 64 tiles.

SK_CASES = [
    # M, N, K, dtype, trans
    (1024, 1024, 4096, F16, NN),
    (512, 768, 1000, BF16, TN),
    (296, 520, 2048, F16, NT),
    (256, 512, 4096, BF16, TT),
    (256, 256, 64, F16, NN),
    (2048, 2048, 2080, F16, NN),
]


@pytest.mark.parametrize("case", SK_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-d{c[3]}-t{c[4]}")
def test_stream_k(case):
    import tiled_gemm_02_amd as tg
    M, N, K, dtype, trans = case
    _say("case stream-K", case)
    p = make_problem(M, N, K, dtype, trans, "normal", seed=61)
    opts = dict(split_k=tg.TG_SPLIT_STREAM_K)
    pl = tg.tg_gemm_plan(M, N, K, dtype, trans, opts)
    assert pl["split_k"] == tg.TG_SPLIT_STREAM_K
    r, _, _ = check_full(p, options=opts, out_pad=4)
    assert r["ok"], (case, r)
    r, _, _ = check_scaled(p, 0.75, -0.5, epilogue="leaky_relu", options=opts, c_seed=9)
    assert r["ok"], (case, r)


def test_stream_k_full_size_sampled():
    """2304 x 4096 x 4096 (144 tiles on 256 CUs), in the configuration the
    quantization sweep runs, checked at sampled outputs."""
    import tiled_gemm_02_amd as tg
    _say("case stream-K 2304x4096x4096")
    p = make_problem(2304, 4096, 4096, F16, NN, "normal", seed=62)
    r = check_sampled(p, options=dict(split_k=tg.TG_SPLIT_STREAM_K))
    assert r["ok"], r


# ---------------------------------------------------------------- aligned copies
#
# Operands off the 16-byte grid (K odd, padded leading dimensions) in products
# large enough to copy them into aligned buffers first.

ALIGN_CASES = [
    # M, N, K, dtype, trans, ld_pad
    (1024, 1024, 521, F16, NN, 0),
    (1024, 512, 1031, BF16, TN, 3),
    (512, 1024, 1029, F16, NT, 1),
    (1024, 512, 1030, BF16, TT, 5),
    (1024, 512, 1027, F32, NN, 1),
]


@pytest.mark.parametrize("case", ALIGN_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-d{c[3]}-t{c[4]}-p{c[5]}")
def test_unaligned_operands_copied(case):
    import tiled_gemm_02_amd as tg
    M, N, K, dtype, trans, pad = case
    _say("case aligned copy", case)
    p = make_problem(M, N, K, dtype, trans, "uniform", seed=51, ld_pad=pad)
    # float32 in a layout other than NT copies into the NT layout (3)
    want = 3 if dtype == F32 and trans != NT else 2
    assert tg.tg_plan_model(M, N, K, dtype, trans)["vector_io"] == want
    r, _, _ = check_full(p)
    assert r["ok"], (case, r)
    r, _, _ = check_scaled(p, 0.5, -1.0, epilogue="leaky_relu", c_seed=6)
    assert r["ok"], (case, r)


# M or N off the grid as well (ragged tails in every dimension, padded C
# rows, scaled forms).  Where the off-grid size is the one the 16-byte chunks
# run along (M with A stored transposed, N with B stored plain), the copies
# are padded in M and N too and the macro-tile kernel stores only the M x N
# corner; a 16-bit M with A plain or N with B transposed is read in place (the
# LDS-DMA kernels clamp rows past M and N); a narrow product copies B alone.
PADDED_MN_CASES = [
    # M, N, K, dtype, trans, ld_pad, (path, vector_io)
    (1025, 1000, 1031, F16, NN, 0, ("mfma", 2)),
    (999, 1024, 1024, BF16, TN, 2, ("mfma", 2)),
    (1024, 1003, 600, F16, NT, 0, ("mfma", 1)),
    (517, 1021, 1000, BF16, TT, 1, ("mfma", 2)),
    (1001, 1000, 999, F32, NN, 0, ("mfma", 3)),
    (8191, 100, 1000, F16, NN, 0, ("skinny", 4)),
    (1003, 1024, 1000, F16, NN, 0, ("mfma", 1)),
    (1003, 1001, 1024, BF16, NT, 0, ("mfma", 1)),
    (3, 4096, 4096, F16, NN, 0, ("mfma", 1)),
    (12, 2048, 1024, BF16, NT, 0, ("mfma", 1)),
]


@pytest.mark.parametrize("case", PADDED_MN_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-d{c[3]}-t{c[4]}-p{c[5]}")
def test_unaligned_rows_and_columns(case):
    import tiled_gemm_02_amd as tg
    M, N, K, dtype, trans, pad, (path, vio) = case
    _say("case ragged M / N", case)
    p = make_problem(M, N, K, dtype, trans, "uniform", seed=53, ld_pad=pad)
    pl = tg.tg_plan_model(M, N, K, dtype, trans)
    assert (pl["path_name"], pl["vector_io"]) == (path, vio), pl
    r, _, _ = check_full(p, out_pad=3)
    assert r["ok"], (case, r)
    r, _, _ = check_scaled(p, 0.5, -1.0, epilogue="leaky_relu", c_seed=7)
    assert r["ok"], (case, r)


# One operand off the grid beside a large aligned one: only the small operand
# is copied (the workspace holds a few columns or rows, not the large
# operand), the large one is read in place.
ONE_COPY_CASES = [
    # M, N, K, dtype, trans: A stored transposed and aligned, B K x 7 copied
    (2048, 7, 4096, F16, TN),
    # A stored K x 7 copied, B stored N x K read in place
    (7, 2048, 4096, BF16, TT),
    # A plain with M ragged read in place, B K x 5 copied
    (3001, 5, 2048, F16, NN),
]


@pytest.mark.parametrize("case", ONE_COPY_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-d{c[3]}-t{c[4]}")
def test_only_the_off_grid_operand_is_copied(case):
    import tiled_gemm_02_amd as tg
    M, N, K, dtype, trans = case
    _say("case one copy", case)
    p = make_problem(M, N, K, dtype, trans, "uniform", seed=55)
    pl = tg.tg_plan_model(M, N, K, dtype, trans)
    assert pl["vector_io"] in (2, 4), pl
    assert pl["workspace_bytes"] < 2 * max(M, N) * K // 8, pl
    r, _, _ = check_full(p)
    assert r["ok"], (case, r)
    r, _, _ = check_scaled(p, 0.5, -1.0, epilogue="leaky_relu", c_seed=9)
    assert r["ok"], (case, r)


def test_padded_copy_with_forced_split():
    p = make_problem(1025, 1000, 4100, F16, NN, "uniform", seed=54)
    for split in (1, 3):
        _say("case padded split", split)
        r, _, _ = check_full(p, options=dict(split_k=split, tile_m=128, tile_n=128))
        assert r["ok"], (split, r)
        r, _, _ = check_scaled(p, 2.0, 0.5, options=dict(split_k=split), c_seed=8)
        assert r["ok"], (split, r)


def test_unaligned_copy_with_a_small_workspace_falls_back():
    """A caller workspace too small for the copies: the element-wise kernel runs."""
    import torch
    p = make_problem(1024, 1024, 521, F16, NN, "uniform", seed=52)
    small = torch.empty(4096, dtype=torch.uint8, device="cuda:0")
    r, _, _ = check_full(p, workspace=small)
    assert r["ok"], r



# ---------------------------------------------------------------- the boundary's own entry point

@pytest.mark.parametrize("dtype,trans,shape,epi", [
    (F16, NN, (520, 264, 1000), None),
    (BF16, NT, (300, 520, 136), "leaky_relu"),
    (F32, TN, (136, 200, 264), "leaky_relu"),
    (F16, NN, (2048, 128, 2048), None),   # skinny, split K: the library's own workspace
])
def test_raw_tg_gemm_symbol(dtype, trans, shape, epi):
    """Full products through the exported tg_gemm symbol itself (the
    spec signature: sizes, pointers, leading dimensions, dtype, trans,
    epilogue, stream), called through ctypes with device pointers."""
    import ctypes
    import torch
    import tiled_gemm_02_amd as tg
    from tests.gpu_helpers import from_device, oracle_full, torch_dtype
    import oracle
    M, N, K = shape
    _say("case raw tg_gemm", dtype, trans, shape, epi)
    p = make_problem(M, N, K, dtype, trans, "normal", seed=44)
    A = to_device(p.A, dtype)
    B = to_device(p.B, dtype)
    C = torch.full((M, N), float("nan"), dtype=torch_dtype(dtype), device="cuda:0")
    e = tg.Epilogue(tg.TG_EPI_LEAKY_RELU, 0.01, 0, 1.0, 0.0) if epi else None
    lib = tg.load()
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.tg_gemm(M, N, K, A.data_ptr(), p.lda, B.data_ptr(), p.ldb, C.data_ptr(), N,
                     dtype, trans, ctypes.pointer(e) if e else None, stream)
    assert rc == tg.TG_OK, tg.tg_last_error()
    torch.cuda.synchronize()
    got = from_device(C, dtype)
    ref, absab = oracle_full(p, epi)
    r = oracle.check(got, ref, absab, dtype)
    assert r["ok"], r
