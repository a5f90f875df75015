"""The planner's tile/wave quantization model (CPU only).

Pins: the integer figures of "Matrix Multiplication Background User's Guide"
sections 2-3 (A100 with 108 SMs, one 256x128 tile per SM per wave), the
arithmetic intensities of its section 2, the grid ceil-division of the GEMM
kernels note, and properties of the MI355X plans.
"""
from __future__ import annotations

import pytest

import tiled_gemm_02_amd as tg

F16 = tg.TG_F16
FORCE_256x128 = dict(tile_m=256, tile_n=128, split_k=1)


def a100(M, N, K, tile=(256, 128)):
    return tg.tg_plan_model(M, N, K, F16, tg.TG_NN, num_cus=108, occupancy=1,
                            options=dict(tile_m=tile[0], tile_n=tile[1], split_k=1))


def test_arithmetic_intensity_examples():
    # section 2: 8192 x 128 x 8192 -> 124.1 FLOP/B; 8192^3 -> 2730; GEMV < 1
    assert round(tg.tg_plan_model(8192, 128, 8192, F16)["arith_intensity"], 1) == 124.1
    assert int(tg.tg_plan_model(8192, 8192, 8192, F16)["arith_intensity"]) == 2730
    assert tg.tg_plan_model(1, 8192, 8192, F16)["arith_intensity"] < 1
    assert tg.tg_plan_model(8192, 1, 8192, F16)["arith_intensity"] < 1


def test_wave_quantization_fig8():
    # M = 2304, K = 4096, 256x128 tiles, 108 SMs: N = 1536 is one full wave of 108 tiles
    p = a100(2304, 1536, 4096)
    assert p["tiles"] == 108 and p["waves"] == 1 and p["wave_eff"] == 1.0
    # N = 1544 .. 1664: 9 x 13 = 117 tiles, a tail wave of 9 tiles (8.33% of the SMs)
    for N in (1544, 1600, 1664):
        p = a100(2304, N, 4096)
        assert p["tiles"] == 117 and p["waves"] == 2
        assert p["tiles"] - 108 == 9 and round(9 / 108 * 100, 2) == 8.33
    # throughput roughly halves from 1536 to 1544 (time doubles)
    assert a100(2304, 1544, 4096)["pred_us"] == pytest.approx(2 * a100(2304, 1536, 4096)["pred_us"])
    # the same step after 3072, 4608 and 6144
    for n0 in (3072, 4608, 6144):
        assert a100(2304, n0 + 8, 4096)["waves"] == a100(2304, n0, 4096)["waves"] + 1


def test_tile_quantization_fig7():
    # M = 27648, K = 4096, forced 256x128: N = 136..256 keeps 2 tiles per row, 216 tiles
    for N in range(136, 257, 8):
        p = a100(27648, N, 4096)
        assert p["tiles"] == 216
    assert a100(27648, 128, 4096)["tiles"] == 108
    # at N = 136 only 8 of the second tile's 128 columns are useful
    p = a100(27648, 136, 4096)
    assert p["tile_eff"] == pytest.approx(136 / 256)
    assert (136 - 128) / 128 == 0.0625
    # time is flat while the tile count is flat
    assert a100(27648, 136, 4096)["pred_us"] == pytest.approx(a100(27648, 256, 4096)["pred_us"])


def test_tile_quantization_fig6():
    # 128x128 tiles: 256x256 -> 4 tiles, 257x256 -> 6 tiles: 1.5x the math for +0.39% work
    a = a100(256, 256, 1024, tile=(128, 128))
    b = a100(257, 256, 1024, tile=(128, 128))
    assert a["tiles"] == 4 and b["tiles"] == 6
    assert b["tiles"] / a["tiles"] == 1.5
    assert round((257 * 256 / (256 * 256) - 1) * 100, 2) == 0.39


def test_tile_sizes_fig5():
    # 6912 x 2048: 256x128 gives 432 = 4 x 108 tiles; 64x64 gives 8x the tiles
    big = a100(6912, 2048, 4096, tile=(256, 128))
    small = a100(6912, 2048, 4096, tile=(64, 64))
    assert big["tiles"] == 432 == 4 * 108
    assert small["tiles"] == 8 * big["tiles"]


def test_grid_is_ceil_division():
    # 16 x 16 blocks over N = 1000: (1000 + 15) / 16 = 63 blocks per dimension
    p = tg.tg_plan_model(1000, 1000, 64, F16, tg.TG_NN, num_cus=108, occupancy=1,
                         options=dict(tile_m=16, tile_n=16, split_k=1))
    assert p["tiles"] == 63 * 63 == ((1000 + 15) // 16) ** 2


def test_mi355x_plans():
    p = tg.tg_plan_model(8192, 8192, 8192, F16)
    assert p["path_name"] == "mfma" and p["tile_m"] * p["tile_n"] == 256 * 256
    assert p["tiles"] == 1024 and p["waves"] == 4 and p["wave_eff"] == 1.0
    p = tg.tg_plan_model(1, 8192, 8192, F16)
    assert p["path_name"] == "gemv"
    p = tg.tg_plan_model(8192, 1, 8192, F16)
    assert p["path_name"] == "gemv"
    # K == 0 and empty outputs are quick returns
    assert tg.tg_plan_model(64, 64, 0, F16)["path_name"] == "none"
    assert tg.tg_plan_model(0, 64, 64, F16)["path_name"] == "none"
    # small M and N with large K split K (whole splits, or stream-K's runs)
    p = tg.tg_plan_model(256, 256, 65536, F16)
    if p["split_k"] == tg.TG_SPLIT_STREAM_K:
        assert p["workgroups"] == 256 and p["workspace_bytes"] == 2 * 256 * 256 * 256 * 4
    else:
        assert p["split_k"] > 1 and p["workspace_bytes"] == p["split_k"] * 256 * 256 * 4
    p = tg.tg_plan_model(256, 256, 65536, F16, options=dict(split_k=16))
    assert p["split_k"] == 16 and p["workspace_bytes"] == 16 * 256 * 256 * 4
    # on 256 CUs a forced 256x128 tile steps from one to two waves between N = 3584 and 3592
    f = dict(tile_m=256, tile_n=128, split_k=1)
    a = tg.tg_plan_model(2304, 3584, 4096, F16, occupancy=1, options=f)
    b = tg.tg_plan_model(2304, 3592, 4096, F16, occupancy=1, options=f)
    assert (a["tiles"], a["waves"], b["tiles"], b["waves"]) == (252, 1, 261, 2)


def test_flop_formula_against_page_numbers():
    # Triton tutorial, T4: 2*M*N*K FLOP over the median latency.  Its X is 8192 x 6144 and Y is
    # 6144 x 4096 (BLAS M = 8192, K = 6144, N = 4096); 130.7831 ms -> 3.1533 TFLOPS and
    # 261.9420 ms -> 1.5741 TFLOPS (printed means of per-run ratios; agree to 3 digits).
    flop = 2 * 8192 * 4096 * 6144
    assert flop / 130.7831e-3 / 1e12 == pytest.approx(3.1533, rel=2e-3)
    assert flop / 261.9420e-3 / 1e12 == pytest.approx(1.5741, rel=1e-3)


def round256(x):
    return (x + 255) // 256 * 256


def test_unaligned_operands_are_copied_when_it_pays():
    """K (or a leading dimension) off the 16-byte grid: a large product plans
    an aligned, zero-padded copy of A and B (vector_io 2) with the copies at the
    start of the workspace; a small one keeps the element-wise kernel."""
    F = tg.TG_F16
    big = tg.tg_plan_model(4096, 4096, 4097, F, tg.TG_NN)
    assert big["vector_io"] == 2 and big["path_name"] == "mfma"
    kp = 4104   # K rounded up to 8 elements
    copies = 4096 * kp * 2 + kp * 4096 * 2
    assert big["workspace_bytes"] >= copies
    assert tg.tg_plan_model(4096, 4096, 4096, F, tg.TG_NN)["vector_io"] == 1
    small = tg.tg_plan_model(64, 64, 65, F, tg.TG_NN)
    assert small["vector_io"] == 0 and small["workspace_bytes"] == 0
    # M or N off the grid too: the copies are padded to M' x K' and K' x N',
    # and the macro-tile kernel (loads bounded by M', N', stores by M, N) runs it
    padded = tg.tg_plan_model(4097, 4090, 4097, F, tg.TG_NN)
    assert padded["vector_io"] == 2 and padded["path_name"] == "mfma"
    mp, np_ = 4104, 4096
    copies = round256(mp * kp * 2) + round256(kp * np_ * 2)
    assert padded["workspace_bytes"] >= copies
    assert padded["tiles"] == -(-4097 // padded["tile_m"]) * -(-4090 // padded["tile_n"])
    # a narrow padded product leaves the skinny path for the macro-tile one
    narrow = tg.tg_plan_model(8191, 100, 8191, F, tg.TG_NN)
    assert narrow["vector_io"] == 2 and narrow["path_name"] == "mfma"
    # a forced skinny path is not turned into a macro-tile product:
    # with N off the grid it is unsupported, with only K off it is copied
    with pytest.raises(tg.TgError):
        tg.tg_plan_model(8191, 100, 8191, F, tg.TG_NN, options=dict(path="skinny"))
    sk = tg.tg_plan_model(8192, 96, 8191, F, tg.TG_NN, options=dict(path="skinny"))
    assert sk["vector_io"] == 2 and sk["path_name"] == "skinny"



def test_two_k_group_plans():
    """128 x 128 tiles with two K groups per workgroup (eight waves splitting
    the workgroup's K range, summed in LDS): one workgroup per CU, so the plan
    uses them where the tiles about fill the CUs once and K is long enough to
    share; a K split of two without partials, workspace or a second launch."""
    F = tg.TG_F16
    for n in (1536, 1664, 1792):     # 216-252 tiles on 256 CUs
        p = tg.tg_plan_model(2304, n, 4096, F)
        assert (p["tile_m"], p["tile_n"], p["k_groups"], p["split_k"]) == (128, 128, 2, 1), p
        assert p["occupancy"] == 1 and p["waves"] == 1 and p["workspace_bytes"] == 0
        # one group: the same tile needs a split of two (float32 partials) to fill the CUs
        q = tg.tg_plan_model(2304, n, 4096, F, options=dict(k_groups=1))
        assert q["k_groups"] == 1 and q["pred_us"] > p["pred_us"]
    # 270 tiles would need two waves: not used there, nor for large products
    assert tg.tg_plan_model(2304, 1920, 4096, F)["k_groups"] == 1
    assert tg.tg_plan_model(8192, 8192, 8192, F)["k_groups"] == 1
    # a forced tile keeps one group unless two are asked for
    f = tg.tg_plan_model(2304, 1536, 4096, F, options=dict(tile_m=128, tile_n=128, split_k=2))
    assert f["k_groups"] == 1 and f["workspace_bytes"] == 2 * 2304 * 1536 * 4
    f = tg.tg_plan_model(2304, 1536, 4096, F, options=dict(tile_m=128, tile_n=128, split_k=2, k_groups=2))
    assert f["k_groups"] == 2 and f["split_k"] == 2 and f["workgroups"] == 2 * 216
    # other paths report one group
    assert tg.tg_plan_model(1, 8192, 8192, F)["k_groups"] == 1
    assert tg.tg_plan_model(8192, 128, 8192, F)["k_groups"] == 1
    # no such kernel: K groups with stream-K, other paths, off-grid operands; bad values
    # (a forced tile the model prices whatever it is)
    for args, opts in [((1024, 1024, 4096, F), dict(k_groups=2, split_k=tg.TG_SPLIT_STREAM_K)),
                       ((1, 1024, 4096, F), dict(k_groups=2, path=tg.TG_PATH_GEMV)),
                       ((300, 282, 130, F), dict(k_groups=2)),
                       ((1024, 1024, 4096, F), dict(k_groups=3)),
                       ((1024, 1024, 4096, F), dict(k_groups=8)),
                       ((1024, 1024, 4096, F), dict(k_groups=-1))]:
        with pytest.raises(tg.TgError):
            tg.tg_plan_model(*args, tg.TG_NN, options=opts)


def test_f32_k_group_plans():
    """float32 on the register-staged kernel with K groups: 32 x 32 with four
    groups for the smallest products (256^3: 64 workgroups of sixteen waves, one
    launch), 64 x 64 with four where few tiles meet a long K (1024^3: 256 tiles),
    128 x 128 with two where the tiles fill the CUs once (2048^3); the 256 x 256
    ping-pong tile and large products keep one group."""
    F = tg.TG_F32
    p = tg.tg_plan_model(256, 256, 256, F)
    assert (p["tile_m"], p["k_groups"], p["split_k"], p["workspace_bytes"]) == (32, 4, 1, 0), p
    p = tg.tg_plan_model(1024, 1024, 1024, F)
    assert (p["tile_m"], p["k_groups"], p["split_k"], p["workspace_bytes"]) == (64, 4, 1, 0), p
    p = tg.tg_plan_model(2048, 2048, 2048, F)
    assert (p["tile_m"], p["k_groups"], p["split_k"]) == (128, 2, 1), p
    p = tg.tg_plan_model(8192, 8192, 8192, F, tg.TG_NT)
    assert (p["tile_m"], p["k_groups"]) == (256, 1), p
    f = tg.tg_plan_model(256, 256, 256, F, options=dict(tile_m=64, tile_n=64, k_groups=4, split_k=1))
    assert (f["k_groups"], f["workgroups"], f["occupancy"]) == (4, 16, 1), f


def test_stream_k_plans():
    """Stream-K (split_k = TG_SPLIT_STREAM_K): one workgroup per CU over all
    tiles' 32-deep K stages, 256 x 256 tiles, two float32 tile pieces of
    workspace per workgroup; only with fewer tiles than CUs."""
    F = tg.TG_F16
    SK = tg.TG_SPLIT_STREAM_K
    p = tg.tg_plan_model(2304, 4096, 4096, F, tg.TG_NN, options=dict(split_k=SK))
    assert p["split_k"] == SK and (p["tile_m"], p["tile_n"]) == (256, 256)
    assert p["tiles"] == 9 * 16 and p["workgroups"] == 256
    assert p["workspace_bytes"] == 2 * 256 * 256 * 256 * 4
    # fewer K stages than CUs: one workgroup per stage
    q = tg.tg_plan_model(256, 256, 64, F, tg.TG_NN, options=dict(split_k=SK))
    assert q["workgroups"] == 2
    # not offered: float32, unaligned sizes, as many tiles as CUs, other tiles
    for args, opts in [((1024, 1024, 4096, tg.TG_F32), dict(split_k=SK)),
                       ((256, 252, 1024, F), dict(split_k=SK)),
                       ((8192, 8192, 8192, F), dict(split_k=SK)),
                       ((1024, 1024, 4096, F), dict(split_k=SK, tile_m=128, tile_n=128))]:
        with pytest.raises(tg.TgError):
            tg.tg_plan_model(*args, tg.TG_NN, options=opts)
    with pytest.raises(tg.TgError):
        tg.tg_plan_model(1024, 1024, 4096, F, tg.TG_NN, options=dict(split_k=-2))


def test_f32_tiles():
    """float32: the 256 x 256 tile (ping-pong kernel) only for K-contiguous A
    and B (NT) with leading dimensions up to 2^21; 128 x 128 otherwise."""
    F = tg.TG_F32
    p = tg.tg_plan_model(8192, 8192, 8192, F, tg.TG_NT)
    assert (p["tile_m"], p["tile_n"], p["tiles"], p["vector_io"]) == (256, 256, 1024, 1)
    p = tg.tg_plan_model(1024, 1024, 1024, F, tg.TG_NT, options=dict(tile_m=256, tile_n=256))
    assert p["tile_m"] == 256
    # the other layouts without copies: the register-staged 128 x 128 kernel
    for tr in (tg.TG_NN, tg.TG_TN, tg.TG_TT):
        p = tg.tg_plan_model(8192, 8192, 8192, F, tr, options=dict(tile_m=128, tile_n=128, split_k=1))
        assert (p["tile_m"], p["tile_n"], p["vector_io"]) == (128, 128, 1)


def test_f32_nt_copies():
    """Large float32 products stored in another layout copy the operands that
    are M/N-contiguous into K-contiguous buffers (transposing them) and run
    the NT product on the 256 x 256 kernel (vector_io 3); aligned operands
    already K-contiguous are read in place; small products stay direct."""
    F = tg.TG_F32
    n = 8192
    plane = n * n * 4
    for tr, copied in [(tg.TG_NN, 1), (tg.TG_TN, 2), (tg.TG_TT, 1)]:
        p = tg.tg_plan_model(n, n, n, F, tr)
        assert (p["tile_m"], p["tile_n"], p["vector_io"]) == (256, 256, 3), (tr, p)
        assert p["workspace_bytes"] == copied * plane
        # the copies are priced: the plan costs more than the NT product alone
        assert p["pred_us"] > tg.tg_plan_model(n, n, n, F, tg.TG_NT)["pred_us"]
    assert tg.tg_plan_model(1024, 1024, 1024, F, tg.TG_NN)["vector_io"] == 1
    assert tg.tg_plan_model(300, 200, 100, F, tg.TG_NN)["vector_io"] == 1
    # unaligned float32: both operands copied, padded, laid out for NT
    p = tg.tg_plan_model(4097, 4095, 4099, F, tg.TG_NN)
    assert p["vector_io"] == 3
    kp, mp, np_ = 4100, 4100, 4096
    assert p["workspace_bytes"] >= round256(mp * kp * 4) + round256(np_ * kp * 4)
    # 16-bit products never take the NT copies
    assert tg.tg_plan_model(n, n, n, tg.TG_F16, tg.TG_NN)["vector_io"] == 1
    assert tg.tg_plan_model(4097, 4095, 4099, tg.TG_F16, tg.TG_NN)["vector_io"] == 2
