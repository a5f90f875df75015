"""The C-ABI library: loads, exports every declared symbol, validates arguments
and reports a missing GPU, all without launching anything (CPU only)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import tiled_gemm_02_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "tg_gemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z_]+)\s*\(", src)))


def test_header_declares_entry_points():
    names = _declared_functions()
    for must in ("tg_gemm", "tg_gemm_ex", "tg_gemm_plan", "tg_plan_model", "tg_workspace_size",
                 "tg_workspace_bytes", "tg_set_workspace", "tg_device_cus", "tg_last_error",
                 "tg_version"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tg.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} declared in tg_gemm.h but not exported"


def test_version():
    assert tg.tg_version() == 107


def test_epilogue_struct_matches_header(tmp_path):
    """The binding's tg_epilogue mirror has the header's field offsets and size
    (checked with the host C compiler on the header itself)."""
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "tg_gemm.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(tg_epilogue), '
                   'offsetof(tg_epilogue, kind), offsetof(tg_epilogue, slope), '
                   'offsetof(tg_epilogue, flags), offsetof(tg_epilogue, alpha), '
                   'offsetof(tg_epilogue, beta)); return 0; }\n')
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    E = tg.Epilogue
    assert got == [ctypes.sizeof(E), E.kind.offset, E.slope.offset, E.flags.offset,
                   E.alpha.offset, E.beta.offset]


def test_argument_errors():
    F16 = tg.TG_F16
    # unknown enums
    assert tg.tg_gemm(4, 4, 4, 1, 4, 1, 4, 1, 4, 7, 0) == tg.TG_ERR_ARG
    assert tg.tg_gemm(4, 4, 4, 1, 4, 1, 4, 1, 4, F16, 9) == tg.TG_ERR_ARG
    assert tg.tg_gemm(4, 4, 4, 1, 4, 1, 4, 1, 4, F16, 0, (5, 0.1)) == tg.TG_ERR_ARG
    assert tg.tg_gemm(4, 4, 4, 1, 4, 1, 4, 1, 4, F16, 0, tg.Epilogue(0, 0.0, 6, 1.0, 0.0)) == tg.TG_ERR_ARG
    # negative sizes and short leading dimensions
    assert tg.tg_gemm(-1, 4, 4, 1, 4, 1, 4, 1, 4, F16, 0) == tg.TG_ERR_ARG
    assert tg.tg_gemm(4, 4, 4, 1, 3, 1, 4, 1, 4, F16, 0) == tg.TG_ERR_ARG
    assert "lda" in tg.tg_last_error()
    assert tg.tg_gemm(4, 4, 8, 1, 8, 1, 3, 1, 4, F16, 0) == tg.TG_ERR_ARG
    assert tg.tg_gemm(4, 4, 8, 1, 8, 1, 4, 1, 3, F16, 0) == tg.TG_ERR_ARG
    # transposed operands need ld >= M (A) and >= K (B)
    assert tg.tg_gemm(6, 4, 8, 1, 5, 1, 8, 1, 4, F16, tg.TG_TT) == tg.TG_ERR_ARG
    assert tg.tg_gemm(6, 4, 8, 1, 6, 1, 7, 1, 4, F16, tg.TG_TT) == tg.TG_ERR_ARG
    # NULL operands with elements
    assert tg.tg_gemm(4, 4, 4, None, 4, 1, 4, 1, 4, F16, 0) == tg.TG_ERR_NULL
    assert tg.tg_gemm(4, 4, 4, 1, 4, None, 4, 1, 4, F16, 0) == tg.TG_ERR_NULL
    assert tg.tg_gemm(4, 4, 4, 1, 4, 1, 4, None, 4, F16, 0) == tg.TG_ERR_NULL


def test_quick_returns_need_no_device():
    # M == 0 or N == 0: nothing to do, valid even with NULL operands
    assert tg.tg_gemm(0, 4, 4, None, 4, None, 4, None, 4, tg.TG_F16, 0) == tg.TG_OK
    assert tg.tg_gemm(4, 0, 4, None, 4, None, 1, None, 1, tg.TG_F16, 0) == tg.TG_OK
    assert tg.tg_last_error() == ""


def test_no_device_is_reported():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc = tg.tg_gemm(4, 4, 4, 1, 4, 1, 4, 1, 4, tg.TG_F16, 0)
    assert rc == tg.TG_ERR_DEVICE
    assert tg.tg_device_cus() == tg.TG_ERR_DEVICE
    assert tg.load().tg_tune_cache_size() == tg.TG_ERR_DEVICE
    assert tg.load().tg_tune_cache_clear() == tg.TG_ERR_DEVICE
    with pytest.raises(tg.TgError):
        tg.tg_gemm_plan(64, 64, 64, tg.TG_F16)


def test_plan_model_rejects_bad_input():
    with pytest.raises(tg.TgError):
        tg.tg_plan_model(4, 4, 4, 9)
    with pytest.raises(tg.TgError):
        tg.tg_plan_model(4, 4, 4, tg.TG_F16, num_cus=0)
    with pytest.raises(tg.TgError):
        tg.tg_plan_model(4, 4, 4, tg.TG_F16, options=dict(path=tg.TG_PATH_GEMV))
    with pytest.raises(tg.TgError):
        tg.tg_plan_model(4, 4, 4, tg.TG_F16, options=dict(tile_m=64))


def test_set_workspace_argument_checks():
    """tg_set_workspace needs no device: NULL with a size and a misaligned
    pointer are argument errors; (NULL, 0) clears."""
    with pytest.raises(tg.TgError):
        tg.tg_set_workspace(None, 1024)
    with pytest.raises(tg.TgError):
        tg.tg_set_workspace(0x1000 + 16, 1024)
    assert tg.tg_set_workspace(None, 0) == 0


def _kernel_stubs():
    """Demangled names of the kernel launch stubs the library holds (host side)."""
    import subprocess
    out = subprocess.run(["nm", "-C", tg.LIB_PATH], check=True, capture_output=True, text=True).stdout
    return out


@pytest.mark.parametrize("dtype", ["F16", "BF16"])
def test_every_planned_16bit_tile_has_kernels(dtype):
    """Every macro tile the planner may pick for 16-bit operands has its kernel
    compiled for all four layouts (256 x 256 and 192 x 256: the ping-pong
    kernel; the others: the four-wave LDS-DMA kernel, 128 x 128 also with two
    K groups and 64 x 64 with four), so no plan can reach a launcher without an
    instance."""
    import re
    stubs = _kernel_stubs()
    for bm, bn, kg in [(256, 128, 1), (128, 128, 1), (128, 64, 1), (64, 64, 1), (128, 128, 2), (64, 64, 4)]:
        found = set(re.findall(
            rf"tg::mfma_gemm3_kernel<tg::{dtype}, {bm}, {bn}, \d+, 2, 2, (\w+), (\w+), {kg}, \d+>", stubs))
        assert len(found) == 4, (bm, bn, kg, found)
    # the ping-pong tiles in two forms: whole tile to C (1), K splits and old C (0)
    for bm in (256, 192):
        found = set(re.findall(rf"tg::mfma_pingpong_kernel<tg::{dtype}, \d, 16, (\w+), (\w+), false, {bm}, (\d)>",
                               stubs))
        assert len(found) == (8 if bm == 256 else 4), (bm, found)


def test_every_planned_f32_register_tile_has_kernels():
    """The float32 register-staged tiles the planner may pick (128 x 128 with one
    or two K groups, 64 x 64 with one or four, 32 x 32 with four) exist for all
    four layouts."""
    import re
    stubs = _kernel_stubs()
    for bm, kg in [(128, 1), (128, 2), (64, 1), (64, 4), (32, 4)]:
        found = set(re.findall(rf"tg::mfma_gemm_kernel<tg::F32, {bm}, {bm}, (\w+), (\w+), true, {kg}>", stubs))
        assert len(found) == 4, (bm, kg, found)
