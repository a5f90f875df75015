"""Python binding of libtg_gemm.so, the gfx950 GEMM library.

Argument marshalling only: every step of a product runs in the library's HIP
kernels.  The raw functions carry the C ABI's names and arguments (device
pointers as integers); ``gemm`` derives sizes, leading dimensions and the
stream from torch tensors.  PyTorch supplies device memory and streams.

The library must have been built (``python -m tiled_gemm_02_amd.build``);
nothing here falls back to another implementation when it is missing.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtg_gemm.so")

TG_F32, TG_F16, TG_BF16 = 0, 1, 2
TG_NN, TG_TN, TG_NT, TG_TT = 0, 1, 2, 3
TG_TRANS_A, TG_TRANS_B = 1, 2
TG_EPI_NONE, TG_EPI_LEAKY_RELU = 0, 1
TG_OK, TG_ERR_ARG, TG_ERR_NULL, TG_ERR_UNSUPPORTED, TG_ERR_DEVICE, TG_ERR_LAUNCH = 0, -1, -2, -3, -4, -5
TG_PATH_AUTO, TG_PATH_NONE, TG_PATH_MFMA, TG_PATH_SKINNY, TG_PATH_GEMV = -1, 0, 1, 2, 3
PATH_NAMES = {TG_PATH_NONE: "none", TG_PATH_MFMA: "mfma", TG_PATH_SKINNY: "skinny",
              TG_PATH_GEMV: "gemv"}


class TgError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"tg error {code}: {msg}")
        self.code = code


TG_EPI_SCALE = 1   # tg_epilogue.flags: use alpha and beta
TG_SPLIT_STREAM_K = -1   # tg_options.split_k: stream-K


class Epilogue(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_uint32), ("slope", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float)]


class Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("k_groups", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("occupancy", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("vector_io", ctypes.c_int32), ("tiles", ctypes.c_int64),
                ("workgroups", ctypes.c_int64), ("waves", ctypes.c_int64),
                ("tile_eff", ctypes.c_double), ("wave_eff", ctypes.c_double),
                ("pred_eff", ctypes.c_double), ("pred_us", ctypes.c_double),
                ("arith_intensity", ctypes.c_double), ("workspace_bytes", ctypes.c_uint64),
                ("k_groups", ctypes.c_int32)]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["path_name"] = PATH_NAMES.get(self.path, str(self.path))
        return d


_lib = None


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tiled_gemm_02_amd.build`")
    # PyTorch ships its own HIP runtime under the same soname as the system's.
    # Imported first, it is the runtime this library binds to, so torch's
    # allocations, streams and graph captures and this library's launches share
    # one runtime.  Loaded the other way round, the process would hold two
    # runtimes and torch would find no device.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - the library also runs without torch
        pass
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    ep, op, pp = ctypes.POINTER(Epilogue), ctypes.POINTER(Options), ctypes.POINTER(Plan)
    lib.tg_gemm.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, i32, ep, vp]
    lib.tg_gemm.restype = i32
    lib.tg_gemm_ex.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, i32, ep, op, vp,
                               ctypes.c_size_t, vp]
    lib.tg_gemm_ex.restype = i32
    lib.tg_autotune.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, i32, ep, vp,
                                ctypes.c_size_t, vp, i32, op, ctypes.POINTER(ctypes.c_float)]
    lib.tg_autotune.restype = i32
    lib.tg_gemm_noalloc.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, i32, ep, op, vp]
    lib.tg_gemm_noalloc.restype = i32
    lib.tg_gemm_plan.argtypes = [i64, i64, i64, i32, i32, op, pp]
    lib.tg_gemm_plan.restype = i32
    lib.tg_plan_model.argtypes = [i64, i64, i64, i32, i32, i32, i32, op, pp]
    lib.tg_plan_model.restype = i32
    lib.tg_workspace_size.argtypes = [i64, i64, i64, i32, i32, op]
    lib.tg_workspace_size.restype = ctypes.c_size_t
    lib.tg_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    lib.tg_workspace_bytes.restype = ctypes.c_size_t
    lib.tg_set_workspace.argtypes = [vp, ctypes.c_size_t]
    lib.tg_set_workspace.restype = i32
    lib.tg_softmax.argtypes = [i64, i64, vp, i64, vp, i64, i32, vp]
    lib.tg_softmax.restype = i32
    lib.tg_softmax_shape.argtypes = [i64, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.tg_softmax_shape.restype = i32
    lib.tg_tune_cache_clear.argtypes = []
    lib.tg_tune_cache_clear.restype = i32
    lib.tg_tune_cache_size.argtypes = []
    lib.tg_tune_cache_size.restype = i64
    lib.tg_device_cus.argtypes = []
    lib.tg_device_cus.restype = i32
    lib.tg_last_error.argtypes = []
    lib.tg_last_error.restype = ctypes.c_char_p
    lib.tg_version.argtypes = []
    lib.tg_version.restype = i32
    _lib = lib
    return lib


def _check(rc: int) -> int:
    if rc != TG_OK:
        raise TgError(rc, tg_last_error())
    return rc


def _epi(epilogue, alpha=1.0, beta=0.0) -> ctypes.POINTER(Epilogue) | None:
    """tg_epilogue for (kind or (kind, slope) or "leaky_relu"/"none" or None, alpha, beta)."""
    scaled = alpha != 1.0 or beta != 0.0
    if isinstance(epilogue, Epilogue):
        return ctypes.pointer(epilogue)
    if epilogue is None and not scaled:
        return None
    if epilogue is None:
        kind, slope = TG_EPI_NONE, 0.0
    elif isinstance(epilogue, tuple):
        kind, slope = epilogue
    elif epilogue in ("leaky_relu", TG_EPI_LEAKY_RELU):
        kind, slope = TG_EPI_LEAKY_RELU, 0.01
    elif epilogue in ("none", TG_EPI_NONE):
        kind, slope = TG_EPI_NONE, 0.0
    else:
        raise ValueError(f"unknown epilogue {epilogue!r}")
    if kind == "leaky_relu":
        kind = TG_EPI_LEAKY_RELU
    return ctypes.pointer(Epilogue(int(kind), float(slope), TG_EPI_SCALE if scaled else 0,
                                   float(alpha), float(beta)))


def _opts(options) -> ctypes.POINTER(Options) | None:
    if options is None:
        return None
    if isinstance(options, Options):
        return ctypes.pointer(options)
    o = Options(TG_PATH_AUTO, 0, 0, 0, 0)
    for k, v in dict(options).items():
        if k == "path" and isinstance(v, str):
            v = {n: c for c, n in PATH_NAMES.items()}[v]
        setattr(o, k, int(v))
    return ctypes.pointer(o)


# ---------------------------------------------------------------- raw C-ABI mirrors

def tg_gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, epilogue=None, stream=None) -> int:
    """Raw call: device pointers as integers; returns the status (does not raise)."""
    return load().tg_gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, _epi(epilogue), stream)


def tg_softmax(M, N, X, ldx, Y, ldy, dtype, stream=None) -> int:
    """Raw call: device pointers as integers; returns the status (does not raise)."""
    return load().tg_softmax(M, N, X, ldx, Y, ldy, dtype, stream)


def tg_gemm_ex(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, epilogue=None, options=None,
               workspace=None, workspace_bytes=0, stream=None) -> int:
    return load().tg_gemm_ex(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, _epi(epilogue),
                             _opts(options), workspace, workspace_bytes, stream)


def tg_gemm_noalloc(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, epilogue=None, options=None,
                    stream=None) -> int:
    """Raw call of the entry point that allocates nothing (its workspace is the
    library's static scratch); returns the status (does not raise)."""
    return load().tg_gemm_noalloc(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, _epi(epilogue),
                                  _opts(options), stream)


def tg_gemm_plan(M, N, K, dtype, trans=TG_NN, options=None) -> dict:
    p = Plan()
    _check(load().tg_gemm_plan(M, N, K, dtype, trans, _opts(options), ctypes.byref(p)))
    return p.as_dict()


def tg_plan_model(M, N, K, dtype, trans=TG_NN, num_cus=256, occupancy=0, options=None) -> dict:
    p = Plan()
    _check(load().tg_plan_model(M, N, K, dtype, trans, num_cus, occupancy, _opts(options),
                                ctypes.byref(p)))
    return p.as_dict()


def tg_workspace_size(M, N, K, dtype, trans=TG_NN, options=None) -> int:
    return int(load().tg_workspace_size(M, N, K, dtype, trans, _opts(options)))


def tg_workspace_bytes(M, N, K, dtype, trans=TG_NN) -> int:
    return int(load().tg_workspace_bytes(M, N, K, dtype, trans))


def tg_set_workspace(ptr, nbytes: int) -> int:
    return _check(load().tg_set_workspace(ptr, nbytes))


def tg_device_cus() -> int:
    return int(load().tg_device_cus())


def tg_last_error() -> str:
    return load().tg_last_error().decode()


def tg_version() -> int:
    return int(load().tg_version())


# ---------------------------------------------------------------- torch convenience

def _torch_dtype_code(t) -> int:
    import torch
    m = {torch.float32: TG_F32, torch.float16: TG_F16, torch.bfloat16: TG_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ld(t) -> int:
    """Leading dimension (row stride, elements) of a row-major 2-D tensor.

    Rows must not overlap: a row stride below the row width (an expanded or
    overlapping view) is refused, since the kernels address row r at r * ld."""
    if t.dim() != 2:
        raise ValueError("operands must be 2-D")
    rows, cols = t.shape
    if t.numel() == 0:
        return max(cols, 1)   # no element is addressed; any ld >= the width is valid
    if cols > 1 and t.stride(1) != 1:
        raise ValueError("operands must be row-major (last stride 1); pass a transpose flag instead")
    if rows == 1:
        return max(cols, 1)
    ld = int(t.stride(0))
    if ld < cols:
        raise ValueError(f"row stride {ld} is below the row width {cols}: rows overlap "
                         "(expanded or overlapping views are not supported; make the tensor contiguous)")
    return ld


def _require_cuda(*tensors) -> None:
    """The library reads and writes device memory only: refuse host tensors
    before any pointer reaches a kernel."""
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise TypeError(f"expected a CUDA (device) tensor, got one on {t.device}")


def gemm(A, B, *, trans_a: bool = False, trans_b: bool = False, epilogue=None, out=None,
         alpha: float = 1.0, beta: float = 0.0, options=None, workspace=None, stream=None):
    """C = epilogue(alpha * op(A) . op(B) + beta * C) on the tensors' device.

    A is the stored array: M x K, or K x M when ``trans_a``; B is K x N, or
    N x K when ``trans_b``.  Returns C (M x N, row-major, A's dtype); ``out``
    may be a preallocated (possibly strided) M x N tensor, and holds the old C
    when ``beta`` is not 0 (it is not read when ``beta`` is 0).
    """
    import torch
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    _require_cuda(A, B, out, workspace)
    dtype = _torch_dtype_code(A)
    M, K = (A.shape[1], A.shape[0]) if trans_a else (A.shape[0], A.shape[1])
    Kb, N = (B.shape[1], B.shape[0]) if trans_b else (B.shape[0], B.shape[1])
    if Kb != K:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs out= (the old C)")
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    elif out.shape != (M, N) or out.dtype != A.dtype:
        raise ValueError("out has the wrong shape or dtype")
    trans = (TG_TRANS_A if trans_a else 0) | (TG_TRANS_B if trans_b else 0)
    lda, ldb, ldc = _ld(A), _ld(B), _ld(out)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    ws_ptr, ws_bytes = (None, 0)
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if M == 0 or N == 0:
        return out
    epi = _epi(epilogue, alpha, beta)
    rc = load().tg_gemm_ex(M, N, K, A.data_ptr() if A.numel() else None, lda,
                           B.data_ptr() if B.numel() else None, ldb, out.data_ptr(), ldc,
                           dtype, trans, epi, _opts(options), ws_ptr, ws_bytes, stream)
    _check(rc)
    return out


def softmax(X, *, out=None, stream=None):
    """Row softmax of the 2-D tensor X (tg_softmax): returns Y with Y[i] =
    softmax(X[i]).  Rows may be strided (X.stride(1) must be 1); ``out`` may be
    a preallocated tensor of X's shape and dtype, X itself included (in place)."""
    import torch
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    _require_cuda(X, out)
    dtype = _torch_dtype_code(X)
    M, N = X.shape
    if out is None:
        out = torch.empty((M, N), dtype=X.dtype, device=X.device)
    elif out.shape != X.shape or out.dtype != X.dtype:
        raise ValueError("out has the wrong shape or dtype")
    ldx, ldy = _ld(X), _ld(out)
    if M == 0 or N == 0:
        return out
    if stream is None:
        stream = torch.cuda.current_stream(X.device).cuda_stream
    _check(load().tg_softmax(M, N, X.data_ptr(), ldx, out.data_ptr(), ldy, dtype, stream))
    return out


_ws_keep = threading.local()


def set_workspace(buf) -> None:
    """Make the uint8 device tensor ``buf`` the calling thread's default
    workspace (tg_set_workspace); None clears it.  The tensor is kept alive
    until replaced."""
    if buf is None:
        tg_set_workspace(None, 0)
        _ws_keep.buf = None
        return
    _require_cuda(buf)
    tg_set_workspace(buf.data_ptr(), buf.numel() * buf.element_size())
    _ws_keep.buf = buf


def tune_cache_clear() -> None:
    """Forget the plans tg_autotune recorded on the current device."""
    _check(load().tg_tune_cache_clear())


def tune_cache_size() -> int:
    """Plans tg_autotune has recorded on the current device."""
    n = int(load().tg_tune_cache_size())
    if n < 0:
        _check(n)
    return n


def softmax_shape(N: int, dtype) -> tuple[int, int]:
    """(waves per row, 16-byte chunks per lane) of tg_softmax for rows of N
    elements; (0, 0) = the two-pass long-row kernel."""
    q, c = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().tg_softmax_shape(int(N), int(dtype), ctypes.byref(q), ctypes.byref(c)))
    return q.value, c.value


def autotune(A, B, *, trans_a: bool = False, trans_b: bool = False, epilogue=None, out=None,
             workspace=None, reps: int = 5, stream=None) -> tuple[dict, float]:
    """Time every candidate plan for these operands (tg_autotune) and return
    (options for ``gemm``, mean microseconds of the fastest).  ``out`` (or a
    scratch tensor) is overwritten."""
    import torch
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    _require_cuda(A, B, out, workspace)
    dtype = _torch_dtype_code(A)
    M, K = (A.shape[1], A.shape[0]) if trans_a else (A.shape[0], A.shape[1])
    Kb, N = (B.shape[1], B.shape[0]) if trans_b else (B.shape[0], B.shape[1])
    if Kb != K:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    elif out.shape != (M, N) or out.dtype != A.dtype:
        raise ValueError("out has the wrong shape or dtype")
    trans = (TG_TRANS_A if trans_a else 0) | (TG_TRANS_B if trans_b else 0)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    ws_ptr, ws_bytes = (None, 0)
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    best = Options(TG_PATH_AUTO, 0, 0, 0, 0)
    us = ctypes.c_float(0.0)
    _check(load().tg_autotune(M, N, K, A.data_ptr() if A.numel() else None, _ld(A),
                              B.data_ptr() if B.numel() else None, _ld(B), out.data_ptr(), _ld(out),
                              dtype, trans, _epi(epilogue), ws_ptr, ws_bytes, stream, int(reps),
                              ctypes.byref(best), ctypes.byref(us)))
    opts = dict(path=best.path, tile_m=best.tile_m, tile_n=best.tile_n, split_k=best.split_k,
                k_groups=best.k_groups)
    return opts, float(us.value)


def plan_for(A, B, *, trans_a=False, trans_b=False, options=None) -> dict:
    """The plan ``gemm`` would use for these tensors' shapes (packed operands)."""
    dtype = _torch_dtype_code(A)
    M, K = (A.shape[1], A.shape[0]) if trans_a else (A.shape[0], A.shape[1])
    N = B.shape[0] if trans_b else B.shape[1]
    trans = (TG_TRANS_A if trans_a else 0) | (TG_TRANS_B if trans_b else 0)
    return tg_gemm_plan(M, N, K, dtype, trans, options)
