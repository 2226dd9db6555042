"""ctypes binding of libgemm_f16.so: the C entry points under the same names, arguments only.

Every call goes straight to the library; there is no fallback of any kind.  If the library is
missing, loading raises.  torch is imported before the library is loaded so that the process
uses one HIP runtime (the library's libamdhip64 dependency then resolves to the one torch has
already mapped).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime first; see module docstring)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgemm_f16.so")

GEMM_F16_OK = 0
GEMM_F16_ERR_DIM = -1
GEMM_F16_ERR_LD = -2
GEMM_F16_ERR_NULL = -3
GEMM_F16_ERR_OPTS = -4
GEMM_F16_ERR_TOO_LARGE = -5
GEMM_F16_ERR_LAUNCH = -6
GEMM_F16_ERR_ALIGN = -7
GEMM_F16_ERR_WORKSPACE = -8

TILE_AUTO = 0
TILE_256x256 = 1
TILE_128x128 = 2
TILE_64x64 = 3
TILE_256x128 = 4
TILE_128x128_K4 = 5
TILE_NAMES = {1: "256x256", 2: "128x128", 3: "64x64", 4: "256x128", 5: "128x128k4"}
PATH_AUTO = 0
PATH_REGISTER = 1


class gemm_f16_f32_opts(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("xcd_remap", ctypes.c_int32), ("path", ctypes.c_int32)]


class gemm_f16_f32_plan_t(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("bm", ctypes.c_int32), ("bn", ctypes.c_int32),
                ("bk", ctypes.c_int32), ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("group_m", ctypes.c_int32), ("xcd_remap", ctypes.c_int32), ("vec_a", ctypes.c_int32),
                ("vec_b", ctypes.c_int32), ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64),
                ("grid", ctypes.c_int64), ("split_at", ctypes.c_int64), ("tile2", ctypes.c_int32),
                ("split_dim", ctypes.c_int32), ("grid2", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


# (name, argtypes, restype) for every entry point declared in include/gemm_f16.h
_I64, _P, _F32, _I32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int32
SIGNATURES = {
    "gemm_f16_f32": ([_I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _F32, _P], ctypes.c_int),
    "gemm_f16_f32_ex": ([_I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _F32, _P,
                         ctypes.POINTER(gemm_f16_f32_opts)], ctypes.c_int),
    "gemm_f16_f32_plan": ([_I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64,
                           ctypes.POINTER(gemm_f16_f32_opts), ctypes.POINTER(gemm_f16_f32_plan_t)],
                          ctypes.c_int),
    "gemm_f16_f32_tile_order": ([_I64, _I64, _I32, _I32, _I64, _P, _P], ctypes.c_int),
    "gemm_f16_f32_tt": ([_I32, _I32, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _F32, _P,
                         ctypes.POINTER(gemm_f16_f32_opts)], ctypes.c_int),
    "gemm_f16_f32_plan_tt": ([_I32, _I32, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64,
                              ctypes.POINTER(gemm_f16_f32_opts), ctypes.POINTER(gemm_f16_f32_plan_t)], ctypes.c_int),
    "gemm_f16_f32_splitk": ([_I32, _I32, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _F32, _I32, _P,
                             ctypes.c_size_t, _P, ctypes.POINTER(gemm_f16_f32_opts)], ctypes.c_int),
    "gemm_f16_f32_splitk_workspace": ([_I64, _I64, _I32], ctypes.c_size_t),
    "gemm_f16_f32_splitk_noalloc": ([_I32, _I32, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _F32, _I32, _P,
                                     ctypes.POINTER(gemm_f16_f32_opts)], ctypes.c_int),
    "gemm_f16_f32_splitk_choose": ([_I64, _I64, _I64], ctypes.c_int),
    "softmax_rows_f32": ([_I64, _I64, _P, _I64, _P, _I64, _P], ctypes.c_int),
    "gemm_f16_f32_strerror": ([ctypes.c_int], ctypes.c_char_p),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once).  Raises OSError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError("libgemm_f16.so is not built (%s); run python -m dense_tiled_gemm_f16_amd.build" % path)
    lib = ctypes.CDLL(path)
    for name, (argtypes, restype) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    _lib = lib
    return lib


def load_variant(path: str) -> ctypes.CDLL:
    """A separately built library with the same C ABI (e.g. the measurement variant without the LDS
    swizzle), loaded beside the product library and not cached.  Raises OSError if it is missing."""
    if not os.path.exists(path):
        raise OSError("%s is not built; run python -m dense_tiled_gemm_f16_amd.build" % path)
    lib = ctypes.CDLL(path)
    for name, (argtypes, restype) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    return lib


class GemmError(RuntimeError):
    def __init__(self, code: int):
        super().__init__("gemm_f16_f32 error %d: %s" % (code, gemm_f16_f32_strerror(code)))
        self.code = code


def _opts(opts) -> ctypes.POINTER(gemm_f16_f32_opts) | None:
    if opts is None:
        return None
    if isinstance(opts, dict):
        o = gemm_f16_f32_opts(int(opts.get("tile", 0)), int(opts.get("group_m", 0)),
                              int(opts.get("xcd_remap", -1)), int(opts.get("path", 0)))
    else:
        o = opts
    return ctypes.pointer(o)


def gemm_f16_f32(M, N, K, A, lda, B, ldb, C, ldc, beta, stream) -> int:
    """C entry point gemm_f16_f32; pointers and stream are integers (device addresses)."""
    return load().gemm_f16_f32(M, N, K, A, lda, B, ldb, C, ldc, beta, stream)


def gemm_f16_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, beta, stream, opts=None) -> int:
    return load().gemm_f16_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, beta, stream, _opts(opts))


def gemm_f16_f32_tt(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, beta, stream, opts=None) -> int:
    return load().gemm_f16_f32_tt(int(trans_a), int(trans_b), M, N, K, A, lda, B, ldb, C, ldc, beta, stream,
                                  _opts(opts))


def gemm_f16_f32_plan_tt(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, opts=None) -> tuple[int, dict | None]:
    plan = gemm_f16_f32_plan_t()
    rc = load().gemm_f16_f32_plan_tt(int(trans_a), int(trans_b), M, N, K, A, lda, B, ldb, C, ldc, _opts(opts),
                                     ctypes.byref(plan))
    return rc, (plan.as_dict() if rc == 0 else None)


def gemm_f16_f32_splitk(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, beta, splits, workspace, workspace_bytes,
                        stream, opts=None) -> int:
    return load().gemm_f16_f32_splitk(int(trans_a), int(trans_b), M, N, K, A, lda, B, ldb, C, ldc, beta, splits,
                                      workspace, workspace_bytes, stream, _opts(opts))


def gemm_f16_f32_splitk_noalloc(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, beta, splits, stream,
                                opts=None) -> int:
    """C entry point gemm_f16_f32_splitk_noalloc (split-K with the library's fixed scratch)."""
    return load().gemm_f16_f32_splitk_noalloc(int(trans_a), int(trans_b), M, N, K, A, lda, B, ldb, C, ldc, beta,
                                              splits, stream, _opts(opts))


SCRATCH_BYTES = 32 << 20   # GEMM_F16_SCRATCH_BYTES


def gemm_f16_f32_splitk_workspace(M, N, splits) -> int:
    return int(load().gemm_f16_f32_splitk_workspace(M, N, splits))


def gemm_f16_f32_splitk_choose(M, N, K) -> int:
    return int(load().gemm_f16_f32_splitk_choose(M, N, K))


def gemm_f16_f32_plan(M, N, K, A, lda, B, ldb, C, ldc, opts=None) -> tuple[int, dict | None]:
    plan = gemm_f16_f32_plan_t()
    rc = load().gemm_f16_f32_plan(M, N, K, A, lda, B, ldb, C, ldc, _opts(opts), ctypes.byref(plan))
    return rc, (plan.as_dict() if rc == 0 else None)


def gemm_f16_f32_tile_order(tiles_m, tiles_n, group_m, xcd_remap, count=None):
    """(rc, pid_m list, pid_n list) for workgroups 0..count-1."""
    count = tiles_m * tiles_n if count is None else count
    pm = (ctypes.c_int64 * max(count, 1))()
    pn = (ctypes.c_int64 * max(count, 1))()
    rc = load().gemm_f16_f32_tile_order(tiles_m, tiles_n, group_m, xcd_remap, count,
                                         ctypes.cast(pm, ctypes.c_void_p), ctypes.cast(pn, ctypes.c_void_p))
    return rc, list(pm[:count]), list(pn[:count])


def softmax_rows_f32(M, N, X, ldx, Y, ldy, stream) -> int:
    """C entry point softmax_rows_f32; pointers and stream are integers (device addresses)."""
    return load().softmax_rows_f32(M, N, X, ldx, Y, ldy, stream)


def gemm_f16_f32_strerror(code: int) -> str:
    return load().gemm_f16_f32_strerror(code).decode()
