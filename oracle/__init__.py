"""Reference oracles for the FP16-input, FP32-output matrix product and the row softmax.
TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The GPU library never calls it, and it shares no code with the GPU library:
the arithmetic lives in ``oracle_gemm.c`` and ``oracle_softmax.c`` (plain C, built with gcc), and
this module only builds them, loads them with ctypes and marshals numpy arrays.  The row softmax
oracle and its pins are described in ``oracle_softmax.c`` and tests/test_softmax_oracle_pins.py.

The oracle computes the definition of the product,

    D[i, j] = sum_{k ascending} double(A[i, k]) * double(B[k, j])  +  beta * Cin[i, j],

in FP64, which is the high-precision reference the pages compare their tensor-core and block
kernels against (04_tensor_cores.py, demos 1-2; 06_triton_style.py, demos 1 and 4).

Pins (tests/test_oracle_pins.py) tie it to things outside itself: exact rational arithmetic on
16x8x16 tiles, A.I = A and I.B = B, linearity and power-of-two scaling, numpy's binary16 decoding
over all 65536 patterns, an FP64 library product within its error bound, the pages' fact that
FP16 x FP16 products are exact in FP32 (checked over every finite pair), and the error levels the
pages print for one tensor-core instruction and for FP16 vs FP32 accumulation.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_SRC_SOFTMAX = os.path.join(_HERE, "oracle_softmax.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_gemm.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle_gemm.c and oracle_softmax.c with gcc into liboracle_gemm.so next to them."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-shared", "-fPIC", _SRC, _SRC_SOFTMAX, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm.argtypes = [i64, i64, i64, p, i64, p, i64, ctypes.c_double, p, i64, p, i64]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_count_inexact_f16_products.argtypes = [ctypes.POINTER(ctypes.c_int64)]
    lib.oracle_count_inexact_f16_products.restype = ctypes.c_int64
    lib.oracle_count_inexact_products.argtypes = [p, i64, p, i64]
    lib.oracle_count_inexact_products.restype = ctypes.c_int64
    lib.oracle_softmax_rows.argtypes = [i64, i64, p, i64, p, i64]
    lib.oracle_softmax_rows.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None) -> int | None:
    return None if a is None else a.ctypes.data


def gemm(A: np.ndarray, B: np.ndarray, beta: float = 0.0, C: np.ndarray | None = None) -> np.ndarray:
    """FP64 result of A.B + beta*C for float16 A (M x K) and B (K x N), float32 C (M x N).

    Row-major arrays with a unit column stride are accepted as they are (row strides are passed
    through, so slices of larger arrays work); anything else is copied to a contiguous array.
    """
    if A.dtype != np.float16 or B.dtype != np.float16:
        raise TypeError("oracle.gemm takes float16 A and B")
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError("shape mismatch: A %s, B %s" % (A.shape, B.shape))
    M, K = A.shape
    N = B.shape[1]
    A = _rowmajor(A)
    B = _rowmajor(B)
    lda = A.strides[0] // 2 if M > 0 else max(K, 1)
    ldb = B.strides[0] // 2 if K > 0 else max(N, 1)
    lda = max(lda, K, 1)
    ldb = max(ldb, N)
    Cp, ldc = None, N
    if beta != 0.0:
        if C is None or C.shape != (M, N) or C.dtype != np.float32:
            raise ValueError("beta != 0 needs a float32 C of shape (M, N)")
        C = _rowmajor(C)
        Cp, ldc = C, (max(C.strides[0] // 4, N) if M > 0 else N)
    D = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm(M, N, K, _ptr(A), lda, _ptr(B), ldb, float(beta), _ptr(Cp), ldc,
                             _ptr(D), N)
    if rc != 0:
        raise RuntimeError("oracle_gemm failed with code %d" % rc)
    return D


def softmax_rows(x: np.ndarray) -> np.ndarray:
    """FP64 row softmax of a float32 (M x N) array (oracle_softmax.c)."""
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError("oracle.softmax_rows takes a 2-D float32 array")
    M, N = x.shape
    x = _rowmajor(x)
    ldx = max(x.strides[0] // 4, N, 1) if M > 0 else max(N, 1)
    y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_softmax_rows(M, N, _ptr(x), ldx, _ptr(y), max(N, 1))
    if rc != 0:
        raise RuntimeError("oracle_softmax_rows failed with code %d" % rc)
    return y


def _rowmajor(x: np.ndarray) -> np.ndarray:
    if x.size == 0:
        return np.ascontiguousarray(x)
    if x.strides[1] == x.itemsize and x.strides[0] >= x.shape[1] * x.itemsize and x.strides[0] % x.itemsize == 0:
        return x
    return np.ascontiguousarray(x)


def f16_to_f64(bits: int) -> float:
    """The oracle's own decoding of one binary16 bit pattern."""
    return _load().oracle_f16_to_f64(bits & 0xFFFF)


def count_inexact_f16_products() -> tuple[int, int]:
    """(pairs whose FP32 product is inexact, pairs checked) over every pair of finite binary16 values."""
    checked = ctypes.c_int64(0)
    bad = _load().oracle_count_inexact_f16_products(ctypes.byref(checked))
    return int(bad), int(checked.value)


def count_inexact_products(x: np.ndarray, y: np.ndarray) -> int:
    """Pairs (x[i], y[j]) whose FP32 product is inexact, through the same routine as the FP16 scan
    (the control for count_inexact_f16_products).  Values must be exact FP32 numbers."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    n = _load().oracle_count_inexact_products(_ptr(x), x.size, _ptr(y), y.size)
    if n < 0:
        raise ValueError("count_inexact_products takes finite FP32-representable values")
    return int(n)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())
