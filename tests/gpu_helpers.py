"""Helpers for the GPU parity tests: place numpy operands in device memory (optionally with padded
rows and NaN guard bands), call the library through its C ABI, and read the result back; the row
softmax's run-and-check pair (rows inside NaN padding, the per-element bound against the oracle)."""
from __future__ import annotations

import numpy as np
import torch

import dense_tiled_gemm_f16_amd as lib
import oracle

GUARD = 4096  # elements of NaN guard band before and after every operand


class DevMat:
    """A row-major matrix inside a device buffer: [guard | rows x ld (padding NaN) | guard].
    ``offset`` shifts the start by that many elements (to break 16-byte alignment)."""

    def __init__(self, x: np.ndarray, ld: int | None = None, offset: int = 0, fill=np.nan):
        rows, cols = x.shape
        self.rows, self.cols = rows, cols
        self.ld = max(ld if ld is not None else cols, cols, 1)
        self.offset = offset
        n = GUARD + offset + max(rows, 1) * self.ld + GUARD
        host = np.full(n, fill, dtype=x.dtype)
        body = host[GUARD + offset: GUARD + offset + rows * self.ld].reshape(rows, self.ld) if rows else None
        if rows:
            body[:, :cols] = x
        self.host_init = host
        self.buf = torch.from_numpy(host).cuda()
        self.ptr = self.buf.data_ptr() + (GUARD + offset) * x.itemsize

    def read(self) -> np.ndarray:
        host = self.buf.cpu().numpy()
        if self.rows == 0:
            return np.zeros((0, self.cols), host.dtype)
        body = host[GUARD + self.offset: GUARD + self.offset + self.rows * self.ld].reshape(self.rows, self.ld)
        return body[:, :self.cols].copy()

    def outside_untouched(self) -> bool:
        """True if every element outside the logical matrix still holds its initial bits."""
        host = self.buf.cpu().numpy()
        mask = np.ones(host.shape, bool)
        if self.rows:
            idx = GUARD + self.offset + (np.arange(self.rows)[:, None] * self.ld + np.arange(self.cols)[None, :])
            mask[idx.ravel()] = False
        a = host[mask].view(np.uint16 if host.dtype == np.float16 else np.uint32)
        b = self.host_init[mask].view(np.uint16 if host.dtype == np.float16 else np.uint32)
        return bool(np.array_equal(a, b))


def run(A: np.ndarray, B: np.ndarray, C: np.ndarray | None = None, beta: float = 0.0, opts=None,
        lda=None, ldb=None, ldc=None, offs=(0, 0, 0), c_fill=np.nan, check_guards=True,
        trans_a: bool = False, trans_b: bool = False, splits: int | None = None, library=None) -> np.ndarray:
    """C_out = A.B + beta*C through gemm_f16_f32_tt (or gemm_f16_f32_splitk when `splits` is given,
    with a NaN-filled workspace inside guard bands); checks that nothing outside C was written.

    A (M x K) and B (K x N) are the mathematical operands; with trans_a / trans_b they are stored
    transposed (K x M / N x K) and passed with the transpose flag.  `library`: another build of the
    same C ABI (a ctypes library from _abi.load_variant) to call instead of the product library."""
    M, K = A.shape
    N = B.shape[1]
    dA = DevMat(np.ascontiguousarray(A.T) if trans_a else A, lda, offs[0])
    dB = DevMat(np.ascontiguousarray(B.T) if trans_b else B, ldb, offs[1])
    C0 = C if C is not None else np.full((M, N), c_fill, np.float32)
    dC = DevMat(C0.astype(np.float32), ldc, offs[2])
    stream = torch.cuda.current_stream().cuda_stream
    if library is not None:
        from dense_tiled_gemm_f16_amd import _abi
        rc = library.gemm_f16_f32_tt(int(trans_a), int(trans_b), M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr, dC.ld,
                                     float(beta), stream, _abi._opts(opts))
    elif splits is None:
        rc = lib.gemm_f16_f32_tt(trans_a, trans_b, M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr, dC.ld, float(beta),
                                 stream, opts)
    else:
        need = lib.gemm_f16_f32_splitk_workspace(M, N, splits)
        dW = DevMat(np.full((1, max(need // 4, 1)), np.nan, np.float32))
        rc = lib.gemm_f16_f32_splitk(trans_a, trans_b, M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr, dC.ld,
                                     float(beta), splits, dW.ptr, need, stream, opts)
    assert rc == 0, lib.gemm_f16_f32_strerror(rc)
    torch.cuda.synchronize()
    if splits is not None and check_guards:
        assert dW.outside_untouched(), "write outside the workspace"
    if check_guards:
        assert dC.outside_untouched(), "write outside C"
        assert dA.outside_untouched() and dB.outside_untouched()
    return dC.read()


# ---------------------------------------------------------------- row softmax
U = 2.0 ** -24


def softmax_run(x, ldx=None, ldy=None, offs=(0, 0), inplace=False):
    """Row softmax of host matrix x through the library, X and Y placed `offs` elements into
    NaN-filled buffers with row strides ldx, ldy (Y = X when inplace); checks that nothing outside
    Y's rows was written and returns Y."""
    M, N = x.shape
    ldx = ldx or N
    ldy = ldy or N
    bx = torch.full((M * ldx + offs[0] + 8,), float("nan"), dtype=torch.float32, device="cuda")
    X = bx[offs[0]:offs[0] + M * ldx].view(M, ldx)[:, :N]
    X.copy_(torch.from_numpy(x))
    if inplace:
        Y, by = X, bx
    else:
        by = torch.full((M * ldy + offs[1] + 8,), float("nan"), dtype=torch.float32, device="cuda")
        Y = by[offs[1]:offs[1] + M * ldy].view(M, ldy)[:, :N]
    lib.softmax_rows(X, Y)
    torch.cuda.synchronize()
    out = Y.cpu().numpy()
    full = by.cpu().numpy()
    mask = np.ones(full.shape, bool)
    base = offs[1] if not inplace else offs[0]
    ld = ldy if not inplace else ldx
    for i in range(M):
        mask[base + i * ld: base + i * ld + N] = False
    assert np.all(np.isnan(full[mask])), "write outside Y"
    return out


def softmax_check(x, y):
    """Per element |y - y_oracle| <= y_oracle (N + 2R + 16) 2^-24 + 1e-37, R the row's largest
    |x - max| (the FP32 roundings of x - max, exp, the row sum and the scaling); returns the
    largest error."""
    ref = oracle.softmax_rows(x)
    xd = x.astype(np.float64)
    R = (xd.max(1, keepdims=True) - xd).max(1, keepdims=True)
    tol = ref * (x.shape[1] + 2 * R + 16) * U + 1e-37
    assert np.all(np.isfinite(y)), "non-finite output"
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= tol), float(np.max(err / tol))
    return float(np.max(err))
