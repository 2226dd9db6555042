"""FP16-input, FP32-accumulate block-tiled matrix product for MI355X (gfx950).

The compute path is the hand-written HIP library ``libgemm_f16.so`` (C ABI in
``include/gemm_f16.h``).  This package only marshals arguments: torch tensors supply device
memory and the current stream, the library does all the work.  There is no CPU fallback.

    import torch, dense_tiled_gemm_f16_amd as g
    C = g.gemm(A, B)                  # A: (M, K) float16, B: (K, N) float16, on the GPU
    g.gemm(A, B, C, beta=1.0)         # C <- A.B + C in place (C float32)
"""
from __future__ import annotations

import torch

from ._abi import (GEMM_F16_OK, PATH_AUTO, PATH_REGISTER, TILE_128x128, TILE_128x128_K4, TILE_256x128,
                   TILE_256x256, TILE_64x64, TILE_AUTO, TILE_NAMES, GemmError, gemm_f16_f32, gemm_f16_f32_ex,
                   gemm_f16_f32_plan, gemm_f16_f32_plan_tt, gemm_f16_f32_strerror, gemm_f16_f32_tile_order,
                   gemm_f16_f32_splitk, gemm_f16_f32_splitk_choose, gemm_f16_f32_splitk_noalloc,
                   gemm_f16_f32_splitk_workspace, gemm_f16_f32_tt, load, softmax_rows_f32)

__all__ = ["gemm", "gemm_splitk", "gemm_splitk_noalloc", "gemm_f16_f32_splitk_noalloc", "plan", "softmax_rows", "softmax_rows_f32", "gemm_f16_f32", "gemm_f16_f32_tt",
           "gemm_f16_f32_splitk", "gemm_f16_f32_splitk_workspace", "gemm_f16_f32_splitk_choose",
           "gemm_f16_f32_plan_tt", "gemm_f16_f32_ex", "gemm_f16_f32_plan",
           "gemm_f16_f32_tile_order", "gemm_f16_f32_strerror", "GemmError", "load",
           "TILE_AUTO", "TILE_256x256", "TILE_128x128", "TILE_64x64", "TILE_256x128", "TILE_128x128_K4",
           "TILE_NAMES", "PATH_AUTO", "PATH_REGISTER"]


def _ld(t: torch.Tensor) -> int:
    rows, cols = t.shape
    if t.numel() and t.stride(1) != 1:
        raise ValueError("matrices must have a unit column stride (row-major)")
    return max(t.stride(0) if rows > 1 else cols, cols, 1)


def _args(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, trans_a: bool = False, trans_b: bool = False):
    if A.dtype != torch.float16 or B.dtype != torch.float16:
        raise TypeError("A and B must be float16")
    if C.dtype != torch.float32:
        raise TypeError("C must be float32")
    if A.dim() != 2 or B.dim() != 2 or C.dim() != 2:
        raise ValueError("A, B, C must be 2-D")
    M, K = (A.shape[1], A.shape[0]) if trans_a else A.shape
    K2, N = (B.shape[1], B.shape[0]) if trans_b else B.shape
    if K != K2 or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape), tuple(C.shape)))
    for t in (A, B, C):
        if t.numel() and not t.is_cuda:
            raise ValueError("operands must be GPU tensors")
    return M, N, K


def gemm(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor | None = None, beta: float = 0.0,
         opts: dict | str | None = None, stream: torch.cuda.Stream | None = None, trans_a: bool = False,
         trans_b: bool = False, splits: int | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """C <- op(A).op(B) + beta*C on the GPU; returns C (allocated when None).

    splits=None with opts=None: the library's cost model (gemm_f16_f32_splitk_choose) decides
    whether K is split across workgroups.  Skinny and deep-K problems (a few rows or columns, long
    K) then run as gemm_f16_f32_splitk: the product kernel writes partial products into a
    workspace (`workspace`, else one from torch's allocator) and a fixed-order reduction adds them
    into C.  Otherwise, and always with splits=1 or options that override the library's choice
    (a non-empty dict, or a tuned record of one), the call is gemm_f16_f32_tt: one
    launch, or two when the library splits C's rows or columns against wave quantisation (plan()
    shows which).  Either way the result is deterministic.

    trans_a: A is given as the K x M transpose (op(A) = A^T); trans_b: B is given as N x K.
    opts: None (the library chooses), a dict of gemm_f16_f32_opts fields, or "tuned" (the options
    autotune.tune recorded for operands of this shape and layout; the library's choice if none)."""
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        M = A.shape[1] if trans_a else A.shape[0]
        N = B.shape[0] if trans_b else B.shape[1]
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if isinstance(opts, str):
        if opts != "tuned":
            raise ValueError("opts must be None, a dict or 'tuned'")
        from . import autotune
        opts = autotune.tuned_opts(A, B, C, beta) if not (trans_a or trans_b) else None
    if isinstance(opts, dict) and not opts:
        opts = None   # no overrides (also a tuned record whose winner was the library's own call)
    M, N, K = _args(A, B, C, trans_a, trans_b)
    if splits is None:
        splits = gemm_f16_f32_splitk_choose(M, N, K) if opts is None else 1
    if splits > 1:
        return gemm_splitk(A, B, C, splits=splits, beta=beta, workspace=workspace, opts=opts, stream=stream,
                           trans_a=trans_a, trans_b=trans_b)
    s = stream if stream is not None else torch.cuda.current_stream(C.device.index if C.is_cuda else None)
    rc = gemm_f16_f32_tt(trans_a, trans_b, M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), C.data_ptr(),
                         _ld(C), float(beta), s.cuda_stream, opts)
    if rc != GEMM_F16_OK:
        raise GemmError(rc)
    return C


def gemm_splitk(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, splits: int | None = None, beta: float = 0.0,
                workspace: torch.Tensor | None = None, opts: dict | None = None,
                stream: torch.cuda.Stream | None = None, trans_a: bool = False, trans_b: bool = False) -> torch.Tensor:
    """C <- op(A).op(B) + beta*C with K split `splits` ways (gemm_f16_f32_splitk; None: the count
    gemm_f16_f32_splitk_choose gives).  The workspace is a caller-owned device tensor (allocated
    here through torch when None)."""
    M, N, K = _args(A, B, C, trans_a, trans_b)
    if splits is None:
        splits = gemm_f16_f32_splitk_choose(M, N, K)
    need = gemm_f16_f32_splitk_workspace(M, N, splits)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=C.device)
    s = stream if stream is not None else torch.cuda.current_stream(C.device.index if C.is_cuda else None)
    rc = gemm_f16_f32_splitk(trans_a, trans_b, M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), C.data_ptr(),
                             _ld(C), float(beta), int(splits), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), s.cuda_stream, opts)
    if rc != GEMM_F16_OK:
        raise GemmError(rc)
    return C


def gemm_splitk_noalloc(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, splits: int, beta: float = 0.0,
                        opts: dict | None = None, stream: torch.cuda.Stream | None = None, trans_a: bool = False,
                        trans_b: bool = False) -> torch.Tensor:
    """gemm_splitk with the partial products in the library's fixed scratch
    (gemm_f16_f32_splitk_noalloc): nothing is allocated, here or in the library."""
    M, N, K = _args(A, B, C, trans_a, trans_b)
    s = stream if stream is not None else torch.cuda.current_stream(C.device.index if C.is_cuda else None)
    rc = gemm_f16_f32_splitk_noalloc(trans_a, trans_b, M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B),
                                     C.data_ptr(), _ld(C), float(beta), int(splits), s.cuda_stream, opts)
    if rc != GEMM_F16_OK:
        raise GemmError(rc)
    return C


def plan(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, opts: dict | None = None, trans_a: bool = False,
         trans_b: bool = False) -> dict:
    """The launch the library would make for these operands (host only)."""
    M, N, K = _args(A, B, C, trans_a, trans_b)
    rc, p = gemm_f16_f32_plan_tt(trans_a, trans_b, M, N, K, A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), C.data_ptr(),
                                 _ld(C), opts)
    if rc != GEMM_F16_OK:
        raise GemmError(rc)
    return p


def softmax_rows(X: torch.Tensor, Y: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Y <- row softmax of X (float32, M x N, unit column stride) through softmax_rows_f32; Y may be X."""
    if X.dtype != torch.float32 or X.dim() != 2:
        raise TypeError("X must be a 2-D float32 tensor")
    if Y is None:
        Y = torch.empty_like(X, memory_format=torch.contiguous_format)
    if Y.dtype != torch.float32 or tuple(Y.shape) != tuple(X.shape):
        raise ValueError("Y must be float32 with the shape of X")
    M, N = X.shape
    s = stream if stream is not None else torch.cuda.current_stream(X.device.index if X.is_cuda else None)
    rc = softmax_rows_f32(M, N, X.data_ptr(), _ld(X), Y.data_ptr(), _ld(Y), s.cuda_stream)
    if rc != GEMM_F16_OK:
        raise GemmError(rc)
    return Y
