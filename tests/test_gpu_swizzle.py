"""The LDS XOR swizzle changes where data sits in LDS, not what is computed (04_tensor_cores.py,
CS349E lecture 10, "Tensor Core kernels", demo 2 observations: the swizzled and plain layouts give
the same errors).  A variant of the library built with the swizzle off (every panel row's chunks
in order; libgemm_f16_noswizzle.so, measurement only) must give the product library's bits on
every tile, layout and staging path, on ragged shapes with a K tail, and both must match the
oracle."""
import numpy as np
import pytest

import oracle
from gemm_inputs import normal_problem
from tolerance import max_abs_err, tol_normal

pytestmark = pytest.mark.gpu

TILES = (1, 2, 3, 4, 5)
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


@pytest.fixture(scope="module")
def plain_lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dense_tiled_gemm_f16_amd as lib
    from dense_tiled_gemm_f16_amd import _abi, build
    lib.load()
    return _abi.load_variant(build.NOSWIZZLE_LIB_PATH)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(300, 200, 150), (1000, 1100, 704), (129, 65, 33), (513, 257, 192)])
def test_swizzle_off_gives_the_same_bits(plain_lib, ta, tb, shape):
    from gpu_helpers import run
    M, N, K = shape
    print("case swizzle", shape, ta, tb, flush=True)
    A, B, C = normal_problem(M, N, K, 2100 + M + K, with_c=True)
    D = oracle.gemm(A, B, beta=1.0, C=C)
    for tile in TILES:
        for path in (0, 1):
            opts = {"tile": tile, "path": path}
            ref = run(A, B, C, beta=1.0, opts=opts, trans_a=ta, trans_b=tb)
            out = run(A, B, C, beta=1.0, opts=opts, trans_a=ta, trans_b=tb, library=plain_lib)
            assert np.array_equal(out, ref), (tile, path)
            assert max_abs_err(out, D) <= tol_normal(K), (tile, path)
