"""GPU parity on randomly drawn problems: shapes, strides, misalignment, layouts, beta, tile, load
path and split-K drawn together from one seeded generator, each call against the FP64 oracle; and
row softmax problems drawn the same way (row count and length, strides, alignment, in place).
Large problems (multi-wave grids, row and column splits into two launches) are drawn separately
and compared on stratified rows and columns.

The directed tests take one feature at a time; these cases cross them (an NT product on the
register path with a padded, misaligned C and a forced tile, split three ways, ...).  Every
operand sits inside NaN guard bands with NaN row padding (tests/gpu_helpers.py), so a read of
padding or a write outside C or the workspace shows up.  Bar: max |C_gpu - C_oracle| <= 1e-4 sqrt(K)
for N(0,1) inputs; with beta = 0, C starts NaN-filled and must not be read.
"""
import numpy as np
import pytest

import oracle
from gemm_inputs import normal_problem
from tolerance import max_abs_err, tol_normal

CASES = 1000
SEED = 4242


def _log_uniform(rng, lo, hi):
    return int(round(np.exp(rng.uniform(np.log(lo), np.log(hi)))))


def _draw(i):
    rng = np.random.default_rng(SEED + i)
    M = _log_uniform(rng, 1, 1500)
    N = _log_uniform(rng, 1, 1500)
    K = _log_uniform(rng, 1, 5000)
    ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
    pads = (0, 0, 1, 3, 8, 13)
    lda = (M if ta else K) + int(rng.choice(pads))
    ldb = (K if tb else N) + int(rng.choice(pads))
    ldc = N + int(rng.choice(pads))
    offs = (int(rng.choice((0, 0, 1, 3, 8))), int(rng.choice((0, 0, 2, 5, 8))), int(rng.choice((0, 0, 1, 3))))
    beta = float(rng.choice((0.0, 0.0, 1.0, -0.5)))
    route = int(rng.integers(4))
    opts, splits = None, None
    if route == 1:
        opts = {"tile": int(rng.integers(1, 6))}
    elif route == 2:
        opts = {"tile": int(rng.integers(0, 6)), "path": 1}
    elif route == 3:
        splits = int(rng.integers(1, 10))
        if rng.integers(2):
            opts = {"tile": int(rng.integers(1, 6))}
    return dict(M=M, N=N, K=K, ta=ta, tb=tb, lda=lda, ldb=ldb, ldc=ldc, offs=offs, beta=beta, opts=opts,
                splits=splits)


def test_draws_cover_the_features():
    """The seeded draws reach every layout, every tile, both load paths, split-K, beta != 0 and
    misaligned operands (a check on the case list itself)."""
    cs = [_draw(i) for i in range(CASES)]
    assert {(c["ta"], c["tb"]) for c in cs} == {(False, False), (False, True), (True, False), (True, True)}
    assert {c["opts"]["tile"] for c in cs if c["opts"] and c["opts"].get("tile")} == {1, 2, 3, 4, 5}
    assert any(c["opts"] and c["opts"].get("path") == 1 for c in cs)
    assert sum(c["splits"] is not None and c["splits"] > 1 for c in cs) >= 10
    assert any(c["beta"] != 0.0 for c in cs) and any(c["beta"] == 0.0 for c in cs)
    assert any(c["offs"][0] % 8 for c in cs) and any(c["offs"][1] % 8 for c in cs) and any(c["offs"][2] for c in cs)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(CASES))
def test_random_case(i):
    from gpu_helpers import run
    c = _draw(i)
    print("case random", i, c, flush=True)
    A, B, C = normal_problem(c["M"], c["N"], c["K"], 5000 + i, with_c=True)
    D = oracle.gemm(A, B, beta=c["beta"], C=C)
    out = run(A, B, C if c["beta"] != 0.0 else None, beta=c["beta"], opts=c["opts"], lda=c["lda"], ldb=c["ldb"],
              ldc=c["ldc"], offs=c["offs"], trans_a=c["ta"], trans_b=c["tb"], splits=c["splits"])
    assert np.all(np.isfinite(out)), "non-finite output"
    err = max_abs_err(out, D)
    assert err <= tol_normal(c["K"]), (err, tol_normal(c["K"]))


SOFTMAX_CASES = 300


def _draw_softmax(i):
    """Rows, row length (1 to 200000, at most 2^23 elements in all), padded strides, starts off
    16-byte alignment, in place or not, value scale."""
    rng = np.random.default_rng(SEED + 100000 + i)
    N = _log_uniform(rng, 1, 200000)
    M = min(_log_uniform(rng, 1, 3000), max(1, (1 << 23) // N))
    pads = (0, 0, 0, 1, 3, 4, 8)
    ldx = N + int(rng.choice(pads))
    ldy = N + int(rng.choice(pads))
    offs = (int(rng.choice((0, 0, 1, 2, 3, 4))), int(rng.choice((0, 0, 1, 2, 3, 4))))
    inplace = bool(rng.random() < 0.2)
    scale = float(rng.choice((1.0, 1.0, 10.0, 80.0)))
    return dict(M=M, N=N, ldx=ldx, ldy=ldy, offs=offs, inplace=inplace, scale=scale)


def test_softmax_draws_cover_the_kernels():
    """Row lengths in every kernel band (wave per row up to 2048, four-, eight- and sixteen-wave
    blocks, the hybrid past 65536), row counts that fill several workgroups, aligned and
    misaligned starts, in place (a check on the case list itself)."""
    cs = [_draw_softmax(i) for i in range(SOFTMAX_CASES)]
    ns = [c["N"] for c in cs]
    for lo, hi in ((1, 2048), (2049, 8192), (8193, 32768), (32769, 65536), (65537, 200000)):
        assert any(lo <= n <= hi for n in ns), (lo, hi)
    assert any(c["M"] > 256 for c in cs)
    assert any(c["offs"][0] % 4 for c in cs) and any(c["inplace"] for c in cs)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(SOFTMAX_CASES))
def test_random_softmax_case(i):
    from gpu_helpers import softmax_check as _check, softmax_run as _run
    c = _draw_softmax(i)
    print("case random softmax", i, c, flush=True)
    x = (np.random.default_rng(7000 + i).standard_normal((c["M"], c["N"])) * c["scale"]).astype(np.float32)
    if c["inplace"]:
        _check(x, _run(x, ldx=c["ldx"], offs=(c["offs"][0], 0), inplace=True))
    else:
        _check(x, _run(x, ldx=c["ldx"], ldy=c["ldy"], offs=c["offs"]))


LARGE_CASES = 24


def _draw_large(i):
    """Large problems: grids of several waves, where the library may split rows or columns into
    two launches; layout, strides, misalignment and beta drawn as above; the library's own choice
    of tile and path, or a forced tile."""
    rng = np.random.default_rng(SEED + 200000 + i)
    M = _log_uniform(rng, 1000, 6000)
    N = _log_uniform(rng, 1000, 6000)
    K = _log_uniform(rng, 64, 2048)
    ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
    pads = (0, 0, 0, 1, 8)
    lda = (M if ta else K) + int(rng.choice(pads))
    ldb = (K if tb else N) + int(rng.choice(pads))
    ldc = N + int(rng.choice(pads))
    offs = (int(rng.choice((0, 0, 0, 1))), int(rng.choice((0, 0, 0, 3))), int(rng.choice((0, 0, 1))))
    beta = float(rng.choice((0.0, 1.0)))
    opts = None if rng.random() < 0.6 else {"tile": int(rng.integers(1, 6))}
    return dict(M=M, N=N, K=K, ta=ta, tb=tb, lda=lda, ldb=ldb, ldc=ldc, offs=offs, beta=beta, opts=opts)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(LARGE_CASES))
def test_random_large_case(i):
    from gpu_helpers import run
    from sampling import strata
    c = _draw_large(i)
    print("case random large", i, c, flush=True)
    A, B, C = normal_problem(c["M"], c["N"], c["K"], 9000 + i, with_c=True)
    out = run(A, B, C if c["beta"] != 0.0 else None, beta=c["beta"], opts=c["opts"], lda=c["lda"], ldb=c["ldb"],
              ldc=c["ldc"], offs=c["offs"], trans_a=c["ta"], trans_b=c["tb"])
    assert np.all(np.isfinite(out)), "non-finite output"
    rows, cols = strata(c["M"]), strata(c["N"])
    Cr = np.ascontiguousarray(C[rows]) if c["beta"] != 0.0 else None
    Cc = np.ascontiguousarray(C[:, cols]) if c["beta"] != 0.0 else None
    assert max_abs_err(out[rows], oracle.gemm(np.ascontiguousarray(A[rows]), B, beta=c["beta"], C=Cr)) <= tol_normal(c["K"])
    assert max_abs_err(out[:, cols], oracle.gemm(A, np.ascontiguousarray(B[:, cols]), beta=c["beta"], C=Cc)) <= \
        tol_normal(c["K"])
