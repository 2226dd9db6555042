"""The library inside captured HIP graphs and on concurrent streams.

Every entry point launches its kernels on the caller's stream, synchronizes nothing and records no
memset, so its calls can be captured into a graph and replayed, and calls on different streams can
run at the same time.  Checks:

- graphs: each case is captured once and replayed several times, with the output overwritten by
  NaN before every replay and the program's own eager work (other library calls, a
  synchronization) between replays; every replay must give the eager call's bits, and the eager
  result meets the oracle's bar (1e-4 sqrt(K) for N(0,1) GEMM inputs, the softmax bound of
  test_gpu_softmax);
- streams: several different calls are issued on four streams without waiting in between; the
  results must equal, bit for bit, the same calls made one after another.
"""
import sys

import numpy as np
import pytest

import oracle
from gemm_inputs import normal_problem
from sampling import strata
from tolerance import max_abs_err, tol_normal

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dense_tiled_gemm_f16_amd as lib
    lib.load()
    yield


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _bits(t):
    import torch
    return t.contiguous().view(torch.int32).cpu().numpy()


def _gemm_case(name):
    """(launch, output tensor, oracle check) for one GEMM case; launch() writes the output in full."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    if name == "plain beta 1":
        M, N, K = 700, 900, 1000
        A, B, C = normal_problem(M, N, K, 301, with_c=True)
        dA, dB, dC0 = _dev(A), _dev(B), _dev(C)
        dC = torch.empty_like(dC0)

        def launch():
            dC.copy_(dC0)
            lib.gemm(dA, dB, dC, beta=1.0)

        return launch, dC, lambda out: _check_rows(out, A, B, K, 1.0, C)
    if name == "two launches (row split)":
        M, N, K = 4352, 4352, 512
        A, B, _ = normal_problem(M, N, K, 302)
        dA, dB = _dev(A), _dev(B)
        dC = torch.empty(M, N, dtype=torch.float32, device="cuda")
        p = lib.plan(dA, dB, dC)
        assert p["split_at"] < M and p["grid2"] > 0, p   # the case must exercise the second launch
        return (lambda: lib.gemm(dA, dB, dC)), dC, lambda out: _check_rows(out, A, B, K)
    if name == "register path, unaligned rows":
        M, N, K = 513, 257, 1001
        A, B, _ = normal_problem(M, N, K, 303)
        dA, dB = _dev(A), _dev(B)
        dC = torch.empty(M, N, dtype=torch.float32, device="cuda")
        return (lambda: lib.gemm(dA, dB, dC)), dC, lambda out: _check_rows(out, A, B, K)
    if name == "B transposed":
        M, N, K = 600, 500, 700
        A, B, _ = normal_problem(M, N, K, 304)
        dA, dBt = _dev(A), _dev(B.T)
        dC = torch.empty(M, N, dtype=torch.float32, device="cuda")
        return (lambda: lib.gemm(dA, dBt, dC, trans_b=True)), dC, lambda out: _check_rows(out, A, B, K)
    if name == "library call, skinny (split-K, workspace from torch)":
        M, N, K = 16, 4096, 8192
        assert lib.gemm_f16_f32_splitk_choose(M, N, K) > 1
        A, B, _ = normal_problem(M, N, K, 306)
        dA, dB = _dev(A), _dev(B)
        dC = torch.empty(M, N, dtype=torch.float32, device="cuda")
        return (lambda: lib.gemm(dA, dB, dC)), dC, lambda out: _check_rows(out, A, B, K)
    if name in ("split-K workspace beta 1", "split-K fixed scratch"):
        M, N, K = 256, 256, 8192
        beta = 1.0 if name.endswith("beta 1") else 0.0
        A, B, C = normal_problem(M, N, K, 305, with_c=True)
        dA, dB, dC0 = _dev(A), _dev(B), _dev(C)
        dC = torch.empty_like(dC0)
        ws = torch.empty(lib.gemm_f16_f32_splitk_workspace(M, N, 8) // 4, dtype=torch.float32, device="cuda")

        def launch():
            dC.copy_(dC0)
            if beta:
                lib.gemm_splitk(dA, dB, dC, splits=8, beta=beta, workspace=ws)
            else:
                lib.gemm_splitk_noalloc(dA, dB, dC, splits=8)

        return launch, dC, lambda out: _check_rows(out, A, B, K, beta, C)
    raise KeyError(name)


def _check_rows(out, A, B, K, beta=0.0, C=None):
    """Stratified rows of a result against the oracle (every row when there are few)."""
    rows = strata(A.shape[0]) if A.shape[0] > 1024 else np.arange(A.shape[0])
    res = out.cpu().numpy()[rows]
    assert np.all(np.isfinite(res)), "non-finite output"
    ref = oracle.gemm(np.ascontiguousarray(A[rows]), B, beta=beta,
                      C=(np.ascontiguousarray(C[rows]) if C is not None else None))
    err = max_abs_err(res, ref)
    assert err <= tol_normal(K), (err, tol_normal(K))


def _softmax_case(shape):
    import torch
    import dense_tiled_gemm_f16_amd as lib
    M, N = shape
    x = np.random.default_rng(310 + N).standard_normal((M, N)).astype(np.float32)
    dX = _dev(x)
    dY = torch.empty_like(dX)

    def check(out):
        rows = min(M, 64)
        y = out[:rows].cpu().numpy()
        ref = oracle.softmax_rows(x[:rows])
        xd = x[:rows].astype(np.float64)
        R = (xd.max(1, keepdims=True) - xd).max(1, keepdims=True)
        tol = ref * (N + 2 * R + 16) * U + 1e-37
        assert np.all(np.isfinite(y)), "non-finite output"
        assert np.all(np.abs(y.astype(np.float64) - ref) <= tol)

    return (lambda: lib.softmax_rows(dX, dY)), dY, check


GEMM_CASES = ["plain beta 1", "two launches (row split)", "register path, unaligned rows", "B transposed",
              "split-K workspace beta 1", "split-K fixed scratch", "library call, skinny (split-K, workspace from torch)"]
# one shape per softmax kernel family: wave per row, four-wave block, sixteen-wave block with
# grouped exponentials, two-rows-per-CU hybrid (LDS), one-row hybrid (LDS and a twice-read rest)
SOFTMAX_SHAPES = [(4096, 1024), (64, 6000), (8, 60000), (300, 40000), (4, 150000)]


def _eager_noise():
    """Unrelated eager work between replays: a library call on other operands."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    a = torch.ones(192, 160, dtype=torch.float16, device="cuda")
    b = torch.ones(160, 224, dtype=torch.float16, device="cuda")
    c = lib.gemm(a, b)
    torch.cuda.synchronize()
    assert float(c[0, 0]) == 160.0


def _replay_matches_eager(launch, out, check, replays=4):
    import torch
    launch()
    torch.cuda.synchronize()
    eager = _bits(out)
    check(out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    for r in range(replays):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), eager), ("replay", r)
        _eager_noise()


@pytest.mark.parametrize("name", GEMM_CASES)
def test_gemm_graph_replays_match_eager(name):
    _say("case graph gemm", name)
    _replay_matches_eager(*_gemm_case(name))


@pytest.mark.parametrize("shape", SOFTMAX_SHAPES)
def test_softmax_graph_replays_match_eager(shape):
    _say("case graph softmax", shape)
    _replay_matches_eager(*_softmax_case(shape))


def test_concurrent_streams_match_serial():
    """Seven different calls (two-launch GEMM, register path, transposed B, split-K with its own
    workspace, the library's split-K call with a workspace from torch, two softmax kernels) spread
    over four streams and issued three times each without waiting give the bits of the same calls
    made one after another."""
    import torch
    _say("case streams")
    cases = [_gemm_case(n) for n in ("two launches (row split)", "register path, unaligned rows", "B transposed",
                                     "split-K workspace beta 1", "library call, skinny (split-K, workspace from torch)")]
    cases += [_softmax_case(s) for s in ((4096, 1024), (4, 150000))]
    serial = []
    for launch, out, _ in cases:
        launch()
        torch.cuda.synchronize()
        serial.append(_bits(out))
    for _, out, _ in cases:
        out.fill_(float("nan"))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for i, (launch, _, _) in enumerate(cases):
            with torch.cuda.stream(streams[i % 4]):
                launch()
    torch.cuda.synchronize()
    for i, (_, out, _) in enumerate(cases):
        assert np.array_equal(_bits(out), serial[i]), i
