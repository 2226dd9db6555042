"""GPU: the autotuner times real launches, records a winner, and the winner still matches the oracle."""
import numpy as np
import pytest

import oracle
from gemm_inputs import normal_problem
from tolerance import max_abs_err, tol_normal

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (1792, 1792, 1792), (16, 4096, 8192)])
def test_tune_records_a_winner_that_matches_the_oracle(shape, tmp_path):
    """The last shape is skinny: the library's own call splits K there, so the recorded winner is
    either that call (empty options) or a single launch that beat it."""
    import torch
    import dense_tiled_gemm_f16_amd as g
    from dense_tiled_gemm_f16_amd import autotune
    M, N, K = shape
    print("case autotune", shape, flush=True)
    A, B, _ = normal_problem(M, N, K, 1200 + M)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    dC = torch.empty((M, N), dtype=torch.float32, device="cuda")
    cache = autotune.Cache(str(tmp_path / "tune.json"))
    r = autotune.tune(dA, dB, dC, top_k=6, cache=cache)
    assert len(r["results"]) == 6 and r["us"] <= r["default_us"]
    assert autotune.tuned_opts(dA, dB, dC, cache=cache) == r["opts"]
    dC.fill_(float("nan"))
    g.gemm(dA, dB, dC, opts=r["opts"])
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    rows = np.arange(0, M, max(1, M // 48))
    err = max_abs_err(out[rows], oracle.gemm(A[rows], B))
    assert np.all(np.isfinite(out)) and err <= tol_normal(K), err


def test_empty_options_are_the_library_call():
    """opts={} (no overrides, also what a tuned record holds when the library's own call won) runs
    the library's call, split-K included, bit for bit."""
    import torch
    import dense_tiled_gemm_f16_amd as g
    M, N, K = 16, 4096, 8192
    assert g.gemm_f16_f32_splitk_choose(M, N, K) > 1
    A, B, _ = normal_problem(M, N, K, 1300)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    c0 = g.gemm(dA, dB)
    c1 = g.gemm(dA, dB, opts={})
    c2 = g.gemm(dA, dB, splits=1)
    torch.cuda.synchronize()
    assert torch.equal(c0.view(torch.int32), c1.view(torch.int32))
    err = max_abs_err(c0.cpu().numpy(), oracle.gemm(A, B))
    assert err <= tol_normal(K), err
    assert max_abs_err(c2.cpu().numpy(), oracle.gemm(A, B)) <= tol_normal(K)
