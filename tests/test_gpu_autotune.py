"""GPU: the autotuner times real launches, records a winner, and the winner still matches the oracle."""
import numpy as np
import pytest

import oracle
from gemm_inputs import normal_problem
from tolerance import max_abs_err, tol_normal

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(1024, 1024, 1024), (1792, 1792, 1792)])
def test_tune_records_a_winner_that_matches_the_oracle(shape, tmp_path):
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
