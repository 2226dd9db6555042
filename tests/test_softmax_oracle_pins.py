"""Pins for the row-softmax oracle (oracle_softmax.c), tied to facts outside the oracle itself.

06_triton_style.py (CS349E lecture 10, block programming), demo 3 defines the operation: subtract
the row maximum, exponentiate, divide by the row sum.
"""
import math

import numpy as np
import pytest

import oracle
from dense_tiled_gemm_f16_amd import model


def _rows(seed, M, N, scale=1.0):
    return (np.random.default_rng(seed).standard_normal((M, N)) * scale).astype(np.float32)


def test_rows_sum_to_one_and_are_positive():
    y = oracle.softmax_rows(_rows(1, 64, 1000))
    assert np.all(y > 0)
    assert np.max(np.abs(y.sum(1) - 1.0)) <= 1000 * 2.0 ** -52


def test_two_element_rows_are_the_logistic_function():
    """softmax([a, b])[0] = 1 / (1 + e^(b - a)), a different expression of the same number."""
    x = _rows(2, 200, 2, scale=4.0)
    y = oracle.softmax_rows(x)
    a, b = x[:, 0].astype(np.float64), x[:, 1].astype(np.float64)
    logistic = np.array([1.0 / (1.0 + math.exp(bb - aa)) for aa, bb in zip(a, b)])
    assert np.max(np.abs(y[:, 0] - logistic)) <= 4 * 2.0 ** -52


def test_special_rows():
    x = np.array([[0.0, math.log(2.0)], [1000.0, 1000.0], [7.0, 7.0]], np.float32)
    y = oracle.softmax_rows(x)
    two = math.exp(float(np.float32(math.log(2.0))))          # e^(ln 2 rounded to FP32)
    assert abs(y[0, 0] - 1.0 / (1.0 + two)) <= 1e-15 and abs(y[0, 1] - two / (1.0 + two)) <= 1e-15
    assert np.array_equal(y[1], [0.5, 0.5]) and np.array_equal(y[2], [0.5, 0.5])
    const = oracle.softmax_rows(np.full((3, 7), -3.25, np.float32))
    assert np.all(const == 1.0 / 7.0)
    # exp(-1000) underflows to exactly 0 in FP64 after the row maximum is subtracted
    big = oracle.softmax_rows(np.array([[1000.0, 0.0, 1000.0]], np.float32))
    assert big[0, 1] == 0.0 and big[0, 0] == 0.5


def test_shift_invariance_on_exact_inputs():
    """Adding the same integer to a row of small integers (exact in FP32) leaves the softmax
    unchanged: every x - max is the same FP32 value."""
    x = np.random.default_rng(3).integers(-20, 20, size=(50, 33)).astype(np.float32)
    shift = np.random.default_rng(4).integers(-1000, 1000, size=(50, 1)).astype(np.float32)
    assert np.array_equal(oracle.softmax_rows(x), oracle.softmax_rows(x + shift))


def test_matches_a_library_computation():
    x = _rows(5, 40, 513, scale=3.0)
    ref = x.astype(np.float64)
    ref = np.exp(ref - ref.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    assert np.max(np.abs(oracle.softmax_rows(x) - ref) / ref) <= 2000 * 2.0 ** -52


def test_strided_input():
    big = _rows(6, 20, 300)
    assert np.array_equal(oracle.softmax_rows(big[:, :257]), oracle.softmax_rows(np.ascontiguousarray(big[:, :257])))


@pytest.mark.parametrize("mistake", ["no_max", "wrong_axis", "drop_last"])
def test_planted_mistakes_fail_the_pins(mistake):
    """Plausible mistakes in a softmax fail the logistic or row-sum pins."""
    x = _rows(7, 30, 2, scale=40.0)
    xd = x.astype(np.float64)
    if mistake == "no_max":
        with np.errstate(over="ignore", invalid="ignore"):
            e = np.exp(xd * 30.0)                  # large rows overflow without the maximum
            y = e / e.sum(1, keepdims=True)
        assert not np.all(np.isfinite(y))
        return
    if mistake == "wrong_axis":
        e = np.exp(xd - xd.max(0, keepdims=True))
        y = e / e.sum(0, keepdims=True)
    else:
        e = np.exp(xd - xd.max(1, keepdims=True))
        y = e / e[:, :-1].sum(1, keepdims=True)
    assert np.max(np.abs(y.sum(1) - 1.0)) > 1e-6


def test_traffic_counts_match_the_page(golden):
    g = golden["page_launch_counts"]["softmax_traffic"]
    M, N = g["M"], g["N"]
    rd, wr = model.softmax_traffic(M, N, fused=False)
    assert (rd, wr) == (5 * M * N + 2 * M, 3 * M * N + 2 * M)
    assert (g["unfused_reads"], g["unfused_writes"]) == ("5MN + 2M", "3MN + 2M")
    assert model.softmax_traffic(M, N, fused=True) == (M * N, M * N)
    assert round((rd + wr) / (2 * M * N), 1) == g["traffic_ratio_one_decimal"]
