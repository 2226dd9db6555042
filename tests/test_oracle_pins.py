"""Pins for the oracle: each test ties it to something other than itself.

A plausible mistake in the oracle -- a dropped term, a wrong sign or index, a transposed operand,
a mis-decoded FP16 value, a beta term applied wrongly -- fails at least one of these; the last
test plants such mistakes (on the CPU, by mis-calling the oracle) and checks that they are caught.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gemm_inputs import integer_problem, normal_problem, subnormal_problem

U64 = 2.0 ** -53


# ---------------------------------------------------------------- binary16 decoding
def test_decoder_matches_numpy_on_all_patterns():
    """The oracle's own binary16 decoder against numpy's, for all 65536 bit patterns."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (got == ref))
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24),
    (0x0400, 2.0 ** -14), (0x7BFF, 65504.0), (0x3555, 1365 * 2.0 ** -12), (0x7C00, math.inf),
])
def test_decoder_definition_values(bits, value):
    """Values fixed by the binary16 definition (bias 15, 10 fraction bits, subnormals 2^-24 apart)."""
    assert oracle.f16_to_f64(bits) == value


# ---------------------------------------------------------------- exact arithmetic
def _exact(A, B, beta=0.0, C=None):
    M, K = A.shape
    N = B.shape[1]
    Af = [[Fraction(float(x)) for x in row] for row in A]
    Bf = [[Fraction(float(x)) for x in row] for row in B]
    S = [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    absS = [[sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    if beta != 0.0:
        for i in range(M):
            for j in range(N):
                c = Fraction(beta) * Fraction(float(C[i, j]))
                S[i][j] += c
                absS[i][j] += abs(c)
    return S, absS


@pytest.mark.parametrize("shape", [(16, 8, 16), (1, 1, 1), (3, 5, 7), (16, 16, 16)])
def test_matches_exact_rational_sum(shape):
    """Brute force: exact rational arithmetic over the FP16 values.  FP64 accumulation of K exact
    products is within K*2^-53*sum|terms| of the exact sum (and is nearly always equal to it
    after rounding)."""
    M, N, K = shape
    exact_hits = total = 0
    for seed in range(25 if shape == (16, 8, 16) else 6):
        A, B, _ = normal_problem(M, N, K, 1000 + seed)
        D = oracle.gemm(A, B)
        S, absS = _exact(A, B)
        for i in range(M):
            for j in range(N):
                err = abs(Fraction(float(D[i, j])) - S[i][j])
                assert err <= K * Fraction(U64) * absS[i][j], (seed, i, j)
                exact_hits += float(S[i][j]) == D[i, j]
                total += 1
    assert exact_hits >= 0.99 * total


def test_matches_exact_rational_sum_with_beta():
    for seed, beta in ((0, 1.0), (1, 0.5), (2, -1.25)):
        A, B, C = normal_problem(16, 8, 16, 2000 + seed, with_c=True)
        D = oracle.gemm(A, B, beta=beta, C=C)
        S, absS = _exact(A, B, beta, C)
        for i in range(16):
            for j in range(8):
                err = abs(Fraction(float(D[i, j])) - S[i][j])
                assert err <= (16 + 2) * Fraction(U64) * absS[i][j]


def test_empty_k_gives_beta_c():
    A = np.zeros((4, 0), np.float16)
    B = np.zeros((0, 3), np.float16)
    C = np.arange(12, dtype=np.float32).reshape(4, 3)
    assert np.array_equal(oracle.gemm(A, B), np.zeros((4, 3)))
    assert np.array_equal(oracle.gemm(A, B, beta=2.0, C=C), 2.0 * C.astype(np.float64))


def test_empty_m_or_n():
    A, B, _ = normal_problem(0, 5, 7, 1)
    assert oracle.gemm(A, B).shape == (0, 5)
    A, B, _ = normal_problem(5, 0, 7, 1)
    assert oracle.gemm(A, B).shape == (5, 0)


# ---------------------------------------------------------------- identities and linearity
def test_identity_right_and_left():
    """A.I = A and I.B = B exactly (FP16 values are exact in FP64; the sum has one nonzero term)."""
    A, B, _ = normal_problem(37, 53, 41, 11)
    I41 = np.eye(41, dtype=np.float16)
    I37 = np.eye(37, dtype=np.float16)
    assert np.array_equal(oracle.gemm(A, I41), A.astype(np.float64))
    assert np.array_equal(oracle.gemm(I37, A), A.astype(np.float64))
    Z = np.zeros((37, 41), np.float32)
    assert np.array_equal(oracle.gemm(A, I41, beta=1.0, C=Z), A.astype(np.float64))


def test_permutation_picks_rows_and_columns():
    """Multiplying by a permutation matrix reorders exactly: catches transposed indexing."""
    A, _, _ = normal_problem(19, 1, 23, 12)
    rng = np.random.default_rng(5)
    p = rng.permutation(23)
    P = np.zeros((23, 23), np.float16)
    P[np.arange(23), p] = 1          # (A.P)[:, p[k]] = A[:, k]
    D = oracle.gemm(A, P)
    assert np.array_equal(D[:, p], A.astype(np.float64))


def test_linearity_exact_on_integers():
    """With integer entries every FP64 operation is exact, so linearity holds bit for bit."""
    A, B1, _ = integer_problem(31, 29, 47, 21)
    _, B2, _ = integer_problem(31, 29, 47, 22)
    lhs = oracle.gemm(A, B1) + oracle.gemm(A, B2)
    rhs = oracle.gemm(A, (B1.astype(np.float32) + B2.astype(np.float32)).astype(np.float16))
    assert np.array_equal(lhs, rhs)
    assert np.array_equal(oracle.gemm(A, B1), A.astype(np.float64) @ B1.astype(np.float64))


def test_linearity_within_rounding_on_normals():
    A, B1, _ = normal_problem(24, 40, 64, 31)
    B2 = np.round(np.random.default_rng(32).standard_normal((64, 40)) * 4).astype(np.float16)
    Bs = (B1.astype(np.float64) + B2.astype(np.float64))
    lhs = oracle.gemm(A, B1) + oracle.gemm(A, B2)
    # B1 + B2 is not always an FP16 value, so compare against the exact sum of the two products
    absprod = np.abs(A.astype(np.float64)) @ (np.abs(B1.astype(np.float64)) + np.abs(B2.astype(np.float64)))
    rhs = A.astype(np.float64) @ Bs
    assert np.all(np.abs(lhs - rhs) <= 3 * 64 * U64 * absprod)


@pytest.mark.parametrize("p", [1, 2, 4])
def test_power_of_two_scaling_exact(p):
    A, B, _ = normal_problem(33, 35, 70, 40 + p)
    As = (A.astype(np.float64) * 2.0 ** p)
    assert np.array_equal(As.astype(np.float16).astype(np.float64), As)
    assert np.array_equal(oracle.gemm(As.astype(np.float16), B), 2.0 ** p * oracle.gemm(A, B))


@pytest.mark.parametrize("beta", [0.5, -1.25, 1.0])
def test_beta_term_added_once(beta):
    """D = (sum) + beta*C with one FP64 product and one FP64 add."""
    A, B, C = normal_problem(17, 13, 29, 50, with_c=True)
    D0 = oracle.gemm(A, B)
    assert np.array_equal(oracle.gemm(A, B, beta=beta, C=C), D0 + beta * C.astype(np.float64))


def test_beta_zero_never_reads_c():
    A, B, _ = normal_problem(8, 9, 10, 51)
    C = np.full((8, 9), np.nan, np.float32)
    D = oracle.gemm(A, B, beta=0.0, C=C)
    assert np.all(np.isfinite(D))


def test_strided_operands():
    """Row strides larger than the logical width (padding filled with NaN) are honoured."""
    from gemm_inputs import padded
    A, B, C = normal_problem(21, 19, 27, 52, with_c=True)
    Ap, Bp, Cp = padded(A, 40), padded(B, 33), padded(C, 25)
    assert np.array_equal(oracle.gemm(Ap, Bp, beta=1.0, C=Cp), oracle.gemm(A, B, beta=1.0, C=C))


# ---------------------------------------------------------------- a library FP64 product
def test_within_error_bound_of_library_fp64_product():
    """numpy's FP64 matmul (a different summation order) agrees within the FP64 bound."""
    A, B, _ = normal_problem(97, 131, 257, 60)
    D = oracle.gemm(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    absprod = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    assert np.all(np.abs(D - ref) <= 2 * 257 * U64 * absprod)


def test_subnormal_inputs_honoured():
    """Subnormal FP16 inputs are decoded, not flushed: with B around 2^10 every product is normal."""
    A, B, _ = subnormal_problem(9, 7, 12, 61)
    D = oracle.gemm(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert np.all(np.abs(A.astype(np.float64)) < 2.0 ** -14)
    assert np.max(np.abs(ref)) > 1e-4
    absprod = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    assert np.all(np.abs(D - ref) <= 2 * 12 * U64 * absprod)


# ---------------------------------------------------------------- the pages' facts
def test_fp16_products_exact_in_fp32_every_finite_pair():
    """The pages' fact (04_tensor_cores.py, demo 1 observations): two 11-bit significands multiply
    into at most 22 bits, so every FP16 x FP16 product is exact in FP32.  Checked over all
    63488^2 pairs of finite binary16 values."""
    bad, checked = oracle.count_inexact_f16_products()
    assert checked == 63488 ** 2
    assert bad == 0


def test_inexact_product_count_controls():
    """Controls for the exactness count above (the same routine in the oracle counts both): sets
    whose FP32 products are known to round must be counted.

    - Every value v(1 + 2^-12), v a nonzero normal FP16 value, is an FP32 number (at most 23
      significant bits).  The product of two of them is vw(1 + 2^-11 + 2^-24): its lowest set bit
      lies 24 places below the lowest set bit of vw, and so at least 24 places below its highest,
      which is 25 or more significant bits.  Every pair is inexact: the count is exactly nx * ny.
    - A mix of FP16 values and full-precision FP32 values: the expected count comes from exact
      rational products (fractions.Fraction) against numpy's FP32 multiply, pair by pair.  A count
      taken with the product in double would report 0 for both sets."""
    from fractions import Fraction
    rng = np.random.default_rng(123)
    v = rng.standard_normal(160).astype(np.float16).astype(np.float64)
    v = v[(np.abs(v) >= 2.0 ** -14)]                      # nonzero normals
    x = v * (1.0 + 2.0 ** -12)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    assert oracle.count_inexact_products(x, x) == x.size * x.size
    assert oracle.count_inexact_products(v, v) == 0       # plain FP16 values: exact, as above
    mix = np.concatenate([rng.standard_normal(60).astype(np.float16).astype(np.float64),
                          rng.standard_normal(60).astype(np.float32).astype(np.float64),
                          np.array([0.5, -2.0, 1.0, 0.0])])
    expected = 0
    for a in mix:
        for b in mix:
            p32 = np.float32(a) * np.float32(b)
            expected += Fraction(float(p32)) != Fraction(float(a)) * Fraction(float(b))
    assert 0 < expected < mix.size ** 2
    assert oracle.count_inexact_products(mix, mix) == expected
    with pytest.raises(ValueError):
        oracle.count_inexact_products(np.array([1.0 + 2.0 ** -30]), np.array([1.0]))


def test_page_one_instruction_error_level(golden):
    """04_tensor_cores.py demo 1: 100 random D = A.B + C (16x16 . 16x8 + C) in FP32 against the
    FP64 reference; the page prints an error of about 2e-6."""
    g = golden["page_error_levels"]["one_instruction"]
    rng = np.random.default_rng(0)
    errs = []
    for _ in range(100):
        Am = rng.standard_normal((16, 16)).astype(np.float16)
        Bm = rng.standard_normal((16, 8)).astype(np.float16)
        Cm = rng.standard_normal((16, 8)).astype(np.float32)
        acc = Cm.copy()
        for k in range(16):                      # FP32 accumulation of exact products
            acc = acc + Am[:, k:k + 1].astype(np.float32) * Bm[k:k + 1, :].astype(np.float32)
        errs.append(np.abs(acc.astype(np.float64) - oracle.gemm(Am, Bm, beta=1.0, C=Cm)).max())
    lo, hi = g["accept_band"]
    assert lo <= max(errs) <= hi


def test_page_block_gemm_error_level(golden):
    """04_tensor_cores.py demo 2: 128^3 FP16 product with FP32 accumulation in k16 instruction steps
    lands about 5e-6 from the FP64 reference."""
    g = golden["page_error_levels"]["block_gemm_128"]
    rng = np.random.default_rng(1)
    A = rng.standard_normal((128, 128)).astype(np.float16)
    B = rng.standard_normal((128, 128)).astype(np.float16)
    # the page's block kernel accumulates one 16-deep instruction at a time: the 16 exact products
    # and the running FP32 accumulator are summed and rounded to FP32 once per instruction
    acc = np.zeros((128, 128), np.float64)
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    for k0 in range(0, 128, 16):
        acc = (acc + A64[:, k0:k0 + 16] @ B64[k0:k0 + 16, :]).astype(np.float32).astype(np.float64)
    err = np.abs(acc - oracle.gemm(A, B)).max()
    lo, hi = g["accept_band"]
    assert lo <= err <= hi


def test_page_fp16_vs_fp32_accumulation_table(golden):
    """06_triton_style.py demo 4, second table: FP16 accumulation is several thousand times worse
    than FP32 accumulation, and the FP32 error divided by sqrt(K) grows with K."""
    g = golden["page_error_levels"]["fp16_vs_fp32_accumulation"]
    rng = np.random.default_rng(3)
    for (M, N, K) in [(64, 64, 64), (128, 64, 96), (1, 1, 1), (17, 33, 65), (100, 70, 50), (64, 64, 40)]:
        rng.standard_normal((M, K)).astype(np.float32)     # the edge-shape draws come first
        rng.standard_normal((K, N)).astype(np.float32)
    ratios, e32 = [], []
    for K in (64, 256, 1024, 4096):
        a = rng.standard_normal((64, K)).astype(np.float16)
        b = rng.standard_normal((K, 64)).astype(np.float16)
        ref = oracle.gemm(a, b)
        acc32 = np.zeros((64, 64), np.float32)
        acc16 = np.zeros((64, 64), np.float16)
        for k in range(K):
            prod = a[:, k:k + 1].astype(np.float32) * b[k:k + 1, :].astype(np.float32)
            acc32 += prod
            acc16 = (acc16.astype(np.float32) + prod).astype(np.float16)
        err32 = np.abs(acc32 - ref).max()
        err16 = np.abs(acc16 - ref).max()
        ratios.append(err16 / err32)
        e32.append(err32 / math.sqrt(K))
    lo, hi = g["accept_band"]
    assert all(lo <= r <= hi for r in ratios), ratios
    assert all(x < y for x, y in zip(e32, e32[1:])), e32


# ---------------------------------------------------------------- planted mistakes are caught
def _rational_pin_passes(fn, seed=7):
    A, B, _ = normal_problem(16, 8, 16, seed)
    D = fn(A, B)
    S, absS = _exact(A, B)
    return all(abs(Fraction(float(D[i, j])) - S[i][j]) <= 16 * Fraction(U64) * absS[i][j]
               for i in range(16) for j in range(8))


def test_planted_mistakes_fail_the_pins():
    assert _rational_pin_passes(oracle.gemm)
    mutants = {
        "dropped last k term": lambda A, B: oracle.gemm(A[:, :-1], B[:-1, :]),
        "dropped first k term": lambda A, B: oracle.gemm(A[:, 1:], B[1:, :]),
        "wrong sign": lambda A, B: -oracle.gemm(A, B),
        "B read transposed": lambda A, B: oracle.gemm(A, np.ascontiguousarray(
            np.resize(B.T, B.shape))),
        "A rows shifted": lambda A, B: oracle.gemm(np.roll(A, 1, axis=0), B),
        "operand rounded to FP16 output": lambda A, B: oracle.gemm(A, B).astype(np.float16).astype(np.float64),
    }
    for name, fn in mutants.items():
        assert not _rational_pin_passes(fn), name
