"""Pins for the oracle's dense GEMMs (CPU only).

The oracle follows the definition of the matrix fused multiply-add,
d_ij = sum_l a_il b_lj + c_ij ("Accurate Models of AMD Matrix Cores",
Section 2, Eq. (1)).  These tests pin it to things other than itself:
closed forms, identity/permutation matrices, exact small-integer products
(int64 numpy as witness), brute force with exact rationals on 4x4x4 tiles,
numpy float64 matmul as a library witness, layout invariance, and exact
power-of-two scaling.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

LAYOUTS = ["k_contig", "mn_contig"]
FLOATS = ["bf16", "f16", "e4m3", "e5m2"]


def store_A(vals_codes_MK, layout):
    return vals_codes_MK if layout == "k_contig" else np.ascontiguousarray(vals_codes_MK.T)


def store_B(vals_codes_KN, layout):
    return np.ascontiguousarray(vals_codes_KN.T) if layout == "k_contig" else vals_codes_KN


def ld_of(stored):
    return stored.shape[1]


def codes_from_values(dt, values):
    """Raw codes of exactly representable values (torch conversion)."""
    t = torch.as_tensor(values, dtype=torch.float64)
    if dt == "i8":
        return t.to(torch.int8).numpy()
    return W.codes_of(t.to(torch.float32).to(W.TORCH_DTYPE[dt]), dt)


def run_float(dtA, dtB, layA, layB, Avals, Bvals, C=None, alpha=1.0, beta=0.0, sA=1.0, sB=1.0):
    M, K = Avals.shape
    N = Bvals.shape[1]
    A = store_A(codes_from_values(dtA, Avals), layA)
    B = store_B(codes_from_values(dtB, Bvals), layB)
    return oracle.gemm_float(dtA, dtB, layA, layB, M, N, K, A, ld_of(A), B, ld_of(B),
                             C, N, alpha, beta, sA, sB)


def run_i8(layA, layB, Avals, Bvals, C=None, alpha=1, beta=0):
    M, K = Avals.shape
    N = Bvals.shape[1]
    A = store_A(np.asarray(Avals, np.int8), layA)
    B = store_B(np.asarray(Bvals, np.int8), layB)
    return oracle.gemm_i8(layA, layB, M, N, K, A, ld_of(A), B, ld_of(B), C, N, alpha, beta)


# ------------------------------------------------------------------ int8 pins

@pytest.mark.parametrize("layA", LAYOUTS)
@pytest.mark.parametrize("layB", LAYOUTS)
def test_i8_closed_forms(layA, layB):
    M, N, K = 5, 7, 96
    C = np.arange(M * N, dtype=np.int32).reshape(M, N) - 17
    d = run_i8(layA, layB, np.ones((M, K)), np.ones((K, N)), C, 1, 1)
    assert np.array_equal(d, K + C)
    d = run_i8(layA, layB, np.full((M, K), -128), np.full((K, N), -128))
    assert np.all(d == 16384 * K)


def test_i8_all_minus128_at_4096_is_2_pow_26():
    K = 4096
    d = run_i8("k_contig", "k_contig", np.full((2, K), -128), np.full((K, 3), -128))
    assert np.all(d == 2 ** 26)


def test_i8_permutation_and_identity():
    rng = np.random.default_rng(0)
    n = 24
    P = np.eye(n, dtype=np.int64)[rng.permutation(n)]
    B = rng.integers(-128, 128, (n, 9))
    C = rng.integers(-1000, 1000, (n, 9)).astype(np.int32)
    for layA in LAYOUTS:
        for layB in LAYOUTS:
            assert np.array_equal(run_i8(layA, layB, P, B), P @ B)
            assert np.array_equal(run_i8(layA, layB, np.eye(n), B, C, 1, 1), B + C)


def test_i8_numpy_witness_and_layout_invariance():
    rng = np.random.default_rng(1)
    M, N, K = 19, 23, 77
    A = rng.integers(-128, 128, (M, K))
    B = rng.integers(-128, 128, (K, N))
    C = rng.integers(-(1 << 20), (1 << 20) + 1, (M, N)).astype(np.int32)
    want = (3 * (A @ B) - 2 * C.astype(np.int64)).astype(np.int64)
    for layA in LAYOUTS:
        for layB in LAYOUTS:
            assert np.array_equal(run_i8(layA, layB, A, B, C, 3, -2), want.astype(np.int32))


def test_i8_brute_force_4x4x4():
    rng = np.random.default_rng(2)
    for trial in range(20):
        A = rng.integers(-128, 128, (4, 4))
        B = rng.integers(-128, 128, (4, 4))
        C = rng.integers(-(1 << 20), 1 << 20, (4, 4)).astype(np.int32)
        want = [[sum(int(A[i][l]) * int(B[l][j]) for l in range(4)) + int(C[i][j])
                 for j in range(4)] for i in range(4)]
        assert np.array_equal(run_i8("k_contig", "mn_contig", A, B, C, 1, 1),
                              np.array(want, np.int32))


def test_i8_wraps_mod_2_32():
    A = np.full((1, 4), 127)
    B = np.full((4, 1), 127)
    alpha = 40000  # 40000 * 4 * 127^2 = 2580640000 > 2^31
    got = run_i8("k_contig", "k_contig", A, B, None, alpha, 0)
    want = (alpha * 4 * 127 * 127) % (1 << 32)
    want = want - (1 << 32) if want >= (1 << 31) else want
    assert int(got[0, 0]) == want


def test_i8_sampled_equals_full():
    rng = np.random.default_rng(3)
    M, N, K = 13, 11, 40
    A = np.asarray(rng.integers(-128, 128, (M, K)), np.int8)
    B = np.asarray(rng.integers(-128, 128, (N, K)), np.int8)
    C = rng.integers(-100, 100, (M, N)).astype(np.int32)
    full = oracle.gemm_i8("k_contig", "k_contig", M, N, K, A, K, B, K, C, N, 1, 1)
    rows, cols = W.sample_coords(M, N, n_random=50, full_rows=[2], full_cols=[5])
    part = oracle.gemm_i8("k_contig", "k_contig", M, N, K, A, K, B, K, C, N, 1, 1, rows, cols)
    assert np.array_equal(part, full[rows, cols])


def test_i8_beta_zero_does_not_read_c():
    A = np.ones((2, 8))
    B = np.ones((8, 2))
    # C=None with beta=0 must be accepted
    assert np.all(run_i8("k_contig", "k_contig", A, B, None, 1, 0) == 8)


# ----------------------------------------------------------------- float pins

SMALL = {"bf16": 8, "f16": 8, "e4m3": 16, "e5m2": 8}


@pytest.mark.parametrize("dt", FLOATS)
@pytest.mark.parametrize("layA", LAYOUTS)
@pytest.mark.parametrize("layB", LAYOUTS)
def test_float_small_integers_exact(dt, layA, layB):
    # Integer values small enough that every partial sum is an integer below
    # 2^24: the rounded result must equal the exact int64 product bit for bit.
    rng = np.random.default_rng(4)
    M, N, K = 9, 14, 64
    r = SMALL[dt]
    A = rng.integers(-r, r + 1, (M, K))
    B = rng.integers(-r, r + 1, (K, N))
    C = rng.integers(-1000, 1000, (M, N)).astype(np.float32)
    d, s = run_float(dt, dt, layA, layB, A, B, C, 1.0, 1.0)
    assert np.array_equal(d, (A @ B + C.astype(np.int64)).astype(np.float32))
    assert np.array_equal(s, np.abs(A)[:, :, None].__mul__(np.abs(B)[None, :, :]).sum(1))


def test_float_mixed_fp8_small_integers_exact():
    rng = np.random.default_rng(5)
    A = rng.integers(-16, 17, (6, 32))
    B = rng.integers(-8, 9, (32, 5))
    d, _ = run_float("e4m3", "e5m2", "k_contig", "k_contig", A, B)
    assert np.array_equal(d, (A @ B).astype(np.float32))


def fraction_to_f32(x: Fraction) -> np.float32:
    """Round an exact rational to binary32, nearest even (brute force)."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    e = max(e, -126)                      # subnormal range keeps the same step
    step = Fraction(2) ** (e - 23)
    q = x / step
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(n * step))


@pytest.mark.parametrize("dt", FLOATS)
def test_float_brute_force_4x4x4_exact_rationals(dt):
    gen = torch.Generator().manual_seed(6)
    for trial in range(10):
        Aq, _ = W.quantize(torch.randn((4, 4), generator=gen) * 3, dt)
        Bq, _ = W.quantize(torch.randn((4, 4), generator=gen) * 3, dt)
        Ac, Bc = W.codes_of(Aq, dt), W.codes_of(Bq.t().contiguous(), dt)  # B column-major
        C = torch.randn((4, 4), generator=gen).numpy().astype(np.float32)
        alpha, beta = 0.75, -1.25
        d, _ = oracle.gemm_float(dt, dt, "k_contig", "k_contig", 4, 4, 4, Ac, 4, Bc, 4,
                                 C, 4, alpha, beta)
        Af = [[Fraction(float(v)) for v in row] for row in Aq.to(torch.float64).tolist()]
        Bf = [[Fraction(float(v)) for v in row] for row in Bq.to(torch.float64).tolist()]
        for i in range(4):
            for j in range(4):
                t = Fraction(alpha) * sum(Af[i][l] * Bf[l][j] for l in range(4)) \
                    + Fraction(beta) * Fraction(float(C[i, j]))
                assert d[i, j] == fraction_to_f32(t), (trial, i, j)


@pytest.mark.parametrize("dt", FLOATS)
def test_float_numpy_float64_witness(dt):
    gen = torch.Generator().manual_seed(7)
    M, N, K = 17, 31, 200
    Aq, _ = W.quantize(torch.randn((M, K), generator=gen), dt)
    Bq, _ = W.quantize(torch.randn((K, N), generator=gen), dt)
    C = torch.randn((M, N), generator=gen).numpy().astype(np.float32)
    A64, B64 = Aq.to(torch.float64).numpy(), Bq.to(torch.float64).numpy()
    want = (A64 @ B64 + C.astype(np.float64)).astype(np.float32)
    for layA in LAYOUTS:
        for layB in LAYOUTS:
            A = W.store(Aq, "A", layA)[0]
            B = W.store(Bq, "B", layB)[0]
            d, s = oracle.gemm_float(dt, dt, layA, layB, M, N, K, W.codes_of(A, dt),
                                     A.shape[1], W.codes_of(B, dt), B.shape[1], C, N, 1.0, 1.0)
            ulp = np.spacing(np.abs(want)).astype(np.float64)
            assert np.all(np.abs(d.astype(np.float64) - want) <= ulp)
            assert np.allclose(s, np.abs(A64) @ np.abs(B64), rtol=1e-12)


def test_float_power_of_two_alpha_is_exact_and_scales_apply():
    gen = torch.Generator().manual_seed(8)
    Aq, _ = W.quantize(torch.randn((8, 64), generator=gen), "bf16")
    Bq, _ = W.quantize(torch.randn((64, 8), generator=gen), "bf16")
    A = W.codes_of(Aq, "bf16")
    B = W.codes_of(Bq.t().contiguous(), "bf16")
    d1, _ = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", 8, 8, 64, A, 64, B, 64)
    d8, _ = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", 8, 8, 64, A, 64, B, 64,
                              alpha=8.0)
    assert np.array_equal(d8, d1 * np.float32(8))
    ds, _ = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", 8, 8, 64, A, 64, B, 64,
                              sA=0.5, sB=16.0)
    assert np.array_equal(ds, d8)


def test_float_permutation_and_identity_with_c():
    rng = np.random.default_rng(9)
    n = 16
    P = np.eye(n)[rng.permutation(n)]
    gen = torch.Generator().manual_seed(9)
    Bq, _ = W.quantize(torch.randn((n, 6), generator=gen), "bf16")
    Bv = Bq.to(torch.float64).numpy()
    d, _ = run_float("bf16", "bf16", "k_contig", "mn_contig", P, Bv)
    assert np.array_equal(d, (P @ Bv).astype(np.float32))
    C = torch.randn((n, 6), generator=gen).numpy().astype(np.float32)
    d, _ = run_float("bf16", "bf16", "mn_contig", "k_contig", np.eye(n), Bv, C, 1.0, 1.0)
    assert np.array_equal(d, (Bv + C.astype(np.float64)).astype(np.float32))


def test_float_padded_leading_dimensions():
    gen = torch.Generator().manual_seed(10)
    M, N, K = 6, 5, 12
    Aq, _ = W.quantize(torch.randn((M, K), generator=gen), "f16")
    Bq, _ = W.quantize(torch.randn((K, N), generator=gen), "f16")
    C = torch.randn((M, 9), generator=gen).numpy().astype(np.float32)
    A1, lda1 = W.store(Aq, "A", "k_contig")
    A2, lda2 = W.store(Aq, "A", "k_contig", ld=20)
    B1, ldb1 = W.store(Bq, "B", "mn_contig")
    B2, ldb2 = W.store(Bq, "B", "mn_contig", ld=8)
    d1, _ = oracle.gemm_float("f16", "f16", "k_contig", "mn_contig", M, N, K, W.codes_of(A1, "f16"),
                              lda1, W.codes_of(B1, "f16"), ldb1, C, 9, 1.0, 1.0)
    d2, _ = oracle.gemm_float("f16", "f16", "k_contig", "mn_contig", M, N, K, W.codes_of(A2, "f16"),
                              lda2, W.codes_of(B2, "f16"), ldb2, C, 9, 1.0, 1.0)
    assert np.array_equal(d1, d2)


def test_float_k_zero_gives_beta_c():
    C = np.array([[1.5, -2.0]], np.float32)
    A = np.zeros((1, 0), np.uint16)
    B = np.zeros((2, 0), np.uint16)
    d, s = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", 1, 2, 0, A, 1, B, 1,
                             C, 2, 1.0, 2.0)
    assert np.array_equal(d, 2 * C)
    assert np.all(s == 0)
