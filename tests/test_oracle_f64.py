"""Pins for the oracle's binary64 GEMM (CPU only).

The oracle computes d_ij = alpha * sum_l a_il b_lj + beta * c_ij
("Accurate Models of AMD Matrix Cores", Section 2, Eq. (1), with BLAS alpha and
beta) for binary64 operands, the operand format of the FP64-accumulate
builtins ("CDNA3 dense MFMA builtins", FP64-accumulate builtins), as exact
products summed in binary128 and rounded once to binary64.  These tests pin it
to things other than itself: exact rationals (Python fractions) on small
tiles, cancellations that plain binary64 summation gets wrong, permutation
matrices, integer-valued products against numpy int64, numpy's float64
matmul as a library witness within its error bound, and the BLAS beta = 0
convention.  The acceptance checker for binary64 results is mutation-tested
at the end.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

LAYOUTS = ["k_contig", "mn_contig"]


def store_A(vals_MK, layout):
    return np.ascontiguousarray(vals_MK if layout == "k_contig" else vals_MK.T)


def store_B(vals_KN, layout):
    return np.ascontiguousarray(vals_KN.T if layout == "k_contig" else vals_KN)


def run(A, B, C=None, alpha=1.0, beta=0.0, layA="k_contig", layB="k_contig", rows=None, cols=None):
    M, K = A.shape
    N = B.shape[1]
    As, Bs = store_A(A, layA), store_B(B, layB)
    return oracle.gemm_f64(layA, layB, M, N, K, As, As.shape[1] if As.ndim == 2 and As.size else max(K, 1),
                           Bs, Bs.shape[1] if Bs.ndim == 2 and Bs.size else max(K, 1),
                           C, N, alpha, beta, rows, cols)


def exact(A, B, C, alpha, beta, i, j):
    t = Fraction(alpha) * sum((Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(A.shape[1])),
                              Fraction(0))
    if beta != 0.0:
        t += Fraction(beta) * Fraction(float(C[i, j]))
    return t


def rand_sig(shape, seed):
    """Values +-[1, 2) with full 53-bit significands."""
    g = W.gen(seed)
    u = torch.rand(shape, generator=g, dtype=torch.float64).numpy()
    s = torch.randint(0, 2, shape, generator=g).numpy() * 2 - 1
    return s * (1.0 + u)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (4, 4, 4), (3, 5, 7), (5, 3, 2)])
@pytest.mark.parametrize("layA", LAYOUTS)
@pytest.mark.parametrize("layB", LAYOUTS)
def test_brute_force_exact_rationals(M, N, K, layA, layB):
    """Significands in [1, 2), K <= 7, alpha = 0.75, beta = -1.25: the exact
    value fits binary128, so the oracle equals the exact rational rounded once
    to nearest (Python's Fraction -> float conversion)."""
    A = rand_sig((M, K), 10 + M)
    B = rand_sig((K, N), 20 + N)
    C = rand_sig((M, N), 30 + K)
    d, s = run(A, B, C, 0.75, -1.25, layA, layB)
    for i in range(M):
        for j in range(N):
            assert d[i, j] == float(exact(A, B, C, 0.75, -1.25, i, j)), (i, j)
            assert s[i, j] == float(sum(abs(Fraction(A[i, k]) * Fraction(B[k, j])) for k in range(K)))


def test_wide_exponent_range_matches_exact_rationals():
    """Magnitudes over about 2^-17 .. 2^17 (K = 24): still the correctly rounded
    exact value."""
    M, N, K = 6, 5, 24
    A = W.draw("lognormal", (M, K), 41, torch.float64).numpy()
    B = W.draw("lognormal", (K, N), 42, torch.float64).numpy()
    C = W.draw("lognormal", (M, N), 43, torch.float64).numpy()
    d, _ = run(A, B, C, -0.3, 0.7)
    for i in range(M):
        for j in range(N):
            assert d[i, j] == float(exact(A, B, C, -0.3, 0.7, i, j))


def test_products_exact_and_cancellation():
    """Results that binary64 products or binary64 summation get wrong:
    (1 + 2^-52)^2 - (1 + 2^-51) = 2^-104, and 2^60 + 1 - 2^60 = 1."""
    e = 2.0 ** -52
    A = np.array([[1 + e, -1.0, 0.0], [2.0 ** 60, 1.0, -(2.0 ** 60)]])
    B = np.array([[1 + e], [1 + 2 * e], [1.0]])
    B2 = np.ones((3, 1))
    d1, _ = run(A[:1, :2], B[:2])
    assert d1[0, 0] == 2.0 ** -104
    # the same through a plain binary64 loop would give 0
    assert (1 + e) * (1 + e) - (1 + 2 * e) == 0.0
    d2, s2 = run(A[1:], B2)
    assert d2[0, 0] == 1.0 and s2[0, 0] == 2.0 ** 61 + 1
    assert (2.0 ** 60 + 1.0) - 2.0 ** 60 == 0.0


@pytest.mark.parametrize("layA", LAYOUTS)
@pytest.mark.parametrize("layB", LAYOUTS)
def test_permutation_rows_exact(layA, layB):
    K, N = 33, 17
    perm = torch.randperm(K, generator=W.gen(5)).numpy()
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0
    B = W.draw("normal", (K, N), 6, torch.float64).numpy()
    d, _ = run(P, B, layA=layA, layB=layB)
    assert np.array_equal(d, B[perm])


def test_integer_valued_matches_int64():
    M, N, K = 19, 23, 300
    g = W.gen(7)
    Ai = torch.randint(-1000, 1001, (M, K), generator=g).numpy()
    Bi = torch.randint(-1000, 1001, (K, N), generator=g).numpy()
    Ci = torch.randint(-1000, 1001, (M, N), generator=g).numpy()
    d, _ = run(Ai.astype(np.float64), Bi.astype(np.float64), Ci.astype(np.float64), 3.0, -2.0)
    want = 3 * (Ai.astype(np.int64) @ Bi.astype(np.int64)) - 2 * Ci
    assert np.array_equal(d, want.astype(np.float64))


@pytest.mark.parametrize("layA", LAYOUTS)
@pytest.mark.parametrize("layB", LAYOUTS)
def test_numpy_float64_witness(layA, layB):
    """numpy's binary64 matmul is within K u S of the exact value; the oracle
    must agree with it to that bound (a transposed operand or a dropped term
    is far outside it)."""
    M, N, K = 37, 29, 301
    A = W.draw("normal", (M, K), 8, torch.float64).numpy()
    B = W.draw("normal", (K, N), 9, torch.float64).numpy()
    d, s = run(A, B, layA=layA, layB=layB)
    ref = A @ B
    assert np.all(np.abs(d - ref) <= 2.0 * K * 2.0 ** -53 * s)
    assert np.allclose(s, np.abs(A) @ np.abs(B), rtol=1e-12)


def test_beta_zero_never_reads_c_and_k_zero():
    A = np.ones((2, 3))
    B = np.ones((3, 2))
    C = np.full((2, 2), np.nan)
    d, _ = run(A, B, C, 2.0, 0.0)
    assert np.array_equal(d, np.full((2, 2), 6.0))
    Cc = np.array([[1.5, -2.0], [0.25, 3.0]])
    d0, s0 = oracle.gemm_f64("k_contig", "k_contig", 2, 2, 0, np.zeros(1), 1, np.zeros(1), 1, Cc, 2, 5.0, -2.0)
    assert np.array_equal(d0, -2.0 * Cc) and np.all(s0 == 0)


def test_sampled_equals_full():
    M, N, K = 40, 30, 50
    A = W.draw("normal", (M, K), 11, torch.float64).numpy()
    B = W.draw("normal", (K, N), 12, torch.float64).numpy()
    C = W.draw("normal", (M, N), 13, torch.float64).numpy()
    d, s = run(A, B, C, 1.5, 0.5)
    rows, cols = W.sample_coords(M, N, 200, full_rows=(0,), full_cols=(N - 1,))
    ds, ss = run(A, B, C, 1.5, 0.5, rows=rows, cols=cols)
    assert np.array_equal(ds, d[rows, cols]) and np.array_equal(ss, s[rows, cols])


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.gemm_f64("k_contig", "k_contig", 2, 2, 2, np.zeros(4), 2, np.zeros(4), 2, None, 2, 1.0, 1.0)
    with pytest.raises(ValueError):
        oracle.gemm_f64("k_contig", "k_contig", 2, 2, 2, np.zeros(4), 2, np.zeros(4), 2, rows=[2], cols=[0])


# ---------------------------------------------------------------- checker

def setup(M=48, N=40, K=200):
    A = W.operand("A", "f64", M, K, "normal")
    B = W.operand("B", "f64", K, N, "normal")
    d, s = oracle.gemm_f64("k_contig", "k_contig", M, N, K, A.codes, A.ld, B.codes, B.ld)
    return A, B, d, s


def test_checker_exact_passes_and_just_outside_fails():
    _, _, d, s = setup()
    assert oracle.check_f64(d, d, s, 200)["ok"]
    b = oracle.f64_bound(d, s, 200)
    assert oracle.check_f64(d + 0.5 * b, d, s, 200)["ok"]
    out = np.nextafter(np.nextafter(d + b, np.inf), np.inf)
    r = oracle.check_f64(out, d, s, 200)
    assert not r["ok"] and r["violations"] == d.size


def test_checker_catches_binary32_accumulation_and_dropped_slab():
    M, N, K = 48, 40, 200
    A, B, d, s = setup(M, N, K)
    # a binary32 result is far outside the binary64 bound
    d32 = d.astype(np.float32).astype(np.float64)
    assert oracle.check_f64(d32, d, s, K)["violations"] > 0.9 * d.size
    Ac = A.codes.copy()
    Ac[:, 16:32] = 0.0
    d_bad, _ = oracle.gemm_f64("k_contig", "k_contig", M, N, K, Ac, A.ld, B.codes, B.ld)
    assert oracle.check_f64(d_bad, d, s, K)["violations"] > 0.9 * d.size


def test_checker_nan_and_index_shift_fail():
    _, _, d, s = setup()
    bad = d.copy()
    bad[3, 7] = np.nan
    r = oracle.check_f64(bad, d, s, 200)
    assert not r["ok"] and r["violations"] == 1
    assert not oracle.check_f64(np.roll(d, 1, axis=1), d, s, 200)["ok"]
