"""Mutation tests for the acceptance checker (CPU).

A correct result passes; results with a plausible kernel mistake -- a value
just outside the bound, a dropped K-slab, a NaN, an off-by-one output index,
a transposed operand -- fail.
"""
import numpy as np
import torch

import oracle
import workloads as W


def setup(M=64, N=48, K=256, dt="bf16"):
    A = W.operand("A", dt, M, K, "uniform", "k_contig")
    B = W.operand("B", dt, K, N, "uniform", "k_contig")
    d, s = oracle.gemm_float(dt, dt, "k_contig", "k_contig", M, N, K, A.codes, A.ld,
                             B.codes, B.ld)
    return A, B, d, s


def test_exact_result_passes():
    _, _, d, s = setup()
    assert oracle.check_float(d, d, s, 256)["ok"]


def test_just_outside_bound_fails_just_inside_passes():
    _, _, d, s = setup()
    b = oracle.float_bound(d, s, 256)
    inside = (d.astype(np.float64) + 0.5 * b).astype(np.float32)
    assert oracle.check_float(inside, d, s, 256)["ok"]
    outside = np.nextafter((d.astype(np.float64) + b).astype(np.float32), np.float32(np.inf))
    outside = np.where(d.astype(np.float64) + b >= outside, np.nextafter(outside, np.float32(np.inf)), outside)
    r = oracle.check_float(outside, d, s, 256)
    assert not r["ok"] and r["violations"] == d.size


def test_dropped_k_slab_fails():
    M, N, K = 64, 48, 256
    A, B, d, s = setup(M, N, K)
    # zero one 32-wide slab of K in A: what a kernel that skips a k-step computes
    Ac = A.codes.copy()
    Ac[:, 96:128] = 0
    d_bad, _ = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", M, N, K, Ac, A.ld,
                                 B.codes, B.ld)
    r = oracle.check_float(d_bad, d, s, K)
    assert not r["ok"] and r["violations"] > 0.9 * d.size


def test_nan_fails():
    _, _, d, s = setup()
    bad = d.copy()
    bad[3, 7] = np.nan
    r = oracle.check_float(bad, d, s, 256)
    assert not r["ok"] and r["violations"] == 1 and r["first_bad"] == [3 * d.shape[1] + 7]


def test_off_by_one_index_fails():
    _, _, d, s = setup()
    assert not oracle.check_float(np.roll(d, 1, axis=1), d, s, 256)["ok"]
    assert not oracle.check_float(np.roll(d, 1, axis=0), d, s, 256)["ok"]


def test_transposed_operand_fails():
    M = N = K = 64
    A = W.operand("A", "bf16", M, K, "uniform", "k_contig")
    B = W.operand("B", "bf16", K, N, "uniform", "k_contig")
    d, s = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", M, N, K, A.codes, A.ld,
                             B.codes, B.ld)
    # reading A as column-major is what a kernel with swapped A indices computes
    d_t, _ = oracle.gemm_float("bf16", "bf16", "mn_contig", "k_contig", M, N, K, A.codes, A.ld,
                               B.codes, B.ld)
    assert not oracle.check_float(d_t, d, s, K)["ok"]


def test_exact_checker():
    a = np.arange(10, dtype=np.int32)
    assert oracle.check_exact(a, a.copy())["ok"]
    b = a.copy()
    b[4] += 1
    r = oracle.check_exact(b, a)
    assert not r["ok"] and r["first_bad"] == [4]


def test_bound_scales_with_alpha_and_fp8_scales():
    d = np.array([1.0], np.float32)
    s = np.array([10.0])
    b1 = oracle.float_bound(d, s, 100)
    b2 = oracle.float_bound(d, s, 100, alpha=2.0, sA=0.5, sB=4.0)
    u = 2.0 ** -24
    assert np.isclose(b1[0], 4 * u * 102 * 10 + u)
    assert np.isclose(b2[0], 4 * u * 102 * 10 * 4 + u)
