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


# ---------------------------------------------------------------------------
# 16-bit outputs.  A bfloat16 / binary16 D is the kernel's binary32 result y
# (|y - x| <= e, x the exact value, e the binary32 bound) rounded once more,
# while the oracle's D_ref is x rounded once to the same format.  Both
# roundings are at most half an ulp of the output format (u_out |.| in the
# normal range, half the smallest subnormal below it), so a correct D lies
# within e + u_out (2 |D_ref| + e) + 2 h of D_ref; with precision p (Table 1
# of "Accurate Models of AMD Matrix Cores": 8 for bfloat16, 11 for binary16)
# u_out = 2^-p.  At D_ref = 1 that is one ulp above 1 (2^(1-p)) plus e, so a
# correct D is at most one ulp away there, and two ulps must fail.

FMT = {"bf16": (8, -133), "f16": (11, -24)}  # precision, exponent of the smallest subnormal


def _round16(x, out):
    """Round binary64 values once to the 16-bit output format (nearest even),
    through numpy / bit arithmetic that does not use the oracle."""
    x = np.asarray(x, np.float64)
    if out == "f16":
        return x.astype(np.float16).astype(np.float64)
    # bfloat16: round the binary32 image to nearest even on its top 16 bits;
    # first round binary64 -> binary32 by truncation plus a sticky bit so the
    # result is a single rounding of x (x is representable in 31 bits here)
    f = x.astype(np.float32)
    assert np.all(f.astype(np.float64) == x), "test values must be exact in binary32"
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_bound_16bit_hand_value():
    # D_ref = 1, S = 1, K = 2: e = 4u(K+2) S + u |D_ref| = 17 u (u = 2^-24)
    u = 2.0 ** -24
    e = 17 * u
    for out, (p, emin) in FMT.items():
        uo = 2.0 ** -p
        h = 2.0 ** (emin - 1)
        b = oracle.float_bound(np.array([1.0]), np.array([1.0]), 2, out=out)[0]
        assert b == e + uo * (2.0 + e) + 2 * h, (out, b)
        # one ulp above 1 plus e: the bound admits exactly one ulp of the format
        assert 2.0 ** (1 - p) < b < 2.0 ** (1 - p) + 2.0 ** (-p)


def test_bound_16bit_one_ulp_passes_two_ulps_fail():
    for out, (p, _) in FMT.items():
        ulp = 2.0 ** (1 - p)                   # ulp of [1, 2)
        ref = np.array([1.0, 1.0, -1.0, 1.5])
        S = np.array([1.0, 1.0, 1.0, 1.5])
        # below 1 the format's ulp halves: 1 - ulp is two of its steps away but
        # still one ulp of [1, 2) in distance, which is what the bound measures
        one = np.array([1.0 + ulp, 1.0 - ulp, -1.0 - ulp, 1.5 + ulp])
        two = np.array([1.0 + 2 * ulp, 1.0 - 1.5 * ulp, -1.0 - 2 * ulp, 1.5 + 2 * ulp])
        assert oracle.check_float(one, ref, S, 2, out=out)["ok"], out
        r = oracle.check_float(two, ref, S, 2, out=out)
        assert r["violations"] == 4, (out, r)


def test_bound_16bit_subnormal_range():
    # D_ref = 0 with S = 0: the kernel's binary32 result is exact, and one
    # smallest subnormal is the most two roundings can move it; two fail
    for out, (p, emin) in FMT.items():
        sub = 2.0 ** emin
        zero = np.zeros(2)
        assert oracle.check_float(np.array([sub, -sub]), zero, zero, 8, out=out)["ok"]
        assert oracle.check_float(np.array([2 * sub, -2 * sub]), zero, zero, 8, out=out)["violations"] == 2


def test_bound_16bit_admits_every_double_rounding():
    # exact values x just below / above a midpoint of the 16-bit format; every
    # binary32 result y within the binary32 bound e of x, rounded once more,
    # must pass -- including the cases where y and x round to different
    # neighbours (the double rounding the bound accounts for)
    rng = np.random.default_rng(5)
    for out, (p, _) in FMT.items():
        ulp = 2.0 ** (1 - p)
        n = 4000
        base = 1.0 + rng.integers(0, 2 ** (p - 1), n) * ulp          # representable in [1, 2)
        S = rng.uniform(0.5, 4.0, n)
        K = 64
        e = 4 * 2.0 ** -24 * (K + 2) * S + 2.0 ** -24 * 2.0
        off = rng.uniform(-1, 1, n) * e
        x = base + ulp / 2 + np.where(rng.integers(0, 2, n) == 1, 1, -1) * rng.uniform(0, 1, n) * e
        x = x.astype(np.float32).astype(np.float64)                   # exact value, binary32-representable
        y = (x + off).astype(np.float32).astype(np.float64)           # a kernel's binary32 result
        y = np.clip(y, x - e, x + e)
        y = np.where(np.abs(y - x) <= e, y, x)
        d_gpu = _round16(y, out)
        d_ref = _round16(x, out)
        flips = int(np.sum(d_gpu != d_ref))
        assert flips > n // 10, (out, flips)                          # the adversarial case occurs
        r = oracle.check_float(d_gpu, d_ref, S, K, out=out)
        assert r["ok"], (out, r)
