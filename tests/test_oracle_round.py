"""Pins of the oracle's rounding to the output formats (bfloat16, binary16).

The oracle rounds the exact binary64 value of an output element once to the
output format (nearest, ties to even, gradual underflow, overflow to infinity;
format parameters of "Accurate Models of AMD Matrix Cores", Table 1).  These
tests hold that rounding against things other than the oracle itself:
  - a brute-force nearest-value search over every finite value of the format
    (all 2^16 codes, decoded by torch), with exact rational comparisons and
    ties resolved to the code with an even significand;
  - numpy's direct float64 -> float16 conversion as a library witness;
  - closed forms: representable values are fixed points, midpoints between
    neighbours go to the even one, the overflow threshold.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

FMT = {"bf16": torch.bfloat16, "f16": torch.float16}


def finite_table(fmt):
    """Sorted distinct finite values of the format with, for each, whether its
    code has an even significand (its lowest bit clear)."""
    codes = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    vals = codes.view(FMT[fmt]).double().numpy()
    c = codes.numpy().astype(np.uint16)
    keep = np.isfinite(vals)
    vals, c = vals[keep], c[keep]
    order = np.argsort(vals, kind="stable")
    vals, c = vals[order], c[order]
    # +0 and -0 compare equal: keep one entry (both have even significands)
    uniq, first = np.unique(vals, return_index=True)
    return uniq, (c[first] & 1) == 0


def brute_round(fmt, t, table):
    vals, even = table
    big = vals[-1]
    # overflow threshold: the largest finite value plus half its ulp
    ulp_top = float(vals[-1] - vals[-2])
    if abs(t) >= big + ulp_top / 2:
        return np.inf if t > 0 else -np.inf
    i = np.searchsorted(vals, t)
    if i < len(vals) and vals[i] == t:
        return float(vals[i])
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = Fraction(t) - Fraction(float(lo)), Fraction(float(hi)) - Fraction(t)
    if dlo < dhi:
        return float(lo)
    if dhi < dlo:
        return float(hi)
    return float(lo) if even[i - 1] else float(hi)


def random_doubles(fmt, n, seed):
    """Magnitudes log-uniform from deep in the subnormal range to beyond the
    largest finite value, random signs, random low-order bits."""
    g = np.random.default_rng(seed)
    lo, hi = (-140, 129) if fmt == "bf16" else (-27, 17)
    e = g.uniform(lo, hi, n)
    x = np.exp2(e) * g.choice([-1.0, 1.0], n)
    return x


def midpoints(fmt, table, n, seed):
    """Exact midpoints between neighbouring finite values (ties), and values one
    binary64 ulp either side of them."""
    vals, _ = table
    g = np.random.default_rng(seed)
    i = g.integers(0, len(vals) - 1, n)
    mid = (vals[i] + vals[i + 1]) / 2.0  # exact in binary64
    return np.concatenate([mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)])


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_round_matches_brute_force(fmt):
    table = finite_table(fmt)
    x = np.concatenate([random_doubles(fmt, 3000, 1), midpoints(fmt, table, 1000, 2)])
    got = oracle.round_to(fmt, x)
    want = np.array([brute_round(fmt, float(t), table) for t in x])
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_representable_values_are_fixed_points(fmt):
    vals, _ = finite_table(fmt)
    assert np.array_equal(oracle.round_to(fmt, vals), vals)


def test_f16_matches_numpy_conversion():
    x = np.concatenate([random_doubles("f16", 20000, 3),
                        midpoints("f16", finite_table("f16"), 5000, 4)])
    got = oracle.round_to("f16", x)
    with np.errstate(over="ignore"):  # magnitudes beyond 65520 become infinities, as intended
        want = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, want)


def test_ties_to_even_and_overflow_closed_forms():
    # bfloat16: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1 (even)
    assert oracle.round_to("bf16", [1 + 2.0 ** -8])[0] == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6 (even)
    assert oracle.round_to("bf16", [1 + 3 * 2.0 ** -8])[0] == 1 + 2.0 ** -6
    # binary16: largest finite 65504; 65520 is the overflow threshold
    assert oracle.round_to("f16", [65519.99])[0] == 65504.0
    assert np.isinf(oracle.round_to("f16", [65520.0])[0])
    # bfloat16 overflow threshold (2 - 2^-8) * 2^127
    big = (2 - 2.0 ** -7) * 2.0 ** 127
    assert oracle.round_to("bf16", [big])[0] == big
    assert np.isinf(oracle.round_to("bf16", [(2 - 2.0 ** -8) * 2.0 ** 127])[0])
    # binary16 gradual underflow: half the smallest subnormal rounds to 0 (even),
    # three halves of it to two smallest subnormals (even)
    s = 2.0 ** -24
    assert oracle.round_to("f16", [s / 2])[0] == 0.0
    assert oracle.round_to("f16", [1.5 * s])[0] == 2 * s
    # binary32 output keeps the C cast
    assert oracle.round_to("f32", [1 + 2.0 ** -30])[0] == 1.0


def test_gemm_output_rounding_is_single():
    """The GEMM's bfloat16 output is the exact result rounded once, not via
    binary32.  With K = 3 products 1*1 + 1*2^-8 + 1*2^-30 the exact sum
    1 + 2^-8 + 2^-30 lies just above the bfloat16 midpoint 1 + 2^-8, so it
    rounds up to 1 + 2^-7; binary32 would first give 1 + 2^-8 exactly (a tie
    that rounds down to 1)."""
    A = np.array([0x3F80, 0x3F80, 0x3F80], np.uint16)  # bfloat16 1.0 three times
    B = torch.tensor([1.0, 2.0 ** -8, 2.0 ** -30], dtype=torch.float32).to(torch.bfloat16)
    Bc = B.view(torch.int16).numpy().view(np.uint16)
    d, _ = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", 1, 1, 3, A, 3, Bc, 3,
                             out="bf16")
    assert float(d[0, 0]) == 1 + 2.0 ** -7
    d32, _ = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", 1, 1, 3, A, 3, Bc, 3)
    assert float(d32[0, 0]) == float(np.float32(1 + 2.0 ** -8 + 2.0 ** -30))
