"""Randomised test vectors for single matrix-core instructions, and the Bayesian
bound on the mismatch probability of a model of them.

Follows "Accurate Models of AMD Matrix Cores", Section 5:
  - exponent-mantissa sampling (Section 5.1, Algorithm 3): every element is
    s * 2^e with the exponent e an integer drawn uniformly between per-operand
    limits and the significand s drawn uniformly from [-2 + 2^(1-f), 2 - 2^(1-f)]
    on the format's significand grid (f = precision of the format, Table 1), from
    a Mersenne Twister (MT19937) seeded with 0;
  - independent bit sampling (Section 5.2): every bit of every code is an
    independent fair coin; a code that decodes to an infinity or a NaN gets its
    exponent field drawn again;
  - the bound (Section 5.4): with N samples and m mismatches under a uniform prior,
    the posterior of the mismatch probability is Beta(m + 1, N - m + 1); the
    epsilon-upper bound p_eps solves P(p < p_eps) = 1 - eps, which for m = 0 is
    p_eps = 1 - eps^(1 / (N + 1)).

Test infrastructure only: this module draws inputs; the library under test never
sees anything but the codes it produces.
"""
from __future__ import annotations

import math

import numpy as np

# format -> (precision f, exponent bits, mantissa bits, bias, numpy code type)
FORMATS = {
    "bf16": (8, 8, 7, 127, np.uint16),
    "f16": (11, 5, 10, 15, np.uint16),
    "e4m3": (4, 4, 3, 7, np.uint8),
    "e5m2": (3, 5, 2, 15, np.uint8),
}


def rng(seed: int = 0) -> np.random.Generator:
    """The Mersenne Twister of Algorithm 3 (MT19937, seed 0 by default)."""
    return np.random.Generator(np.random.MT19937(seed))


def _decode(fmt: str, codes: np.ndarray) -> np.ndarray:
    """Exact values of codes (binary64), including subnormals; NaN/Inf as such."""
    f, eb, mb, bias, _ = FORMATS[fmt]
    c = codes.astype(np.int64)
    sign = np.where((c >> (eb + mb)) & 1, -1.0, 1.0)
    e = (c >> mb) & ((1 << eb) - 1)
    m = c & ((1 << mb) - 1)
    val = np.where(e == 0, m * 2.0 ** (1 - bias - mb), (m + (1 << mb)) * 2.0 ** (e.astype(np.float64) - bias - mb))
    special = _is_special(fmt, codes)
    return np.where(special, np.nan, sign * val)


def _is_special(fmt: str, codes: np.ndarray) -> np.ndarray:
    f, eb, mb, bias, _ = FORMATS[fmt]
    c = codes.astype(np.int64)
    e = (c >> mb) & ((1 << eb) - 1)
    m = c & ((1 << mb) - 1)
    if fmt == "e4m3":  # OCP E4M3: only S.1111.111 is special (NaN)
        return (e == (1 << eb) - 1) & (m == (1 << mb) - 1)
    return e == (1 << eb) - 1


def _encode_exact(fmt: str, x: np.ndarray) -> np.ndarray:
    """Codes of values that are exactly representable in `fmt` (asserted)."""
    f, eb, mb, bias, ct = FORMATS[fmt]
    out = np.zeros(x.shape, np.int64)
    sign = (x < 0).astype(np.int64)
    a = np.abs(x)
    nz = a > 0
    e = np.zeros(x.shape, np.int64)
    e[nz] = np.floor(np.log2(a[nz])).astype(np.int64)
    emin = 1 - bias
    sub = nz & (e < emin)
    # normal: exponent field e + bias, mantissa (a / 2^e - 1) * 2^mb
    ef = np.where(sub | ~nz, 0, e + bias)
    m = np.where(sub, a / 2.0 ** (emin - mb), a / np.where(nz, 2.0 ** e.astype(np.float64), 1.0) * 2 ** mb - 2 ** mb)
    m = np.where(nz, m, 0.0)
    assert np.all(m == np.round(m)), "value not representable in the format"
    out = (sign << (eb + mb)) | (ef << mb) | m.astype(np.int64)
    back = _decode(fmt, out.astype(ct))
    assert np.array_equal(back, x), "encoding is not exact"
    return out.astype(ct)


def exponent_mantissa(fmt: str, n: int, k: int, ea: tuple[int, int], eb_: tuple[int, int], ec: tuple[int, int],
                      gen: np.random.Generator):
    """Algorithm 3: n test vectors of k elements of a and of b in `fmt`, and n binary32
    accumulators c.  Exponents are uniform integers in [lo, hi]; significands are
    uniform on the grid m * 2^(1 - f), |m| <= 2^f - 1 (the range [-2 + 2^(1-f),
    2 - 2^(1-f)]); values below the format's smallest subnormal spacing are
    rounded to it (nearest even) so that every element is a code of the format.
    Returns (codes_a (n, k), codes_b (n, k), c float32 (n,))."""
    f = FORMATS[fmt][0]

    def draw(lo, hi, shape):
        e = gen.integers(lo, hi + 1, size=shape)
        m = gen.integers(-(2 ** f - 1), 2 ** f, size=shape)
        return m.astype(np.float64) * np.exp2((e - (f - 1)).astype(np.float64))

    def to_codes(x):
        _, ebits, mb, bias, _ = FORMATS[fmt]
        q = 2.0 ** (1 - bias - mb)  # smallest subnormal: values snap to its multiples
        x = np.where(np.abs(x) < 2.0 ** (1 - bias), np.round(x / q) * q, x)  # numpy rounds half to even
        return _encode_exact(fmt, x)

    a = to_codes(draw(*ea, (n, k)))
    b = to_codes(draw(*eb_, (n, k)))
    e = gen.integers(ec[0], ec[1] + 1, size=n)
    m = gen.integers(-(2 ** 24 - 1), 2 ** 24, size=n)
    c = (m.astype(np.float64) * np.exp2((e - 23).astype(np.float64))).astype(np.float32)
    return a, b, c


def independent_bits(fmt: str, n: int, k: int, gen: np.random.Generator, emax: int | None = None):
    """Section 5.2: every bit of every code a fair coin; codes that decode to an
    infinity or a NaN get a fresh exponent field until they do not.  c is drawn
    the same way as a binary32 bit pattern.  emax (optional) also redraws
    exponent fields whose unbiased exponent exceeds it (bfloat16 products of
    random bit patterns would otherwise overflow binary32 in most vectors)."""
    _, ebits, mb, bias, ct = FORMATS[fmt]
    width = 1 + ebits + mb

    def draw(shape):
        c = gen.integers(0, 2 ** width, size=shape, dtype=np.int64)
        while True:
            bad = _is_special(fmt, c.astype(ct))
            if emax is not None:
                bad = bad | (((c >> mb) & ((1 << ebits) - 1)) - bias > emax)
            if not bad.any():
                return c.astype(ct)
            newe = gen.integers(0, 2 ** ebits, size=int(bad.sum()), dtype=np.int64)
            c[bad] = (c[bad] & ~(((1 << ebits) - 1) << mb)) | (newe << mb)

    a, b = draw((n, k)), draw((n, k))
    cbits = gen.integers(0, 2 ** 32, size=n, dtype=np.int64)
    while True:
        bad = ((cbits >> 23) & 0xFF) == 0xFF
        if not bad.any():
            break
        cbits[bad] = (cbits[bad] & ~(0xFF << 23)) | (gen.integers(0, 256, size=int(bad.sum()), dtype=np.int64) << 23)
    c = cbits.astype(np.uint32).view(np.float32)
    return a, b, c


def decode(fmt: str, codes: np.ndarray) -> np.ndarray:
    return _decode(fmt, codes)


def bayes_upper_bound(n: int, m: int, eps: float = 1e-6) -> float:
    """Smallest p with P(p_S < p | n samples, m mismatches) >= 1 - eps under a
    uniform prior (the Beta(m + 1, n - m + 1) posterior).  m = 0 has the closed
    form 1 - eps^(1 / (n + 1)); otherwise the regularised incomplete beta function
    is inverted by bisection."""
    if m == 0:
        return 1.0 - math.exp(math.log(eps) / (n + 1))
    from scipy.special import betainc
    lo, hi = 0.0, 1.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if betainc(m + 1, n - m + 1, mid) >= 1 - eps:
            hi = mid
        else:
            lo = mid
    return hi
