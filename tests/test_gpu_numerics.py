"""Numerical features of single gfx950 matrix-core instructions, measured with
targeted test vectors in the manner of "Accurate Models of AMD Matrix Cores"
(Section 3; the CDNA3 feature tests of Section 4.3).  Each vector drives one
output element d = sum_l a_l b_l + c of one instruction through the C ABI's
mcg_mfma_eval; products are fed as exact a_l * b_l.

What these tests pin for gfx950 (CDNA4, not covered by the pages):
  bf16 / f16 (16x16x32 and 32x32x16):
    - products are summed in groups of 8 consecutive operand slots; the group
      result is rounded to binary32 before the next group is added;
    - at least one alignment bit beyond binary32 within a group;
    - the final rounding is to nearest, ties to even;
    - c is aligned to the group's largest product and rounded down (toward
      minus infinity) at the alignment stage;
    - no odd/even interleaving of products.
  fp8 E4M3 / E5M2 (f8f6f4 16x16x128 and 32x32x64):
    - groups of 8 consecutive slots, rounded to binary32 between groups;
    - inside a group, products are aligned to the largest one and truncated
      (toward zero) to 13 fractional bits: a product 2^-14 below the largest
      is lost, one 2^-13 below is kept exactly;
    - c is combined with a group's sum at binary32 precision.
  binary64 (v_mfma_f64_16x16x4_f64 and v_mfma_f64_4x4x4_4b_f64):
    - d is a chain of IEEE binary64 fused multiply-adds in slot order,
      d = fma(a3, b3, fma(a2, b2, fma(a1, b1, fma(a0, b0, c)))), each rounded to
      nearest, ties to even; random test vectors match this model bit for bit.
The last fp8 fact is why the fp8 paths widen to bfloat16 below K = 6144."""
import itertools
from fractions import Fraction

import pytest
import torch

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f16": torch.float16, "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2,
      "f64": torch.float64}
U = 2.0 ** -24


def run(mcg, dt, shape, cases):
    """cases: list of (dict slot -> (a, b), c); returns d per case (python floats)."""
    k = mcg.mfma_eval_k(dt, shape)
    assert k > 0
    n = len(cases)
    A = torch.zeros((n, k), dtype=torch.float64)
    B = torch.zeros((n, k), dtype=torch.float64)
    C = torch.zeros(n, dtype=torch.float64)
    for t, (ps, c) in enumerate(cases):
        for i, (x, y) in ps.items():
            A[t, i], B[t, i] = x, y
        C[t] = c
    if dt == "f64":
        d = torch.full((n,), float("nan"), dtype=torch.float64, device="cuda")
        mcg.mfma_eval(dt, shape, n, A.cuda(), B.cuda(), C.cuda(), d)
        torch.cuda.synchronize()
        return [float(x) for x in d.cpu()]
    Aq, Bq = A.to(TD[dt]), B.to(TD[dt])
    assert torch.equal(Aq.double(), A) and torch.equal(Bq.double(), B), "test inputs not representable"
    assert torch.equal(C.float().double(), C)
    view = torch.int16 if dt in ("bf16", "f16") else torch.uint8
    d = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    mcg.mfma_eval(dt, shape, n, Aq.view(view).cuda(), Bq.view(view).cuda(), C.float().cuda(), d)
    torch.cuda.synchronize()
    return [float(x) for x in d.cpu()]


def prod(p):
    """An exact product p = a * b with a, b representable in bf16 and f16."""
    return (p * 2.0 ** 12, 2.0 ** -12) if abs(p) < 2.0 ** -12 else (p, 1.0)


H16 = [("bf16", 16), ("bf16", 32), ("f16", 16), ("f16", 32)]
F8 = [("e4m3", 16), ("e4m3", 32), ("e5m2", 16), ("e5m2", 32)]


@pytest.mark.parametrize("dt,shape", H16)
def test_final_rounding_nearest_even(dt, shape):
    mcg = need_gpu()
    # 1.5, 0.5 and 2.5 units in the last place above 1: ties go to the even neighbour
    got = run(mcg, dt, shape, [({0: prod(1.0)}, 3 * U), ({0: prod(1.0)}, U), ({0: prod(-1.0)}, -3 * U),
                               ({0: prod(1.0)}, 5 * U), ({0: prod(1.0)}, 7 * U)])
    assert got == [1 + 2 ** -22, 1.0, -(1 + 2 ** -22), 1 + 2 ** -22, 1 + 2 ** -21]


@pytest.mark.parametrize("dt,shape", H16)
def test_c_alignment_rounds_down(dt, shape):
    """c = +-1.5 * 2^-24 against a product +-1: bits of c below the window are
    rounded toward minus infinity before the sum is rounded to nearest."""
    mcg = need_gpu()
    got = run(mcg, dt, shape, [({0: prod(1.0)}, 1.5 * U), ({0: prod(-1.0)}, -1.5 * U)])
    assert got == [1.0, -(1 + 2 ** -23)]


@pytest.mark.parametrize("dt,shape", H16)
def test_extra_alignment_bit(dt, shape):
    """1, 2^-24, 2^-24 in any placement over c, p1, p2 give 1 + 2^-23."""
    mcg = need_gpu()
    cases = []
    for c, p1, p2 in set(itertools.permutations([1.0, U, U])):
        cases.append(({0: prod(p1), 1: prod(p2)}, c))
    assert all(d == 1 + 2 * U for d in run(mcg, dt, shape, cases))


@pytest.mark.parametrize("dt,shape", H16)
def test_groups_of_eight_rounded_between(dt, shape):
    """c = 1, p0 = pj = 2^-24: the two small products only survive together
    when they share a group of 8 slots (j < 8)."""
    mcg = need_gpu()
    k = mcg.mfma_eval_k(dt, shape)
    got = run(mcg, dt, shape, [({0: prod(U), j: prod(U)}, 1.0) for j in range(1, k)])
    together = [j for j, d in zip(range(1, k), got) if d == 1 + 2 * U]
    say(f"{dt} {shape}: p0 and pj summed exactly for j in {together}")
    assert together == list(range(1, 8))
    assert all(d == 1.0 for j, d in zip(range(1, k), got) if j >= 8)


@pytest.mark.parametrize("dt,shape", H16)
def test_no_interleaving(dt, shape):
    mcg = need_gpu()
    cases = []
    for sgn in (1.0, -1.0):
        for perm in set(itertools.permutations([1.0, 0.0, U + U / 2])):
            cases.append(({i: prod(sgn * x) for i, x in enumerate(perm)}, 0.0))
    got = run(mcg, dt, shape, cases)
    assert got[:len(got) // 2] == [1.0] * (len(got) // 2)
    assert got[len(got) // 2:] == [-1.0] * (len(got) // 2)


def f8prod(e):
    """An exact fp8 product 2^-e (e <= 18) for both E4M3 and E5M2."""
    ea = min(e // 2, 9)
    return (2.0 ** -ea, 2.0 ** -(e - ea))


@pytest.mark.parametrize("dt,shape", F8)
def test_fp8_groups_of_eight(dt, shape):
    """p0 = 1, pj = 2^-14: lost inside p0's group, kept from the next group on."""
    mcg = need_gpu()
    k = mcg.mfma_eval_k(dt, shape)
    got = run(mcg, dt, shape, [({0: (1.0, 1.0), j: f8prod(14)}, 0.0) for j in range(1, k)])
    assert all(d == 1.0 for j, d in zip(range(1, k), got) if j < 8)
    assert all(d == 1.0 + 2.0 ** -14 for j, d in zip(range(1, k), got) if j >= 8)


@pytest.mark.parametrize("dt,shape", F8)
def test_fp8_group_window_13_bits_truncating(dt, shape):
    """Inside a group, a product 2^-e below the largest survives exactly for
    e <= 13 and is dropped (toward zero, either sign) for e >= 14."""
    mcg = need_gpu()
    es = list(range(6, 19))
    cases = [({0: (1.0, 1.0), 1: (s * f8prod(e)[0], f8prod(e)[1])}, 0.0) for s in (1.0, -1.0) for e in es]
    got = run(mcg, dt, shape, cases)
    want = [1.0 + s * 2.0 ** -e if e <= 13 else 1.0 for s in (1.0, -1.0) for e in es]
    assert got == want


@pytest.mark.parametrize("dt,shape", F8)
def test_fp8_c_keeps_binary32_precision(dt, shape):
    """c = 1 with a single product 2^-e: the product is kept exactly for every
    e up to 18 (the group sum meets c at binary32 precision)."""
    mcg = need_gpu()
    es = list(range(6, 19))
    got = run(mcg, dt, shape, [({0: f8prod(e)}, 1.0) for e in es])
    assert got == [1.0 + 2.0 ** -e for e in es]


F64 = [("f64", 16), ("f64", 4)]


def fma_chain(a, b, c):
    """binary64 fused multiply-adds in slot order, each correctly rounded (Python's
    Fraction -> float conversion rounds to nearest, ties to even)."""
    d = c
    for x, y in zip(a, b):
        d = float(Fraction(x) * Fraction(y) + Fraction(d))
    return d


@pytest.mark.parametrize("dt,shape", F64)
def test_f64_products_fused(dt, shape):
    """(1 + 2^-30)^2 - (1 + 2^-29) = 2^-60 exactly: the product is not rounded."""
    mcg = need_gpu()
    e = 1 + 2.0 ** -30
    assert run(mcg, dt, shape, [({0: (e, e)}, -(1 + 2.0 ** -29))]) == [2.0 ** -60]


@pytest.mark.parametrize("dt,shape", F64)
def test_f64_sequential_order_and_ties(dt, shape):
    """Every order of the products 2^53, -2^53, 1, 1 (and c = 2^53 against 1, -2^53
    in every pair of slots) gives the result of rounding after each slot in slot
    order; 1 + 2^-53 ties to 1, 1 + 3 * 2^-53 to 1 + 2^-51, two 2^-53 added to 1
    one after the other are both lost."""
    mcg = need_gpu()
    E = 2.0 ** 53
    cases = [({i: (v, 1.0) for i, v in enumerate(perm)}, 0.0) for perm in sorted(set(itertools.permutations([E, -E, 1.0, 1.0])))]
    for j in range(4):
        for k in range(4):
            if j != k:
                cases.append(({j: (1.0, 1.0), k: (-E, 1.0)}, E))
    u = 2.0 ** -53
    cases += [({0: (u, 1.0), 1: (u, 1.0)}, 1.0), ({0: (1.0, 1.0)}, u), ({0: (1.0, 1.0)}, 3 * u),
              ({0: (1.0, 1.0), 1: (2.0 ** -80, 1.0)}, u)]
    got = run(mcg, dt, shape, cases)
    want = []
    for ps, c in cases:
        a = [ps.get(i, (0.0, 0.0))[0] for i in range(4)]
        b = [ps.get(i, (0.0, 0.0))[1] for i in range(4)]
        want.append(fma_chain(a, b, c))
    assert got == want
    assert got[-4:] == [1.0, 1.0, 1 + 2.0 ** -51, 1.0]


@pytest.mark.parametrize("dt,shape", F64)
def test_f64_random_vectors_match_fma_chain(dt, shape):
    """Random vectors (signs random, exponents over 2^-40 .. 2^40, c likewise):
    every result equals the binary64 fused multiply-add chain in slot order."""
    mcg = need_gpu()
    n = 20000
    g = torch.Generator().manual_seed(4242 + shape)
    def draw(shape_):
        m = torch.rand(shape_, generator=g, dtype=torch.float64) + 1.0
        e = torch.randint(-20, 21, shape_, generator=g).to(torch.float64)
        sgn = torch.randint(0, 2, shape_, generator=g).to(torch.float64) * 2 - 1
        return sgn * m * torch.pow(2.0, e)
    A, B, C = draw((n, 4)), draw((n, 4)), draw((n,))
    d = torch.full((n,), float("nan"), dtype=torch.float64, device="cuda")
    mcg.mfma_eval(dt, shape, n, A.cuda(), B.cuda(), C.cuda(), d)
    torch.cuda.synchronize()
    got = d.cpu().tolist()
    a, b, c = A.tolist(), B.tolist(), C.tolist()
    bad = [t for t in range(n) if got[t] != fma_chain(a[t], b[t], c[t])]
    say(f"{dt} {shape}: {len(bad)} of {n} random vectors differ from the fma chain")
    assert not bad, bad[:5]


def test_eval_rejects_unsupported():
    mcg = need_gpu()
    assert mcg.mfma_eval_k("i8", 16) == 0
    assert mcg.mfma_eval_k("bf16", 8) == 0
    assert mcg.mfma_eval_k("bf16", 4) == 0
    assert mcg.mfma_eval_k("f64", 32) == 0
    assert mcg.mfma_eval_k("f64", 4) == 4 and mcg.mfma_eval_k("f64", 16) == 4
    with pytest.raises(mcg.MCGError):
        mcg.mfma_eval("i8", 16, 1, None, None, None, None)
