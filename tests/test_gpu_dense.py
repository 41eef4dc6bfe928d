"""GPU parity of gemm_dense against the CPU oracle (MI355X).

Float paths must satisfy |D_gpu - D_ref| <= 4*2^-24*(K+2)*|alpha*sA*sB|*S + 2^-24*|D_ref|
element-wise (S = sum_k |a_ik b_kj|); int8 must be bit-exact; inputs whose
partial sums are all exactly representable must be bit-exact on every path.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import compare, dev, need_gpu, oracle_dense, run_dense, say

pytestmark = pytest.mark.gpu

PAIRS = [("bf16", "bf16"), ("f16", "f16"), ("i8", "i8"), ("e4m3", "e4m3"), ("e4m3", "e5m2"),
         ("e5m2", "e4m3"), ("e5m2", "e5m2")]
LAYOUTS = [("k_contig", "k_contig"), ("k_contig", "mn_contig"), ("mn_contig", "k_contig"),
           ("mn_contig", "mn_contig")]


SMALL = {"bf16": 8, "f16": 8, "e4m3": 16, "e5m2": 8}


def operands(dtA, dtB, layA, layB, M, N, K, dist=None, pad=0, seed=0, scaled=True):
    dist = dist or ("int8" if dtA == "i8" else "normal")
    fp8 = scaled and dtA in ("e4m3", "e5m2")
    ldA = (K if layA == "k_contig" else M) + pad
    ldB = (K if layB == "k_contig" else N) + pad
    A = W.operand("A", dtA, M, K, dist, layA, seed=10 * seed, ld=ldA, fp8_scaled=fp8)
    B = W.operand("B", dtB, K, N, dist, layB, seed=10 * seed + 1, ld=ldB, fp8_scaled=fp8)
    return A, B


def check_case(mcg, dtA, dtB, layA, layB, M, N, K, pad=0, beta=1.0, alpha=None, ldc_pad=0, seed=0,
               dist=None, expect_path=None):
    say(f"case {dtA}x{dtB} {layA}/{layB} M={M} N={N} K={K} pad={pad} beta={beta}")
    A, B = operands(dtA, dtB, layA, layB, M, N, K, dist, pad, seed)
    ldc = N + ldc_pad
    i8 = dtA == "i8"
    if alpha is None:
        alpha = 3 if i8 else 1.5
    C = None
    if beta != 0:
        C = W.c_matrix(M, N, "int20" if i8 else "normal", seed=10 * seed + 2, ldc=ldc)
    d = run_dense(mcg, dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc, alpha,
                  beta, A.scale, B.scale, expect_path=expect_path)
    ref, s = oracle_dense(dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc,
                          alpha, beta, A.scale, B.scale)
    compare(dtA, d[:M, :N], ref, s, K, alpha, A.scale, B.scale, beta,
            None if C is None else C[:M, :N], what=f"{dtA}x{dtB} {layA}/{layB} {M}x{N}x{K}")
    if ldc_pad:  # padding columns of D untouched
        if i8:
            assert np.all(d[:M, N:] == -0x5A5A5A5A)
        else:
            assert np.all(np.isnan(d[:M, N:]))


def test_config_bf16_256_cubed():
    """bf16 256^3, A row-major, B column-major, C = 0, alpha = 1, beta = 0,
    entries uniform in [-1, 1] rounded to bf16: full comparison."""
    mcg = need_gpu()
    wl = W.standard_workloads()[0]
    A = W.operand("A", "bf16", 256, 256, "uniform", "k_contig")
    B = W.operand("B", "bf16", 256, 256, "uniform", "k_contig")
    d = run_dense(mcg, "bf16", "bf16", "k_contig", "k_contig", 256, 256, 256, A.codes, A.ld,
                  B.codes, B.ld)
    ref, s = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", 256, 256, 256, A.codes,
                               A.ld, B.codes, B.ld)
    r = compare("bf16", d, ref, s, 256, what=wl.name)
    say("config bf16 256^3 max |delta|/bound", r["max_ratio"])


@pytest.mark.parametrize("dtA,dtB", PAIRS)
@pytest.mark.parametrize("layA,layB", LAYOUTS)
def test_multi_tile_ragged(dtA, dtB, layA, layB):
    """Several tiles with ragged tails in M, N and K (vector-load path)."""
    mcg = need_gpu()
    check_case(mcg, dtA, dtB, layA, layB, 300, 200, 300, pad=20, ldc_pad=4, expect_path=0)


# Shapes taken by the 256 x 256 kernel for every dtype and layout (at least 128
# output tiles of 256 x 256, K and every leading dimension a multiple of 16
# elements): ragged M and N tiles, K ending inside a 128-byte stage, a single
# partial stage, padded leading dimensions.  Outputs are compared on every
# element of the rows and columns at tile boundaries and 4096 random ones.
FAST_SHAPES = [(2832, 3088, 208, 16), (3072, 2832, 80, 0), (2320, 3344, 1040, 32)]


def tile_edges(n, t=256):
    """First and last index of the first tile, of the last whole tile, and of the
    ragged tail (when there is one)."""
    last = (n // t) * t
    e = {0, t - 1, t, last - 1, n - 1}
    if last < n:
        e.add(last)
    return tuple(sorted(x for x in e if 0 <= x < n))


def check_case_sampled(mcg, dtA, dtB, layA, layB, M, N, K, pad=0, ldc_pad=0, seed=0, dist=None,
                       alpha=None, beta=1.0, expect_path=None, exact=False):
    say(f"sampled case {dtA}x{dtB} {layA}/{layB} M={M} N={N} K={K} pad={pad}")
    # exact checks use the small integers unscaled (fp8 scaling would make them inexact)
    A, B = operands(dtA, dtB, layA, layB, M, N, K, dist, pad, seed, scaled=not exact)
    ldc = N + ldc_pad
    i8 = dtA == "i8"
    alpha = (3 if i8 else 1.5) if alpha is None else alpha
    C = None
    if beta != 0:
        C = W.c_matrix(M, N, "int20" if i8 else "normal", seed=10 * seed + 2, ldc=ldc)
        if exact and not i8:
            C = np.round(C * 1000).astype(np.float32)
    d = run_dense(mcg, dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc, alpha,
                  beta, A.scale, B.scale, expect_path=expect_path)
    rows, cols = W.sample_coords(M, N, n_random=4096, full_rows=tile_edges(M), full_cols=tile_edges(N))
    ref, s = oracle_dense(dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc,
                          alpha, beta, A.scale, B.scale, rows, cols)
    if exact:
        assert np.array_equal(d[rows, cols], ref)
    else:
        compare(dtA, d[rows, cols], ref, s, K, alpha, A.scale, B.scale, beta,
                None if C is None else C[rows, cols], what=f"{dtA}x{dtB} {layA}/{layB} {M}x{N}x{K}")
    if ldc_pad:  # padding columns of D untouched
        if i8:
            assert np.all(d[:M, N:] == -0x5A5A5A5A)
        else:
            assert np.all(np.isnan(d[:M, N:]))


@pytest.mark.parametrize("dtA,dtB", PAIRS)
@pytest.mark.parametrize("layA,layB", LAYOUTS)
@pytest.mark.parametrize("shape", FAST_SHAPES, ids=["2832x3088x208", "3072x2832x80", "2320x3344x1040"])
def test_256_tile_path_ragged(dtA, dtB, layA, layB, shape):
    mcg = need_gpu()
    M, N, K, pad = shape
    check_case_sampled(mcg, dtA, dtB, layA, layB, M, N, K, pad=pad, ldc_pad=4, seed=3, expect_path=1)


@pytest.mark.parametrize("dtA,dtB", PAIRS)
def test_256_tile_path_every_output(dtA, dtB):
    """One ragged shape of the 256 x 256 kernel per input pair (the layout pair
    rotates over the input pairs), compared with the oracle on every output."""
    mcg = need_gpu()
    layA, layB = LAYOUTS[PAIRS.index((dtA, dtB)) % len(LAYOUTS)]
    M, N, K, pad = FAST_SHAPES[0]
    check_case(mcg, dtA, dtB, layA, layB, M, N, K, pad=pad, ldc_pad=4, seed=31, expect_path=1)


# Shapes taken by the 128 x 128 form of the same kernel (too few 256 x 256 tiles to
# fill the chip, K long enough for it to beat the general kernel): ragged M and N
# tiles, K ending inside a stage, padded leading dimensions.
MID_SHAPES = [(1936, 1808, 2064, 16), (1040, 2064, 2080, 32), (2000, 1008, 2128, 0)]


@pytest.mark.parametrize("dtA,dtB", PAIRS)
@pytest.mark.parametrize("layA,layB", LAYOUTS)
@pytest.mark.parametrize("shape", MID_SHAPES, ids=["1936x1808x2064", "1040x2064x2080", "2000x1008x2128"])
def test_128_tile_path_ragged(dtA, dtB, layA, layB, shape):
    mcg = need_gpu()
    M, N, K, pad = shape
    check_case_sampled(mcg, dtA, dtB, layA, layB, M, N, K, pad=pad, ldc_pad=4, seed=23, expect_path=6)


@pytest.mark.parametrize("dtA,dtB", [p for p in PAIRS if p[0] != "i8"])
@pytest.mark.parametrize("layA,layB", LAYOUTS)
def test_small_integers_bit_exact_128_tiles(dtA, dtB, layA, layB):
    """Exactly representable partial sums on the 128 x 128 form (ragged M and N, K
    ending inside a stage): the sampled outputs must equal the oracle bit for bit."""
    mcg = need_gpu()
    M, N, K = 1808, 1808, 2128
    r = min(SMALL[dtA], SMALL[dtB])
    check_case_sampled(mcg, dtA, dtB, layA, layB, M, N, K, seed=25, dist=f"smallint{r}", alpha=1.0,
                       beta=1.0, expect_path=6, exact=True)


FP8_PAIRS = [p for p in PAIRS if p[0] in ("e4m3", "e5m2")]


@pytest.mark.parametrize("dtA,dtB", FP8_PAIRS)
@pytest.mark.parametrize("layA,layB", LAYOUTS)
@pytest.mark.parametrize("exact", [False, True], ids=["normal", "smallint"])
def test_128_tile_fp8_native(dtA, dtB, layA, layB, exact):
    """K = 6160 (ragged, past 6144): the 128 x 128 form with the native fp8 instruction
    (32 bytes of K per lane); N(0,1) within the bound, small integers bit for bit."""
    mcg = need_gpu()
    r = min(SMALL[dtA], SMALL[dtB])
    check_case_sampled(mcg, dtA, dtB, layA, layB, 1040, 1168, 6160, pad=16, ldc_pad=4, seed=27,
                       dist=f"smallint{r}" if exact else None, alpha=1.0 if exact else None,
                       expect_path=6, exact=exact)


@pytest.mark.parametrize("dtA,dtB", [p for p in PAIRS if p[0] != "i8"])
@pytest.mark.parametrize("layA,layB", LAYOUTS)
def test_small_integers_bit_exact_256_tiles(dtA, dtB, layA, layB):
    """Exactly representable partial sums on the 256 x 256 kernel (ragged M and N,
    K ending inside a stage): the sampled outputs must equal the oracle bit for bit."""
    mcg = need_gpu()
    M, N, K = 2832, 2832, 1104
    r = min(SMALL[dtA], SMALL[dtB])
    check_case_sampled(mcg, dtA, dtB, layA, layB, M, N, K, seed=15, dist=f"smallint{r}", alpha=1.0,
                       beta=1.0, expect_path=1, exact=True)


@pytest.mark.parametrize("dtA,dtB", PAIRS)
@pytest.mark.parametrize("shape", [(1, 1, 1), (17, 33, 65), (255, 257, 129), (64, 48, 3)])
def test_small_odd_shapes_element_path(dtA, dtB, shape):
    """Odd sizes with unpadded leading dimensions take the element-load path."""
    mcg = need_gpu()
    M, N, K = shape
    for layA, layB in LAYOUTS:
        check_case(mcg, dtA, dtB, layA, layB, M, N, K, pad=0)


@pytest.mark.parametrize("dtA,dtB", PAIRS)
def test_beta_zero_and_alpha(dtA, dtB):
    mcg = need_gpu()
    check_case(mcg, dtA, dtB, "k_contig", "k_contig", 130, 140, 256, beta=0.0)
    check_case(mcg, dtA, dtB, "mn_contig", "k_contig", 130, 140, 256, beta=-2 if dtA == "i8" else 0.5,
               alpha=-1 if dtA == "i8" else -0.25)


@pytest.mark.parametrize("dtA,dtB", [p for p in PAIRS if p[0] != "i8"])
@pytest.mark.parametrize("layA,layB", LAYOUTS)
def test_small_integers_bit_exact(dtA, dtB, layA, layB):
    """Integer-valued inputs with all partial sums below 2^24: any accumulation
    order or alignment scheme gives the exact result, so the GPU must match the
    oracle bit for bit."""
    mcg = need_gpu()
    M, N, K = 192, 160, 512
    r = min(SMALL[dtA], SMALL[dtB])
    A = W.operand("A", dtA, M, K, f"smallint{r}", layA, seed=5)
    B = W.operand("B", dtB, K, N, f"smallint{r}", layB, seed=6)
    C = np.round(W.c_matrix(M, N, "normal", seed=7) * 1000).astype(np.float32)
    d = run_dense(mcg, dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, N, 1.0, 1.0)
    ref, _ = oracle.gemm_float(dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, N,
                               1.0, 1.0)
    assert np.array_equal(d, ref)


@pytest.mark.parametrize("dt", ["bf16", "f16", "i8", "e4m3"])
@pytest.mark.parametrize("layA,layB", LAYOUTS)
def test_permutation_bit_exact(dt, layA, layB):
    """D = P.B (+ C): every output is one input value (plus C), rounded once."""
    mcg = need_gpu()
    n, N = 256, 136
    perm = np.random.default_rng(3).permutation(n)
    Pm = torch.zeros((n, n), dtype=torch.float32)
    Pm[torch.arange(n), torch.from_numpy(perm)] = 1.0
    Pq, _ = W.quantize(Pm if dt != "i8" else Pm.to(torch.int64), dt)
    Ps, lda = W.store(Pq, "A", layA)
    B = W.operand("B", dt, n, N, "int8" if dt == "i8" else "normal", layB, seed=8)
    C = W.c_matrix(n, N, "int20" if dt == "i8" else "normal", seed=9)
    d = run_dense(mcg, dt, dt, layA, layB, n, N, n, W.codes_of(Ps, dt), lda, B.codes, B.ld, C, N,
                  1, 1)
    ref, _ = oracle_dense(dt, dt, layA, layB, n, N, n, W.codes_of(Ps, dt), lda, B.codes, B.ld, C, N,
                          1, 1)
    assert np.array_equal(d, ref)


def test_every_output_written_and_c_not_read_when_beta_zero():
    mcg = need_gpu()
    M, N, K = 333, 222, 96
    A, B = operands("bf16", "bf16", "k_contig", "k_contig", M, N, K)
    c_nan = torch.full((M, N), float("nan"), device="cuda")
    d = run_dense(mcg, "bf16", "bf16", "k_contig", "k_contig", M, N, K, A.codes, A.ld, B.codes,
                  B.ld, None, N, 1.0, 0.0, c_dev=c_nan)
    assert not np.isnan(d).any()


def test_k_zero_gives_beta_c_and_m_zero_is_noop():
    mcg = need_gpu()
    M, N = 70, 90
    C = W.c_matrix(M, N, "normal")
    A = np.zeros((M, 8), np.uint16)
    B = np.zeros((N, 8), np.uint16)
    d = run_dense(mcg, "bf16", "bf16", "k_contig", "k_contig", M, N, 0, A, 8, B, 8, C, N, 1.0, 2.0)
    assert np.array_equal(d, (2.0 * C).astype(np.float32))
    D = torch.full((4, 4), 7.0, device="cuda")
    mcg.gemm_dense("bf16", "bf16", 0, 0, 0, 4, 4, None, 4, None, 4, None, D, 4, "f32")
    torch.cuda.synchronize()
    assert torch.all(D == 7.0)


def test_d_aliases_c():
    mcg = need_gpu()
    M, N, K = 200, 136, 192
    A, B = operands("f16", "f16", "k_contig", "mn_contig", M, N, K)
    C = W.c_matrix(M, N, "normal")
    cd = dev(C)
    mcg.gemm_dense("f16", "f16", "k_contig", "mn_contig", M, N, K, dev(A.codes), A.ld, dev(B.codes),
                   B.ld, cd, cd, N, "f32", 1.0, 1.0)
    torch.cuda.synchronize()
    ref, s = oracle.gemm_float("f16", "f16", "k_contig", "mn_contig", M, N, K, A.codes, A.ld,
                               B.codes, B.ld, C, N, 1.0, 1.0)
    compare("f16", cd.cpu().numpy(), ref, s, K, beta=1.0, c=C)


def test_int8_wraps_mod_2_32():
    mcg = need_gpu()
    M, N, K = 64, 64, 512
    A = np.full((M, K), 127, np.int8)
    B = np.full((N, K), 127, np.int8)
    C = np.full((M, N), 2 ** 30, np.int32)
    d = run_dense(mcg, "i8", "i8", "k_contig", "k_contig", M, N, K, A, K, B, K, C, N, 7, 3)
    ref = oracle.gemm_i8("k_contig", "k_contig", M, N, K, A, K, B, K, C, N, 7, 3)
    assert np.array_equal(d, ref)


def test_streams_are_honoured():
    mcg = need_gpu()
    M = N = K = 512
    A, B = operands("bf16", "bf16", "k_contig", "k_contig", M, N, K)
    dA, dB = dev(A.codes), dev(B.codes)
    s = torch.cuda.Stream()
    D = torch.empty((M, N), device="cuda")
    with torch.cuda.stream(s):
        mcg.gemm_dense("bf16", "bf16", 0, 0, M, N, K, dA, A.ld, dB, B.ld, None, D, N, "f32")
    s.synchronize()
    ref, sref = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", M, N, K, A.codes, A.ld,
                                  B.codes, B.ld)
    compare("bf16", D.cpu().numpy(), ref, sref, K)


# ------------------------------------------------------- full-size configurations

def sampled_check(mcg, wl, seed=0):
    """Full-size run in the benchmark's launch configuration; the oracle
    computes sampled outputs one by one (whole rows, whole columns, random
    elements, corners)."""
    say(f"full-size: {wl.name}")
    M, N, K = wl.M, wl.N, wl.K
    A = W.operand("A", wl.dtA, M, K, wl.dist, wl.layA, fp8_scaled=wl.fp8_scaled)
    B = W.operand("B", wl.dtB, K, N, wl.dist, wl.layB, fp8_scaled=wl.fp8_scaled)
    C = W.c_matrix(M, N, wl.c_dist) if wl.c_dist else None
    d = run_dense(mcg, wl.dtA, wl.dtB, wl.layA, wl.layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C,
                  N, wl.alpha, wl.beta, A.scale, B.scale, expect_path=1)
    rows, cols = W.sample_coords(M, N, n_random=4096, full_rows=(0, M // 2 + 5, M - 1),
                                 full_cols=(1, N - 1))
    ref, s = oracle_dense(wl.dtA, wl.dtB, wl.layA, wl.layB, M, N, K, A.codes, A.ld, B.codes, B.ld,
                          C, N, wl.alpha, wl.beta, A.scale, B.scale, rows, cols)
    r = compare(wl.dtA, d[rows, cols], ref, s, K, wl.alpha, A.scale, B.scale, wl.beta,
                None if C is None else C[rows, cols], what=wl.name)
    if wl.dtA != "i8":
        assert not np.isnan(d).any()
    say(f"  sampled {r['n']} outputs ok; max |delta|/bound = {r.get('max_ratio')}")
    return d


FULL = [w for w in W.standard_workloads() if not w.sparse and w.M > 256]


@pytest.mark.parametrize("wl", FULL, ids=[w.name.split(",")[0] for w in FULL])
def test_full_size_configurations(wl):
    mcg = need_gpu()
    d = sampled_check(mcg, wl)
    if wl.dtA == "i8":
        # the exact path: every output equal to the oracle's
        M, N, K = wl.M, wl.N, wl.K
        A = W.operand("A", wl.dtA, M, K, wl.dist, wl.layA)
        B = W.operand("B", wl.dtB, K, N, wl.dist, wl.layB)
        C = W.c_matrix(M, N, wl.c_dist) if wl.c_dist else None
        ref = oracle.gemm_i8(wl.layA, wl.layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, N,
                             int(wl.alpha), int(wl.beta))
        r = oracle.check_exact(d, ref)
        assert r["ok"], f"{wl.name}: {r}"
        say(f"  every one of {r['n']} outputs bit-exact")


# ------------------------------------------------ fp8 accumulation-precision cases

def adversarial_fp8(M, N, K, dtA, dtB, seed=21):
    """Per group of eight consecutive k: one product of magnitude 2^8 and seven
    of magnitude 2^-6 (14 binades below), with random signs."""
    big = {"e4m3": 16.0, "e5m2": 16.0}
    rng = np.random.default_rng(seed)
    k = np.arange(K)
    Av = np.where(k % 8 == 0, big[dtA], 0.125)[None, :] * rng.choice([-1.0, 1.0], (M, K))
    Bv = np.where(k % 8 == 0, big[dtB], 0.125)[:, None] * rng.choice([-1.0, 1.0], (K, N))
    Aq, _ = W.quantize(torch.from_numpy(Av).float(), dtA)
    Bq, _ = W.quantize(torch.from_numpy(Bv).float(), dtB)
    As, lda = W.store(Aq, "A", "k_contig")
    Bs, ldb = W.store(Bq, "B", "k_contig")
    return W.codes_of(As, dtA), lda, W.codes_of(Bs, dtB), ldb


@pytest.mark.parametrize("dtA,dtB", [("e4m3", "e4m3"), ("e4m3", "e5m2")])
@pytest.mark.parametrize("K", [8, 65, 1000, 6143, 6144, 8192])
def test_fp8_wide_dynamic_range_meets_bound(dtA, dtB, K):
    """The bound must hold for every K, including where one product per
    eight-element group dwarfs the others (the regime where the native fp8
    instruction's short alignment window loses the small products)."""
    mcg = need_gpu()
    M, N = 32, 48
    A, lda, B, ldb = adversarial_fp8(M, N, K, dtA, dtB)
    d = run_dense(mcg, dtA, dtB, "k_contig", "k_contig", M, N, K, A, lda, B, ldb)
    ref, s = oracle.gemm_float(dtA, dtB, "k_contig", "k_contig", M, N, K, A, lda, B, ldb)
    r = compare(dtA, d, ref, s, K, what=f"fp8 dynamic range K={K}")
    say(f"fp8 {dtA}x{dtB} K={K}: max |delta|/bound = {r['max_ratio']:.3f}")


@pytest.mark.parametrize("dtA,dtB", [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("layA,layB", LAYOUTS)
def test_fp8_native_path_at_threshold(dtA, dtB, layA, layB):
    """K = 6144: the first K served by the native fp8 instruction; full check."""
    mcg = need_gpu()
    check_case(mcg, dtA, dtB, layA, layB, 96, 80, 6144, pad=16)
