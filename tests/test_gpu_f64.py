"""GPU parity of the binary64 GEMM (FP64 matrix instructions) against the CPU
oracle (exact products summed in binary128, rounded once to binary64).

Every result must meet the binary64 acceptance bound
4 * 2^-53 * (K + 2) * |alpha| * S + 2^-53 * |D_ref| (+ 2^-53 |beta c| for
beta not 0 or +-1), S = sum_k |a_ik b_kj|.  Cases span several 128 x 128 tiles
with ragged M, N and K tails, all four operand layouts, odd leading
dimensions, beta = 0 (C never read), D aliasing C, K = 0, split K (atomic
partial sums, beta * C added after) and the full 8192^3 workload on sampled
outputs."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import dev, need_gpu, say

pytestmark = pytest.mark.gpu

LAYOUTS = ["k_contig", "mn_contig"]
F64_KERNEL = 5


def operands(layA, layB, M, N, K, pad=0, seed=0, dist="normal"):
    A = W.operand("A", "f64", M, K, dist, layA, seed=70 + seed, ld=(K if layA == "k_contig" else M) + pad)
    B = W.operand("B", "f64", K, N, dist, layB, seed=80 + seed, ld=(K if layB == "k_contig" else N) + pad)
    return A, B


def run_case(mcg, layA, layB, M, N, K, alpha=1.25, beta=0.5, pad=0, ldc_pad=0, seed=0, split=False,
             sample=None, dist="normal", inplace=False):
    A, B = operands(layA, layB, M, N, K, pad, seed, dist)
    ldc = N + ldc_pad
    C = None if beta == 0 else W.c_matrix(M, N, dist, seed=90 + seed, ldc=ldc, dtype="f64")
    dA, dB = dev(A.codes), dev(B.codes)
    if inplace:
        D = dev(C)
        dC = D
    else:
        dC = None if C is None else dev(C)
        D = torch.full((max(M, 1), ldc), float("nan"), dtype=torch.float64, device="cuda")
    assert mcg.dense_path("f64", layA, layB, M, N, K, dA, A.ld, dB, B.ld) == F64_KERNEL
    got_split = mcg.dense_splits("f64", layA, layB, M, N, K, dA, A.ld, dB, B.ld, dC, D, "f64", beta)
    say(f"f64 {layA}/{layB} {M}x{N}x{K} pad {pad} beta {beta}: splits {got_split}")
    if split is True:
        assert got_split > 1
    elif split is False:
        assert got_split == 1
    mcg.gemm_dense("f64", "f64", layA, layB, M, N, K, dA, A.ld, dB, B.ld, dC, D, ldc, "f64", alpha, beta)
    torch.cuda.synchronize()
    d = D.cpu().numpy()
    rows, cols = sample if sample is not None else (None, None)
    ref, s = oracle.gemm_f64(layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc, alpha, beta, rows, cols)
    got = d[:M, :N] if rows is None else d[rows, cols]
    c = None if C is None else (C[:M, :N] if rows is None else C[rows, cols])
    r = oracle.check_f64(got, ref, s, K, alpha, beta, c)
    assert r["ok"], f"f64 {layA}/{layB} {M}x{N}x{K}: {r}"
    if ldc_pad and not inplace:  # padding columns of D untouched
        assert np.all(np.isnan(d[:, N:]))
    return r, got


# (M, N, K): several tiles with ragged tails in every dimension, K tails of
# 1..15 inside a tile of 16, single rows/columns, one tile exactly.
SHAPES = [(300, 260, 200), (129, 131, 17), (128, 128, 16), (64, 200, 1), (1, 1, 1), (517, 129, 333),
          (3, 700, 45), (700, 5, 64)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("layA", LAYOUTS)
@pytest.mark.parametrize("layB", LAYOUTS)
def test_f64_full_compare(M, N, K, layA, layB):
    mcg = need_gpu()
    run_case(mcg, layA, layB, M, N, K)


@pytest.mark.parametrize("layA", LAYOUTS)
@pytest.mark.parametrize("layB", LAYOUTS)
def test_f64_odd_leading_dims_and_wide_range(layA, layB):
    """Leading dimensions with odd element counts (no 16-byte row alignment),
    a padded ldc, and magnitudes over about 2^-17 .. 2^17."""
    mcg = need_gpu()
    run_case(mcg, layA, layB, 259, 141, 149, alpha=-0.7, beta=1.0, pad=3, ldc_pad=5, dist="lognormal")


def test_f64_beta_zero_never_reads_c():
    mcg = need_gpu()
    M, N, K = 200, 150, 96
    A, B = operands("k_contig", "k_contig", M, N, K)
    Cnan = torch.full((M, N), float("nan"), dtype=torch.float64, device="cuda")
    D = torch.full((M, N), float("nan"), dtype=torch.float64, device="cuda")
    mcg.gemm_dense("f64", "f64", "k_contig", "k_contig", M, N, K, dev(A.codes), A.ld, dev(B.codes), B.ld, Cnan, D,
                   N, "f64", 2.0, 0.0)
    torch.cuda.synchronize()
    ref, s = oracle.gemm_f64("k_contig", "k_contig", M, N, K, A.codes, A.ld, B.codes, B.ld, None, N, 2.0, 0.0)
    assert oracle.check_f64(D.cpu().numpy(), ref, s, K, 2.0)["ok"]


def test_f64_in_place_c_is_d():
    """D aliasing C with beta != 0 (never split: C must be read before D is written)."""
    mcg = need_gpu()
    run_case(mcg, "k_contig", "mn_contig", 140, 270, 4096, beta=-1.5, inplace=True, split=False)


def test_f64_k_zero_gives_beta_c():
    mcg = need_gpu()
    M, N = 70, 33
    C = W.c_matrix(M, N, "normal", seed=5, dtype="f64")
    D = torch.full((M, N), float("nan"), dtype=torch.float64, device="cuda")
    z = torch.zeros(1, dtype=torch.float64, device="cuda")
    mcg.gemm_dense("f64", "f64", "k_contig", "k_contig", M, N, 0, z, 1, z, 1, dev(C), D, N, "f64", 1.0, -3.0)
    torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy(), -3.0 * C)


@pytest.mark.parametrize("layA,layB,M,N,K,beta", [
    ("k_contig", "k_contig", 200, 190, 8192, 0.0),     # 4 tiles, long K: split
    ("mn_contig", "k_contig", 130, 257, 6000, 0.75),   # ragged, beta * C added after the partial sums
    ("k_contig", "mn_contig", 31, 500, 4111, 1.0),     # K tail inside the last range
])
def test_f64_split_k(layA, layB, M, N, K, beta):
    mcg = need_gpu()
    run_case(mcg, layA, layB, M, N, K, beta=beta, split=True)


def test_f64_unsplit_is_deterministic():
    mcg = need_gpu()
    M, N, K = 384, 384, 400
    A, B = operands("k_contig", "k_contig", M, N, K)
    dA, dB = dev(A.codes), dev(B.codes)
    assert mcg.dense_splits("f64", "k_contig", "k_contig", M, N, K, dA, A.ld, dB, B.ld, None, dA, "f64", 0.0) == 1
    outs = []
    for _ in range(2):
        D = torch.empty((M, N), dtype=torch.float64, device="cuda")
        mcg.gemm_dense("f64", "f64", "k_contig", "k_contig", M, N, K, dA, A.ld, dB, B.ld, None, D, N, "f64", 1.0, 0.0)
        torch.cuda.synchronize()
        outs.append(D.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_f64_rejects_mixed_and_wrong_output():
    mcg = need_gpu()
    z = torch.zeros(16, dtype=torch.float64, device="cuda")
    with pytest.raises(mcg.MCGError):
        mcg.gemm_dense("f64", "bf16", "k_contig", "k_contig", 2, 2, 2, z, 2, z, 2, None, z, 2, "f64", 1.0, 0.0)
    with pytest.raises(mcg.MCGError):
        mcg.gemm_dense("f64", "f64", "k_contig", "k_contig", 2, 2, 2, z, 2, z, 2, None, z, 2, "f32", 1.0, 0.0)


@pytest.mark.parametrize("layA,layB", [("k_contig", "k_contig"), ("mn_contig", "mn_contig")])
def test_f64_full_size_sampled(layA, layB):
    """The 8192^3 binary64 workload (alpha = beta = 1, C ~ N(0, 1)) on sampled
    outputs: random coordinates, a full row and column, and the edges of the
    first and last tiles."""
    mcg = need_gpu()
    M = N = K = 8192
    edges = (0, 127, 128, 8063, 8064, 8191)
    rows, cols = W.sample_coords(M, N, 4096, full_rows=(5,), full_cols=(8190,))
    er, ec = np.meshgrid(np.array(edges), np.array(edges), indexing="ij")
    rows = np.concatenate([rows, er.ravel()]).astype(np.int64)
    cols = np.concatenate([cols, ec.ravel()]).astype(np.int64)
    r, _ = run_case(mcg, layA, layB, M, N, K, alpha=1.0, beta=1.0, sample=(rows, cols))
    say(f"full size {layA}/{layB}: max |delta|/bound {r['max_ratio']:.3g}")


def kernel_order_model(A, B, C, alpha, beta, i, j):
    """d_ij as the binary64 kernel computes it when K is not split: its FP64 matrix
    instructions are chains of correctly rounded fused multiply-adds in slot order
    (tests/test_gpu_numerics.py), one accumulator per output element, fed K tile by
    K tile (16 deep); inside a tile, lane group g supplies K index 4g + 2h + e of the
    instruction for pair h and element e, so the K order of one tile is
    0, 4, 8, 12, 1, 5, 9, 13, 2, 6, 10, 14, 3, 7, 11, 15.  Then alpha * acc is rounded
    and beta * c added with one fused multiply-add."""
    K = A.shape[1]
    acc = 0.0
    for t in range(0, K, 16):
        for h in range(2):
            for e in range(2):
                for g in range(4):
                    k = t + 4 * g + 2 * h + e
                    if k < K:
                        acc = float(Fraction(float(A[i, k])) * Fraction(float(B[k, j])) + Fraction(acc))
                    # k >= K: the tile holds zeros there, and fma(0, 0, acc) = acc
    v = alpha * acc
    if beta != 0.0:
        v = float(Fraction(beta) * Fraction(float(C[i, j])) + Fraction(v))
    return v


@pytest.mark.parametrize("layA,layB", [("k_contig", "k_contig"), ("mn_contig", "k_contig"), ("k_contig", "mn_contig"),
                                       ("mn_contig", "mn_contig")])
def test_f64_bit_exact_against_instruction_model(layA, layB):
    """Unsplit results equal, bit for bit, the kernel's order of binary64 fused
    multiply-adds built from the measured instruction model, on tile edges and
    random outputs of a 2 x 2-tile problem with a ragged K tail (and the edge
    tiles' checked loads)."""
    mcg = need_gpu()
    M, N, K = 150, 140, 45
    alpha, beta = 1.25, -0.75
    A, B = operands(layA, layB, M, N, K, seed=3)
    C = W.c_matrix(M, N, "normal", seed=93, dtype="f64")
    D = torch.full((M, N), float("nan"), dtype=torch.float64, device="cuda")
    assert mcg.dense_splits("f64", layA, layB, M, N, K, dev(A.codes), A.ld, dev(B.codes), B.ld, None, D, "f64",
                            beta) == 1
    mcg.gemm_dense("f64", "f64", layA, layB, M, N, K, dev(A.codes), A.ld, dev(B.codes), B.ld, dev(C), D, N, "f64",
                   alpha, beta)
    torch.cuda.synchronize()
    d = D.cpu().numpy()
    Al = A.codes[:M, :K] if layA == "k_contig" else A.codes[:K, :M].T
    Bl = B.codes[:N, :K].T if layB == "k_contig" else B.codes[:K, :N]
    rows, cols = W.sample_coords(M, N, 400, full_rows=(0, 127, 128, M - 1), full_cols=(127,))
    bad = [(i, j) for i, j in zip(rows, cols) if d[i, j] != kernel_order_model(Al, Bl, C, alpha, beta, i, j)]
    say(f"{layA}/{layB}: {len(bad)} of {len(rows)} outputs differ from the instruction-order model")
    assert not bad, bad[:5]


@pytest.mark.parametrize("layA,layB", [("k_contig", "k_contig"), ("mn_contig", "k_contig"), ("k_contig", "mn_contig"),
                                       ("mn_contig", "mn_contig")])
def test_f64_odd_leading_dims_bit_exact(layA, layB):
    """Leading dimensions of odd length (rows not 16-byte aligned: interior tiles load
    with 4-byte DMA, edge tiles element by element) give exactly the instruction-order
    model's results, over several interior tiles and a K tail."""
    mcg = need_gpu()
    M, N, K = 300, 290, 90
    alpha, beta = 0.5, 1.5
    A, B = operands(layA, layB, M, N, K, pad=1, seed=5)
    assert A.ld % 2 == 1 and B.ld % 2 == 1
    C = W.c_matrix(M, N, "normal", seed=95, dtype="f64")
    D = torch.full((M, N), float("nan"), dtype=torch.float64, device="cuda")
    mcg.gemm_dense("f64", "f64", layA, layB, M, N, K, dev(A.codes), A.ld, dev(B.codes), B.ld, dev(C), D, N, "f64",
                   alpha, beta)
    torch.cuda.synchronize()
    d = D.cpu().numpy()
    Al = A.codes[:M, :K] if layA == "k_contig" else A.codes[:K, :M].T
    Bl = B.codes[:N, :K].T if layB == "k_contig" else B.codes[:K, :N]
    rows, cols = W.sample_coords(M, N, 300, full_rows=(0, 127, 128, 255), full_cols=(0, 129, 255))
    bad = [(i, j) for i, j in zip(rows, cols) if d[i, j] != kernel_order_model(Al, Bl, C, alpha, beta, i, j)]
    say(f"{layA}/{layB} odd ld: {len(bad)} of {len(rows)} outputs differ from the instruction-order model")
    assert not bad, bad[:5]
    ref, s = oracle.gemm_f64(layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, N, alpha, beta)
    assert oracle.check_f64(d, ref, s, K, alpha, beta, C)["ok"]
