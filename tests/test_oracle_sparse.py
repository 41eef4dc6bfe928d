"""Pins for the oracle's 2:4 compressor, decompressor and sparse GEMM (CPU).

The format follows "RDNA4 sparse WMMA builtins", Structured sparsity (2:4
pattern) and Common parameters (the index operand): two values kept per group
of four along K, each position encoded in two bits.  The worked example the
page gives (positions 0 and 2 kept in every group) is a stored fixture.
"""
import itertools
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sparse24_even_positions.txt")


def read_golden():
    out = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, *v = line.split()
                out[k] = v
    return out


def test_pages_even_position_example():
    g = read_golden()
    p0, p1 = (int(x) for x in g["positions"])
    K = 64
    A = np.zeros((3, K), np.int8)
    vals = np.arange(1, 3 * K // 2 + 1).reshape(3, K // 2) % 100 + 1
    A[:, p0::4] = vals[:, 0::2]
    A[:, p1::4] = vals[:, 1::2]
    c, idx, viol = oracle.compress24("i8", A)
    assert viol == 0
    assert np.all(idx == np.uint32(int(g["word"][0], 16)))
    assert (int(idx[0, 0]) & 0xF) == int(g["group_code"][0], 16)
    # compressed values: each group's two kept values in ascending position order
    assert np.array_equal(c, vals.astype(np.int8))
    assert np.array_equal(oracle.decompress24("i8", c, idx, K), A)


@pytest.mark.parametrize("dt", ["bf16", "f16", "i8", "e4m3", "e5m2"])
def test_every_zero_mask_of_a_group(dt):
    # All 16 non-zero patterns of one group of four.
    one = {"bf16": 0x3F80, "f16": 0x3C00, "i8": 1, "e4m3": 0x38, "e5m2": 0x3C}[dt]
    npdt = W.CODE_NP[dt]
    for mask in range(16):
        nz = [p for p in range(4) if mask >> p & 1]
        A = np.zeros((1, 4), npdt)
        for n, p in enumerate(nz):
            A[0, p] = np.array(one + n, dtype=np.int64).astype(npdt)
        c, idx, viol = oracle.compress24(dt, A)
        if len(nz) > 2:
            assert viol == 1
            continue
        assert viol == 0
        code = int(idx[0, 0]) & 0xF
        p0, p1 = code & 3, code >> 2
        assert p0 < p1
        # the non-zeros are selected; padding uses the lowest free positions
        want = sorted(nz + [p for p in range(4) if p not in nz][: 2 - len(nz)])
        assert [p0, p1] == want
        assert np.array_equal(oracle.decompress24(dt, c, idx, 4), A)
        assert int(idx[0, 0]) >> 4 == 0  # unused codes of the word stay zero


def test_signed_zero_counts_as_zero_and_nan_as_nonzero():
    A = np.array([[0x8000, 0x3F80, 0x0000, 0x4000]], np.uint16)   # -0, 1, +0, 2 (bf16)
    c, idx, viol = oracle.compress24("bf16", A)
    assert viol == 0 and (int(idx[0, 0]) & 0xF) == (1 | 3 << 2)
    A = np.array([[0x7FC0, 0x3F80, 0x0000, 0x4000]], np.uint16)   # NaN, 1, 0, 2
    _, _, viol = oracle.compress24("bf16", A)
    assert viol == 1


def test_code_domain_and_round_trips():
    for dt_ in ("bf16", "i8", "e4m3"):
        M, K = 33, 200
        A = W.sparse24_dense(dt_, M, K, dist="int8" if dt_ == "i8" else "normal")
        c, idx, viol = oracle.compress24(dt_, A)
        assert viol == 0
        assert c.shape == (M, K // 2) and idx.shape == (M, (K + 31) // 32)
        codes = [(int(w) >> (4 * s)) & 0xF for w in idx.ravel() for s in range(8)]
        allowed = {p0 | p1 << 2 for p0, p1 in itertools.combinations(range(4), 2)} | {0}
        assert set(codes) <= allowed
        # decompress . compress = identity on valid 2:4 matrices
        assert np.array_equal(oracle.decompress24(dt_, c, idx, K), A)
        # compress . decompress = identity on canonical metadata
        c2, idx2, v2 = oracle.compress24(dt_, oracle.decompress24(dt_, c, idx, K))
        assert v2 == 0 and np.array_equal(c2, c) and np.array_equal(idx2, idx)


def test_trailing_partial_word_is_zero_padded():
    K = 40  # 10 groups: the second word holds 2 codes, 6 unused
    A = W.sparse24_dense("bf16", 4, K)
    _, idx, _ = oracle.compress24("bf16", A)
    assert np.all((idx[:, 1] >> 8) == 0)


def test_bad_index_rejected():
    vals = np.ones((1, 2), np.int8)
    for code in (0x0, 0x5, 0xF, 0x1):   # (0,0), (1,1), (3,3), (1,0)
        with pytest.raises(ValueError):
            oracle.decompress24("i8", vals, np.array([[code]], np.uint32), 4)


def test_sparse_gemm_equals_dense_gemm_on_decompressed():
    M, N, K = 20, 24, 128
    A = W.sparse24_dense("bf16", M, K)
    B = W.operand("B", "bf16", K, N, "normal", "k_contig")
    c, idx, viol = oracle.compress24("bf16", A)
    assert viol == 0
    d_s, s_s = oracle.gemm_sparse24("bf16", "bf16", "k_contig", M, N, K, c, idx, B.codes, B.ld)
    d_d, s_d = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", M, N, K, A, K,
                                 B.codes, B.ld)
    assert np.array_equal(d_s, d_d) and np.array_equal(s_s, s_d)
    # witness: numpy float64 on the decoded dense matrix
    Ad = oracle.decode("bf16", A).reshape(M, K)
    Bd = W.to_tensor(B.codes, "bf16").to(torch.float64).numpy().reshape(N, K).T
    want = (Ad @ Bd).astype(np.float32)
    assert np.all(np.abs(d_s.astype(np.float64) - want) <= np.spacing(np.abs(want)))


def test_generator_gives_exactly_two_nonzeros_per_group():
    A = W.sparse24_dense("bf16", 64, 256)
    nz = (A.reshape(64, 64, 4) & 0x7FFF) != 0
    assert np.all(nz.sum(-1) == 2)


def _brute_sparse_int(vals, idx, K, B, ldb, layB, N, C, alpha, beta):
    """Python-int walk over the compressed form itself: for every group of four,
    its 4-bit code names the two dense positions of its two kept values."""
    M = vals.shape[0]
    out = np.zeros((M, N), np.int64)
    for i in range(M):
        for j in range(N):
            acc = 0
            for g in range(K // 4):
                code = (int(idx[i, g // 8]) >> (4 * (g % 8))) & 0xF
                for slot, pos in enumerate((code & 3, code >> 2)):
                    k = 4 * g + pos
                    b = int(B[j * ldb + k]) if layB == "k_contig" else int(B[k * ldb + j])
                    acc += int(vals[i, 2 * g + slot]) * b
            t = alpha * acc + (beta * int(C[i, j]) if beta else 0)
            out[i, j] = ((t + 2**31) % 2**32) - 2**31
    return out.astype(np.int32)


@pytest.mark.parametrize("layB", ["k_contig", "mn_contig"])
def test_sparse_int8_gemm_matches_brute_force(layB):
    M, N, K = 5, 7, 72
    A = W.sparse24_dense("i8", M, K, dist="int8", seed=5)
    B = W.operand("B", "i8", K, N, "int8", layB, seed=6)
    C = W.c_matrix(M, N, "int20", seed=7)
    vals, idx, viol = oracle.compress24("i8", A)
    assert viol == 0
    d, s = oracle.gemm_sparse24("i8", "i8", layB, M, N, K, vals, idx, B.codes, B.ld, C, N, -3, 2)
    assert s is None
    want = _brute_sparse_int(vals, idx, K, B.codes.ravel(), B.ld, layB, N, C, -3, 2)
    assert np.array_equal(d, want)


def test_sparse_int8_wraps_mod_2_32():
    """All products 127 * 127 over K = 1024 with alpha = 2^30: the int32 result wraps."""
    M, N, K = 2, 3, 1024
    A = np.zeros((M, K), np.int8)
    A[:, 0::4] = 127
    A[:, 3::4] = 127
    B = np.full((N, K), 127, np.int8)
    vals, idx, _ = oracle.compress24("i8", A)
    d, _ = oracle.gemm_sparse24("i8", "i8", "k_contig", M, N, K, vals, idx, B, K, alpha=2**30)
    exact = 2**30 * (K // 2) * 127 * 127
    assert np.all(d == np.int32(((exact + 2**31) % 2**32) - 2**31))


@pytest.mark.parametrize("dtA,dtB", [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
def test_sparse_fp8_gemm_matches_float64(dtA, dtB):
    """fp8 2:4 reference against numpy float64 on the decoded dense operands
    (scales folded into alpha), rounded once to binary32."""
    M, N, K = 9, 11, 96
    A = W.sparse24_dense(dtA, M, K, seed=8)
    B = W.operand("B", dtB, K, N, "normal", "k_contig", seed=9, fp8_scaled=True)
    vals, idx, viol = oracle.compress24(dtA, A)
    assert viol == 0
    alpha = 0.375 * B.scale
    d, _ = oracle.gemm_sparse24(dtA, dtB, "k_contig", M, N, K, vals, idx, B.codes, B.ld, alpha=alpha)
    Ad = oracle.decode(dtA, A).reshape(M, K)
    Bd = oracle.decode(dtB, B.codes).reshape(N, K).T
    want = (alpha * (Ad @ Bd)).astype(np.float32)
    assert np.array_equal(d, want)
