"""GPU parity of the 2:4 path: the device compressor must equal the oracle's
byte for byte; gemm_sparse24 must meet the float bound against "decompress,
then the dense oracle" (bit-exact on integer-valued inputs)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import compare, dev, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", ["bf16", "f16", "i8", "e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [(1, 4), (7, 36), (130, 200), (64, 1024), (3, 4100), (5, 272), (33, 8208)])
def test_compress24_matches_oracle(dt, shape):
    mcg = need_gpu()
    M, K = shape
    say(f"compress24 {dt} {shape}")
    A = W.sparse24_dense(dt, M, K, dist="int8" if dt == "i8" else "normal")
    nw = (K + 31) // 32
    vals = torch.full((M, K // 2), 0x5A, dtype=torch.uint8 if W.ELEM_BYTES[dt] == 1 else torch.int16,
                      device="cuda")
    idx = torch.full((M, nw), -1, dtype=torch.int32, device="cuda")
    viol = torch.full((1,), 123, dtype=torch.int32, device="cuda")
    mcg.compress24(dt, M, K, dev(A), K, vals, K // 2, idx, nw, viol)
    torch.cuda.synchronize()
    ov, oi, ovio = oracle.compress24(dt, A)
    assert int(viol.item()) == ovio == 0
    assert np.array_equal(vals.cpu().numpy().view(W.CODE_NP[dt]).reshape(ov.shape), ov)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), oi)


@pytest.mark.parametrize("dt", ["i8", "bf16"])
@pytest.mark.parametrize("K", [256, 36])  # vector path (K * elem_bytes % 16 == 0) and general path
def test_compress24_counts_violations(dt, K):
    mcg = need_gpu()
    rng = np.random.default_rng(1)
    M = 40
    ints = rng.integers(-2, 3, (M, K))
    if dt == "i8":
        A = ints.astype(np.int8)
        vals = torch.zeros((M, K // 2), dtype=torch.int8, device="cuda")
    else:
        A = torch.from_numpy(ints.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        vals = torch.zeros((M, K // 2), dtype=torch.int16, device="cuda")
    nw = (K + 31) // 32
    idx = torch.zeros((M, nw), dtype=torch.int32, device="cuda")
    viol = torch.zeros((1,), dtype=torch.int32, device="cuda")
    mcg.compress24(dt, M, K, dev(A), K, vals, K // 2, idx, nw, viol)
    torch.cuda.synchronize()
    ov, oi, ovio = oracle.compress24(dt, A)
    assert ovio > 0 and int(viol.item()) == ovio
    assert np.array_equal(vals.cpu().numpy().view(ov.dtype).reshape(ov.shape), ov)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), oi)


def run_sparse(mcg, dt, layB, M, N, K, A_dense, B, C=None, alpha=1.0, beta=0.0, via_device=True):
    """Compress A (device compressor) and run gemm_sparse24; returns D, vals, idx."""
    nw = (K + 31) // 32
    if via_device:
        vals = torch.empty((M, K // 2), dtype=torch.int16, device="cuda")
        idx = torch.empty((M, nw), dtype=torch.int32, device="cuda")
        viol = torch.zeros((1,), dtype=torch.int32, device="cuda")
        mcg.compress24(dt, M, K, dev(A_dense), K, vals, K // 2, idx, nw, viol)
    else:
        v, i, _ = oracle.compress24(dt, A_dense)
        vals, idx = dev(v), dev(i.view(np.int32))
    D = torch.full((M, N), float("nan"), device="cuda")
    mcg.gemm_sparse24(dt, dt, layB, M, N, K, vals, K // 2, idx, nw, dev(B.codes), B.ld,
                      None if C is None else dev(C), D, N, "f32", alpha, beta)
    torch.cuda.synchronize()
    if via_device:
        assert int(viol.item()) == 0
    return D.cpu().numpy(), vals, idx


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("layB", ["k_contig", "mn_contig"])
@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 200, 388), (17, 33, 4), (130, 140, 1000)])
def test_sparse_gemm_matches_oracle(dt, layB, shape):
    mcg = need_gpu()
    M, N, K = shape
    say(f"sparse {dt} B {layB} {shape}")
    A = W.sparse24_dense(dt, M, K)
    B = W.operand("B", dt, K, N, "normal", layB, seed=11)
    C = W.c_matrix(M, N, "normal", seed=12)
    d, vals, idx = run_sparse(mcg, dt, layB, M, N, K, A, B, C, 0.75, 1.0)
    v, i, _ = oracle.compress24(dt, A)
    ref, s = oracle.gemm_sparse24(dt, dt, layB, M, N, K, v, i, B.codes, B.ld, C, N, 0.75, 1.0)
    compare(dt, d, ref, s, K, 0.75, beta=1.0, c=C, what=f"sparse {dt} {layB} {shape}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("layB", ["k_contig", "mn_contig"])
@pytest.mark.parametrize("shape,pads", [
    ((300, 520, 400), (8, 3, 16)),     # ragged M and N, K % 32 == 16 (partial last stage)
    ((512, 768, 1024), (0, 0, 0)),     # whole tiles, unpadded
    ((257, 304, 16), (16, 1, 8)),      # one stage, one row past a tile
    ((600, 256, 2000), (24, 5, 40)),   # many stages, odd index stride
])
def test_sparse_256_tile_path(dt, layB, shape, pads):
    """Shapes taken by the 256 x 256 sparse kernel (M, N >= 256, K % 16 == 0, aligned),
    with padded leading dimensions of the kept values, the index and B."""
    mcg = need_gpu()
    M, N, K = shape
    pad_v, pad_i, pad_b = pads
    say(f"sparse 256-tile {dt} B {layB} {shape} pads {pads}")
    A = W.sparse24_dense(dt, M, K, seed=21)
    B = W.operand("B", dt, K, N, "normal", layB, seed=22,
                  ld=(K if layB == "k_contig" else N) + pad_b)
    C = W.c_matrix(M, N, "normal", seed=23)
    v, i, _ = oracle.compress24(dt, A)
    nw = (K + 31) // 32
    lda_c, ld_idx = K // 2 + pad_v, nw + pad_i
    vp = np.zeros((M, lda_c), v.dtype)
    vp[:, :K // 2] = v
    ip = np.full((M, ld_idx), 0xFFFFFFFF, np.uint32)  # padding words: read only for groups past K
    ip[:, :nw] = i
    D = torch.full((M, N), float("nan"), device="cuda")
    dv, di, dbb = dev(vp), dev(ip.view(np.int32)), dev(B.codes)
    assert mcg.sparse24_path(dt, layB, M, N, K, dv, lda_c, di, ld_idx, dbb, B.ld) == 1
    mcg.gemm_sparse24(dt, dt, layB, M, N, K, dv, lda_c, di, ld_idx, dbb, B.ld, dev(C), D, N, "f32",
                      1.5, -0.5)
    torch.cuda.synchronize()
    ref, s = oracle.gemm_sparse24(dt, dt, layB, M, N, K, v, i, B.codes, B.ld, C, N, 1.5, -0.5)
    compare(dt, D.cpu().numpy(), ref, s, K, 1.5, beta=-0.5, c=C, what=f"sparse256 {dt} {layB} {shape}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_sparse_small_integers_bit_exact(dt):
    mcg = need_gpu()
    M, N, K = 160, 192, 512
    _sparse_smallint_case(mcg, dt, M, N, K)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_sparse_small_integers_bit_exact_256_tiles(dt):
    """The 256 x 256 kernel: every partial sum is an exact small integer, so the
    result must equal the oracle bit for bit (pins the operand and index layouts)."""
    mcg = need_gpu()
    _sparse_smallint_case(mcg, dt, 512, 512, 1024)


def _sparse_smallint_case(mcg, dt, M, N, K):
    A = W.sparse24_dense(dt, M, K, dist="smallint8")
    B = W.operand("B", dt, K, N, "smallint8", "k_contig", seed=13)
    d, _, _ = run_sparse(mcg, dt, "k_contig", M, N, K, A, B)
    v, i, _ = oracle.compress24(dt, A)
    ref, _ = oracle.gemm_sparse24(dt, dt, "k_contig", M, N, K, v, i, B.codes, B.ld)
    assert np.array_equal(d, ref)


def test_sparse_with_host_compressed_operand():
    """Operand compressed by the oracle (not the device) gives the same result."""
    mcg = need_gpu()
    M, N, K = 256, 128, 512
    A = W.sparse24_dense("bf16", M, K)
    B = W.operand("B", "bf16", K, N, "normal", "k_contig", seed=14)
    d1, _, _ = run_sparse(mcg, "bf16", "k_contig", M, N, K, A, B)
    d2, _, _ = run_sparse(mcg, "bf16", "k_contig", M, N, K, A, B, via_device=False)
    assert np.array_equal(d1, d2)


def test_full_size_sparse_configuration():
    """2:4 bf16 8192^3 in the benchmark's launch configuration; sampled outputs."""
    mcg = need_gpu()
    wl = [w for w in W.standard_workloads() if w.sparse][0]
    M, N, K = wl.M, wl.N, wl.K
    say(f"full-size: {wl.name}")
    A = W.sparse24_dense("bf16", M, K)
    B = W.operand("B", "bf16", K, N, "normal", "k_contig")
    d, vals, idx = run_sparse(mcg, "bf16", "k_contig", M, N, K, A, B)
    assert not np.isnan(d).any()
    rows, cols = W.sample_coords(M, N, n_random=4096, full_rows=(0, M - 1), full_cols=(N // 3,))
    # the device-compressed operand equals the oracle's on sampled rows
    v, i, _ = oracle.compress24("bf16", A[np.unique(rows)])
    assert np.array_equal(vals.cpu().numpy().view(np.uint16)[np.unique(rows)], v)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32)[np.unique(rows)], i)
    ref, s = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", M, N, K, A, K, B.codes, B.ld,
                               rows=rows, cols=cols)
    r = compare("bf16", d[rows, cols], ref, s, K, what=wl.name)
    say(f"  sampled {r['n']} outputs ok; max |delta|/bound = {r['max_ratio']}")


# ------------------------------------------------------------ 8-bit sparse (int8, fp8)

SP8 = [("i8", "i8"), ("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]


def sparse8_case(mcg, dtA, dtB, layB, M, N, K, path, pads=(0, 0, 0), seed=0, alpha=None, beta=1.0,
                 sample=None, A=None, B=None):
    """Compress A on the device into padded buffers, run gemm_sparse24, compare
    with the oracle (int8 bit-exact, float inputs within the bound; fp8 scales in
    alpha).  path: the kernel the call must take, or None for any."""
    i8 = dtA == "i8"
    pad_v, pad_i, pad_b = pads
    if A is None:
        A = W.sparse24_dense(dtA, M, K, dist="int8" if i8 else "normal", seed=70 + seed)
    if B is None:
        B = W.operand("B", dtB, K, N, "int8" if i8 else "normal", layB, seed=71 + seed,
                      ld=(K if layB == "k_contig" else N) + pad_b, fp8_scaled=not i8)
    if alpha is None:
        alpha = 3 if i8 else 1.25 * B.scale
    C = None if beta == 0 else W.c_matrix(M, N, "int20" if i8 else "normal", seed=72 + seed)
    nw = (K + 31) // 32
    lda_c, ld_idx = K // 2 + pad_v, nw + pad_i
    # M x lda_c kept values of the input's width
    vals = torch.full((M, lda_c), 0x5A, dtype=torch.uint8 if W.ELEM_BYTES[dtA] == 1 else torch.int16,
                      device="cuda")
    idx = torch.full((M, ld_idx), -1, dtype=torch.int32, device="cuda")
    viol = torch.zeros((1,), dtype=torch.int32, device="cuda")
    mcg.compress24(dtA, M, K, dev(A), K, vals, lda_c, idx, ld_idx, viol)
    dbb = dev(B.codes)
    if path is not None:
        assert mcg.sparse24_path(dtA, layB, M, N, K, vals, lda_c, idx, ld_idx, dbb, B.ld) == path
    D = torch.full((M, N), -0x5A5A5A5A if i8 else float("nan"), dtype=torch.int32 if i8 else torch.float32,
                   device="cuda")
    mcg.gemm_sparse24(dtA, dtB, layB, M, N, K, vals, lda_c, idx, ld_idx, dbb, B.ld,
                      None if C is None else dev(C), D, N, "i32" if i8 else "f32", alpha, beta)
    torch.cuda.synchronize()
    assert int(viol.item()) == 0
    v, ix, _ = oracle.compress24(dtA, A)
    rows, cols = sample if sample is not None else (None, None)
    ref, s = oracle.gemm_sparse24(dtA, dtB, layB, M, N, K, v, ix, B.codes, B.ld, C, N, alpha, beta,
                                  rows=rows, cols=cols)
    d = D.cpu().numpy()
    got = d if rows is None else d[rows, cols]
    c = None if C is None else (C if rows is None else C[rows, cols])
    return compare(dtA, got, ref, s, K, alpha, beta=beta, c=c,
                   what=f"sparse {dtA}x{dtB} {layB} {M}x{N}x{K}")


@pytest.mark.parametrize("dtA,dtB", SP8)
@pytest.mark.parametrize("layB", ["k_contig", "mn_contig"])
@pytest.mark.parametrize("shape", [(130, 140, 1000), (300, 200, 388), (17, 33, 4), (64, 96, 6176)])
def test_sparse8_general_kernel(dtA, dtB, layB, shape):
    """General kernel: ragged tiles, K ending inside a tile; fp8 widened to
    bfloat16 below K = 6144 and native above."""
    mcg = need_gpu()
    M, N, K = shape
    say(f"sparse8 general {dtA}x{dtB} {layB} {shape}")
    sparse8_case(mcg, dtA, dtB, layB, M, N, K, 0, seed=1)


@pytest.mark.parametrize("dtA,dtB", SP8)
@pytest.mark.parametrize("layB", ["k_contig", "mn_contig"])
@pytest.mark.parametrize("shape,pads", [
    ((512, 512, 6144), (0, 0, 0)),       # whole tiles
    ((300, 528, 6176), (16, 3, 32)),     # ragged M and N, last stage partial, padded ld's
    ((257, 304, 6400), (32, 1, 16)),     # one row past a tile
])
def test_sparse8_256_tile_path(dtA, dtB, layB, shape, pads):
    """The 256 x 256 sparse kernel with 8-bit operands (native fp8 from K = 6144)."""
    mcg = need_gpu()
    M, N, K = shape
    say(f"sparse8 256-tile {dtA}x{dtB} {layB} {shape} pads {pads}")
    sparse8_case(mcg, dtA, dtB, layB, M, N, K, 1, pads=pads, seed=2)


@pytest.mark.parametrize("layB", ["k_contig", "mn_contig"])
def test_sparse_int8_256_tile_short_k(layB):
    """int8 takes the 256 x 256 kernel at any K that is a multiple of 32."""
    mcg = need_gpu()
    sparse8_case(mcg, "i8", "i8", layB, 512, 288, 1056, 1, alpha=-7, beta=2, seed=3)
    sparse8_case(mcg, "i8", "i8", layB, 256, 256, 32, 1, alpha=1, beta=0, seed=4)


@pytest.mark.parametrize("dtA,dtB", [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("K", [256, 2048, 6144])
def test_sparse_fp8_wide_dynamic_range_meets_bound(dtA, dtB, K):
    """Kept values of magnitude 16 at the first kept position of every other
    group and 1/8 elsewhere (14 binades between products): the regime where the
    native fp8 instruction drops small products.  Widened below K = 6144,
    native from there; the bound must hold either way."""
    mcg = need_gpu()
    M, N = 256, 256
    rng = np.random.default_rng(5)
    g = np.arange(K) // 4
    vals = np.where((np.arange(K) % 4 == 0) & (g % 2 == 0), 16.0, 0.125)
    keep = (np.arange(K) % 4) < 2
    Av = np.where(keep, vals, 0.0)[None, :] * rng.choice([-1.0, 1.0], (M, K))
    Bv = np.where(np.arange(K) % 8 == 0, 16.0, 0.125)[:, None] * rng.choice([-1.0, 1.0], (K, N))
    Aq, _ = W.quantize(torch.from_numpy(Av).float(), dtA)
    A = W.codes_of(Aq, dtA)
    Bq, _ = W.quantize(torch.from_numpy(Bv).float(), dtB)
    Bs, ldb = W.store(Bq, "B", "k_contig")
    B = W.Operand(dtB, "k_contig", W.codes_of(Bs, dtB), ldb, 1.0)
    r = sparse8_case(mcg, dtA, dtB, "k_contig", M, N, K, 1 if K >= 6144 else 0, alpha=1.0, beta=0.0,
                     A=A, B=B)
    say(f"sparse fp8 {dtA}x{dtB} K={K}: max |delta|/bound = {r['max_ratio']:.3f}")


@pytest.mark.parametrize("dtA,dtB", [("i8", "i8"), ("e4m3", "e4m3")])
def test_full_size_sparse8(dtA, dtB):
    """8192^3 in the benchmark's launch configuration (C absent); sampled outputs."""
    mcg = need_gpu()
    M = N = K = 8192
    rows, cols = W.sample_coords(M, N, n_random=4096, full_rows=(0, M - 1), full_cols=(N // 3,))
    r = sparse8_case(mcg, dtA, dtB, "k_contig", M, N, K, 1, beta=0.0, alpha=1 if dtA == "i8" else None,
                     sample=(rows, cols), seed=6)
    say(f"  full-size sparse {dtA}: sampled {r['n']} outputs ok; max ratio {r.get('max_ratio', 0)}")
