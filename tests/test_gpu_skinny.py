"""GPU parity of the skinny and few-tile dense paths against the CPU oracle:
the streaming kernel (N <= 32 or M <= 32, any storage order), the general
kernel with 128 x 32 / 32 x 128 tiles (a small MN-contiguous wide operand), and split K (partial
sums added into D with atomic adds, beta * C added after).  Float results must
meet the accuracy bound, int8 results must be bit-exact; every case asserts
the kernel and split the library reports for it, so each code path is known
to have run."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import compare, dev, need_gpu, oracle_dense, say

pytestmark = pytest.mark.gpu

PAIRS = [("bf16", "bf16"), ("f16", "f16"), ("i8", "i8"), ("e4m3", "e4m3"), ("e4m3", "e5m2"),
         ("e5m2", "e4m3"), ("e5m2", "e5m2")]
GENERAL, FAST, SKINNY_N, SKINNY_M, STREAM = 0, 1, 2, 3, 4


def operands(dtA, dtB, layA, layB, M, N, K, pad=0, seed=0, dist=None):
    dist = dist or ("int8" if dtA == "i8" else "normal")
    fp8 = dtA in ("e4m3", "e5m2")
    A = W.operand("A", dtA, M, K, dist, layA, seed=40 + seed,
                  ld=(K if layA == "k_contig" else M) + pad, fp8_scaled=fp8)
    B = W.operand("B", dtB, K, N, dist, layB, seed=50 + seed,
                  ld=(K if layB == "k_contig" else N) + pad, fp8_scaled=fp8)
    return A, B


def run_case(mcg, dtA, dtB, layA, layB, M, N, K, kernel, split, alpha=None, beta=1.0, pad=0,
             ldc_pad=0, seed=0, sample=None):
    """Run one problem; assert the kernel and whether K is split (split: True,
    False, or an exact count); compare with the oracle (all outputs, or the
    sampled coordinates `sample` = (rows, cols))."""
    i8 = dtA == "i8"
    alpha = (3 if i8 else 1.25) if alpha is None else alpha
    A, B = operands(dtA, dtB, layA, layB, M, N, K, pad, seed)
    ldc = N + ldc_pad
    C = None if beta == 0 else W.c_matrix(M, N, "int20" if i8 else "normal", seed=60 + seed, ldc=ldc)
    dA, dB = dev(A.codes), dev(B.codes)
    dC = None if C is None else dev(C)
    fill = -0x5A5A5A5A if i8 else float("nan")
    D = torch.full((M, ldc), fill, dtype=torch.int32 if i8 else torch.float32, device="cuda")
    dtD = "i32" if i8 else "f32"
    got_kernel = mcg.dense_path(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld)
    got_split = mcg.dense_splits(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld, dC, D, dtD, beta)
    say(f"{dtA}x{dtB} {layA}/{layB} {M}x{N}x{K}: kernel {got_kernel}, splits {got_split}")
    assert got_kernel == kernel
    if split is None:
        pass
    elif split is True:
        assert got_split > 1
    elif split is False:
        assert got_split == 1
    else:
        assert got_split == split
    mcg.gemm_dense(dtA, dtB, layA, layB, M, N, K, dA, A.ld, dB, B.ld, dC, D, ldc, dtD, alpha, beta,
                   A.scale, B.scale)
    torch.cuda.synchronize()
    d = D.cpu().numpy()
    rows, cols = sample if sample is not None else (None, None)
    ref, s = oracle_dense(dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc,
                          alpha, beta, A.scale, B.scale, rows, cols)
    got = d[:M, :N] if rows is None else d[rows, cols]
    c = None if C is None else (C[:M, :N] if rows is None else C[rows, cols])
    r = compare(dtA, got, ref, s, K, alpha, A.scale, B.scale, beta, c,
                what=f"{dtA}x{dtB} {layA}/{layB} {M}x{N}x{K}")
    if ldc_pad:  # padding columns of D untouched
        assert np.all(d[:, N:] == fill) if i8 else np.all(np.isnan(d[:, N:]))
    return r


# ------------------------------------------------------------ streaming kernel

# (M, N, K, split): N-skinny (A streamed) and M-skinny (B streamed); ragged
# wide dimension, K ending inside a 128-byte tile, tiny N, 128-row blocks.
STREAM_SHAPES = [
    (1000, 16, 4096, True),    # 32 blocks of 32 rows: K split in two, atomic adds
    (777, 5, 4160, True),      # ragged M, N = 5, K ends inside a tile
    (7, 1500, 4096, True),     # M-skinny: B streamed, ragged N
    (8192, 16, 1040, False),   # 256 blocks, K ends inside a tile
    (20000, 3, 512, False),    # 128-row blocks (M >= 16384), ragged last block
    (24, 17000, 256, False),   # M-skinny with 128-column blocks
]


@pytest.mark.parametrize("dtA,dtB", PAIRS)
@pytest.mark.parametrize("shape", STREAM_SHAPES, ids=lambda s: "x".join(map(str, s[:3])))
def test_stream_kernel(dtA, dtB, shape):
    mcg = need_gpu()
    M, N, K, split = shape
    run_case(mcg, dtA, dtB, "k_contig", "k_contig", M, N, K, STREAM, split, ldc_pad=4, seed=1)


@pytest.mark.parametrize("dtA,dtB", [("bf16", "bf16"), ("i8", "i8"), ("e4m3", "e5m2")])
def test_stream_kernel_beta_zero_alpha(dtA, dtB):
    """Split (alpha folded into every partial sum, no C pass) and unsplit."""
    mcg = need_gpu()
    i8 = dtA == "i8"
    for M, N, K, split in [(1000, 16, 4096, True), (8192, 16, 1040, False)]:
        run_case(mcg, dtA, dtB, "k_contig", "k_contig", M, N, K, STREAM, split, beta=0.0,
                 alpha=-2 if i8 else -0.75, seed=2)
        run_case(mcg, dtA, dtB, "k_contig", "k_contig", M, N, K, STREAM, split, beta=-3 if i8 else 0.5,
                 alpha=5 if i8 else 2.0, seed=3)


def test_stream_native_fp8_long_k_split():
    """fp8 with K >= 6144 (native f8f6f4 accumulation) and a split K."""
    mcg = need_gpu()
    run_case(mcg, "e4m3", "e5m2", "k_contig", "k_contig", 300, 16, 8192, STREAM, True, seed=4)
    run_case(mcg, "e4m3", "e4m3", "k_contig", "k_contig", 16, 300, 8192, STREAM, True, seed=5)


def test_tiny_output_long_k():
    """16 x 16 output, K = 65536: many K ranges on one block."""
    mcg = need_gpu()
    run_case(mcg, "bf16", "bf16", "k_contig", "k_contig", 16, 16, 65536, STREAM, True, seed=6)
    run_case(mcg, "i8", "i8", "k_contig", "k_contig", 16, 16, 65536, STREAM, True, seed=6)


@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_stream_kernel_16bit_output(out):
    """16-bit C and D: no split (partial sums need a binary32 D); rounded once."""
    mcg = need_gpu()
    M, N, K = 1000, 16, 3008
    A, B = operands("bf16", "bf16", "k_contig", "k_contig", M, N, K, seed=7)
    tdt = torch.bfloat16 if out == "bf16" else torch.float16
    Ct = W.draw("normal", (M, N), 70).to(torch.float32).to(tdt)
    Cc = Ct.view(torch.int16).numpy().view(np.uint16)
    dA, dB = dev(A.codes), dev(B.codes)
    dC = dev(Cc.view(np.int16))
    D = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    assert mcg.dense_path("bf16", "k_contig", "k_contig", M, N, K, dA, A.ld, dB, B.ld) == STREAM
    assert mcg.dense_splits("bf16", "k_contig", "k_contig", M, N, K, dA, A.ld, dB, B.ld, dC, D, out, 1.0) == 1
    mcg.gemm_dense("bf16", "bf16", "k_contig", "k_contig", M, N, K, dA, A.ld, dB, B.ld, dC, D, N, out,
                   0.5, 1.0)
    torch.cuda.synchronize()
    got = D.cpu().view(tdt).double().numpy()
    ref, s = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", M, N, K, A.codes, A.ld, B.codes,
                               B.ld, Cc, N, 0.5, 1.0, out=out)
    r = oracle.check_float(got, ref, s, K, 0.5, beta=1.0, c=Ct.double().numpy(), out=out)
    assert r["ok"], r


def test_stream_split_int8_is_deterministic():
    """Split K: int32 sums are exact, so repeated runs agree bit for bit."""
    mcg = need_gpu()
    M, N, K = 1000, 16, 4096
    A, B = operands("i8", "i8", "k_contig", "k_contig", M, N, K, seed=8)
    dA, dB = dev(A.codes), dev(B.codes)
    outs = []
    for _ in range(3):
        D = torch.zeros((M, N), dtype=torch.int32, device="cuda")
        assert mcg.dense_splits("i8", 0, 0, M, N, K, dA, A.ld, dB, B.ld, None, D, "i32", 0.0) > 1
        mcg.gemm_dense("i8", "i8", 0, 0, M, N, K, dA, A.ld, dB, B.ld, None, D, N, "i32", 1, 0)
        torch.cuda.synchronize()
        outs.append(D.cpu().numpy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    ref, _ = oracle_dense("i8", "i8", "k_contig", "k_contig", M, N, K, A.codes, A.ld, B.codes, B.ld)
    assert np.array_equal(outs[0], ref)


# ------------------------------------------------------------ general kernel, skinny tiles

def skinny_kernel(layA, layB, M, N):
    """The library's choice for an aligned skinny problem: the streaming kernel,
    or the general kernel's 128 x 32 / 32 x 128 tiles when the wide operand is
    MN-contiguous with fewer than 2048 rows."""
    wide_a = N <= 32 and N <= M
    wide, lay = (M, layA) if wide_a else (N, layB)
    if lay == "mn_contig" and wide < 2048:
        return SKINNY_N if wide_a else SKINNY_M
    return STREAM


@pytest.mark.parametrize("dtA,dtB", [("bf16", "bf16"), ("i8", "i8"), ("e4m3", "e5m2"), ("f16", "f16")])
@pytest.mark.parametrize("layA,layB", [("k_contig", "mn_contig"), ("mn_contig", "k_contig"),
                                       ("mn_contig", "mn_contig")])
def test_skinny_other_layouts(dtA, dtB, layA, layB):
    """MN-contiguous operands: the streaming kernel (transposing reads of the wide
    and the narrow tiles), or the general kernel's skinny tiles for a small
    MN-contiguous wide operand; split and unsplit, padded leading dimensions,
    ragged edges."""
    mcg = need_gpu()
    K = 3008 if dtA in ("bf16", "f16") else 6016  # 47 K tiles of 128 bytes: split
    for M, N, K, split, kw in ((1024, 16, K, True, dict(ldc_pad=4, seed=9)), (16, 1024, K, True, dict(seed=10)),
                               (304, 32, 256, False, dict(pad=16, seed=11)),
                               (16, 4112, 1040, None, dict(pad=16, seed=18)),
                               (2048, 32, 2048, None, dict(seed=19))):
        run_case(mcg, dtA, dtB, layA, layB, M, N, K, skinny_kernel(layA, layB, M, N), split, **kw)


def test_unaligned_skinny_takes_general_kernel():
    """A leading dimension that is not a whole number of 16-byte chunks: the
    general 128 x 128 kernel (element loads), still split."""
    mcg = need_gpu()
    run_case(mcg, "bf16", "bf16", "k_contig", "k_contig", 1000, 16, 3000, GENERAL, True, pad=3, seed=12)
    run_case(mcg, "i8", "i8", "k_contig", "k_contig", 1000, 16, 3001, GENERAL, True, pad=1, seed=12)


# ------------------------------------------------------------ general kernel, split K

@pytest.mark.parametrize("dtA,dtB", PAIRS)
def test_general_split_k(dtA, dtB):
    """Few 128 x 128 tiles and a long K: K ranges on separate workgroups."""
    mcg = need_gpu()
    run_case(mcg, dtA, dtB, "k_contig", "k_contig", 300, 264, 8320, GENERAL, True, ldc_pad=4, seed=13)
    run_case(mcg, dtA, dtB, "mn_contig", "mn_contig", 264, 300, 8320, GENERAL, True, seed=14)


def test_general_split_k_native_fp8_and_alpha_beta():
    mcg = need_gpu()
    run_case(mcg, "e4m3", "e5m2", "k_contig", "mn_contig", 256, 200, 8192, GENERAL, True, alpha=-0.5,
             beta=2.0, seed=15)
    run_case(mcg, "i8", "i8", "mn_contig", "k_contig", 256, 200, 8192, GENERAL, True, alpha=-7,
             beta=0.0, seed=15)


def test_split_skipped_when_d_is_c():
    """D aliasing C with beta != 0 cannot be zeroed first: no split, same result."""
    mcg = need_gpu()
    for dt in ("bf16", "i8"):
        M, N, K = 300, 264, 8320
        A, B = operands(dt, dt, "k_contig", "k_contig", M, N, K, seed=16)
        C = W.c_matrix(M, N, "int20" if dt == "i8" else "normal", seed=17)
        D = dev(C)
        dA, dB = dev(A.codes), dev(B.codes)
        dtD = "i32" if dt == "i8" else "f32"
        assert mcg.dense_splits(dt, 0, 0, M, N, K, dA, A.ld, dB, B.ld, D, D, dtD, 1.0) == 1
        assert mcg.dense_splits(dt, 0, 0, M, N, K, dA, A.ld, dB, B.ld, D, D, dtD, 0.0) > 1
        mcg.gemm_dense(dt, dt, 0, 0, M, N, K, dA, A.ld, dB, B.ld, D, D, N, dtD, 1, 1)
        torch.cuda.synchronize()
        ref, s = oracle_dense(dt, dt, "k_contig", "k_contig", M, N, K, A.codes, A.ld, B.codes, B.ld, C,
                              N, 1, 1)
        compare(dt, D.cpu().numpy(), ref, s, K, beta=1.0, c=C, what=f"alias {dt}")


def test_split_does_not_read_c_when_beta_zero():
    mcg = need_gpu()
    M, N, K = 1000, 16, 3008
    A, B = operands("bf16", "bf16", "k_contig", "k_contig", M, N, K, seed=18)
    c_nan = torch.full((M, N), float("nan"), device="cuda")
    D = torch.empty((M, N), device="cuda")
    mcg.gemm_dense("bf16", "bf16", 0, 0, M, N, K, dev(A.codes), A.ld, dev(B.codes), B.ld, c_nan, D, N,
                   "f32", 1.0, 0.0)
    torch.cuda.synchronize()
    assert not torch.isnan(D).any()


# ------------------------------------------------------------ full-size skinny workloads

@pytest.mark.parametrize("M,N,K", [(32768, 16, 8192), (16, 32768, 8192), (8192, 16, 8192)])
def test_full_size_skinny(M, N, K):
    """The skinny benchmark shapes (bf16, C absent): sampled outputs, including
    every output of the first and last narrow column / row."""
    mcg = need_gpu()
    if N <= 32:
        sample = W.sample_coords(M, N, n_random=4096, full_cols=(0, N - 1))
    else:
        sample = W.sample_coords(M, N, n_random=4096, full_rows=(0, M - 1))
    r = run_case(mcg, "bf16", "bf16", "k_contig", "k_contig", M, N, K, STREAM, False, alpha=1.0,
                 beta=0.0, seed=19, sample=sample)
    say(f"  sampled {r['n']} outputs; max |delta|/bound = {r['max_ratio']}")


@pytest.mark.parametrize("dt,layA,layB,M,N,K", [
    ("bf16", "mn_contig", "k_contig", 32768, 16, 8192), ("bf16", "k_contig", "mn_contig", 16, 32768, 8192),
    ("bf16", "mn_contig", "mn_contig", 8192, 16, 8192), ("i8", "mn_contig", "k_contig", 32768, 16, 8192)])
def test_full_size_skinny_mn_contiguous(dt, layA, layB, M, N, K):
    """The skinny benchmark shapes with a column-major (MN-contiguous) wide
    operand on the streaming kernel: sampled outputs, including every output
    of the first and last narrow column / row (int8 bit-exact)."""
    mcg = need_gpu()
    if N <= 32:
        sample = W.sample_coords(M, N, n_random=4096, full_cols=(0, N - 1))
    else:
        sample = W.sample_coords(M, N, n_random=4096, full_rows=(0, M - 1))
    r = run_case(mcg, dt, dt, layA, layB, M, N, K, STREAM, None, alpha=2 if dt == "i8" else 1.0,
                 beta=0.0, seed=20, sample=sample)
    say(f"  sampled outputs checked: {r}")
