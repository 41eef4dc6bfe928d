"""Seeded random dense problems through gemm_dense, every output compared with the
oracle: sizes from 1 to several tiles with ragged tails, all four layouts, every
input pair, padded and unpadded leading dimensions, alpha and beta drawn from a
small set (beta = 0 included).  Whatever kernel the library picks (general,
skinny, streaming or pipelined) must meet the same bound; the case is printed
before it runs.  Further seeded cases: 2:4 problems, large problems on the
pipelined kernel, and problems whose plan takes the stream-K form
(gemm_dense_ws)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import dev, need_gpu, say
from test_gpu_dense import LAYOUTS, PAIRS, check_case

pytestmark = pytest.mark.gpu

SIZES = [1, 3, 16, 31, 33, 64, 100, 127, 128, 129, 200, 255, 256, 257, 300, 384]
KS = [1, 2, 15, 16, 17, 64, 96, 130, 256, 300, 512, 700]


def draw_case(seed):
    """Case `seed`: a numpy generator seeded with it picks every parameter."""
    r = np.random.default_rng(1000 + seed)
    dtA, dtB = PAIRS[r.integers(len(PAIRS))]
    layA, layB = LAYOUTS[r.integers(len(LAYOUTS))]
    M, N = int(r.choice(SIZES)), int(r.choice(SIZES))
    K = int(r.choice(KS))
    pad = int(r.choice([0, 0, 1, 8, 16]))
    ldc_pad = int(r.choice([0, 4]))
    i8 = dtA == "i8"
    alpha = float(r.choice([1, -3, 2] if i8 else [1.0, -0.75, 2.5]))
    beta = float(r.choice([0, 1, -2] if i8 else [0.0, 1.0, 0.5]))
    return dtA, dtB, layA, layB, M, N, K, pad, ldc_pad, alpha, beta


@pytest.mark.parametrize("seed", range(48))
def test_random_dense_problem(seed):
    mcg = need_gpu()
    dtA, dtB, layA, layB, M, N, K, pad, ldc_pad, alpha, beta = draw_case(seed)
    check_case(mcg, dtA, dtB, layA, layB, M, N, K, pad=pad, beta=beta, alpha=alpha, ldc_pad=ldc_pad,
               seed=50 + seed)


def draw_large_case(seed):
    """Large case `seed`: even seeds draw M, N above 2816 (at least 144 output
    tiles of 256 x 256: the 256 x 256 kernel), odd seeds M, N in [1024, 2048]
    with a long K (the kernel's 128 x 128 form); K and the leading-dimension
    paddings are whole 16-byte chunks for every element width, as both forms
    require."""
    r = np.random.default_rng(3000 + seed)
    dtA, dtB = PAIRS[r.integers(len(PAIRS))]
    layA, layB = LAYOUTS[r.integers(len(LAYOUTS))]
    if seed % 2 == 0:
        M, N = int(r.integers(2833, 3329)), int(r.integers(2833, 3329))
        K = 16 * int(r.integers(1, 25))
        path = 1
    else:
        M, N = int(r.integers(1040, 2049)), int(r.integers(1040, 2049))
        K = 16 * int(r.integers(140, 170))
        path = 6
    # an MN-contiguous operand's leading dimension is M or N plus the padding:
    # that side is a whole number of 16-byte chunks (still ragged against the tiles)
    M = M - M % 16 if layA == "mn_contig" else M
    N = N - N % 16 if layB == "mn_contig" else N
    pad = int(r.choice([0, 16, 32]))
    ldc_pad = int(r.choice([0, 4]))
    i8 = dtA == "i8"
    alpha = float(r.choice([1, -3, 2] if i8 else [1.0, -0.75, 2.5]))
    beta = float(r.choice([0, 1, -2] if i8 else [0.0, 1.0, 0.5]))
    return dtA, dtB, layA, layB, M, N, K, pad, ldc_pad, alpha, beta, path


@pytest.mark.parametrize("seed", range(8))
def test_random_large_dense_problem(seed):
    """Every output of a seeded random problem on the pipelined kernel's two tile
    forms (the path is asserted)."""
    mcg = need_gpu()
    dtA, dtB, layA, layB, M, N, K, pad, ldc_pad, alpha, beta, path = draw_large_case(seed)
    check_case(mcg, dtA, dtB, layA, layB, M, N, K, pad=pad, beta=beta, alpha=alpha, ldc_pad=ldc_pad,
               seed=70 + seed, expect_path=path)


SPARSE_DTYPES = [("bf16", "bf16"), ("f16", "f16"), ("i8", "i8"), ("e4m3", "e4m3"), ("e4m3", "e5m2")]
SPARSE_KS = [4, 8, 28, 32, 64, 100, 128, 260, 512, 1000]


def draw_sparse_case(seed):
    """2:4 case `seed`: sizes, B layout, paddings of the compressed buffers and of B,
    beta, all drawn from a generator seeded with it (K a multiple of 4)."""
    r = np.random.default_rng(5000 + seed)
    dtA, dtB = SPARSE_DTYPES[r.integers(len(SPARSE_DTYPES))]
    layB = ["k_contig", "mn_contig"][r.integers(2)]
    M, N = int(r.choice(SIZES)), int(r.choice(SIZES))
    K = int(r.choice(SPARSE_KS))
    pads = (int(r.choice([0, 2, 8])), int(r.choice([0, 1, 3])), int(r.choice([0, 8, 16])))
    beta = float(r.choice([0.0, 1.0] if dtA != "i8" else [0, 2]))
    return dtA, dtB, layB, M, N, K, pads, beta


@pytest.mark.parametrize("seed", range(32))
def test_random_sparse_problem(seed):
    """compress24 on the device, then gemm_sparse24 on whatever kernel it picks."""
    from test_gpu_sparse import sparse8_case
    mcg = need_gpu()
    dtA, dtB, layB, M, N, K, pads, beta = draw_sparse_case(seed)
    sparse8_case(mcg, dtA, dtB, layB, M, N, K, None, pads=pads, seed=90 + seed, beta=beta)


def draw_streamk_case(seed):
    """Random problem with a stream-K plan: sizes, input pair, layouts, output
    format, alpha/beta, drawn from a generator seeded with its index until the
    plan takes the stream-K form (256 x 256 tiles, or the 128 x 128 form)."""
    import matrix_core_gemm_amd as mcg
    r = np.random.default_rng(7000 + seed)
    pairs = [("bf16", "bf16"), ("f16", "f16"), ("i8", "i8"), ("e4m3", "e5m2")]
    for _ in range(1000):
        dtA, dtB = pairs[r.integers(len(pairs))]
        layA, layB = ["k_contig", "mn_contig"][r.integers(2)], ["k_contig", "mn_contig"][r.integers(2)]
        big = r.integers(2) == 0
        M = 16 * int(r.integers(64, 200) if big else r.integers(30, 120))
        N = 16 * int(r.integers(64, 200) if big else r.integers(30, 120))
        K = 16 * int(r.integers(128, 768))
        if dtA == "e4m3":
            K = max(K, 6144)
        lda = K if layA == "k_contig" else M
        ldb = K if layB == "k_contig" else N
        if mcg.dense_workspace_bytes(dtA, layA, layB, M, N, K, 0x1000, lda, 0x1000, ldb) > 0:
            out = "i32" if dtA == "i8" else ["f32", "bf16", "f16"][r.integers(3)]
            beta = [0.0, 1.0, -0.5][r.integers(3)] if dtA != "i8" else [0, 1, -2][r.integers(3)]
            return dtA, dtB, layA, layB, M, N, K, out, beta
    raise AssertionError("no stream-K shape drawn")


@pytest.mark.parametrize("seed", range(8))
def test_random_streamk_problem(seed):
    """gemm_dense_ws on a random stream-K problem: every output of two remainder
    tiles and sampled others against the oracle."""
    from test_gpu_streamk import grouped_tile, tile_coords, workspace
    mcg = need_gpu()
    dtA, dtB, layA, layB, M, N, K, out, beta = draw_streamk_case(seed)
    say(f"stream-K fuzz {seed}: {dtA}x{dtB} {layA}/{layB} {M}x{N}x{K} -> {out} beta={beta}")
    i8 = dtA == "i8"
    fp8 = dtA in ("e4m3", "e5m2")
    A = W.operand("A", dtA, M, K, "int8" if i8 else "normal", layA, seed=300 + seed, fp8_scaled=fp8)
    B = W.operand("B", dtB, K, N, "int8" if i8 else "normal", layB, seed=310 + seed, fp8_scaled=fp8)
    dA, dB = dev(A.codes), dev(B.codes)
    kernel = mcg.dense_path(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld)
    assert kernel in (1, 6)
    t = 256 if kernel == 1 else 128
    need = mcg.dense_workspace_bytes(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld)
    alpha = 2 if i8 else 1.25
    C = None
    if out == "i32":
        C = W.c_matrix(M, N, "int20", seed=320 + seed)
        D = torch.full((M, N), -0x5A5A5A5A, dtype=torch.int32, device="cuda")
    elif out == "f32":
        C = W.c_matrix(M, N, "normal", seed=320 + seed) if beta != 0 else None
        D = torch.full((M, N), float("nan"), device="cuda")
    else:
        tdt = torch.bfloat16 if out == "bf16" else torch.float16
        C = W.draw("normal", (M, N), 320 + seed).to(tdt).view(torch.int16).numpy().view(np.uint16)
        D = torch.full((M, N), 0x7FC0 if out == "bf16" else 0x7E00, dtype=torch.int32).to(torch.int16).to("cuda")
    dC = None if C is None or (beta == 0) else dev(C.view(np.int16) if out in ("bf16", "f16") else C)
    mcg.gemm_dense_ws(dtA, dtB, layA, layB, M, N, K, dA, A.ld, dB, B.ld, dC, D, N, out, alpha, beta,
                      A.scale, B.scale, workspace=workspace(need))
    torch.cuda.synchronize()
    d = D.cpu().numpy()
    tm, tn = -(-M // t), -(-N // t)
    T = tm * tn
    R = T % torch.cuda.get_device_properties(0).multi_processor_count
    tiles = [grouped_tile(p, tm, tn) for p in (T - R, T - 1)]
    r1, c1 = tile_coords(tiles, M, N, t)
    r2, c2 = W.sample_coords(M, N, n_random=1024, full_rows=(M - 1,), full_cols=(N - 1,))
    rows, cols = np.concatenate([r1, r2]), np.concatenate([c1, c2])
    Cr = C if dC is not None else None
    if i8:
        ref = oracle.gemm_i8(layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, Cr, N, alpha, beta, rows=rows,
                             cols=cols)
        r = oracle.check_exact(d[rows, cols], ref)
    else:
        ref, s = oracle.gemm_float(dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, Cr, N, alpha, beta,
                                   A.scale, B.scale, rows=rows, cols=cols, out=out)
        if out in ("bf16", "f16"):
            tdt = torch.bfloat16 if out == "bf16" else torch.float16
            dec = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(tdt).double().numpy()
            got, cc = dec(d)[rows, cols], None if Cr is None else dec(C)[rows, cols]
        else:
            got, cc = d[rows, cols], None if Cr is None else C[rows, cols]
        r = oracle.check_float(got, ref, s, K, alpha, A.scale, B.scale, beta, cc, out=out)
    say("  ", {k: v for k, v in r.items() if k != "worst"})
    assert r["ok"], r


def draw_sparse_streamk_case(seed):
    """Random 2:4 problem with a stream-K plan: input pair, B layout, sizes, output
    format and beta drawn from a generator seeded with its index until the plan
    takes the stream-K form.  K is a multiple of 32 (the 256 x 256 kernel's
    alignment for every width); the pieces' lengths in kept-value stages vary
    with it, so pieces start at every offset within an index block."""
    import matrix_core_gemm_amd as mcg
    r = np.random.default_rng(9000 + seed)
    for _ in range(1000):
        dtA, dtB = SPARSE_DTYPES[r.integers(len(SPARSE_DTYPES))]
        layB = ["k_contig", "mn_contig"][r.integers(2)]
        M = 16 * int(r.integers(16, 190))
        N = 16 * int(r.integers(16, 190))
        K = 32 * int(r.integers(16, 384))
        if dtA in ("e4m3", "e5m2"):
            K = max(K, 6144)
        ldb = K if layB == "k_contig" else N
        if mcg.sparse24_workspace_bytes(dtA, layB, M, N, K, 0x1000, K // 2, 0x1000, (K + 31) // 32, 0x1000,
                                        ldb) > 0:
            out = "i32" if dtA == "i8" else ["f32", {"bf16": "bf16", "f16": "f16"}.get(dtA, "f32")][r.integers(2)]
            beta = [0.0, 1.0, -0.5][r.integers(3)] if dtA != "i8" else [0, 1, -2][r.integers(3)]
            return dtA, dtB, layB, M, N, K, out, beta
    raise AssertionError("no 2:4 stream-K shape drawn")


@pytest.mark.parametrize("seed", range(6))
def test_random_sparse_streamk_problem(seed):
    """gemm_sparse24_ws on a random stream-K problem: every output of the first and
    the last stream-K tile and sampled others against the oracle."""
    from test_gpu_streamk import grouped_tile, tile_coords, workspace
    mcg = need_gpu()
    dtA, dtB, layB, M, N, K, out, beta = draw_sparse_streamk_case(seed)
    say(f"2:4 stream-K fuzz {seed}: {dtA}x{dtB} B {layB} {M}x{N}x{K} -> {out} beta={beta}")
    i8 = dtA == "i8"
    A = W.sparse24_dense(dtA, M, K, dist="int8" if i8 else "normal", seed=400 + seed)
    B = W.operand("B", dtB, K, N, "int8" if i8 else "normal", layB, seed=410 + seed, fp8_scaled=not i8)
    alpha = 2 if i8 else 1.25 * B.scale
    v, ix, nv = oracle.compress24(dtA, A)
    assert nv == 0
    dv, di, dB = dev(v), dev(ix.view(np.int32)), dev(B.codes)
    lda_c, ld_idx = K // 2, (K + 31) // 32
    assert mcg.sparse24_path(dtA, layB, M, N, K, dv, lda_c, di, ld_idx, dB, B.ld) == 1
    need = mcg.sparse24_workspace_bytes(dtA, layB, M, N, K, dv, lda_c, di, ld_idx, dB, B.ld)
    C = None
    if out == "i32":
        C = W.c_matrix(M, N, "int20", seed=420 + seed)
        D = torch.full((M, N), -0x5A5A5A5A, dtype=torch.int32, device="cuda")
    elif out == "f32":
        C = W.c_matrix(M, N, "normal", seed=420 + seed) if beta != 0 else None
        D = torch.full((M, N), float("nan"), device="cuda")
    else:
        tdt = torch.bfloat16 if out == "bf16" else torch.float16
        C = W.draw("normal", (M, N), 420 + seed).to(tdt).view(torch.int16).numpy().view(np.uint16)
        D = torch.full((M, N), 0x7FC0 if out == "bf16" else 0x7E00, dtype=torch.int32).to(torch.int16).to("cuda")
    dC = None if C is None or beta == 0 else dev(C.view(np.int16) if out in ("bf16", "f16") else C)
    mcg.gemm_sparse24_ws(dtA, dtB, layB, M, N, K, dv, lda_c, di, ld_idx, dB, B.ld, dC, D, N, out, alpha, beta,
                         workspace=workspace(need))
    torch.cuda.synchronize()
    d = D.cpu().numpy()
    tm, tn = -(-M // 256), -(-N // 256)
    T = tm * tn
    R = T % torch.cuda.get_device_properties(0).multi_processor_count
    tiles = [grouped_tile(p, tm, tn) for p in (T - R, T - 1)]
    r1, c1 = tile_coords(tiles, M, N, 256)
    r2, c2 = W.sample_coords(M, N, n_random=1024, full_rows=(M - 1,), full_cols=(N - 1,))
    rows, cols = np.concatenate([r1, r2]), np.concatenate([c1, c2])
    Cr = C if dC is not None else None
    say(f"  {R} stream-K tiles, {need // (256 * 256 * 4)} pieces, {len(rows)} outputs compared")
    ref, s = oracle.gemm_sparse24(dtA, dtB, layB, M, N, K, v, ix, B.codes, B.ld, Cr, N, alpha, beta, rows=rows,
                                  cols=cols, out=out if out in ("f16", "bf16") else "f32")
    if i8:
        r = oracle.check_exact(d[rows, cols], ref)
    else:
        if out in ("bf16", "f16"):
            tdt = torch.bfloat16 if out == "bf16" else torch.float16
            dec = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(tdt).double().numpy()
            got, cc = dec(d)[rows, cols], None if Cr is None else dec(C)[rows, cols]
        else:
            got, cc = d[rows, cols], None if Cr is None else C[rows, cols]
        r = oracle.check_float(got, ref, s, K, alpha, beta=beta, c=cc, out=out if out in ("f16", "bf16") else "f32")
    say("  ", {k: v for k, v in r.items() if k != "worst"})
    assert r["ok"], r
