"""Seeded random dense problems through gemm_dense, every output compared with the
oracle: sizes from 1 to several tiles with ragged tails, all four layouts, every
input pair, padded and unpadded leading dimensions, alpha and beta drawn from a
small set (beta = 0 included).  Whatever kernel the library picks (general,
skinny, streaming or pipelined) must meet the same bound; the case is printed
before it runs."""
import numpy as np
import pytest

from gpu_util import need_gpu
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
