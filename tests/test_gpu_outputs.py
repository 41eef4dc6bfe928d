"""GPU parity for bfloat16 / binary16 outputs (C read and D written in the
output format) on the dense and 2:4 kernels, against the oracle, which rounds
the exact result once to the output format.  The acceptance bound is the fp32
bound plus both roundings to the output format (oracle.float_bound)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import dev, need_gpu, say

pytestmark = pytest.mark.gpu

TORCH_OUT = {"bf16": torch.bfloat16, "f16": torch.float16}
NAN_CODE = {"bf16": 0x7FC0, "f16": 0x7E00}


def c_codes(M, ldc, out, seed):
    """C ~ N(0,1) rounded to the output format; raw 16-bit codes (M, ldc)."""
    c = W.draw("normal", (M, ldc), seed).to(torch.float32).to(TORCH_OUT[out])
    return c.view(torch.int16).numpy().view(np.uint16)


def decode(codes, out):
    t = torch.from_numpy(np.ascontiguousarray(codes).view(np.int16)).view(TORCH_OUT[out])
    return t.double().numpy()


def run_dense16(mcg, dtA, dtB, layA, layB, M, N, K, A, B, C, ldc, out, alpha, beta, expect_path):
    dA, dB = dev(A.codes), dev(B.codes)
    assert mcg.dense_path(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld) == expect_path
    D = torch.full((M, ldc), NAN_CODE[out], dtype=torch.int32).to(torch.int16).to("cuda")
    mcg.gemm_dense(dtA, dtB, layA, layB, M, N, K, dA, A.ld, dB, B.ld,
                   None if C is None else dev(C.view(np.int16)), D, ldc, out, alpha, beta,
                   A.scale, B.scale)
    torch.cuda.synchronize()
    return D.cpu().numpy().view(np.uint16)


DENSE_PAIRS = [("bf16", "bf16"), ("f16", "f16"), ("e4m3", "e4m3"), ("e4m3", "e5m2")]
DENSE_CASES = [  # (M, N, K, pad, expected kernel, sampled)
    (130, 140, 196, 8, 0, False),      # general kernel, ragged (K * 2 bytes not a multiple of 16)
    (1008, 752, 2080, 16, 6, True),    # 128 x 128 form of the fast kernel, ragged M, N and K
    (2832, 2576, 208, 16, 1, True),    # 256 x 256 kernel, ragged M, N and K
    (1024, 16, 1040, 0, 4, False),     # streaming kernel (N <= 32)
]


@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("dtA,dtB", DENSE_PAIRS)
@pytest.mark.parametrize("layA,layB", [("k_contig", "k_contig"), ("mn_contig", "mn_contig")])
@pytest.mark.parametrize("case", DENSE_CASES, ids=["general", "tile128", "tile256", "stream"])
def test_dense_16bit_output(out, dtA, dtB, layA, layB, case):
    mcg = need_gpu()
    M, N, K, pad, path, sampled = case
    if path == 4 and layA != "k_contig":
        path = 2  # a small MN-contiguous wide operand takes the general kernel with 128 x 32 tiles
    say(f"dense {dtA}x{dtB} {layA}/{layB} {M}x{N}x{K} -> {out}")
    fp8 = dtA in ("e4m3", "e5m2")
    A = W.operand("A", dtA, M, K, "normal", layA, seed=31,
                  ld=(K if layA == "k_contig" else M) + pad, fp8_scaled=fp8)
    B = W.operand("B", dtB, K, N, "normal", layB, seed=32,
                  ld=(K if layB == "k_contig" else N) + pad, fp8_scaled=fp8)
    ldc = N + 4
    C = c_codes(M, ldc, out, 33)
    alpha, beta = -0.75, 1.5
    d = run_dense16(mcg, dtA, dtB, layA, layB, M, N, K, A, B, C, ldc, out, alpha, beta, path)
    rows = cols = None
    if sampled:
        rows, cols = W.sample_coords(M, N, n_random=4096, full_rows=(0, 255, 256, M - 1),
                                     full_cols=(0, 255, 256, N - 1))
    ref, s = oracle.gemm_float(dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc,
                               alpha, beta, A.scale, B.scale, rows=rows, cols=cols, out=out)
    got = decode(d, out)
    cdec = decode(C, out)
    if sampled:
        got, cdec = got[rows, cols], cdec[rows, cols]
    else:
        got, cdec = got[:, :N], cdec[:, :N]
    r = oracle.check_float(got, ref, s, K, alpha, A.scale, B.scale, beta, cdec, out=out)
    assert r["ok"], r
    assert np.all(d[:, N:] == NAN_CODE[out])  # padding columns of D untouched


@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("case", [(130, 200, 388, 0), (512, 304, 1024, 1)], ids=["general", "tile256"])
def test_sparse_16bit_output(out, dt, case):
    mcg = need_gpu()
    M, N, K, path = case
    say(f"sparse {dt} {M}x{N}x{K} -> {out}")
    A = W.sparse24_dense(dt, M, K, seed=34)
    B = W.operand("B", dt, K, N, "normal", "k_contig", seed=35)
    v, i, _ = oracle.compress24(dt, A)
    nw = (K + 31) // 32
    dv, di, dbb = dev(v), dev(i.view(np.int32)), dev(B.codes)
    assert mcg.sparse24_path(dt, "k_contig", M, N, K, dv, K // 2, di, nw, dbb, B.ld) == path
    C = c_codes(M, N, out, 36)
    D = torch.full((M, N), NAN_CODE[out], dtype=torch.int32).to(torch.int16).to("cuda")
    mcg.gemm_sparse24(dt, dt, "k_contig", M, N, K, dv, K // 2, di, nw, dbb, B.ld,
                      dev(C.view(np.int16)), D, N, out, 0.5, -1.0)
    torch.cuda.synchronize()
    ref, s = oracle.gemm_sparse24(dt, dt, "k_contig", M, N, K, v, i, B.codes, B.ld, C, N, 0.5,
                                  -1.0, out=out)
    r = oracle.check_float(decode(D.cpu().numpy().view(np.uint16), out), ref, s, K, 0.5, beta=-1.0,
                           c=decode(C, out), out=out)
    assert r["ok"], r


def test_full_size_bf16_in_bf16_out():
    """bf16 8192^3 with C and D in bfloat16 (alpha = beta = 1), in the launch
    configuration of the benchmark's bf16-output entry; sampled outputs."""
    mcg = need_gpu()
    M = N = K = 8192
    A = W.operand("A", "bf16", M, K, "normal", "k_contig")
    B = W.operand("B", "bf16", K, N, "normal", "k_contig")
    C = c_codes(M, N, "bf16", W.SEED_C)
    d = run_dense16(mcg, "bf16", "bf16", "k_contig", "k_contig", M, N, K, A, B, C, N, "bf16",
                    1.0, 1.0, 1)
    rows, cols = W.sample_coords(M, N, n_random=4096, full_rows=(0, M - 1), full_cols=(N // 2,))
    ref, s = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", M, N, K, A.codes, A.ld,
                               B.codes, B.ld, C, N, 1.0, 1.0, rows=rows, cols=cols, out="bf16")
    got = decode(d, "bf16")[rows, cols]
    r = oracle.check_float(got, ref, s, K, beta=1.0, c=decode(C, "bf16")[rows, cols], out="bf16")
    say(f"  sampled {r['n']} outputs; max |delta|/bound = {r['max_ratio']}")
    assert r["ok"], r
