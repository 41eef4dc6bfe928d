"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through its C ABI binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import matrix_core_gemm_amd as mcg  # noqa: F401  (fails loudly if the library is missing)
    return mcg


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def run_dense(mcg, dtA, dtB, layA, layB, M, N, K, A, lda, B, ldb, C=None, ldc=None, alpha=1.0,
              beta=0.0, sA=1.0, sB=1.0, d_fill=float("nan"), c_dev=None, expect_path=None):
    """Run gemm_dense on host code arrays; returns D (numpy, shape (M, ldc)).
    expect_path: asserts the kernel the call runs (0 general, 1 the 256 x 256 kernel,
    6 its 128 x 128 form)."""
    i8 = dtA == "i8"
    ldc = N if ldc is None else ldc
    dA, dB = dev(A), dev(B)
    if expect_path is not None:
        assert mcg.dense_path(dtA, layA, layB, M, N, K, dA, lda, dB, ldb) == expect_path
    if c_dev is None and C is not None:
        c_dev = dev(C)
    if i8:
        D = torch.full((max(M, 1), ldc), -0x5A5A5A5A, dtype=torch.int32, device="cuda")
    else:
        D = torch.full((max(M, 1), ldc), d_fill, dtype=torch.float32, device="cuda")
    mcg.gemm_dense(dtA, dtB, layA, layB, M, N, K, dA, lda, dB, ldb, c_dev, D, ldc,
                   "i32" if i8 else "f32", alpha, beta, sA, sB)
    torch.cuda.synchronize()
    return D.cpu().numpy()


def oracle_dense(dtA, dtB, layA, layB, M, N, K, A, lda, B, ldb, C=None, ldc=None, alpha=1.0,
                 beta=0.0, sA=1.0, sB=1.0, rows=None, cols=None):
    ldc = N if ldc is None else ldc
    if dtA == "i8":
        return oracle.gemm_i8(layA, layB, M, N, K, A, lda, B, ldb, C, ldc, int(alpha), int(beta),
                              rows, cols), None
    return oracle.gemm_float(dtA, dtB, layA, layB, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta,
                             sA, sB, rows, cols)


def compare(dtA, d_gpu, d_ref, s_ref, K, alpha=1.0, sA=1.0, sB=1.0, beta=0.0, c=None, what=""):
    if dtA == "i8":
        r = oracle.check_exact(d_gpu, d_ref)
    else:
        r = oracle.check_float(d_gpu, d_ref, s_ref, K, alpha, sA, sB, beta, c)
    assert r["ok"], f"{what}: {r}"
    return r
