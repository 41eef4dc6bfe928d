"""GPU check of gemm_dense_noalloc, the entry point for callers that cannot
allocate: its stream-K scratch is the library's static device array instead of
a caller workspace.  Called through the C ABI, its output must equal bit for
bit that of gemm_dense_ws with a workspace (same plan, same kernels, pieces
added in a fixed order), on two calls in a row, the second smaller, so that the
second runs over the first one's leftovers in the array.  A problem whose plan
needs more than the array holds is rejected before anything is written; the
optional 256 x 256 stream-K form of a long-K 128 x 128 problem is taken only
when it fits, else the problem runs as gemm_dense."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, need_gpu, say

pytestmark = pytest.mark.gpu


def _args(M, N, K, A, B, D):
    return (0, 0, 0, 0, M, N, K, A.data_ptr(), K, B.data_ptr(), K, None, D.data_ptr(), N, 5, 1.0, 0.0, 1.0,
            1.0)


def test_noalloc_matches_workspace_entry_point():
    mcg = need_gpu()
    lib = mcg.lib()
    limit = lib.mcg_dense_noalloc_scratch_bytes()
    assert limit == 32 << 20
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # 128 x 128 tiles: 1024 x 2048 x 8192 cuts 128 tiles in two, 1024^2 x 4096 cuts
    # 64 tiles in four (16 MiB of slots each)
    for i, (M, N, K) in enumerate([(1024, 2048, 8192), (1024, 1024, 4096)]):
        A = dev(W.operand("A", "bf16", M, K, "normal", "k_contig", seed=61 + i).codes)
        B = dev(W.operand("B", "bf16", K, N, "normal", "k_contig", seed=71 + i).codes)
        need = mcg.dense_workspace_bytes("bf16", "k_contig", "k_contig", M, N, K, A, K, B, K)
        say(f"no-alloc call {i}: {M}x{N}x{K}, plan {need >> 20} MiB of {limit >> 20}")
        assert 0 < need <= limit
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        D_ws = torch.full((M, N), float("nan"), device="cuda")
        D_na = torch.full((M, N), float("nan"), device="cuda")
        assert lib.gemm_dense_ws(*_args(M, N, K, A, B, D_ws), ws.data_ptr(), need, stream) == 0
        assert lib.gemm_dense_noalloc(*_args(M, N, K, A, B, D_na), stream) == 0
        torch.cuda.synchronize()
        a, b = D_ws.cpu().numpy(), D_na.cpu().numpy()
        assert not np.isnan(a).any()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"call {i} differs"


def test_noalloc_rejects_a_plan_beyond_the_array():
    mcg = need_gpu()
    lib = mcg.lib()
    M, N, K = 4096, 4352, 4096  # 16 remainder tiles in 16 pieces of 256 KiB: 64 MiB
    A = torch.zeros(M, K, dtype=torch.int16, device="cuda")
    B = torch.zeros(N, K, dtype=torch.int16, device="cuda")
    assert mcg.dense_workspace_bytes("bf16", "k_contig", "k_contig", M, N, K, A, K, B, K) > \
        lib.mcg_dense_noalloc_scratch_bytes()
    D = torch.full((M, N), float("nan"), device="cuda")
    st = lib.gemm_dense_noalloc(*_args(M, N, K, A, B, D), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 11
    assert torch.isnan(D).all().item()


def test_noalloc_long_k_alternative_beyond_the_array_runs_as_gemm_dense():
    # 1536^2 x 16384 runs on 128 x 128 tiles; its 256 x 256 stream-K alternative
    # (36 tiles in 4 pieces: 36 MiB) is optional, so without room for it the call
    # runs whole tiles, as gemm_dense does, instead of failing
    mcg = need_gpu()
    lib = mcg.lib()
    M, N, K = 1536, 1536, 16384
    A = dev(W.operand("A", "bf16", M, K, "normal", "k_contig", seed=91).codes)
    B = dev(W.operand("B", "bf16", K, N, "normal", "k_contig", seed=92).codes)
    assert mcg.dense_workspace_bytes("bf16", "k_contig", "k_contig", M, N, K, A, K, B, K) > \
        lib.mcg_dense_noalloc_scratch_bytes()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    D_na = torch.full((M, N), float("nan"), device="cuda")
    D_pl = torch.full((M, N), float("nan"), device="cuda")
    assert lib.gemm_dense_noalloc(*_args(M, N, K, A, B, D_na), stream) == 0
    assert lib.gemm_dense(*_args(M, N, K, A, B, D_pl), stream) == 0
    torch.cuda.synchronize()
    a, b = D_na.cpu().numpy(), D_pl.cpu().numpy()
    assert not np.isnan(a).any()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
