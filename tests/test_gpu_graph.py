"""The library's calls under HIP graph capture.  Every entry point launches only
kernels on the caller's stream (no allocation, no memset, no host
synchronisation), so a caller can capture a sequence of calls once and replay it.
Each test captures calls into a graph, then replays it several times with the
program's own eager work and synchronisations between the replays (the outputs
are refilled with NaN patterns eagerly, so a replay that writes nothing fails),
and checks every replay bit for bit against the same calls run eagerly."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, need_gpu, say

pytestmark = pytest.mark.gpu


def replay_and_compare(run, outs, fills, reps=3):
    """run(stream) issues the calls; outs are their output tensors, fills the
    patterns written over them before each run."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for o, f in zip(outs, fills):
            o.fill_(f)
        run(s)
    s.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(s)
    for rep in range(reps):
        for o, f in zip(outs, fills):  # eager work between replays
            o.fill_(f)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"replay {rep} differs"
    say(f"  {reps} replays bit-identical to the eager calls")


def test_graph_dense_launch_bound_batch():
    # the bf16 256^3 workload: 50 calls in one graph (the 128 x 128 form)
    mcg = need_gpu()
    n = 256
    A = W.operand("A", "bf16", n, n, "uniform", "k_contig", seed=1)
    B = W.operand("B", "bf16", n, n, "uniform", "k_contig", seed=2)
    dA, dB = dev(A.codes), dev(B.codes)
    assert mcg.dense_path("bf16", "k_contig", "k_contig", n, n, n, dA, n, dB, n) == 6
    Ds = [torch.empty((n, n), device="cuda") for _ in range(50)]

    def run(s):
        for D in Ds:
            mcg.gemm_dense("bf16", "bf16", 0, 0, n, n, n, dA, n, dB, n, None, D, n, "f32", 1.0, 0.0, stream=s)
    replay_and_compare(run, Ds, [float("nan")] * 50)


def test_graph_dense_paths_and_streamk():
    # the 256 x 256 kernel with C, the general kernel with split K (its zeroing is
    # a kernel), int8, and the stream-K form with a workspace
    mcg = need_gpu()
    A = W.operand("A", "bf16", 1024, 1024, "normal", "k_contig", seed=3)
    B = W.operand("B", "bf16", 1024, 1024, "normal", "k_contig", seed=4)
    dA, dB = dev(A.codes), dev(B.codes)
    C = dev(W.c_matrix(1024, 1024, "normal", seed=5))
    D1 = torch.empty((1024, 1024), device="cuda")
    Ai = dev(W.operand("A", "i8", 300, 2048, "int8", "k_contig", seed=6).codes)
    Bi = dev(W.operand("B", "i8", 2048, 40, "int8", "k_contig", seed=7).codes)
    D2 = torch.empty((300, 40), dtype=torch.int32, device="cuda")
    M3, N3, K3 = 1024, 2048, 8192
    A3 = dev(W.operand("A", "bf16", M3, K3, "normal", "k_contig", seed=8).codes)
    B3 = dev(W.operand("B", "bf16", K3, N3, "normal", "k_contig", seed=9).codes)
    D3 = torch.empty((M3, N3), device="cuda")
    need = mcg.dense_workspace_bytes("bf16", "k_contig", "k_contig", M3, N3, K3, A3, K3, B3, K3)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert mcg.dense_path("bf16", "k_contig", "k_contig", 1024, 1024, 1024, dA, 1024, dB, 1024) in (1, 6)
    D4 = torch.empty((M3, N3), device="cuda")  # the same stream-K problem on the library's static scratch
    assert need <= mcg._lib.mcg_dense_noalloc_scratch_bytes()
    g = torch.Generator(device="cuda").manual_seed(10)
    A5 = torch.randn((384, 320), generator=g, dtype=torch.float64, device="cuda")
    B5 = torch.randn((160, 320), generator=g, dtype=torch.float64, device="cuda")  # column-major K x N
    D5 = torch.empty((384, 160), dtype=torch.float64, device="cuda")

    def run(s):
        mcg.gemm_dense("bf16", "bf16", 0, 0, 1024, 1024, 1024, dA, 1024, dB, 1024, C, D1, 1024, "f32", 1.5, -0.5,
                       stream=s)
        mcg.gemm_dense("i8", "i8", 0, 0, 300, 40, 2048, Ai, 2048, Bi, 2048, None, D2, 40, "i32", 1, 0, stream=s)
        mcg.gemm_dense_ws("bf16", "bf16", 0, 0, M3, N3, K3, A3, K3, B3, K3, None, D3, N3, "f32", 1.0, 0.0,
                          workspace=ws, stream=s)
        mcg.gemm_dense_noalloc("bf16", "bf16", 0, 0, M3, N3, K3, A3, K3, B3, K3, None, D4, N3, "f32", 1.0, 0.0,
                               stream=s)
        mcg.gemm_dense("f64", "f64", 0, 0, 384, 160, 320, A5, 320, B5, 320, None, D5, 160, "f64", 1.0, 0.0,
                       stream=s)
    replay_and_compare(run, [D1, D2, D3, D4, D5], [float("nan"), -0x5A5A5A5A, float("nan"), float("nan"),
                                                   float("nan")])


def test_graph_compress_then_sparse():
    # compress24 on the device, then the 2:4 GEMM on its output, in one graph; and
    # the 2:4 stream-K form with a workspace
    mcg = need_gpu()
    M, N, K = 512, 768, 1024
    M2, N2, K2 = 2048, 2048, 8192
    vals2 = dev(W.sparse24_dense("bf16", M2, K2, seed=13))  # compressed below, eagerly
    v2 = torch.empty((M2, K2 // 2), dtype=torch.int16, device="cuda")
    i2 = torch.empty((M2, K2 // 32), dtype=torch.int32, device="cuda")
    mcg.compress24("bf16", M2, K2, vals2, K2, v2, K2 // 2, i2, K2 // 32, None)
    B2 = dev(W.operand("B", "bf16", K2, N2, "normal", "k_contig", seed=14).codes)
    need = mcg.sparse24_workspace_bytes("bf16", "k_contig", M2, N2, K2, v2, K2 // 2, i2, K2 // 32, B2, K2)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    D2 = torch.empty((M2, N2), device="cuda")
    Ad = dev(W.sparse24_dense("bf16", M, K, seed=11))
    B = dev(W.operand("B", "bf16", K, N, "normal", "k_contig", seed=12).codes)
    vals = torch.empty((M, K // 2), dtype=torch.int16, device="cuda")
    idx = torch.empty((M, K // 32), dtype=torch.int32, device="cuda")
    D = torch.empty((M, N), device="cuda")

    def run(s):
        mcg.compress24("bf16", M, K, Ad, K, vals, K // 2, idx, K // 32, None, stream=s)
        mcg.gemm_sparse24("bf16", "bf16", "k_contig", M, N, K, vals, K // 2, idx, K // 32, B, K, None, D, N, "f32",
                          1.0, 0.0, stream=s)
        mcg.gemm_sparse24_ws("bf16", "bf16", "k_contig", M2, N2, K2, v2, K2 // 2, i2, K2 // 32, B2, K2, None, D2, N2,
                             "f32", 1.0, 0.0, workspace=ws, stream=s)
    replay_and_compare(run, [vals, idx, D, D2], [0x7BCD, 0x7BCDEF01, float("nan"), float("nan")])
