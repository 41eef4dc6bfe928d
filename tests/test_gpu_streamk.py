"""GPU parity of the stream-K form of the pipelined kernel (gemm_dense_ws)
against the CPU oracle.

Shapes whose last round of tiles leaves most compute units idle take
the stream-K form when a workspace is given: the K iterations of the remaining
tiles are split over all CUs and their partial sums added by a second kernel.
Every output of those tiles is compared with the oracle (float: the acceptance
bound; int8: bit for bit), together with one whole-tile workgroup's tile and
sampled outputs elsewhere.  The cases cover both tile sizes (256 x 256 and the
128 x 128 form), 2 to 16 pieces per tile, with and without whole-tile rounds
before them, the MN-contiguous storage orders, bfloat16 and binary16 D, D
aliasing C, int8 with wrapping alpha/beta, native fp8, repeated
calls (deterministic: the pieces are added in a fixed order) and a workspace too
small for the plan (the call runs as gemm_dense, bit for bit).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import dev, need_gpu, say

pytestmark = pytest.mark.gpu

def grouped_tile(pid, tiles_m, tiles_n):
    """The kernels' tile order: groups of four tile rows, column-major inside."""
    g, r = divmod(pid, 4 * tiles_n)
    gsize = min(4, tiles_m - 4 * g)
    return 4 * g + r % gsize, r // gsize


def remainder_tiles(M, N, num_cu, t=256):
    tm, tn = -(-M // t), -(-N // t)
    T = tm * tn
    R = T % num_cu
    return [grouped_tile(p, tm, tn) for p in range(T - R, T)], grouped_tile(0, tm, tn)


def tile_coords(tiles, M, N, t=256):
    rows, cols = [], []
    for tm, tn in tiles:
        r = np.arange(tm * t, min(M, tm * t + t))
        c = np.arange(tn * t, min(N, tn * t + t))
        rr, cc = np.meshgrid(r, c, indexing="ij")
        rows.append(rr.ravel())
        cols.append(cc.ravel())
    return np.concatenate(rows), np.concatenate(cols)


def num_cu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def workspace(nbytes):
    return torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device="cuda").fill_(float("nan"))


CASES = [  # dtA, dtB, layA, layB, M, N, K, out, alpha, beta, D aliases C, kernel (1: 256 x 256, 6: 128 x 128)
    ("bf16", "bf16", "k_contig", "k_contig", 4096, 4352, 4096, "f32", 1.5, 0.5, False, 1),
    ("bf16", "bf16", "mn_contig", "mn_contig", 4096, 4864, 4096, "f32", -0.75, 1.0, True, 1),
    ("f16", "f16", "k_contig", "mn_contig", 4096, 4864, 4096, "bf16", 1.0, -1.25, False, 1),
    ("i8", "i8", "k_contig", "k_contig", 4096, 4352, 8192, "i32", 3, -2, False, 1),
    ("e4m3", "e5m2", "k_contig", "k_contig", 4096, 4352, 8192, "f32", 1.0, 0.0, False, 1),
    ("bf16", "bf16", "k_contig", "k_contig", 1024, 2048, 8192, "f32", 1.0, 0.5, False, 6),
    ("f16", "f16", "mn_contig", "k_contig", 1152, 1280, 12288, "f16", -1.5, 1.0, True, 6),
    ("i8", "i8", "k_contig", "mn_contig", 1024, 1024, 16384, "i32", -1, 1, False, 6),
    # ragged M, N and K: edge tiles among the pieces, a last K tile cut short
    ("bf16", "bf16", "k_contig", "k_contig", 4196, 4316, 4048, "f32", 1.25, -0.5, False, 1),
    ("i8", "i8", "k_contig", "mn_contig", 4196, 4320, 8176, "i32", 2, 3, False, 1),
    ("bf16", "bf16", "mn_contig", "k_contig", 1000, 1944, 8176, "bf16", 1.0, 1.0, True, 6),
]


@pytest.mark.parametrize("case", CASES, ids=["bf16_16_pieces", "bf16_mn_alias_4_pieces", "f16_bf16out",
                                             "i8_wrap", "fp8_native", "mid_bf16", "mid_f16_f16out_alias",
                                             "mid_i8", "ragged_bf16", "ragged_i8_mn", "mid_ragged_bf16out_alias"])
def test_streamk_against_oracle(case):
    mcg = need_gpu()
    dtA, dtB, layA, layB, M, N, K, out, alpha, beta, alias, kernel = case
    t = 256 if kernel == 1 else 128
    say(f"stream-K {dtA}x{dtB} {layA}/{layB} {M}x{N}x{K} -> {out} alias={alias}")
    fp8 = dtA in ("e4m3", "e5m2")
    dist = "int8" if dtA == "i8" else "normal"
    A = W.operand("A", dtA, M, K, dist, layA, seed=41, fp8_scaled=fp8)
    B = W.operand("B", dtB, K, N, dist, layB, seed=42, fp8_scaled=fp8)
    dA, dB = dev(A.codes), dev(B.codes)
    assert mcg.dense_path(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld) == kernel
    need = mcg.dense_workspace_bytes(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld)
    assert need > 0 and need % (t * t * 4) == 0
    ldc = N
    C = None
    if out == "i32":
        C = W.c_matrix(M, N, "int20", seed=43, ldc=ldc)
        D = torch.full((M, ldc), -0x5A5A5A5A, dtype=torch.int32, device="cuda")
    elif out == "f32":
        C = W.c_matrix(M, N, "normal", seed=43, ldc=ldc) if beta != 0 else None
        D = torch.full((M, ldc), float("nan"), dtype=torch.float32, device="cuda")
    else:
        tdt = torch.bfloat16 if out == "bf16" else torch.float16
        c16 = W.draw("normal", (M, ldc), 43).to(torch.float32).to(tdt)
        C = c16.view(torch.int16).numpy().view(np.uint16)
        D = torch.full((M, ldc), 0x7FC0 if out == "bf16" else 0x7E00, dtype=torch.int32).to(torch.int16).to("cuda")
    dC = None if C is None else dev(C.view(np.int16) if out in ("bf16", "f16") else C)
    if alias:
        D = dC
    ws = workspace(need)
    mcg.gemm_dense_ws(dtA, dtB, layA, layB, M, N, K, dA, A.ld, dB, B.ld, dC, D, ldc, out, alpha, beta,
                      A.scale, B.scale, workspace=ws)
    torch.cuda.synchronize()
    d = D.cpu().numpy()
    # every output of the remainder tiles, one whole tile, and sampled others
    sk, first = remainder_tiles(M, N, num_cu(), t)
    r1, c1 = tile_coords(sk + [first], M, N, t)
    r2, c2 = W.sample_coords(M, N, n_random=2048, full_rows=(M - 1,), full_cols=(N - 1,))
    rows, cols = np.concatenate([r1, r2]), np.concatenate([c1, c2])
    say(f"  {len(sk)} stream-K tiles, {need // (t * t * 4)} pieces, {len(rows)} outputs compared")
    if out == "i32":
        ref = oracle.gemm_i8(layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc, alpha, beta,
                             rows=rows, cols=cols)
        r = oracle.check_exact(d[rows, cols], ref)
    else:
        ref, s = oracle.gemm_float(dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc,
                                   alpha, beta, A.scale, B.scale, rows=rows, cols=cols, out=out)
        if out in ("bf16", "f16"):
            tdt = torch.bfloat16 if out == "bf16" else torch.float16
            dec = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(tdt).double().numpy()
            got = dec(d)[rows, cols]
            cc = None if C is None else dec(C)[rows, cols]
        else:
            got = d[rows, cols]
            cc = None if C is None else C[rows, cols]
        r = oracle.check_float(got, ref, s, K, alpha, A.scale, B.scale, beta, cc, out=out)
    say("  ", {k: v for k, v in r.items() if k != "worst"})
    assert r["ok"], r


def test_streamk_deterministic_and_small_workspace_falls_back():
    mcg = need_gpu()
    M, N, K = 4096, 4864, 4096
    A = W.operand("A", "bf16", M, K, "normal", "k_contig", seed=51)
    B = W.operand("B", "bf16", K, N, "normal", "k_contig", seed=52)
    dA, dB = dev(A.codes), dev(B.codes)
    need = mcg.dense_workspace_bytes("bf16", "k_contig", "k_contig", M, N, K, dA, K, dB, K)
    assert need > 0
    outs = []
    for ws_bytes in (need, need, need - 16):
        ws = workspace(need)
        D = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        mcg.gemm_dense_ws("bf16", "bf16", "k_contig", "k_contig", M, N, K, dA, K, dB, K, None, D, N, "f32",
                          workspace=ws, workspace_bytes=ws_bytes)
        torch.cuda.synchronize()
        outs.append(D.cpu().numpy())
    D = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mcg.gemm_dense("bf16", "bf16", "k_contig", "k_contig", M, N, K, dA, K, dB, K, None, D, N, "f32")
    torch.cuda.synchronize()
    plain = D.cpu().numpy()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), "stream-K not deterministic"
    assert np.array_equal(outs[2].view(np.uint32), plain.view(np.uint32)), "small workspace must run gemm_dense"
    # the stream-K tiles differ from the whole-tile order only within the bound
    sk, _ = remainder_tiles(M, N, num_cu())
    rows, cols = tile_coords(sk[:4], M, N)
    ref, s = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", M, N, K, A.codes, K, B.codes, K,
                               rows=rows, cols=cols)
    assert oracle.check_float(outs[0][rows, cols], ref, s, K)["ok"]
    assert oracle.check_float(plain[rows, cols], ref, s, K)["ok"]


SPARSE_CASES = [  # dtA, dtB, layB, M, N, K, out, alpha, beta, D aliases C
    ("bf16", "bf16", "k_contig", 2048, 2048, 8192, "f32", 1.5, 0.5, False),          # 64 tiles, 4 pieces each
    ("i8", "i8", "mn_contig", 2048, 2048, 8192, "i32", 3, -2, False),                # int8, MN-contiguous B
    ("f16", "f16", "k_contig", 4096, 4352, 8192, "f16", -0.75, 1.0, True),          # whole rounds + 16 tiles
    ("e4m3", "e5m2", "k_contig", 2100, 2000, 8192, "f32", 1.0, 0.0, False),         # ragged, native fp8
    # pieces of 3 kept-value stages: most pieces start inside an index block (4
    # stages of 16-bit, 2 of 8-bit elements), whose earlier parts they load first
    ("bf16", "bf16", "k_contig", 1024, 1024, 6144, "f32", 1.0, 0.0, False),         # 16 tiles, 16 pieces each
    ("i8", "i8", "k_contig", 1024, 1536, 6144, "i32", 1, 1, False),                 # 24 tiles, 8 pieces each
]


@pytest.mark.parametrize("case", SPARSE_CASES, ids=["sparse_bf16", "sparse_i8_mn", "sparse_f16_f16out_alias",
                                                    "sparse_fp8_ragged", "sparse_bf16_pieces_of_3",
                                                    "sparse_i8_pieces_of_3"])
def test_sparse_streamk_against_oracle(case):
    """gemm_sparse24_ws: every output of the stream-K tiles, one whole tile and
    sampled others against the oracle (A compressed on the host by the oracle)."""
    mcg = need_gpu()
    dtA, dtB, layB, M, N, K, out, alpha, beta, alias = case
    say(f"sparse stream-K {dtA}x{dtB} B {layB} {M}x{N}x{K} -> {out} alias={alias}")
    i8 = dtA == "i8"
    A = W.sparse24_dense(dtA, M, K, dist="int8" if i8 else "normal", seed=81)
    B = W.operand("B", dtB, K, N, "int8" if i8 else "normal", layB, seed=82, fp8_scaled=not i8)
    if not i8:
        alpha = alpha * B.scale
    v, ix, nv = oracle.compress24(dtA, A)
    assert nv == 0
    dv, di, dB = dev(v), dev(ix.view(np.int32)), dev(B.codes)
    lda_c, ld_idx = K // 2, (K + 31) // 32
    assert mcg.sparse24_path(dtA, layB, M, N, K, dv, lda_c, di, ld_idx, dB, B.ld) == 1
    need = mcg.sparse24_workspace_bytes(dtA, layB, M, N, K, dv, lda_c, di, ld_idx, dB, B.ld)
    assert need > 0 and need % (256 * 256 * 4) == 0
    C = None
    if out == "i32":
        C = W.c_matrix(M, N, "int20", seed=83)
        D = torch.full((M, N), -0x5A5A5A5A, dtype=torch.int32, device="cuda")
    elif out == "f32":
        C = W.c_matrix(M, N, "normal", seed=83) if beta != 0 else None
        D = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    else:
        c16 = W.draw("normal", (M, N), 83).to(torch.float32).to(torch.float16)
        C = c16.view(torch.int16).numpy().view(np.uint16)
        D = torch.full((M, N), 0x7E00, dtype=torch.int32).to(torch.int16).to("cuda")
    dC = None if C is None else dev(C.view(np.int16) if out == "f16" else C)
    if alias:
        D = dC
    ws = workspace(need)
    mcg.gemm_sparse24_ws(dtA, dtB, layB, M, N, K, dv, lda_c, di, ld_idx, dB, B.ld, dC, D, N, out, alpha, beta,
                         workspace=ws)
    torch.cuda.synchronize()
    d = D.cpu().numpy()
    sk, first = remainder_tiles(M, N, num_cu(), 256)
    r1, c1 = tile_coords(sk + [first], M, N, 256)
    r2, c2 = W.sample_coords(M, N, n_random=2048, full_rows=(M - 1,), full_cols=(N - 1,))
    rows, cols = np.concatenate([r1, r2]), np.concatenate([c1, c2])
    say(f"  {len(sk)} stream-K tiles, {need // (256 * 256 * 4)} pieces, {len(rows)} outputs compared")
    ref, s = oracle.gemm_sparse24(dtA, dtB, layB, M, N, K, v, ix, B.codes, B.ld, C, N, alpha, beta,
                                  rows=rows, cols=cols, out=out if out in ("f16", "bf16") else "f32")
    if i8:
        r = oracle.check_exact(d[rows, cols], ref)
    else:
        if out == "f16":
            dec = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.float16).double().numpy()
            got, cc = dec(d)[rows, cols], dec(C)[rows, cols]
        else:
            got, cc = d[rows, cols], None if C is None else C[rows, cols]
        r = oracle.check_float(got, ref, s, K, alpha, beta=beta, c=cc, out=out if out == "f16" else "f32")
    say("  ", {k: v for k, v in r.items() if k != "worst"})
    assert r["ok"], r


LONG_K_CASES = [  # dtA, dtB, layA, layB, M, N, K, out, alpha, beta, D aliases C
    # 144 tiles of 128 x 128 fill no second round and cannot be cut (2 pieces would
    # need 288 CUs): 36 tiles of 256 x 256 in 4 pieces of 64 K tiles instead
    ("bf16", "bf16", "k_contig", "k_contig", 1536, 1536, 16384, "f32", 1.0, 0.5, False),
    ("i8", "i8", "k_contig", "mn_contig", 1536, 1536, 32768, "i32", 2, -1, False),
    # ragged M and N, a last K tile cut short (K = 16592: 260 K tiles, the last a
    # quarter full), 42 tiles in 5 pieces, D aliasing C
    ("bf16", "bf16", "mn_contig", "k_contig", 1504, 1700, 16592, "bf16", -1.0, 1.0, True),
]


@pytest.mark.parametrize("case", LONG_K_CASES, ids=["bf16", "i8_mn", "ragged_bf16out_alias"])
def test_long_k_mid_plan_takes_256_streamk(case):
    """A 128 x 128 plan with no stream-K split of its own and at least 256 K
    tiles runs as 256 x 256 stream-K when a workspace is given."""
    mcg = need_gpu()
    dtA, dtB, layA, layB, M, N, K, out, alpha, beta, alias = case
    say(f"long-K stream-K {dtA} {layA}/{layB} {M}x{N}x{K} -> {out} alias={alias}")
    dist = "int8" if dtA == "i8" else "normal"
    A = W.operand("A", dtA, M, K, dist, layA, seed=81)
    B = W.operand("B", dtB, K, N, dist, layB, seed=82)
    dA, dB = dev(A.codes), dev(B.codes)
    assert mcg.dense_path(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld) == 6
    need = mcg.dense_workspace_bytes(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld)
    tm, tn = -(-M // 256), -(-N // 256)
    assert need > 0 and need % (256 * 256 * 4) == 0 and need // (256 * 256 * 4) % (tm * tn) == 0
    ldc = N
    if out == "i32":
        C = W.c_matrix(M, N, "int20", seed=83, ldc=ldc)
        D = torch.full((M, ldc), -0x5A5A5A5A, dtype=torch.int32, device="cuda")
        dC = dev(C)
    elif out == "f32":
        C = W.c_matrix(M, N, "normal", seed=83, ldc=ldc)
        D = torch.full((M, ldc), float("nan"), dtype=torch.float32, device="cuda")
        dC = dev(C)
    else:
        C = W.draw("normal", (M, ldc), 83).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
        dC = dev(C)
        C = C.view(np.uint16)
        D = torch.full((M, ldc), 0x7FC0, dtype=torch.int16, device="cuda")
    if alias:
        D = dC
    mcg.gemm_dense_ws(dtA, dtB, layA, layB, M, N, K, dA, A.ld, dB, B.ld, dC, D, ldc, out, alpha, beta,
                      A.scale, B.scale, workspace=workspace(need))
    torch.cuda.synchronize()
    d = D.cpu().numpy()
    # four whole tiles (the last one ragged when M, N are) and sampled outputs
    tiles = [(0, 0), (1, 2), (tm - 1, 0), (tm - 1, tn - 1)]
    r1, c1 = tile_coords(tiles, M, N)
    r2, c2 = W.sample_coords(M, N, n_random=2048, full_rows=(M - 1,), full_cols=(N - 1,))
    rows, cols = np.concatenate([r1, r2]), np.concatenate([c1, c2])
    say(f"  {tm * tn} tiles, {need // (256 * 256 * 4)} pieces, {len(rows)} outputs compared")
    if out == "i32":
        ref = oracle.gemm_i8(layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc, alpha, beta,
                             rows=rows, cols=cols)
        r = oracle.check_exact(d[rows, cols], ref)
    else:
        ref, s = oracle.gemm_float(dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc,
                                   alpha, beta, A.scale, B.scale, rows=rows, cols=cols, out=out)
        if out == "bf16":
            dec = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).double().numpy()
            got, cc = dec(d)[rows, cols], dec(C)[rows, cols]
        else:
            got, cc = d[rows, cols], C[rows, cols]
        r = oracle.check_float(got, ref, s, K, alpha, A.scale, B.scale, beta, cc, out=out)
    say("  ", {k: v for k, v in r.items() if k != "worst"})
    assert r["ok"], r


GENERAL_SK_CASES = [  # dtA, dtB, layA, layB, M, N, K, out, alpha, beta, D aliases C
    # 64 tiles of 128 x 128 in 4 pieces of 64 K tiles (without a workspace: the
    # general kernel with K split in 4)
    ("bf16", "bf16", "k_contig", "k_contig", 1024, 1024, 16384, "f32", 1.0, 0.5, False),
    ("bf16", "bf16", "mn_contig", "k_contig", 768, 768, 32768, "bf16", -0.5, 1.0, True),
    # ragged: 9 tiles in 26 pieces of 5 K tiles, the last K tile cut short
    ("i8", "i8", "k_contig", "k_contig", 300, 264, 16592, "i32", 3, -2, False),
    ("e4m3", "e5m2", "k_contig", "k_contig", 256, 384, 8192, "f32", 1.0, 0.0, False),
]


@pytest.mark.parametrize("case", GENERAL_SK_CASES, ids=["bf16", "bf16_mn_bf16out_alias", "i8_ragged", "fp8"])
def test_general_plan_takes_128_streamk(case):
    """A few-tile, long-K problem that the general kernel takes without a
    workspace runs as 128 x 128 stream-K with one; every output is compared."""
    mcg = need_gpu()
    dtA, dtB, layA, layB, M, N, K, out, alpha, beta, alias = case
    say(f"general -> 128 x 128 stream-K {dtA}x{dtB} {layA}/{layB} {M}x{N}x{K} -> {out} alias={alias}")
    fp8 = dtA in ("e4m3", "e5m2")
    dist = "int8" if dtA == "i8" else "normal"
    A = W.operand("A", dtA, M, K, dist, layA, seed=85, fp8_scaled=fp8)
    B = W.operand("B", dtB, K, N, dist, layB, seed=86, fp8_scaled=fp8)
    dA, dB = dev(A.codes), dev(B.codes)
    assert mcg.dense_path(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld) == 0
    need = mcg.dense_workspace_bytes(dtA, layA, layB, M, N, K, dA, A.ld, dB, B.ld)
    assert need > 0 and need % (128 * 128 * 4) == 0
    ldc = N
    if out == "i32":
        C = W.c_matrix(M, N, "int20", seed=87, ldc=ldc)
        D = torch.full((M, ldc), -0x5A5A5A5A, dtype=torch.int32, device="cuda")
        dC = dev(C)
    elif out == "f32":
        C = W.c_matrix(M, N, "normal", seed=87, ldc=ldc) if beta != 0 else None
        D = torch.full((M, ldc), float("nan"), dtype=torch.float32, device="cuda")
        dC = None if C is None else dev(C)
    else:
        C = W.draw("normal", (M, ldc), 87).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
        dC = dev(C)
        C = C.view(np.uint16)
        D = torch.full((M, ldc), 0x7FC0, dtype=torch.int16, device="cuda")
    if alias:
        D = dC
    mcg.gemm_dense_ws(dtA, dtB, layA, layB, M, N, K, dA, A.ld, dB, B.ld, dC, D, ldc, out, alpha, beta,
                      A.scale, B.scale, workspace=workspace(need))
    torch.cuda.synchronize()
    d = D.cpu().numpy()
    say(f"  {need // (128 * 128 * 4)} pieces, {M * N} outputs compared")
    if out == "i32":
        ref = oracle.gemm_i8(layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc, alpha, beta)
        r = oracle.check_exact(d[:M, :N], ref)
    else:
        ref, s = oracle.gemm_float(dtA, dtB, layA, layB, M, N, K, A.codes, A.ld, B.codes, B.ld, C, ldc,
                                   alpha, beta, A.scale, B.scale, out=out)
        if out == "bf16":
            dec = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).double().numpy()
            got, cc = dec(d)[:M, :N], dec(C)[:M, :N]
        else:
            got, cc = d[:M, :N], None if C is None else C[:M, :N]
        r = oracle.check_float(got, ref, s, K, alpha, A.scale, B.scale, beta, cc, out=out)
    say("  ", {k: v for k, v in r.items() if k != "worst"})
    assert r["ok"], r
