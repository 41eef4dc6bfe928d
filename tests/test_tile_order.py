"""CPU checks of the tile order and the stream-K plan.

tile_order.hpp (built into a host program, tests/tile_order_dump.cpp):
  - the grouped order is a bijection of the tile grid, and runs column by
    column through groups of four tile rows;
  - sk_first_piece, a closed form, equals the count of pieces found by walking
    every workgroup's range of K tiles over the tile boundaries.
mcg_dense_workspace_bytes (the library's host-side plan, 256 compute units when
no device is present): one binary32 tile per piece for shapes whose last round
of tiles is short, 0 where whole rounds fill the device or there is too little
to gain.
"""
import os
import subprocess
from collections import defaultdict

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def dump(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("to") / "tile_order_dump")
    subprocess.check_call([HIPCC, "-std=c++17", "-O1", "-I", os.path.join(ROOT, "matrix_core_gemm_amd", "csrc"),
                           os.path.join(ROOT, "tests", "tile_order_dump.cpp"), "-o", exe],
                          stderr=subprocess.DEVNULL)
    out = subprocess.check_output([exe], text=True)
    d = defaultdict(list)
    for line in out.splitlines():
        kind, *vals = line.split()
        d[kind].append(tuple(int(v) for v in vals))
    return d


def test_grouped_order_is_a_bijection_in_row_groups(dump):
    grids = defaultdict(dict)
    for tm_, tn_, pid, tm, tn in dump["tile"]:
        grids[(tm_, tn_)][pid] = (tm, tn)
    assert len(grids) == 8
    for (rows, cols), order in grids.items():
        assert sorted(order.values()) == [(i, j) for i in range(rows) for j in range(cols)]
        for pid, (tm, tn) in order.items():
            # group of four tile rows (the last one may be smaller), column-major inside it
            g, r = divmod(pid, 4 * cols)
            gsize = min(4, rows - 4 * g)
            assert (tm, tn) == (4 * g + r % gsize, r // gsize), (rows, cols, pid)


def brute_pieces(tiles, nk, L):
    """First-piece index of every workgroup, by walking the ranges."""
    total, firsts = 0, []
    w = 0
    while w * L < tiles * nk:
        s, e = w * L, min(w * L + L, tiles * nk)
        firsts.append(total)
        total += (e - 1) // nk - s // nk + 1
        w += 1
    return firsts, total


def test_first_piece_closed_form_matches_the_walk(dump):
    by_case = defaultdict(dict)
    for tiles, nk, L, w, first in dump["piece"]:
        by_case[(tiles, nk, L)][w] = first
    assert len(by_case) == 10
    for (tiles, nk, L), got in by_case.items():
        firsts, _ = brute_pieces(tiles, nk, L)
        assert [got[w] for w in range(len(firsts))] == firsts, (tiles, nk, L)


def _ws(mcg, dt, M, N, K):
    return mcg.dense_workspace_bytes(dt, "k_contig", "k_contig", M, N, K, 0x1000, K, 0x1000, K)


def test_workspace_plan(monkeypatch):
    mcg = pytest.importorskip("matrix_core_gemm_amd")
    slot = 256 * 256 * 4
    # 7168^3 bf16: 784 tiles = 3 rounds + 16; 112 K tiles each cut into 16 pieces of 7
    assert _ws(mcg, "bf16", 7168, 7168, 7168) == 256 * slot
    # 6144^3: 576 = 2 rounds + 64, 4 pieces of 24 per tile
    assert _ws(mcg, "bf16", 6144, 6144, 6144) == 256 * slot
    # int8 7168^3: 56 K tiles of 128 bytes, ranges of 4: 224 workgroups, one piece each
    assert _ws(mcg, "i8", 7168, 7168, 7168) == 224 * slot
    # 16 x 19 tiles = 256 + 48, K = 4096 (64 K tiles): at most 5 pieces per tile,
    # 5 does not divide 64, so 4 pieces of 16 K tiles: 192 workgroups
    assert _ws(mcg, "bf16", 4096, 4864, 4096) == 192 * slot
    # whole rounds, or too little to gain (5120^3: the last round is 144 of 256 tiles)
    assert _ws(mcg, "bf16", 8192, 8192, 8192) == 0
    assert _ws(mcg, "bf16", 4096, 4096, 4096) == 0
    assert _ws(mcg, "bf16", 5120, 5120, 5120) == 0
    # the 128 x 128 form (too few 256 x 256 tiles): 1024 x 2048 is 128 tiles of
    # 128 x 128 with 128 K tiles, each tile cut in two: 256 slots of 64 KiB;
    # 1280^2 x 16384 is 100 tiles, cut in two (three would need 300 CUs)
    assert _ws(mcg, "bf16", 1024, 2048, 8192) == 256 * 128 * 128 * 4
    assert _ws(mcg, "bf16", 1280, 1280, 16384) == 200 * 128 * 128 * 4
    # long K on the 128 x 128 form without a split of its own (1536^2 is 144 tiles:
    # two pieces each would need 288 CUs): from 256 K tiles of 128 bytes on, the
    # 256 x 256 split, here 36 tiles in 4 pieces of 64 K tiles (2560^2: 100 tiles in 2)
    assert _ws(mcg, "bf16", 1536, 1536, 16384) == 144 * slot
    assert _ws(mcg, "i8", 1536, 1536, 32768) == 144 * slot
    assert _ws(mcg, "bf16", 2560, 2560, 16384) == 200 * slot
    assert _ws(mcg, "bf16", 2048, 2048, 16384) == 0  # 256 tiles of 128 x 128: one whole round
    assert _ws(mcg, "bf16", 1536, 1536, 12288) == 0  # 192 K tiles: the two forms are even
    assert _ws(mcg, "i8", 1536, 1536, 16384) == 0
    # few tiles, long K: the general kernel without a workspace, the 128 x 128
    # split with one (1024^2 x 16384: 64 tiles in 4 pieces; 300 x 264: 9 in 26)
    assert _ws(mcg, "bf16", 1024, 1024, 16384) == 256 * 128 * 128 * 4
    assert _ws(mcg, "i8", 300, 264, 16592) == 234 * 128 * 128 * 4
    # not the pipelined kernel (skinny, binary64)
    assert _ws(mcg, "bf16", 32768, 16, 8192) == 0
    assert mcg.dense_workspace_bytes("f64", "k_contig", "k_contig", 7168, 7168, 7168, 0x1000, 7168, 0x1000,
                                     7168) == 0


def test_gemm_dense_ws_argument_errors():
    mcg = pytest.importorskip("matrix_core_gemm_amd")
    lib = mcg.lib()
    args = (0, 0, 0, 0, 256, 256, 256, 0x1000, 256, 0x1000, 256, None, 0x1000, 256, 5, 1.0, 0.0, 1.0, 1.0)
    assert lib.gemm_dense_ws(*args, 0x1008, 1 << 20, None) == 5   # workspace not 16-byte aligned
    assert lib.gemm_dense_ws(*args, 0x1000, -1, None) == 2        # negative size
    # validation of the GEMM arguments comes first, as in gemm_dense
    bad = list(args)
    bad[4] = -1
    assert lib.gemm_dense_ws(*bad, 0x1000, 1 << 20, None) == lib.mcg_validate_dense(*bad)


def _sws(mcg, dt, M, N, K):
    return mcg.sparse24_workspace_bytes(dt, "k_contig", M, N, K, 0x1000, K // 2, 0x1000, (K + 31) // 32, 0x1000, K)


def test_sparse_workspace_plan():
    mcg = pytest.importorskip("matrix_core_gemm_amd")
    slot = 256 * 256 * 4
    # 2048^2 x 8192 bf16: 64 tiles of 256 x 256, 64 kept-value stages each, cut in 4
    assert _sws(mcg, "bf16", 2048, 2048, 8192) == 256 * slot
    # 1536^2: 36 tiles, at most 7 pieces each, 4 divides 64 stages: 144 pieces
    assert _sws(mcg, "bf16", 1536, 1536, 8192) == 144 * slot
    # int8: 256 dense k per stage, 2048^2 x 8192 has 32 stages per tile, cut in 4
    assert _sws(mcg, "i8", 2048, 2048, 8192) == 256 * slot
    # pieces of 3 stages (the GPU tests' cases whose pieces start inside an index
    # block of 4 or 2 stages): bf16 1024^2 x 6144, 48 stages cut in 16; int8
    # 1024 x 1536 x 6144, 24 stages cut in 8
    assert _sws(mcg, "bf16", 1024, 1024, 6144) == 16 * 16 * slot
    assert _sws(mcg, "i8", 1024, 1536, 6144) == 24 * 8 * slot
    # whole rounds, too little to gain, or not the 256 x 256 sparse kernel
    assert _sws(mcg, "bf16", 8192, 8192, 8192) == 0
    assert _sws(mcg, "bf16", 2048, 2048, 2048) == 0
    assert _sws(mcg, "bf16", 200, 2048, 8192) == 0


def test_gemm_sparse24_ws_argument_errors():
    mcg = pytest.importorskip("matrix_core_gemm_amd")
    lib = mcg.lib()
    args = (0, 0, 0, 256, 256, 256, 0x1000, 128, 0x1000, 8, 0x1000, 256, None, 0x1000, 256, 5, 1.0, 0.0)
    assert lib.gemm_sparse24_ws(*args, 0x1008, 1 << 20, None) == 5   # workspace not 16-byte aligned
    assert lib.gemm_sparse24_ws(*args, 0x1000, -1, None) == 2        # negative size
    bad = list(args)
    bad[5] = 6  # K not a multiple of 4
    assert lib.gemm_sparse24_ws(*bad, 0x1000, 1 << 20, None) == lib.mcg_validate_sparse24(*bad) == 2
