"""CPU checks of the fragment-layout module (matrix_core_gemm_amd/csrc/frag_layout.hpp).

A host program built from the module dumps every map.  The checks:
  - every accumulator map is a bijection between (lane, register) and
    (i, j, block) over the shape's range, in both directions;
  - every map agrees with the row-band tables of "CDNA3 dense MFMA builtins",
    Accumulator layout (tests/golden/acc_layout_tables.txt): rows of a band
    sit exactly in the listed lanes and registers;
  - the dense operand maps assign each (row, k) of an instruction to exactly
    one (lane, element), and the 2:4 maps give every row's K/4 groups of four
    exactly two kept elements and every column's K dense k exactly one element.
The gfx950 placement itself (block 0 of the 32 x 32 and 16 x 16 layouts, the
FP64 layouts, the measured operand layouts) is a hardware fact: on the CPU it
is parity unpinned, and the bit-exact GPU GEMM tests (small integers,
permutations, int8, the 2:4 kernels) pin it on the device.
"""
import os
import subprocess
from collections import defaultdict

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SHAPES = {"32x32": (32, 32, 2, 32), "16x16": (16, 16, 4, 16), "4x4": (4, 4, 16, 4),
          "16x16_f64": (16, 16, 1, 4), "4x4_f64": (4, 4, 4, 1)}  # R, C, blocks, registers per lane


@pytest.fixture(scope="module")
def dump(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("fl") / "frag_layout_dump")
    subprocess.check_call([HIPCC, "-std=c++17", "-O1", "-I", os.path.join(ROOT, "matrix_core_gemm_amd", "csrc"),
                           os.path.join(ROOT, "tests", "frag_layout_dump.cpp"), "-o", exe],
                          stderr=subprocess.DEVNULL)
    out = subprocess.check_output([exe], text=True)
    d = defaultdict(list)
    for line in out.splitlines():
        kind, name, *vals = line.split()
        d[(kind, name)].append(tuple(int(v) for v in vals))
    return d


@pytest.mark.parametrize("shape", list(SHAPES))
def test_accumulator_map_is_a_bijection(dump, shape):
    R, C, blocks, regs = SHAPES[shape]
    coord = {(l, r): (i, j, b) for l, r, i, j, b in dump[("coord", shape)]}
    slot = {(i, j, b): (l, r) for i, j, b, l, r in dump[("slot", shape)]}
    # as many registers in the wavefront as output elements
    assert len(coord) == 64 * regs == R * C * blocks == len(slot)
    assert set(coord.values()) == {(i, j, b) for i in range(R) for j in range(C) for b in range(blocks)}
    for lr, ijb in coord.items():
        assert slot[ijb] == lr, (shape, lr, ijb)


def _rng(s):
    if "," in s:
        return [int(x) for x in s.split(",")]
    a, b = (int(x) for x in s.split("-"))
    return list(range(a, b + 1))


def test_accumulator_maps_match_the_printed_tables(dump):
    path = os.path.join(ROOT, "tests", "golden", "acc_layout_tables.txt")
    n = 0
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        shape, rows, blocks, lanes, regs = line.split()
        slot = {(i, j, b): (l, r) for i, j, b, l, r in dump[("slot", shape)]}
        R, C, _, _ = SHAPES[shape]
        # the band's rows of the listed blocks occupy exactly the listed lanes and registers
        got_lanes, got_regs = set(), set()
        for b in _rng(blocks):
            for i in _rng(rows):
                for j in range(C):
                    l, r = slot[(i, j, b)]
                    got_lanes.add(l)
                    got_regs.add(r)
        assert got_lanes == set(_rng(lanes)), (line, sorted(got_lanes))
        assert got_regs == set(_rng(regs)), (line, sorted(got_regs))
        n += 1
    assert n == 27  # every table row of the fixture was checked


def test_gfx950_single_block_maps(dump):
    """The block-0 maps the kernels rely on, as measured on gfx950 (lane l,
    register r): 16 x 16 -> (4 (l >> 4) + r, l & 15); 32 x 32 ->
    (8 (r >> 2) + 4 (l >> 5) + (r & 3), l & 31); FP64 16 x 16 -> (4 r + (l >> 4), l & 15).
    Parity unpinned on the CPU: the GPU bit-exact GEMM tests pin these."""
    c16 = {(l, r): (i, j) for l, r, i, j, b in dump[("coord", "16x16")] if r < 4}
    c32 = {(l, r): (i, j) for l, r, i, j, b in dump[("coord", "32x32")] if r < 16}
    c64 = {(l, r): (i, j) for l, r, i, j, b in dump[("coord", "16x16_f64")]}
    for l in range(64):
        for r in range(4):
            assert c16[(l, r)] == (4 * (l >> 4) + r, l & 15)
            assert c64[(l, r)] == (4 * r + (l >> 4), l & 15)
        for r in range(16):
            assert c32[(l, r)] == (8 * (r >> 2) + 4 * (l >> 5) + (r & 3), l & 31)


DENSE = {"32x32x16_bf16": (32, 8, 16), "16x16x32_bf16": (16, 8, 32), "32x32x32_i8": (32, 16, 32),
         "16x16x64_i8": (16, 16, 64), "32x32x64_f8": (32, 32, 64), "16x16x128_f8": (16, 32, 128)}


@pytest.mark.parametrize("name", list(DENSE))
def test_dense_operand_maps(dump, name):
    S, E, K = DENSE[name]
    rows = dump[("dense", name)]
    seen = set()
    for l, e, row, k, sl, se in rows:
        assert (sl, se) == (l, e)           # slot(row(l), k(l, e)) inverts the map
        seen.add((row, k))
    assert seen == {(r, k) for r in range(S) for k in range(K)}


SPARSE = {"32x32x32_16bit": (32, 32, 8, 16), "32x32x64_8bit": (32, 64, 16, 32),
          "16x16x64_16bit": (16, 64, 8, 16), "16x16x128_8bit": (16, 128, 16, 32)}


@pytest.mark.parametrize("name", list(SPARSE))
def test_sparse_operand_maps(dump, name):
    S, K, kept, ebd = SPARSE[name]
    (geom,) = dump[("sparse_geom", name)]
    assert geom[:3] == (K, kept, ebd)
    groups = defaultdict(int)
    for l, e, row, grp in dump[("sparse_a", name)]:
        groups[(row, grp)] += 1
    # every row's K/4 groups of four hold exactly two kept values
    assert dict(groups) == {(r, g): 2 for r in range(S) for g in range(K // 4)}
    ks = defaultdict(int)
    for l, e, col, k in dump[("sparse_b", name)]:
        ks[(col, k)] += 1
    assert dict(ks) == {(c, k): 1 for c in range(S) for k in range(K)}


def test_sparse_operand_maps_measured_examples(dump):
    """Measured on gfx950 (16-bit 32x32x32): lane group g of the sparse operand
    holds dense k 16g .. 16g + 15, the dense operand k 8g .. 8g + 7 and
    16 + 8g .. 16 + 8g + 7; (8-bit 16x16x128): groups of 32 dense k, dense
    operand k 16g .. 16g + 15 and 64 + 16g ..  Parity unpinned on the CPU."""
    a = {(l, e): g for l, e, _, g in dump[("sparse_a", "32x32x32_16bit")]}
    b = {(l, e): k for l, e, _, k in dump[("sparse_b", "32x32x32_16bit")]}
    for l in range(64):
        g = l // 32
        assert {a[(l, e)] for e in range(8)} == set(range(4 * g, 4 * g + 4))
        assert [b[(l, e)] for e in range(16)] == list(range(8 * g, 8 * g + 8)) + list(range(16 + 8 * g, 24 + 8 * g))
    b8 = {(l, e): k for l, e, _, k in dump[("sparse_b", "16x16x128_8bit")]}
    for l in range(64):
        g = l // 16
        assert [b8[(l, e)] for e in range(32)] == list(range(16 * g, 16 * g + 16)) + list(range(64 + 16 * g, 80 + 16 * g))
