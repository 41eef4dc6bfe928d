"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects bad arguments on the host before touching the device,
and its host compressor matches the oracle byte for byte."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mcg.h")

m = pytest.importorskip("matrix_core_gemm_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("gemm_dense", "gemm_sparse24", "compress24", "compress24_host", "decompress24_host",
               "mcg_status_string"):
        assert fn in names
    assert set(names) == set(m.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(m.LIB_PATH)
    for fn in declared_functions():
        assert hasattr(lib, fn), fn


def test_status_strings():
    for s in range(11):
        assert m.status_string(s) and "unknown" not in m.status_string(s)
    assert "unknown" in m.status_string(999)
    assert m.version() >= 100


FAKE = 0x10000  # a 64 KiB-aligned non-null address; validation never dereferences it


def dense_args(**kw):
    a = dict(dtypeA="bf16", dtypeB="bf16", layoutA="k_contig", layoutB="k_contig", M=64, N=32, K=48,
             A=FAKE, lda=48, B=FAKE, ldb=48, C=None, D=FAKE, ldc=32, dtypeD="f32", alpha=1.0,
             beta=0.0, scaleA=1.0, scaleB=1.0)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    ({"dtypeA": "f16"}, 4),                          # mixed non-fp8 pair
    ({"dtypeA": "i8", "dtypeB": "i8"}, 4),           # int8 needs i32 output
    ({"dtypeA": "i8", "dtypeB": "i8", "dtypeD": "i32"}, 0),
    ({"dtypeA": "e4m3", "dtypeB": "e5m2"}, 0),
    ({"dtypeA": "e4m3", "dtypeB": "bf16"}, 4),
    ({"dtypeA": 9}, 4),
    ({"layoutA": 2}, 4),
    ({"M": -1}, 2),
    ({"K": -5}, 2),
    ({"M": 0, "A": None, "B": None, "D": None}, 0),  # empty output: no-op
    ({"N": 0, "D": None}, 0),
    ({"D": None}, 1),
    ({"A": None}, 1),
    ({"K": 0, "A": None, "B": None, "lda": 1, "ldb": 1}, 0),
    ({"beta": 1.0}, 1),                              # C needed
    ({"beta": 1.0, "C": FAKE}, 0),
    ({"lda": 47}, 3),
    ({"ldb": 47}, 3),
    ({"ldc": 31}, 3),
    ({"layoutA": "mn_contig", "lda": 63}, 3),
    ({"layoutA": "mn_contig", "lda": 64}, 0),
    ({"layoutB": "mn_contig", "ldb": 31}, 3),
    ({"A": FAKE + 1}, 5),                            # bf16 pointer not 2-byte aligned
    ({"D": FAKE + 2}, 5),
    ({"A": FAKE + 2, "lda": 49}, 0),                 # unaligned to 16 is allowed (slow path)
    ({"scaleA": 2.0}, 10),                           # scales only for fp8
    ({"dtypeA": "e4m3", "dtypeB": "e4m3", "scaleA": 0.25}, 0),
    ({"dtypeA": "i8", "dtypeB": "i8", "dtypeD": "i32", "alpha": 1.5}, 10),
    ({"dtypeA": "i8", "dtypeB": "i8", "dtypeD": "i32", "beta": 2.0 ** 31, "C": FAKE}, 10),
    ({"alpha": float("nan")}, 10),
    ({"alpha": 1e39}, 10),                           # finite in binary64, infinite as fp32
    ({"beta": -1e39, "C": FAKE}, 10),
    ({"alpha": 3e38}, 0),                            # still finite as fp32
    ({"dtypeA": "e4m3", "dtypeB": "e4m3", "alpha": 1e30, "scaleA": 1e10}, 10),   # alpha*scaleA*scaleB overflows
    ({"dtypeA": "e4m3", "dtypeB": "e4m3", "alpha": 1e30, "scaleA": 1e-10}, 0),
    ({"dtypeA": "f64", "dtypeB": "f64", "dtypeD": "f64", "alpha": 1e39}, 0),   # binary64 keeps its range
    ({"dtypeD": "bf16"}, 0),                         # 16-bit outputs for float inputs
    ({"dtypeD": "f16", "beta": 1.0, "C": FAKE}, 0),
    ({"dtypeA": "e4m3", "dtypeB": "e5m2", "dtypeD": "bf16"}, 0),
    ({"dtypeD": "bf16", "D": FAKE + 2}, 0),          # 16-bit D needs only 2-byte alignment
    ({"dtypeD": "bf16", "D": FAKE + 1}, 5),
    ({"dtypeD": "f16", "beta": 1.0, "C": FAKE + 1}, 5),
    ({"dtypeD": "i32"}, 4),                          # int32 output only for int8 inputs
    ({"dtypeA": "i8", "dtypeB": "i8", "dtypeD": "bf16"}, 4),
    ({"dtypeD": "e4m3"}, 4),
    ({"dtypeA": "f64", "dtypeB": "f64", "dtypeD": "f64"}, 0),   # binary64
    ({"dtypeA": "f64", "dtypeB": "f64", "dtypeD": "f32"}, 4),   # binary64 output only
    ({"dtypeA": "f64", "dtypeB": "bf16", "dtypeD": "f64"}, 4),
    ({"dtypeA": "bf16", "dtypeB": "f64", "dtypeD": "f64"}, 4),
    ({"dtypeD": "f64"}, 4),                                     # binary64 output only for binary64 inputs
    ({"dtypeA": "f64", "dtypeB": "f64", "dtypeD": "f64", "A": FAKE + 4}, 5),
    ({"dtypeA": "f64", "dtypeB": "f64", "dtypeD": "f64", "D": FAKE + 8, "lda": 49}, 0),
    ({"dtypeA": "f64", "dtypeB": "f64", "dtypeD": "f64", "scaleB": 0.5}, 10),
    ({"dtypeA": "f64", "dtypeB": "f64", "dtypeD": "f64", "beta": float("inf"), "C": FAKE}, 10),
])
def test_dense_validation(kw, status):
    assert m.validate_dense(**dense_args(**kw)) == status


def test_entry_points_reject_before_touching_the_device():
    # These calls fail validation, so no HIP call happens (no GPU here).
    with pytest.raises(m.MCGError) as e:
        m.gemm_dense(**dense_args(lda=1), stream=0)
    assert e.value.status == 3
    with pytest.raises(m.MCGError):
        m.gemm_sparse24("bf16", "bf16", "k_contig", 8, 8, 6, FAKE, 3, FAKE, 1, FAKE, 6, None, FAKE, 8,
                        "f32", stream=0)
    with pytest.raises(m.MCGError):
        m.compress24("bf16", 4, 10, FAKE, 10, FAKE, 5, FAKE, 1, stream=0)
    # empty problems succeed without a device
    m.gemm_dense(**dense_args(M=0), stream=0)


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    ({"K": 10}, 2),
    ({"dtypeA": "i8", "dtypeB": "i8"}, 4),                    # int8 needs an int32 D
    ({"dtypeA": "i8", "dtypeB": "i8", "dtypeD": "i32"}, 0),
    ({"dtypeA": "i8", "dtypeB": "i8", "dtypeD": "i32", "alpha": 0.5}, 10),
    ({"dtypeA": "i8", "dtypeB": "bf16", "dtypeD": "i32"}, 4),
    ({"dtypeA": "e4m3", "dtypeB": "e5m2"}, 0),
    ({"dtypeA": "e5m2", "dtypeB": "e4m3", "dtypeD": "bf16"}, 0),
    ({"dtypeA": "e4m3", "dtypeB": "i8"}, 4),
    ({"dtypeA": "e4m3", "dtypeB": "e4m3", "dtypeD": "i32"}, 4),
    ({"dtypeA": "e4m3", "dtypeB": "e4m3", "A_compressed": FAKE + 1}, 0),   # 1-byte elements
    ({"dtypeD": "i32"}, 4),
    ({"lda_c": 31}, 3),
    ({"ld_idx": 1}, 3),
    ({"A_index": None}, 1),
    ({"A_index": FAKE + 2}, 5),
    ({"layoutB": "mn_contig", "ldb": 48}, 3),
    ({"layoutB": "mn_contig", "ldb": 96}, 0),
    ({"dtypeD": "bf16"}, 0),
    ({"dtypeD": "f16", "D": FAKE + 2}, 0),
    ({"dtypeD": "f16", "D": FAKE + 1}, 5),
    ({"alpha": 1e39}, 10),
    ({"beta": 1e39, "C": FAKE}, 10),
])
def test_sparse_validation(kw, status):
    a = dict(dtypeA="bf16", dtypeB="bf16", layoutB="k_contig", M=64, N=96, K=64, A_compressed=FAKE,
             lda_c=32, A_index=FAKE, ld_idx=2, B=FAKE, ldb=64, C=None, D=FAKE, ldc=96, dtypeD="f32")
    a.update(kw)
    assert m.validate_sparse24(**a) == status


@pytest.mark.parametrize("dt", ["bf16", "f16", "i8", "e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [(1, 4), (7, 36), (33, 200), (16, 256)])
def test_compress24_host_matches_oracle(dt, shape):
    M, K = shape
    A = W.sparse24_dense(dt, M, K, dist="int8" if dt == "i8" else "normal")
    vals = np.zeros((M, K // 2), W.CODE_NP[dt])
    idx = np.zeros((M, (K + 31) // 32), np.uint32)
    assert m.compress24_host(dt, M, K, A, K, vals, K // 2, idx, idx.shape[1]) == 0
    ov, oi, viol = oracle.compress24(dt, A)
    assert viol == 0
    assert np.array_equal(vals, ov) and np.array_equal(idx, oi)


def test_compress24_host_flags_violations_like_oracle():
    rng = np.random.default_rng(0)
    A = rng.integers(-3, 4, (9, 64)).astype(np.int8)   # dense: many groups have > 2 non-zeros
    vals = np.zeros((9, 32), np.int8)
    idx = np.zeros((9, 2), np.uint32)
    assert m.compress24_host("i8", 9, 64, A, 64, vals, 32, idx, 2) == 6
    ov, oi, viol = oracle.compress24("i8", A)
    assert viol > 0
    assert np.array_equal(vals, ov) and np.array_equal(idx, oi)


# Kernel choice is host-only: addresses are never dereferenced.
BASE = 1 << 20


def plan(dt, M, N, K, lay=("k_contig", "k_contig"), pad=0):
    la, lb = lay
    lda = (K if la == "k_contig" else M) + pad
    ldb = (K if lb == "k_contig" else N) + pad
    path = m.dense_path(dt, la, lb, M, N, K, BASE, max(lda, 1), BASE, max(ldb, 1))
    splits = m.dense_splits(dt, la, lb, M, N, K, BASE, max(lda, 1), BASE, max(ldb, 1), None,
                            BASE + (1 << 34), "i32" if dt == "i8" else "f32", 0.0)
    return path, splits


@pytest.mark.parametrize("dt", ["bf16", "f16", "i8", "e4m3"])
@pytest.mark.parametrize("shape", [(64, 48, 0), (300, 264, 0), (2048, 2048, 0), (0, 300, 256),
                                   (300, 0, 256), (0, 0, 0)])
def test_planner_degenerate_sizes(dt, shape):
    """Empty problems plan without splitting (and without a host arithmetic fault)."""
    path, splits = plan(dt, *shape)
    assert path in (0, 1, 2, 3, 4, 6)
    assert splits == 1


@pytest.mark.parametrize("dt", ["bf16", "i8", "e4m3"])
def test_planner_kernel_by_shape(dt):
    """256 x 256 tiles from 128 of them; below that the 128 x 128 form when it beats
    the general kernel's best split (few tiles with long K keep the split general
    kernel); the general kernel for unaligned operands; the streaming kernel for N <= 32."""
    assert plan(dt, 8192, 8192, 8192)[0] == 1
    assert plan(dt, 2048, 2048, 2048) == (6, 1)
    assert plan(dt, 1024, 2048, 8192) == (6, 1)
    assert plan(dt, 2560, 2560, 2560) == (6, 1)        # 400 tiles of 128 x 128: two rounds
    assert plan(dt, 256, 256, 65536)[0] == 0           # 4 tiles, very long K: split K wins
    assert plan(dt, 2048, 2048, 2050, pad=2)[0] == 0   # K * elem_bytes not a multiple of 16
    assert plan(dt, 256, 200, 8192)[0] == 0            # 4 tiles: split K wins
    assert plan(dt, 256, 200, 8192)[1] > 1
    assert plan(dt, 4096, 16, 4096)[0] == 4


# ---------------------------------------------------------------- decompress24_host

@pytest.mark.parametrize("dt", ["bf16", "f16", "i8", "e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [(1, 4), (7, 36), (33, 200), (16, 256)])
def test_decompress24_host_matches_oracle_and_round_trips(dt, shape):
    M, K = shape
    A = W.sparse24_dense(dt, M, K, dist="int8" if dt == "i8" else "normal")
    ov, oi, viol = oracle.compress24(dt, A)
    assert viol == 0
    out = np.full((M, K + 3), 0x55, W.CODE_NP[dt])           # padded ld; padding must survive
    m.decompress24_host(dt, M, K, ov, K // 2, oi, oi.shape[1], out, K + 3)
    assert np.array_equal(out[:, :K], oracle.decompress24(dt, ov, oi, K))
    assert np.array_equal(out[:, :K], A)                      # decompress(compress(A)) == A
    assert np.all(out[:, K:] == 0x55)
    # compress(decompress(v, i)) == (v, i) for canonical metadata
    vals = np.zeros((M, K // 2), W.CODE_NP[dt])
    idx = np.zeros((M, (K + 31) // 32), np.uint32)
    assert m.compress24_host(dt, M, K, np.ascontiguousarray(out[:, :K]), K, vals, K // 2, idx, idx.shape[1]) == 0
    assert np.array_equal(vals, ov) and np.array_equal(idx, oi)


def test_decompress24_host_every_code():
    # one row of 16 groups, one per 4-bit code: the six ascending pairs expand
    # to their positions; any code with p0 >= p1 is MCG_ERR_INVALID_INDEX
    good = [p0 | (p1 << 2) for p0 in range(4) for p1 in range(4) if p0 < p1]
    assert sorted(good) == [4, 8, 9, 12, 13, 14]
    vals = np.arange(1, 3, dtype=np.int8)
    for code in range(16):
        idx = np.array([[code]], np.uint32)
        out = np.full((1, 4), 99, np.int8)
        if code in good:
            m.decompress24_host("i8", 1, 4, vals.reshape(1, 2), 2, idx, 1, out, 4)
            expect = np.zeros(4, np.int8)
            expect[code & 3], expect[code >> 2] = 1, 2
            assert np.array_equal(out[0], expect), code
        else:
            with pytest.raises(m.MCGError) as e:
                m.decompress24_host("i8", 1, 4, vals.reshape(1, 2), 2, idx, 1, out, 4)
            assert e.value.status == 7
            assert np.all(out == 99), "nothing is written on an invalid code"


def test_decompress24_host_invalid_code_anywhere_writes_nothing():
    M, K = 5, 72                                             # 18 groups: the last word holds 2 used codes
    A = W.sparse24_dense("bf16", M, K)
    ov, oi, _ = oracle.compress24("bf16", A)
    bad = oi.copy()
    bad[4, 2] = (bad[4, 2] & ~np.uint32(0xF0)) | np.uint32(0x50)   # group 17 of row 4: code 5 (1, 1)
    out = np.zeros((M, K), np.uint16)
    with pytest.raises(m.MCGError) as e:
        m.decompress24_host("bf16", M, K, ov, K // 2, bad, bad.shape[1], out, K)
    assert e.value.status == 7 and not out.any()
    with pytest.raises(ValueError):
        oracle.decompress24("bf16", ov, bad, K)               # the oracle rejects it too
    # codes past K / 4 in the last word are ignored
    pad = oi.copy()
    pad[:, 2] |= np.uint32(0x55550000)
    m.decompress24_host("bf16", M, K, ov, K // 2, pad, pad.shape[1], out, K)
    assert np.array_equal(out, A)


def test_decompress24_host_argument_errors():
    v = np.zeros((4, 8), np.uint16)
    i = np.zeros((4, 1), np.uint32)
    a = np.zeros((4, 16), np.uint16)
    for args, status in [(("bf16", 4, 18, v, 8, i, 1, a, 16), 2),      # K % 4 != 0
                         (("bf16", 4, 16, v, 7, i, 1, a, 16), 3),
                         (("bf16", 4, 16, v, 8, i, 1, a, 15), 3),
                         (("f32", 4, 16, v, 8, i, 1, a, 16), 4),
                         (("bf16", 4, 16, None, 8, i, 1, a, 16), 1)]:
        with pytest.raises(m.MCGError) as e:
            m.decompress24_host(*args)
        assert e.value.status == status, args
    m.decompress24_host("bf16", 0, 16, None, 8, None, 1, None, 16)   # empty: no-op


@pytest.mark.parametrize("kw,status", [
    ({"dtypeA": "bf16", "dtypeB": "f16"}, 4),       # mixed 16-bit pair
    ({"dtypeA": "i8", "dtypeB": "e4m3"}, 4),
    ({"sparse": 2}, 4),
    ({"instr_per_wave": 0}, 2),
    ({"instr_per_wave": 24}, 2),                    # not a multiple of 16
    ({"instr_per_wave": (1 << 24) + 16}, 2),
    ({"num_wg": 0}, 2),
    ({"num_wg": 65537}, 2),
    ({"a": None}, 1),
    ({"sink": None}, 1),
    ({"clocks": None}, 1),
    ({"sparse": 1, "idx": None}, 1),
    ({"a": FAKE + 8}, 5),
    ({"sparse": 1, "idx": FAKE + 4}, 5),
    ({"clocks": FAKE + 4}, 5),
])
def test_mfma_probe_rejects_bad_arguments_on_the_host(kw, status):
    # every case fails validation before any HIP call (no GPU here)
    a = dict(dtypeA="bf16", dtypeB="bf16", sparse=0, a=FAKE, b=FAKE, idx=None, instr_per_wave=64, num_wg=1,
             sink=FAKE, clocks=FAKE)
    a.update(kw)
    with pytest.raises(m.MCGError) as e:
        m.mfma_probe(**a, stream=0)
    assert e.value.status == status
