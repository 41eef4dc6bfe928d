"""CPU oracle for the matrix-core GEMM library -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never reaches it, and it
never reaches the GPU library: the two share no code, header or constant.

The arithmetic lives in ``oracle.c`` (plain C11 + OpenMP); this module only
builds/loads it and marshals numpy arrays.  What each routine computes, and the
passages it follows, is stated in ``oracle.c``:

* ``gemm_float``   -- D = alpha*sA*sB*(A*B) + beta*C, binary64 accumulation in
  ascending k, rounded once to binary32 ("Accurate Models of AMD Matrix Cores",
  Section 2, Eq. (1)).
* ``gemm_i8``      -- exact int8 x int8 -> int32 (wraps mod 2^32).
* ``gemm_f64``     -- D = alpha*(A*B) + beta*C for binary64 operands: exact
  products summed in binary128 in ascending k, rounded once to binary64 (the
  FP64-accumulate instructions of "CDNA3 dense MFMA builtins").
* ``compress24`` / ``decompress24`` -- the 2:4 compressed form ("RDNA4 sparse
  WMMA builtins", Structured sparsity (2:4 pattern); Common parameters, index).
* ``gemm_sparse24`` -- decompress, then ``gemm_float``.
* ``float_bound`` / ``check_float`` / ``check_exact`` -- the acceptance test:
  |D_gpu - D_ref| <= 4*2^-24*(K+2)*|alpha*sA*sB|*S + 2^-24*|D_ref| (+ 2^-24*|beta*c|
  when beta is not 0 or +-1), S = sum_k |a_ik*b_kj|; integers must be equal.
* ``f64_bound`` / ``check_f64`` -- the same acceptance test for binary64
  results with u = 2^-53.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against closed forms, brute force, library witnesses
and the values the pages print.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "_liboracle.so")

DTYPES = {"bf16": 0, "f16": 1, "i8": 2, "e4m3": 3, "e5m2": 4}
LAYOUTS = {"k_contig": 0, "mn_contig": 1}
# output (and C) formats of the float GEMM; unit roundoff and half the smallest
# subnormal of each (the largest rounding error of a result in that format)
OUTS = {"f32": 0, "bf16": 1, "f16": 2}
OUT_UNIT = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}
OUT_SUBNORMAL_HALF = {"f32": 2.0 ** -150, "bf16": 2.0 ** -134, "f16": 2.0 ** -25}
CODE_NP = {"bf16": np.uint16, "f16": np.uint16, "i8": np.int8, "e4m3": np.uint8, "e5m2": np.uint8}

U = 2.0 ** -24  # unit roundoff of binary32
U64 = 2.0 ** -53  # unit roundoff of binary64

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with the host C compiler (no HIP involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.orc_decode.argtypes = [i32, i64, vp, vp]
        L.orc_gemm_float_elems.argtypes = [i32, i32, i32, i32, i64, i64, i64, vp, i64, vp, i64,
                                           vp, i64, i32, dbl, dbl, dbl, dbl, i64, vp, vp, vp, vp]
        L.orc_gemm_float_full.argtypes = [i32, i32, i32, i32, i64, i64, i64, vp, i64, vp, i64,
                                          vp, i64, i32, dbl, dbl, dbl, dbl, vp, vp]
        L.orc_round.argtypes = [i32, i64, vp, vp]
        L.orc_gemm_i8_elems.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64,
                                        i64, i64, i64, vp, vp, vp]
        L.orc_gemm_i8_full.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64,
                                       i64, i64, vp]
        L.orc_gemm_f64_elems.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64,
                                         dbl, dbl, i64, vp, vp, vp, vp]
        L.orc_gemm_f64_full.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64,
                                        dbl, dbl, vp, vp]
        L.orc_compress24.argtypes = [i32, i64, i64, vp, i64, vp, i64, vp, i64]
        L.orc_compress24.restype = i64
        L.orc_decompress24.argtypes = [i32, i64, i64, vp, i64, vp, i64, vp, i64]
        L.orc_max_threads.argtypes = []
        L.orc_set_threads.argtypes = [i32]
        L.orc_set_threads.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _flat(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)} array, got {a.dtype}")
    return a


def max_threads() -> int:
    return int(lib().orc_max_threads())


def set_threads(n: int) -> None:
    """Number of OpenMP threads the oracle's parallel loops use from now on."""
    lib().orc_set_threads(int(n))


def decode(dtype: str, codes) -> np.ndarray:
    """Exact binary64 values of an array of raw codes of ``dtype``."""
    c = _flat(codes, CODE_NP[dtype])
    out = np.empty(c.shape, dtype=np.float64)
    rc = lib().orc_decode(DTYPES[dtype], c.size, _ptr(c), _ptr(out))
    if rc != 0:
        raise ValueError(f"orc_decode failed ({rc})")
    return out


def round_to(out, x):
    """Round binary64 values once to the output format `out` (f32, bf16, f16):
    nearest, ties to even, gradual underflow, overflow to infinity."""
    x = _flat(np.asarray(x, np.float64), np.float64)
    y = np.empty_like(x)
    rc = lib().orc_round(OUTS[out], x.size, _ptr(x), _ptr(y))
    if rc != 0:
        raise ValueError(f"oracle round rejected its arguments ({rc})")
    return y


def gemm_float(dtA, dtB, layA, layB, M, N, K, A, lda, B, ldb, C=None, ldc=None,
               alpha=1.0, beta=0.0, sA=1.0, sB=1.0, rows=None, cols=None, out="f32"):
    """Reference for the float paths.

    A and B are flat (or any-shape, contiguous) arrays of raw codes addressed
    through (layout, leading dimension) as described in oracle.c.  C is an
    array in the output format `out` (float32, or bfloat16 / binary16 codes as
    uint16) addressed as C[i*ldc + j].  With rows/cols given, only those output
    elements are computed and 1-D arrays are returned; otherwise full M x N
    arrays.  Returns (d_ref float32 holding the value in the output format,
    abs_sum float64).
    """
    A = _flat(A, CODE_NP[dtA])
    B = _flat(B, CODE_NP[dtB])
    if beta != 0.0:
        C = _flat(C, np.float32 if out == "f32" else np.uint16)
    else:
        C = None
    ldc = N if ldc is None else ldc
    L = lib()
    if rows is None:
        d = np.empty((M, N), np.float32)
        s = np.empty((M, N), np.float64)
        rc = L.orc_gemm_float_full(DTYPES[dtA], DTYPES[dtB], LAYOUTS[layA], LAYOUTS[layB],
                                   M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, OUTS[out],
                                   float(alpha), float(beta), float(sA), float(sB),
                                   _ptr(d), _ptr(s))
    else:
        rows = _flat(np.asarray(rows, np.int64), np.int64)
        cols = _flat(np.asarray(cols, np.int64), np.int64)
        assert rows.shape == cols.shape
        d = np.empty(rows.shape, np.float32)
        s = np.empty(rows.shape, np.float64)
        rc = L.orc_gemm_float_elems(DTYPES[dtA], DTYPES[dtB], LAYOUTS[layA], LAYOUTS[layB],
                                    M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, OUTS[out],
                                    float(alpha), float(beta), float(sA), float(sB),
                                    rows.size, _ptr(rows), _ptr(cols), _ptr(d), _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle float GEMM rejected its arguments ({rc})")
    return d, s


def gemm_i8(layA, layB, M, N, K, A, lda, B, ldb, C=None, ldc=None, alpha=1, beta=0,
            rows=None, cols=None):
    """Reference for int8 x int8 -> int32 (exact, wraps mod 2^32)."""
    A = _flat(A, np.int8)
    B = _flat(B, np.int8)
    C = _flat(C, np.int32) if beta != 0 else None
    ldc = N if ldc is None else ldc
    L = lib()
    if rows is None:
        d = np.empty((M, N), np.int32)
        rc = L.orc_gemm_i8_full(LAYOUTS[layA], LAYOUTS[layB], M, N, K, _ptr(A), lda,
                                _ptr(B), ldb, _ptr(C), ldc, int(alpha), int(beta), _ptr(d))
    else:
        rows = _flat(np.asarray(rows, np.int64), np.int64)
        cols = _flat(np.asarray(cols, np.int64), np.int64)
        d = np.empty(rows.shape, np.int32)
        rc = L.orc_gemm_i8_elems(LAYOUTS[layA], LAYOUTS[layB], M, N, K, _ptr(A), lda,
                                 _ptr(B), ldb, _ptr(C), ldc, int(alpha), int(beta),
                                 rows.size, _ptr(rows), _ptr(cols), _ptr(d))
    if rc != 0:
        raise ValueError(f"oracle int8 GEMM rejected its arguments ({rc})")
    return d


def gemm_f64(layA, layB, M, N, K, A, lda, B, ldb, C=None, ldc=None, alpha=1.0, beta=0.0,
             rows=None, cols=None):
    """Reference for binary64 operands: returns (d_ref float64, abs_sum
    float64), full M x N arrays or, with rows/cols, 1-D arrays."""
    A = _flat(A, np.float64)
    B = _flat(B, np.float64)
    C = _flat(C, np.float64) if beta != 0.0 and C is not None else None
    ldc = N if ldc is None else ldc
    L = lib()
    if rows is None:
        d = np.empty((M, N), np.float64)
        s = np.empty((M, N), np.float64)
        rc = L.orc_gemm_f64_full(LAYOUTS[layA], LAYOUTS[layB], M, N, K, _ptr(A), lda, _ptr(B), ldb,
                                 _ptr(C), ldc, float(alpha), float(beta), _ptr(d), _ptr(s))
    else:
        rows = _flat(np.asarray(rows, np.int64), np.int64)
        cols = _flat(np.asarray(cols, np.int64), np.int64)
        assert rows.shape == cols.shape
        d = np.empty(rows.shape, np.float64)
        s = np.empty(rows.shape, np.float64)
        rc = L.orc_gemm_f64_elems(LAYOUTS[layA], LAYOUTS[layB], M, N, K, _ptr(A), lda, _ptr(B), ldb,
                                  _ptr(C), ldc, float(alpha), float(beta), rows.size, _ptr(rows),
                                  _ptr(cols), _ptr(d), _ptr(s))
    if rc != 0:
        raise ValueError(f"oracle binary64 GEMM rejected its arguments ({rc})")
    return d, s


def compress24(dtype, A):
    """2:4-compress a row-major M x K code array.  Returns (vals M x K/2,
    idx M x ceil(K/32) uint32, number of groups with more than two non-zeros)."""
    A = _flat(A, CODE_NP[dtype])
    M, K = A.shape
    vals = np.zeros((M, K // 2), CODE_NP[dtype])
    idx = np.zeros((M, (K + 31) // 32), np.uint32)
    n = lib().orc_compress24(DTYPES[dtype], M, K, _ptr(A), K, _ptr(vals), K // 2,
                             _ptr(idx), idx.shape[1])
    if n < 0:
        raise ValueError(f"oracle compress24 rejected its arguments ({n})")
    return vals, idx, int(n)


def decompress24(dtype, vals, idx, K):
    """Inverse of ``compress24``: a dense row-major M x K code array."""
    vals = _flat(vals, CODE_NP[dtype])
    idx = _flat(idx, np.uint32)
    M = vals.shape[0]
    A = np.zeros((M, K), CODE_NP[dtype])
    rc = lib().orc_decompress24(DTYPES[dtype], M, K, _ptr(vals), vals.shape[1],
                                _ptr(idx), idx.shape[1], _ptr(A), K)
    if rc == -2:
        raise ValueError("index code does not name two ascending positions")
    if rc != 0:
        raise ValueError(f"oracle decompress24 rejected its arguments ({rc})")
    return A


def gemm_sparse24(dtA, dtB, layB, M, N, K, vals, idx, B, ldb, C=None, ldc=None,
                  alpha=1.0, beta=0.0, rows=None, cols=None, out="f32"):
    """Sparse-A reference: decompress A, then the dense GEMM with the dense K
    (A row-major, i.e. K-contiguous).  Float inputs return (d_ref, abs_sum) as
    ``gemm_float``; int8 returns (d_ref int32, None), exact as ``gemm_i8``.
    fp8 dequantisation scales, if any, are part of alpha."""
    A = decompress24(dtA, vals, idx, K)
    if dtA == "i8":
        return gemm_i8("k_contig", layB, M, N, K, A, K, B, ldb, C, ldc, int(alpha), int(beta),
                       rows, cols), None
    return gemm_float(dtA, dtB, "k_contig", layB, M, N, K, A, K, B, ldb, C, ldc,
                      alpha, beta, 1.0, 1.0, rows, cols, out)


def float_bound(d_ref, abs_sum, K, alpha=1.0, sA=1.0, sB=1.0, beta=0.0, c=None, out="f32"):
    """Per-element acceptance bound for float results (binary64).

    For a binary32 result: 4u(K+2)|alpha sA sB| S + u|D_ref| (u = 2^-24), plus
    u|beta c| when beta is not 0 or +-1.  A result delivered in bfloat16 or
    binary16 is the binary32 value rounded once more, while the reference is
    the exact value rounded once, so both roundings to the output format are
    added: e + u_out (2 |D_ref| + e) + 2 * (half the smallest subnormal)."""
    d = np.abs(np.asarray(d_ref, np.float64))
    bound = (4.0 * U * (K + 2) * abs(alpha * sA * sB)) * np.asarray(abs_sum, np.float64) + U * d
    if beta not in (0.0, 1.0, -1.0) and c is not None:
        bound = bound + U * np.abs(beta * np.asarray(c, np.float64))
    if out != "f32":
        bound = bound + OUT_UNIT[out] * (2.0 * d + bound) + 2.0 * OUT_SUBNORMAL_HALF[out]
    return bound


def f64_bound(d_ref, abs_sum, K, alpha=1.0, beta=0.0, c=None):
    """Per-element acceptance bound for binary64 results: the binary32 bound's
    form with u = 2^-53, i.e. 4u(K+2)|alpha| S + u|D_ref| (+ u|beta c| when
    beta is not 0 or +-1)."""
    d = np.abs(np.asarray(d_ref, np.float64))
    bound = (4.0 * U64 * (K + 2) * abs(alpha)) * np.asarray(abs_sum, np.float64) + U64 * d
    if beta not in (0.0, 1.0, -1.0) and c is not None:
        bound = bound + U64 * np.abs(beta * np.asarray(c, np.float64))
    return bound


def check_f64(d_gpu, d_ref, abs_sum, K, alpha=1.0, beta=0.0, c=None):
    """``check_float`` for binary64 results (``f64_bound``)."""
    return _compare(d_gpu, d_ref, f64_bound(d_ref, abs_sum, K, alpha, beta, c))


def check_float(d_gpu, d_ref, abs_sum, K, alpha=1.0, sA=1.0, sB=1.0, beta=0.0, c=None, out="f32"):
    """Compare GPU float results with the oracle.  Returns a dict with ``ok``,
    the number of violations (NaN counts as one), max |delta|/bound and the
    first offending flat indices."""
    return _compare(d_gpu, d_ref, float_bound(d_ref, abs_sum, K, alpha, sA, sB, beta, c, out))


def _compare(d_gpu, d_ref, bound):
    g = np.asarray(d_gpu, np.float64).ravel()
    r = np.asarray(d_ref, np.float64).ravel()
    b = np.asarray(bound, np.float64).ravel()
    delta = np.abs(g - r)
    bad = ~(delta <= b)  # NaN compares false, so it is flagged
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(b > 0, delta / np.where(b > 0, b, 1.0), np.where(delta > 0, np.inf, 0.0))
    finite = ratio[np.isfinite(ratio)]
    return {
        "ok": not bool(bad.any()),
        "violations": int(bad.sum()),
        "max_ratio": float(finite.max()) if finite.size else (float("inf") if bad.any() else 0.0),
        "first_bad": np.flatnonzero(bad)[:8].tolist(),
        "n": int(g.size),
    }


def check_exact(d_gpu, d_ref):
    """Bit-exact comparison (integers, indices, raw codes)."""
    g = np.asarray(d_gpu).ravel()
    r = np.asarray(d_ref).ravel()
    bad = g != r
    return {"ok": not bool(bad.any()), "violations": int(bad.sum()),
            "first_bad": np.flatnonzero(bad)[:8].tolist(), "n": int(g.size)}
