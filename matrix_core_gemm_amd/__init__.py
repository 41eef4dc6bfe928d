"""Python binding of the gfx950 matrix-core GEMM library (include/mcg.h).

Argument marshalling only: every function has the C entry point's name and
argument order, turns torch tensors into device pointers, defaults the stream
to torch's current stream, and raises ``MCGError`` on a non-zero status.  All
arithmetic runs in the HIP kernels of ``_libmcg.so``; there is no fallback.
If the library has not been built, importing this package fails.

dtype and layout arguments take the C enum values or their names:
  dtypes : "bf16", "f16", "i8", "e4m3", "e5m2", "f32", "i32", "f64"
  layouts: "k_contig" (A row-major / B column-major),
           "mn_contig" (A column-major / B row-major)
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so the library binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_libmcg.so")

DTYPES = {"bf16": 0, "f16": 1, "i8": 2, "e4m3": 3, "e5m2": 4, "f32": 5, "i32": 6, "f64": 7}
LAYOUTS = {"k_contig": 0, "mn_contig": 1}
STATUS = {0: "MCG_SUCCESS", 1: "MCG_ERR_NULL_POINTER", 2: "MCG_ERR_INVALID_SIZE",
          3: "MCG_ERR_INVALID_LD", 4: "MCG_ERR_UNSUPPORTED_DTYPE", 5: "MCG_ERR_MISALIGNED",
          6: "MCG_ERR_NOT_2_4_SPARSE", 7: "MCG_ERR_INVALID_INDEX", 8: "MCG_ERR_UNSUPPORTED_ARCH",
          9: "MCG_ERR_HIP", 10: "MCG_ERR_INVALID_VALUE", 11: "MCG_ERR_SCRATCH_LIMIT"}

# Every symbol include/mcg.h declares.
EXPORTS = ("gemm_dense", "gemm_dense_ws", "gemm_dense_noalloc", "mcg_dense_noalloc_scratch_bytes",
           "mcg_dense_workspace_bytes", "gemm_sparse24_ws", "mcg_sparse24_workspace_bytes", "gemm_sparse24", "compress24", "compress24_host", "decompress24_host",
           "mcg_status_string",
           "mcg_version", "mcg_validate_dense", "mcg_validate_sparse24", "mcg_validate_compress24",
           "mcg_dense_path", "mcg_dense_splits", "mcg_sparse24_path", "mcg_mfma_eval", "mcg_mfma_eval_k",
           "mcg_mfma_probe")


class MCGError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.mcg_status_string(status).decode() if _lib is not None else ""
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with matrix_core_gemm_amd.build.build() "
                      "(or __graft_entry__.build()); there is no non-GPU fallback")

_lib = ctypes.CDLL(LIB_PATH)
_i32, _i64, _dbl, _f32, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_float, ctypes.c_void_p
_lib.gemm_dense.argtypes = [_i32, _i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                            _vp, _vp, _i64, _i32, _dbl, _dbl, _f32, _f32, _vp]
_lib.gemm_dense_ws.argtypes = [_i32, _i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                               _vp, _vp, _i64, _i32, _dbl, _dbl, _f32, _f32, _vp, _i64, _vp]
_lib.gemm_dense_noalloc.argtypes = _lib.gemm_dense.argtypes
_lib.mcg_dense_noalloc_scratch_bytes.argtypes = []
_lib.mcg_dense_noalloc_scratch_bytes.restype = _i64
_lib.mcg_dense_workspace_bytes.argtypes = [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64]
_lib.mcg_dense_workspace_bytes.restype = _i64
_lib.gemm_sparse24.argtypes = [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                               _vp, _vp, _i64, _i32, _dbl, _dbl, _vp]
_lib.gemm_sparse24_ws.argtypes = [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                  _vp, _vp, _i64, _i32, _dbl, _dbl, _vp, _i64, _vp]
_lib.mcg_sparse24_workspace_bytes.argtypes = [_i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
_lib.mcg_sparse24_workspace_bytes.restype = _i64
_lib.compress24.argtypes = [_i32, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp]
_lib.compress24_host.argtypes = [_i32, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
_lib.decompress24_host.argtypes = [_i32, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
_lib.mcg_status_string.argtypes = [_i32]
_lib.mcg_status_string.restype = ctypes.c_char_p
_lib.mcg_version.argtypes = []
_lib.mcg_validate_dense.argtypes = [_i32, _i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                                    _vp, _vp, _i64, _i32, _dbl, _dbl, _f32, _f32]
_lib.mcg_validate_sparse24.argtypes = [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                                       _vp, _i64, _vp, _vp, _i64, _i32, _dbl, _dbl]
_lib.mcg_validate_compress24.argtypes = [_i32, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
_lib.mcg_dense_path.argtypes = [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64]
_lib.mcg_dense_splits.argtypes = [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp,
                                  _i32, ctypes.c_double]
_lib.mcg_sparse24_path.argtypes = [_i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
_lib.mcg_mfma_eval.argtypes = [_i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp]
_lib.mcg_mfma_eval_k.argtypes = [_i32, _i32]
_lib.mcg_mfma_probe.argtypes = [_i32, _i32, _i32, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp]


def lib():
    """The loaded ctypes library."""
    return _lib


def _dt(x) -> int:
    return DTYPES[x] if isinstance(x, str) else int(x)


def _lay(x) -> int:
    return LAYOUTS[x] if isinstance(x, str) else int(x)


def _ptr(t):
    """Device (or host) address of a tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.data_ptr()
    if hasattr(t, "ctypes"):  # numpy array (host entry points only)
        return t.ctypes.data
    return int(t)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MCGError(fn, status)


def gemm_dense(dtypeA, dtypeB, layoutA, layoutB, M, N, K, A, lda, B, ldb, C, D, ldc, dtypeD,
               alpha=1.0, beta=0.0, scaleA=1.0, scaleB=1.0, stream=None) -> None:
    _check("gemm_dense", _lib.gemm_dense(
        _dt(dtypeA), _dt(dtypeB), _lay(layoutA), _lay(layoutB), M, N, K, _ptr(A), lda, _ptr(B), ldb,
        _ptr(C), _ptr(D), ldc, _dt(dtypeD), float(alpha), float(beta), float(scaleA), float(scaleB),
        _stream(stream)))


def gemm_dense_ws(dtypeA, dtypeB, layoutA, layoutB, M, N, K, A, lda, B, ldb, C, D, ldc, dtypeD,
                  alpha=1.0, beta=0.0, scaleA=1.0, scaleB=1.0, workspace=None, workspace_bytes=0,
                  stream=None) -> None:
    """gemm_dense with a device workspace (a tensor, whose byte size is taken
    when workspace_bytes is 0, or an address), which the stream-K form of the
    256 x 256 kernel uses for partial sums."""
    if isinstance(workspace, torch.Tensor) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("gemm_dense_ws", _lib.gemm_dense_ws(
        _dt(dtypeA), _dt(dtypeB), _lay(layoutA), _lay(layoutB), M, N, K, _ptr(A), lda, _ptr(B), ldb,
        _ptr(C), _ptr(D), ldc, _dt(dtypeD), float(alpha), float(beta), float(scaleA), float(scaleB),
        _ptr(workspace), int(workspace_bytes), _stream(stream)))


def gemm_dense_noalloc(dtypeA, dtypeB, layoutA, layoutB, M, N, K, A, lda, B, ldb, C, D, ldc, dtypeD,
                       alpha=1.0, beta=0.0, scaleA=1.0, scaleB=1.0, stream=None) -> None:
    """gemm_dense taking stream-K scratch from the library's static device array
    (no allocation); raises MCGError with MCG_ERR_SCRATCH_LIMIT (11) when the
    plan needs more than mcg_dense_noalloc_scratch_bytes()."""
    _check("gemm_dense_noalloc", _lib.gemm_dense_noalloc(
        _dt(dtypeA), _dt(dtypeB), _lay(layoutA), _lay(layoutB), M, N, K, _ptr(A), lda, _ptr(B), ldb,
        _ptr(C), _ptr(D), ldc, _dt(dtypeD), float(alpha), float(beta), float(scaleA), float(scaleB),
        _stream(stream)))


def dense_workspace_bytes(dtypeA, layoutA, layoutB, M, N, K, A, lda, B, ldb) -> int:
    """Workspace bytes gemm_dense_ws uses for these operands (0: no stream-K form)."""
    return _lib.mcg_dense_workspace_bytes(_dt(dtypeA), _lay(layoutA), _lay(layoutB), M, N, K, _ptr(A), lda,
                                          _ptr(B), ldb)


def gemm_sparse24(dtypeA, dtypeB, layoutB, M, N, K, A_compressed, lda_c, A_index, ld_idx, B, ldb,
                  C, D, ldc, dtypeD, alpha=1.0, beta=0.0, stream=None) -> None:
    _check("gemm_sparse24", _lib.gemm_sparse24(
        _dt(dtypeA), _dt(dtypeB), _lay(layoutB), M, N, K, _ptr(A_compressed), lda_c, _ptr(A_index),
        ld_idx, _ptr(B), ldb, _ptr(C), _ptr(D), ldc, _dt(dtypeD), float(alpha), float(beta),
        _stream(stream)))


def gemm_sparse24_ws(dtypeA, dtypeB, layoutB, M, N, K, A_compressed, lda_c, A_index, ld_idx, B, ldb,
                     C, D, ldc, dtypeD, alpha=1.0, beta=0.0, workspace=None, workspace_bytes=0,
                     stream=None) -> None:
    """gemm_sparse24 with a device workspace for the stream-K form (a tensor,
    whose byte size is taken when workspace_bytes is 0, or an address)."""
    if isinstance(workspace, torch.Tensor) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("gemm_sparse24_ws", _lib.gemm_sparse24_ws(
        _dt(dtypeA), _dt(dtypeB), _lay(layoutB), M, N, K, _ptr(A_compressed), lda_c, _ptr(A_index),
        ld_idx, _ptr(B), ldb, _ptr(C), _ptr(D), ldc, _dt(dtypeD), float(alpha), float(beta),
        _ptr(workspace), int(workspace_bytes), _stream(stream)))


def sparse24_workspace_bytes(dtypeA, layoutB, M, N, K, A_compressed, lda_c, A_index, ld_idx, B, ldb) -> int:
    """Workspace bytes gemm_sparse24_ws uses for these operands (0: no stream-K form)."""
    return _lib.mcg_sparse24_workspace_bytes(_dt(dtypeA), _lay(layoutB), M, N, K, _ptr(A_compressed), lda_c,
                                             _ptr(A_index), ld_idx, _ptr(B), ldb)


def compress24(dtype, M, K, A, lda, A_compressed, lda_c, A_index, ld_idx, d_violations=None,
               stream=None) -> None:
    _check("compress24", _lib.compress24(
        _dt(dtype), M, K, _ptr(A), lda, _ptr(A_compressed), lda_c, _ptr(A_index), ld_idx,
        _ptr(d_violations), _stream(stream)))


def compress24_host(dtype, M, K, A, lda, A_compressed, lda_c, A_index, ld_idx) -> int:
    """Host compressor; returns the status (0, or MCG_ERR_NOT_2_4_SPARSE = 6)
    and raises on any other error."""
    st = _lib.compress24_host(_dt(dtype), M, K, _ptr(A), lda, _ptr(A_compressed), lda_c,
                              _ptr(A_index), ld_idx)
    if st not in (0, 6):
        raise MCGError("compress24_host", st)
    return st


def decompress24_host(dtype, M, K, A_compressed, lda_c, A_index, ld_idx, A, lda) -> None:
    """Host decompressor (inverse of compress24_host); raises MCGError, e.g.
    MCG_ERR_INVALID_INDEX (7) for a code with p0 >= p1, in which case A is
    left untouched."""
    _check("decompress24_host", _lib.decompress24_host(_dt(dtype), M, K, _ptr(A_compressed), lda_c,
                                                       _ptr(A_index), ld_idx, _ptr(A), lda))


def validate_dense(dtypeA, dtypeB, layoutA, layoutB, M, N, K, A, lda, B, ldb, C, D, ldc, dtypeD,
                   alpha=1.0, beta=0.0, scaleA=1.0, scaleB=1.0) -> int:
    return _lib.mcg_validate_dense(_dt(dtypeA), _dt(dtypeB), _lay(layoutA), _lay(layoutB), M, N, K,
                                   _ptr(A), lda, _ptr(B), ldb, _ptr(C), _ptr(D), ldc, _dt(dtypeD),
                                   float(alpha), float(beta), float(scaleA), float(scaleB))


def validate_sparse24(dtypeA, dtypeB, layoutB, M, N, K, A_compressed, lda_c, A_index, ld_idx, B,
                      ldb, C, D, ldc, dtypeD, alpha=1.0, beta=0.0) -> int:
    return _lib.mcg_validate_sparse24(_dt(dtypeA), _dt(dtypeB), _lay(layoutB), M, N, K,
                                      _ptr(A_compressed), lda_c, _ptr(A_index), ld_idx, _ptr(B),
                                      ldb, _ptr(C), _ptr(D), ldc, _dt(dtypeD), float(alpha),
                                      float(beta))


def validate_compress24(dtype, M, K, A, lda, A_compressed, lda_c, A_index, ld_idx) -> int:
    return _lib.mcg_validate_compress24(_dt(dtype), M, K, _ptr(A), lda, _ptr(A_compressed), lda_c,
                                        _ptr(A_index), ld_idx)


def dense_path(dtypeA, layoutA, layoutB, M, N, K, A, lda, B, ldb) -> int:
    """Kernel gemm_dense runs for these operands (binary32/int32 D, not C):
    0 general 128 x 128, 1 the 256 x 256 kernel, 2 general 128 x 32 (N <= 32),
    3 general 32 x 128 (M <= 32), 4 streaming kernel, 5 binary64 kernel,
    6 the pipelined kernel with 128 x 128 tiles (mid-size aligned problems)."""
    return _lib.mcg_dense_path(_dt(dtypeA), _lay(layoutA), _lay(layoutB), M, N, K, _ptr(A), lda,
                               _ptr(B), ldb)


def dense_splits(dtypeA, layoutA, layoutB, M, N, K, A, lda, B, ldb, C, D, dtypeD, beta) -> int:
    """Number of K ranges gemm_dense uses with these arguments (1 = no split)."""
    return _lib.mcg_dense_splits(_dt(dtypeA), _lay(layoutA), _lay(layoutB), M, N, K, _ptr(A), lda,
                                 _ptr(B), ldb, _ptr(C), _ptr(D), _dt(dtypeD), float(beta))


def sparse24_path(dtypeA, layoutB, M, N, K, A_compressed, lda_c, A_index, ld_idx, B, ldb) -> int:
    """1 if gemm_sparse24 with these arguments runs the 256 x 256 kernel, else 0."""
    return _lib.mcg_sparse24_path(_dt(dtypeA), _lay(layoutB), M, N, K, _ptr(A_compressed), lda_c,
                                  _ptr(A_index), ld_idx, _ptr(B), ldb)


def status_string(status: int) -> str:
    return _lib.mcg_status_string(status).decode()


def version() -> int:
    return _lib.mcg_version()


def mfma_eval_k(dtype, shape) -> int:
    """Elements per test vector of mfma_eval (0 if unsupported)."""
    return _lib.mcg_mfma_eval_k(_dt(dtype), int(shape))


def mfma_eval(dtype, shape, n, a, b, c, d, stream=None) -> None:
    """One matrix-core instruction per test vector: d[t] = element (0, 0) of the
    instruction fed with a[t*k:], b[t*k:] and c[t] (see mcg.h)."""
    _check("mcg_mfma_eval", _lib.mcg_mfma_eval(_dt(dtype), int(shape), n, _ptr(a), _ptr(b), _ptr(c), _ptr(d),
                                               _stream(stream)))


def mfma_probe(dtypeA, dtypeB, sparse, a, b, idx, instr_per_wave, num_wg, sink, clocks, stream=None) -> None:
    """Matrix-core rate probe on the operand bits of a, b (and idx for 2:4): the
    GEMM kernels' instructions on fragments loaded once, no other traffic (see
    mcg.h).  sink: float32 tensor of num_wg * 512; clocks: int64 tensor of
    2 * num_wg (shader cycles, 100 MHz ticks per workgroup)."""
    _check("mcg_mfma_probe", _lib.mcg_mfma_probe(_dt(dtypeA), _dt(dtypeB), int(sparse), _ptr(a), _ptr(b),
                                                 _ptr(idx), int(instr_per_wave), int(num_wg), _ptr(sink),
                                                 _ptr(clocks), _stream(stream)))
