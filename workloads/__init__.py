"""Seeded synthetic inputs for the matrix-core GEMM library.

This module is shared by the tests, the benchmark and the smoke check, on both
sides of every comparison (GPU library and CPU oracle).  It holds none of the
GEMM arithmetic: it only draws random operands, rounds them to the input
formats with torch's own conversions (round to nearest even), lays them out in
memory, and picks which output coordinates a check samples.

All randomness comes from torch CPU generators (Mersenne Twister) seeded per
operand: A = 0, B = 1, C = 2, sparsity mask = 3, sampled coordinates = 4, plus
a per-call offset so that several calls in one test draw different data.

Operand storage:
  A is logically M x K.  layout "k_contig" stores it row-major (M rows of K,
  leading dimension lda >= K); "mn_contig" stores it column-major (K rows of
  M, lda >= M).
  B is logically K x N.  "k_contig" stores it column-major (N rows of K,
  ldb >= K); "mn_contig" stores it row-major (K rows of N, ldb >= N).
  C and D are row-major M x N.
Arrays returned here are numpy arrays of raw codes (uint16 for bf16/f16,
uint8 for fp8, int8 for int8) shaped (rows, ld) of the storage order.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

SEED_A, SEED_B, SEED_C, SEED_MASK, SEED_COORDS = 0, 1, 2, 3, 4

TORCH_DTYPE = {
    "bf16": torch.bfloat16,
    "f16": torch.float16,
    "e4m3": torch.float8_e4m3fn,
    "e5m2": torch.float8_e5m2,
    "i8": torch.int8,
    "f64": torch.float64,
}
CODE_VIEW = {"bf16": torch.int16, "f16": torch.int16, "e4m3": torch.uint8,
             "e5m2": torch.uint8, "i8": torch.int8, "f64": torch.float64}
CODE_NP = {"bf16": np.uint16, "f16": np.uint16, "e4m3": np.uint8, "e5m2": np.uint8,
           "i8": np.int8, "f64": np.float64}
ELEM_BYTES = {"bf16": 2, "f16": 2, "e4m3": 1, "e5m2": 1, "i8": 1, "f64": 8}
# largest finite value of each fp8 format (OCP encodings)
FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


def gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def codes_of(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Raw codes of a CPU tensor of the input dtype, as a numpy array."""
    return t.contiguous().view(CODE_VIEW[dtype]).numpy().view(CODE_NP[dtype]).copy()


def to_tensor(codes: np.ndarray, dtype: str) -> torch.Tensor:
    """CPU torch tensor of the input dtype holding these raw codes."""
    view = CODE_VIEW[dtype]
    np_view = {torch.int16: np.int16, torch.uint8: np.uint8, torch.int8: np.int8,
               torch.float64: np.float64}[view]
    return torch.from_numpy(np.ascontiguousarray(codes).view(np_view)).view(TORCH_DTYPE[dtype])


def draw(dist: str, shape, seed: int, fdtype=torch.float32) -> torch.Tensor:
    """Logical values (fdtype, float32 unless asked otherwise, or int64 for
    integer distributions)."""
    g = gen(seed)
    if dist == "uniform":          # 2u - 1, u ~ U[0, 1): values in [-1, 1)
        return torch.rand(shape, generator=g, dtype=fdtype) * 2.0 - 1.0
    if dist == "normal":
        return torch.randn(shape, generator=g, dtype=fdtype)
    if dist == "lognormal":        # sign * exp(2 z): magnitudes over about 2^-17 .. 2^17
        z = torch.randn(shape, generator=g, dtype=fdtype)
        sgn = torch.randint(0, 2, shape, generator=g).to(fdtype) * 2.0 - 1.0
        return sgn * torch.exp(2.0 * z)
    if dist == "int8":             # uniform integers in [-128, 127]
        return torch.randint(-128, 128, shape, generator=g, dtype=torch.int64)
    if dist.startswith("smallint"):  # uniform integers in [-r, r], e.g. "smallint8"
        r = int(dist[len("smallint"):])
        return torch.randint(-r, r + 1, shape, generator=g, dtype=torch.int64)
    raise ValueError(dist)


def quantize(values: torch.Tensor, dtype: str, fp8_scaled: bool = False):
    """Round logical values to the input format.  For fp8 with fp8_scaled the
    tensor is first multiplied by q = 0.9*max/max|x| (one fp32 scale per
    tensor) and the returned dequantisation scale is 1/q.
    Returns (tensor of dtype, dequant scale as a python float)."""
    if dtype == "i8":
        return values.to(torch.int8), 1.0
    if dtype == "f64":
        return values.to(torch.float64), 1.0
    scale = 1.0
    v = values.to(torch.float32)
    if dtype in FP8_MAX and fp8_scaled:
        amax = float(v.abs().max())
        q = np.float32(0.9 * FP8_MAX[dtype] / amax) if amax > 0 else np.float32(1.0)
        v = v * torch.tensor(q, dtype=torch.float32)
        scale = float(np.float32(1.0) / q)
    return v.to(TORCH_DTYPE[dtype]), scale


def store(logical: torch.Tensor, role: str, layout: str, ld: int | None = None) -> tuple[torch.Tensor, int]:
    """Lay a logical operand out in memory.  role "A": logical (M, K);
    role "B": logical (K, N).  Returns (storage tensor (rows, ld), ld)."""
    if role == "A":
        s = logical if layout == "k_contig" else logical.t()
    else:
        s = logical.t() if layout == "k_contig" else logical
    s = s.contiguous()
    rows, cols = s.shape
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("leading dimension below the row length")
    if ld != cols:
        pad = torch.zeros((rows, ld), dtype=s.dtype)
        pad[:, :cols] = s
        s = pad
    return s, ld


@dataclass
class Operand:
    dtype: str
    layout: str
    codes: np.ndarray      # storage (rows, ld) of raw codes
    ld: int
    scale: float = 1.0     # dequantisation scale (fp8), else 1.0


def operand(role, dtype, rows, cols, dist, layout="k_contig", seed=None, ld=None,
            fp8_scaled=False) -> Operand:
    """A (rows=M, cols=K) or B (rows=K, cols=N) operand."""
    seed = (SEED_A if role == "A" else SEED_B) if seed is None else seed
    fdtype = torch.float64 if dtype == "f64" else torch.float32  # binary64 draws use all 53 bits
    vals, scale = quantize(draw(dist, (rows, cols), seed, fdtype), dtype, fp8_scaled)
    s, ld = store(vals, role, layout, ld)
    return Operand(dtype, layout, codes_of(s, dtype), ld, scale)


def c_matrix(M, N, dist, seed=SEED_C, ldc=None, dtype="f32") -> np.ndarray:
    """C, row-major (M, ldc): float32 (normal/uniform), float64 (dtype "f64") or
    int32 (dist "int20": uniform integers in [-2^20, 2^20])."""
    g = gen(seed)
    if dist == "int20":
        c = torch.randint(-(1 << 20), (1 << 20) + 1, (M, N), generator=g, dtype=torch.int64)
        c = c.to(torch.int32)
    elif dtype == "f64":
        c = draw(dist, (M, N), seed, torch.float64)
    else:
        c = draw(dist, (M, N), seed).to(torch.float32)
    ldc = N if ldc is None else ldc
    if ldc != N:
        pad = torch.zeros((M, ldc), dtype=c.dtype)
        pad[:, :N] = c
        c = pad
    return c.numpy().copy()


PAIRS = ((0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3))


def sparse24_dense(dtype, M, K, dist="normal", seed=SEED_A, mask_seed=SEED_MASK) -> np.ndarray:
    """Row-major M x K codes with exactly two non-zeros in every group of four
    along K; the pair of positions is drawn uniformly from the six possible
    pairs, independently per (row, group)."""
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    vals, _ = quantize(draw(dist, (M, K), seed), dtype)
    vals = vals.to(torch.float32) if dtype != "i8" else vals.to(torch.int64)
    vals = torch.where(vals == 0, torch.ones_like(vals), vals)  # keep kept entries non-zero
    choice = torch.randint(0, 6, (M, K // 4), generator=gen(mask_seed))
    pairs = torch.tensor(PAIRS, dtype=torch.int64)[choice]          # (M, K/4, 2)
    keep = torch.zeros((M, K // 4, 4), dtype=torch.bool)
    keep.scatter_(2, pairs, True)
    vals = torch.where(keep.reshape(M, K), vals, torch.zeros_like(vals))
    q, _ = quantize(vals, dtype)
    return codes_of(q, dtype)


def sample_coords(M, N, n_random=4096, full_rows=(), full_cols=(), seed=SEED_COORDS):
    """Output coordinates for a sampled check: n_random uniform (i, j) pairs,
    every element of the listed rows and columns, and the four corners."""
    g = gen(seed)
    ri = torch.randint(0, M, (n_random,), generator=g).numpy()
    rj = torch.randint(0, N, (n_random,), generator=g).numpy()
    rows = [ri]
    cols = [rj]
    for r in full_rows:
        rows.append(np.full(N, r))
        cols.append(np.arange(N))
    for c in full_cols:
        rows.append(np.arange(M))
        cols.append(np.full(M, c))
    rows.append(np.array([0, 0, M - 1, M - 1]))
    cols.append(np.array([0, N - 1, 0, N - 1]))
    return np.concatenate(rows).astype(np.int64), np.concatenate(cols).astype(np.int64)


@dataclass
class Workload:
    """One benchmark/parity configuration."""
    name: str
    dtA: str
    dtB: str
    layA: str
    layB: str
    M: int
    N: int
    K: int
    dist: str
    c_dist: str | None
    alpha: float
    beta: float
    fp8_scaled: bool = False
    sparse: bool = False
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


def standard_workloads():
    """The five input recipes this library is validated and measured on."""
    w = [Workload("dense bf16 256^3, A row-major, B column-major, C=0", "bf16", "bf16",
                  "k_contig", "k_contig", 256, 256, 256, "uniform", None, 1.0, 0.0),
         Workload("dense int8 4096^3, i32 out, C int in [-2^20,2^20], alpha=beta=1", "i8", "i8",
                  "k_contig", "k_contig", 4096, 4096, 4096, "int8", "int20", 1, 1)]
    for dt in ("bf16", "f16"):
        for la in ("k_contig", "mn_contig"):
            for lb in ("k_contig", "mn_contig"):
                w.append(Workload(f"dense {dt} 8192^3 A {la} B {lb}, C ~ N(0,1), alpha=beta=1",
                                  dt, dt, la, lb, 8192, 8192, 8192, "normal", "normal", 1.0, 1.0))
    for dtb in ("e4m3", "e5m2"):
        w.append(Workload(f"dense fp8 e4m3 x {dtb} 8192^3, per-tensor scales, C=0", "e4m3", dtb,
                          "k_contig", "k_contig", 8192, 8192, 8192, "normal", None, 1.0, 0.0,
                          fp8_scaled=True))
    w.append(Workload("2:4 sparse bf16 8192^3 (A compressed), C=0", "bf16", "bf16", "k_contig",
                      "k_contig", 8192, 8192, 8192, "normal", None, 1.0, 0.0, sparse=True))
    return w
