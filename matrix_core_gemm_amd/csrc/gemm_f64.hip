// gemm_f64.hip -- binary64 GEMM (DGEMM) on the FP64 matrix instructions of gfx950.
//
// D = alpha * (A . B) + beta * C for binary64 A, B, C and D, accumulated in binary64
// by the FP64-accumulate matrix instructions ("CDNA3 dense MFMA builtins",
// FP64-accumulate builtins; the accumulator layouts of the 4x4 FP64 tile shape).
//
// Instruction.  gfx950 issues the four-block 4x4x4 FP64 instruction at full rate
// (16 cycles; 75.5 TFLOP/s over the chip, measured), while the one-block 16x16x4
// FP64 instruction reaches only about 49 TFLOP/s (about 100 cycles per
// instruction per SIMD, measured).  The broadcast modifiers (cbsz/abid) leave the
// FP64 instructions of gfx950 unchanged (measured), so each of the four blocks
// takes its own A and B.  Operand and result lanes (measured; D as the pages' 4x4
// FP64 layout):
//   A_b[i][k] in lane i + 4b + 16k,  B_b[k][j] in lane j + 4b + 16k,
//   D_b[i][j] in lane 16i + 4b + j          (i, j, k, b in 0..3).
// The kernel gives the four blocks four different groups of 4 rows of A and the
// same 4 columns of B, so one instruction is a 16 x 4 x 4 product: A lane l holds
// row (l & 15) at K index l >> 4, B lane l holds column (l & 3) at K index l >> 4,
// and result lane l holds row 4((l >> 2) & 3) + (l >> 4), column l & 3.  No
// accumulator is redundant and no cross-lane reduction is needed.
//
// Tiling.  128 x 128 output tiles, 8 waves (2 along M x 4 along N, 64 x 32 per
// wave: 4 x 8 instructions per K index group), K in tiles of 16.  Each thread
// moves 4 elements of A and 4 of B per K tile from HBM into registers (8-byte
// loads, any alignment of the leading dimensions, zero outside the matrix) while
// the previous tile is multiplied, then stores them into the other half of a
// 2 x 32 KiB LDS double buffer; one barrier per K tile.  LDS rows hold the 16 K
// values of one row of A (column of B) as eight 16-byte chunks, chunk c of row r at
// position c ^ (r & 7), so the 8 rows a fragment read touches at once use 8
// different chunks.  A lane's fragment read takes K = 4g + 2h and 4g + 2h + 1
// (g = lane >> 4, h = 0, 1) with one 16-byte read; the two instructions that use
// them take the K index sets {4g + 2h} and {4g + 2h + 1}, consistently for A and B.
//
// Split K (few output tiles, long K): grid.y ranges of K tiles; the ranges add
// alpha * partial into a zeroed D with binary64 atomic adds, and beta * C is added
// afterwards (D must not be C then).
#include "arch_gfx950.hpp"
#include "fast_tiles.hpp"
#include "gemm_kernels.hpp"

namespace mcg {
namespace f64 {

constexpr int BM = 128, BN = 128, BK = 16, THREADS = 512;
constexpr int WM = 64, WN = 32;            // wave tile
constexpr int FM = WM / 16, FN = WN / 4;   // instructions per K index group: FM x FN
constexpr int ROW_BYTES = BK * 8;          // one LDS row: 16 binary64 K values
constexpr int A_BYTES = BM * ROW_BYTES;    // 16 KiB
constexpr int STAGE_BYTES = A_BYTES + BN * ROW_BYTES;
constexpr int PER_THREAD = BM * BK / THREADS;  // elements of each operand per thread and K tile
static_assert(BM == BN, "one loader geometry serves both operands");
static_assert(PER_THREAD * THREADS == BM * BK, "loader covers the tile");

typedef double f64x2 __attribute__((ext_vector_type(2)));

// Byte offset of K value k (0..15) of LDS row r.
__device__ __forceinline__ int lds_at(int r, int k) {
  return r * ROW_BYTES + ((((k >> 1) ^ r) & 7) << 4) + ((k & 1) << 3);
}

// Moves one operand's 128 x 16 tile.  LAY 0 (K-contiguous): element (r, k) at
// X[r * ld + k]; LAY 1 (MN-contiguous): at X[k * ld + r].  Thread t moves
// elements e = t + 512 p: (r, k) = (e >> 4, e & 15) for LAY 0, so 16 threads read
// one 128-byte row; (e & 127, e >> 7) for LAY 1, so consecutive threads read
// consecutive rows of one K.
template <int LAY>
struct Loader {
  const double* ptr[PER_THREAD];
  int64_t step;  // elements between consecutive K tiles
  int r[PER_THREAD], k[PER_THREAD];
  bool row_ok[PER_THREAD];
  double v[PER_THREAD];

  __device__ __forceinline__ void init(const double* X, int64_t ld, int64_t r0, int64_t rows, int64_t k0,
                                       int tid) {
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) {
      const int e = tid + THREADS * p;
      r[p] = LAY == 0 ? e >> 4 : e & (BM - 1);
      k[p] = LAY == 0 ? e & (BK - 1) : e >> 7;
      row_ok[p] = r0 + r[p] < rows;
      const int64_t rg = row_ok[p] ? r0 + r[p] : 0;
      ptr[p] = LAY == 0 ? X + rg * ld + k0 + k[p] : X + (k0 + k[p]) * ld + rg;
    }
    step = LAY == 0 ? BK : BK * ld;
  }
  // Load the tile starting at K = k0 (elements with K >= kend or outside the rows read 0) and
  // advance to the next tile.
  __device__ __forceinline__ void load(int64_t k0, int64_t kend) {
    if (k0 + BK <= kend) {
#pragma unroll
      for (int p = 0; p < PER_THREAD; ++p) v[p] = row_ok[p] ? *ptr[p] : 0.0;
    } else {
#pragma unroll
      for (int p = 0; p < PER_THREAD; ++p) v[p] = (row_ok[p] && k0 + k[p] < kend) ? *ptr[p] : 0.0;
    }
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) ptr[p] += step;
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int p = 0; p < PER_THREAD; ++p) *(double*)(lds + lds_at(r[p], k[p])) = v[p];
  }
};

template <int LA, int LB>
__global__ __launch_bounds__(THREADS) void dgemm_kernel(F64Args p) {
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE_BYTES];
  int tm, tn;
  fast::tile_coords<8>(p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = (w & 1) * WM, wn = (w >> 1) * WN;

  // K range of this workgroup (grid.y > 1: split K)
  const int64_t nk_all = (p.K + BK - 1) / BK;
  const int64_t kt0 = (int64_t)blockIdx.y * p.kt_per_split;
  const int64_t nk = nk_all - kt0 < p.kt_per_split ? nk_all - kt0 : p.kt_per_split;
  const int64_t kbeg = kt0 * BK;

  Loader<LA> la;
  Loader<LB> lb;
  la.init(p.A, p.lda, m0, p.M, kbeg, tid);
  lb.init(p.B, p.ldb, n0, p.N, kbeg, tid);

  double acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int c = 0; c < FN; ++c) acc[f][c] = 0.0;

  const int g = lane >> 4;
  const int ra = wm + (lane & 15);  // A row of this lane (+ 16 f)
  const int cb = wn + (lane & 3);   // B column of this lane (+ 4 c)

  if (nk > 0) {
    la.load(kbeg, p.K);
    lb.load(kbeg, p.K);
    la.store(lds);
    lb.store(lds + A_BYTES);
    __syncthreads();
  }
  for (int64_t t = 0; t < nk; ++t) {
    const bool more = t + 1 < nk;
    if (more) {
      la.load(kbeg + (t + 1) * BK, p.K);
      lb.load(kbeg + (t + 1) * BK, p.K);
    }
    const char* sA = lds + (t & 1) * STAGE_BYTES;
    const char* sB = sA + A_BYTES;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f64x2 a[FM], b[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f) a[f] = *(const f64x2*)(sA + lds_at(ra + 16 * f, 4 * g + 2 * h));
#pragma unroll
      for (int c = 0; c < FN; ++c) b[c] = *(const f64x2*)(sB + lds_at(cb + 4 * c, 4 * g + 2 * h));
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
          for (int c = 0; c < FN; ++c)
            acc[f][c] = __builtin_amdgcn_mfma_f64_4x4x4f64(a[f][e], b[c][e], acc[f][c], 0, 0, 0);
    }
    if (more) {
      char* nxt = lds + ((t + 1) & 1) * STAGE_BYTES;
      la.store(nxt);
      lb.store(nxt + A_BYTES);
    }
    __syncthreads();
  }

  // result lane l: row 4((l >> 2) & 3) + (l >> 4), column l & 3 of each 16 x 4 piece
  const int orow = 4 * ((lane >> 2) & 3) + (lane >> 4);
  const int ocol = lane & 3;
  double* D = p.D;
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int64_t row = m0 + wm + 16 * f + orow;
    if (row >= p.M) continue;
#pragma unroll
    for (int c = 0; c < FN; ++c) {
      const int64_t col = n0 + wn + 4 * c + ocol;
      if (col >= p.N) continue;
      const int64_t off = row * p.ldc + col;
      if (gridDim.y > 1) {
        atomicAdd(D + off, p.alpha * acc[f][c]);
      } else {
        double v = p.alpha * acc[f][c];
        if (p.use_c) v = __builtin_fma(p.beta, p.C[off], v);
        D[off] = v;
      }
    }
  }
}

// Split K, before the partial sums: D = 0 over M x N.
__global__ __launch_bounds__(256) void zero_kernel(F64Args p) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= p.N) return;
  for (int64_t m = blockIdx.y; m < p.M; m += gridDim.y) p.D[m * p.ldc + n] = 0.0;
}

// Split K, after the partial sums (only when beta != 0): D = beta * C + D, one rounding.
__global__ __launch_bounds__(256) void finish_kernel(F64Args p) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= p.N) return;
  for (int64_t m = blockIdx.y; m < p.M; m += gridDim.y) {
    const int64_t off = m * p.ldc + n;
    p.D[off] = __builtin_fma(p.beta, p.C[off], p.D[off]);
  }
}

template <int LA, int LB>
static void launch_tiles(const F64Args& a, int splits, hipStream_t s) {
  hipLaunchKernelGGL((dgemm_kernel<LA, LB>), dim3((unsigned)(a.tiles_m * a.tiles_n), (unsigned)splits), dim3(THREADS),
                     0, s, a);
}

}  // namespace f64

F64Plan plan_f64(const F64Args& a, bool can_split) {
  using namespace f64;
  F64Plan plan{1, (int)((a.K + BK - 1) / BK)};
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const int64_t nk = (a.K + BK - 1) / BK;
  if (!can_split || nk < 2 * F64_SPLIT_MIN_KT || tiles >= F64_NUM_CU) return plan;
  // Estimated time of S ranges: waves of resident tiles times the K tiles of one range,
  // plus the atomic adds of the partial sums and the extra launches.
  auto cost = [&](int64_t S) {
    const int64_t per = (nk + S - 1) / S;
    const int64_t rounds = (tiles * S + F64_NUM_CU - 1) / F64_NUM_CU;
    return (double)rounds * (F64_KT_US * (double)per + F64_ROUND_US) +
           F64_ATOMIC_US * (double)S * (double)a.M * (double)a.N + (S > 1 ? F64_SPLIT_US : 0.0);
  };
  int64_t best = 1;
  double best_t = cost(1);
  for (int64_t S = 2; S <= nk / F64_SPLIT_MIN_KT && tiles * S <= 4 * F64_NUM_CU; ++S) {
    const double t = cost(S);
    if (t < best_t) {
      best_t = t;
      best = S;
    }
  }
  const int64_t per = (nk + best - 1) / best;
  plan.splits = (int)((nk + per - 1) / per);  // no empty range
  plan.kt_per_split = (int)per;
  return plan;
}

hipError_t launch_f64(int la, int lb, const F64Args& a0, const F64Plan& plan, hipStream_t s) {
  using namespace f64;
  F64Args a = a0;
  a.tiles_m = (int)((a.M + BM - 1) / BM);
  a.tiles_n = (int)((a.N + BN - 1) / BN);
  a.kt_per_split = plan.kt_per_split;
  const dim3 rows_grid((unsigned)((a.N + 255) / 256), (unsigned)(a.M < 4096 ? a.M : 4096));
  if (plan.splits > 1) {
    hipLaunchKernelGGL(zero_kernel, rows_grid, dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (la == 0 && lb == 0) launch_tiles<0, 0>(a, plan.splits, s);
  else if (la == 0) launch_tiles<0, 1>(a, plan.splits, s);
  else if (lb == 0) launch_tiles<1, 0>(a, plan.splits, s);
  else launch_tiles<1, 1>(a, plan.splits, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1 || !a.use_c) return e;
  hipLaunchKernelGGL(finish_kernel, rows_grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mcg
