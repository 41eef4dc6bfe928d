// dense_general.hpp -- the general dense MFMA GEMM kernel for gfx950, templated
// on its output tile, and its dtype/layout dispatch.
//
// D = alpha * (A . B) + beta * C: the matrix fused multiply-add of "Accurate
// Models of AMD Matrix Cores" (Section 2, Eq. (1)) tiled over a workgroup, one
// MFMA K-step at a time as the builtins are meant to be used ("CDNA3 dense
// MFMA builtins", Naming convention: one instruction per K step, the caller
// loops over K; Using MFMA builtins as a compute policy: block tiles are
// multiples of the instruction tile and K tiles multiples of its K step).
//
// Kernel structure (per workgroup of 256 threads = 4 wavefronts):
//   - a BM x BN output tile (128 x 128, or 128 x 32 / 32 x 128 for skinny
//     problems); waves in a 2 x 2 grid, each owning a (BM/2) x (BN/2) sub-tile
//     of 16x16 instruction tiles;
//   - K is walked in tiles of 128 bytes; each tile of A and B is staged from
//     HBM into LDS (16-byte loads, swizzled rows), double-buffered so the loads
//     of tile t+1 are in flight while tile t is multiplied;
//   - the instruction is issued with P = B fragment and Q = A fragment, so the
//     output registers of a lane hold four consecutive columns of one row of D
//     (one 16-byte store per lane in the epilogue);
//   - split K (grid.y > 1): workgroup y multiplies K tiles
//     [y * kt_per_split, (y + 1) * kt_per_split) and adds alpha times its
//     partial sums into D with device-scope atomic adds; D was zeroed before
//     and beta * C is added after (splitk_zero / splitk_finish);
//   - otherwise the epilogue computes D = alpha*acc + beta*C in fp32 (float
//     inputs) or wrapping int32 (int8 inputs), rounded once to D's format;
//     C is not read when beta == 0.
#pragma once
#include "gemm_kernels.hpp"
#include "tile_io.hpp"
#include "frag_layout.hpp"

namespace mcg {

template <class Op, int LA, int LB, int BM, int BN, bool ALIGNED>
__global__ __launch_bounds__(256) void gemm_dense_kernel(DenseArgs p) {
  constexpr int NT = 256;
  constexpr int EB = Op::ELEM_BYTES;
  constexpr int STEPS = Op::STEPS;
  constexpr int WTM = BM / 2 / 16, WTN = BN / 2 / 16;  // instruction tiles per wave
  using GA = TileGeom<EB, LA, BM>;
  using GB = TileGeom<EB, LB, BN>;
  using RA = FragReader<EB, Op::LANE_BYTES == 32 ? 32 : 16, LA, BM>;
  using RB = FragReader<EB, Op::LANE_BYTES == 32 ? 32 : 16, LB, BN>;
  using acc_t = typename Op::acc_t;

  __shared__ __attribute__((aligned(16))) char smem_raw[2 * (GA::BYTES + GB::BYTES)];
  lds_char* smem = (lds_char*)smem_raw;
  lds_char* ldsA[2] = {smem, smem + GA::BYTES + GB::BYTES};
  lds_char* ldsB[2] = {smem + GA::BYTES, smem + 2 * GA::BYTES + GB::BYTES};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // workgroup -> output tile, grouped by 8 tile rows for L2 reuse
  const int pid = blockIdx.x;
  const int group = 8;
  const int tiles_in_group = group * p.tiles_n;
  const int gid = pid / tiles_in_group;
  const int first_m = gid * group;
  const int gsize = min(p.tiles_m - first_m, group);
  const int tm = first_m + (pid % tiles_in_group) % gsize;
  const int tn = (pid % tiles_in_group) / gsize;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  // this workgroup's range of K tiles
  const int KE = KT_BYTES / EB;  // K elements per tile
  const int nk_all = (int)((p.K + KE - 1) / KE);
  const int kt_begin = (int)blockIdx.y * p.kt_per_split;
  const int nk = min(nk_all - kt_begin, p.kt_per_split);

  // skinny tiles (BN or BM of 32 for N or M <= 32): the other operand is read once
  TileLoader<EB, LA, BM, NT, ALIGNED, KT_BYTES, (BN <= 32)> la;
  TileLoader<EB, LB, BN, NT, ALIGNED, KT_BYTES, (BM <= 32)> lb;
  auto load_tiles = [&](int kt) {
    const int64_t k0 = (int64_t)(kt_begin + kt) * KE;
    if constexpr (LA == LAYOUT_K) la.load(p.A, p.lda, m0, k0, p.M, p.K, tid);
    else la.load(p.A, p.lda, k0, m0, p.K, p.M, tid);
    if constexpr (LB == LAYOUT_K) lb.load(p.B, p.ldb, n0, k0, p.N, p.K, tid);
    else lb.load(p.B, p.ldb, k0, n0, p.K, p.N, tid);
  };

  acc_t acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  if (nk > 0) {
    load_tiles(0);
    la.store(ldsA[0], tid);
    lb.store(ldsB[0], tid);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles(kt + 1);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      typename Op::frag_t fa[WTM];
      typename Op::frag_t fb[WTN];
#pragma unroll
      for (int i = 0; i < WTM; ++i) fa[i] = Op::template frag_a<RA>(ldsA[cur], wm * (BM / 2) + i * 16, s, lane);
#pragma unroll
      for (int j = 0; j < WTN; ++j) fb[j] = Op::template frag_b<RB>(ldsB[cur], wn * (BN / 2) + j * 16, s, lane);
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j) acc[i][j] = Op::mma(fb[j], fa[i], acc[i][j]);
    }
    if (kt + 1 < nk) {
      la.store(ldsA[cur ^ 1], tid);
      lb.store(ldsB[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // epilogue: each instruction multiplied (B fragment) x (A fragment), so element
  // (i', j') of its 16 x 16 accumulator layout is D[m][n] with m = j', n = i'
  // within the block; register r holds (i' + r, j') for (i', j') =
  // ACC::coord(lane, 0): 4 consecutive columns of one row per lane
  using ACC = frag::Acc<frag::ACC_16x16>;
  const int acc_m = ACC::coord(lane, 0).j, acc_n = ACC::coord(lane, 0).i;
  if (gridDim.y > 1) {
    // split K: add alpha * partial sum into the zeroed D (binary32 or wrapping int32)
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const int64_t m = m0 + wm * (BM / 2) + i * 16 + acc_m;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < WTN; ++j) {
        const int64_t n = n0 + wn * (BN / 2) + j * 16 + acc_n;
        const int64_t off = m * p.ldc + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (n + r >= p.N) break;
          if constexpr (Op::INT_ACC)
            atomicAdd((int*)p.D + off + r, (int)((uint32_t)p.alpha_i * (uint32_t)acc[i][j][r]));
          else
            atomicAdd((float*)p.D + off + r, p.alpha * acc[i][j][r]);
        }
      }
    }
    return;
  }
  const bool vec_ok = p.vec_cd;
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
    const int64_t m = m0 + wm * (BM / 2) + i * 16 + acc_m;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int64_t n = n0 + wn * (BN / 2) + j * 16 + acc_n;
      if (n >= p.N) continue;
      const int64_t off = m * p.ldc + n;
      if constexpr (Op::INT_ACC) {
        const int* C = (const int*)p.C;
        int* D = (int*)p.D;
        i32x4 a = acc[i][j];
        i32x4 c = {0, 0, 0, 0};
        const bool full = vec_ok && n + 4 <= p.N;
        if (p.use_c) {
          if (full) c = *(const i32x4*)(C + off);
          else
            for (int r = 0; r < 4; ++r) if (n + r < p.N) c[r] = C[off + r];
        }
        i32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[r] = (int)((uint32_t)p.alpha_i * (uint32_t)a[r] + (uint32_t)p.beta_i * (uint32_t)c[r]);
        if (full) *(i32x4*)(D + off) = o;
        else
          for (int r = 0; r < 4; ++r) if (n + r < p.N) D[off + r] = o[r];
      } else {
        f32x4 a = acc[i][j];
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
        const bool full = vec_ok && n + 4 <= p.N;
        const int out = p.out;
        if (out == OUT_32) {
          const float* C = (const float*)p.C;
          if (p.use_c) {
            if (full) c = *(const f32x4*)(C + off);
            else
              for (int r = 0; r < 4; ++r) if (n + r < p.N) c[r] = C[off + r];
          }
        } else {  // bfloat16 / binary16 C
          const uint16_t* C = (const uint16_t*)p.C;
          if (p.use_c)
            for (int r = 0; r < 4; ++r) if (n + r < p.N) c[r] = from_out_bits(out, C[off + r]);
        }
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = p.use_c ? __builtin_fmaf(p.alpha, a[r], p.beta * c[r]) : p.alpha * a[r];
        if (out == OUT_32) {
          float* D = (float*)p.D;
          if (full) *(f32x4*)(D + off) = o;
          else
            for (int r = 0; r < 4; ++r) if (n + r < p.N) D[off + r] = o[r];
        } else {  // rounded once to the output format
          uint16_t* D = (uint16_t*)p.D;
          for (int r = 0; r < 4; ++r) if (n + r < p.N) D[off + r] = (uint16_t)to_out_bits(out, o[r]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch

template <class Op, int LA, int LB, int BM, int BN, bool AL>
static hipError_t launch_general_one(const DenseArgs& a0, hipStream_t s) {
  DenseArgs a = a0;
  a.tiles_m = (int)((a.M + BM - 1) / BM);
  a.tiles_n = (int)((a.N + BN - 1) / BN);
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff || a.splits < 1 || a.splits > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_dense_kernel<Op, LA, LB, BM, BN, AL>), dim3((unsigned)blocks, (unsigned)a.splits),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class Op, int BM, int BN, bool AL>
static hipError_t launch_general_layouts(int la, int lb, const DenseArgs& a, hipStream_t s) {
  if (la == 0 && lb == 0) return launch_general_one<Op, 0, 0, BM, BN, AL>(a, s);
  if (la == 0 && lb == 1) return launch_general_one<Op, 0, 1, BM, BN, AL>(a, s);
  if (la == 1 && lb == 0) return launch_general_one<Op, 1, 0, BM, BN, AL>(a, s);
  if (la == 1 && lb == 1) return launch_general_one<Op, 1, 1, BM, BN, AL>(a, s);
  return hipErrorInvalidValue;
}

// Launch the general kernel with a BM x BN tile for any supported dtype pair.
template <int BM, int BN, bool AL>
hipError_t launch_general(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s) {
  if (dtA == DT_BF16) return launch_general_layouts<OpBF16, BM, BN, AL>(la, lb, a, s);
  if (dtA == DT_F16) return launch_general_layouts<OpF16, BM, BN, AL>(la, lb, a, s);
  if (dtA == DT_I8) return launch_general_layouts<OpI8, BM, BN, AL>(la, lb, a, s);
  const int fa = f8fmt(dtA), fb = f8fmt(dtB);
  if (a.K >= FP8_NATIVE_MIN_K) {
    // P = B fragment, Q = A fragment: the P format is B's.
    if (fb == 0 && fa == 0) return launch_general_layouts<OpF8<0, 0>, BM, BN, AL>(la, lb, a, s);
    if (fb == 1 && fa == 0) return launch_general_layouts<OpF8<1, 0>, BM, BN, AL>(la, lb, a, s);
    if (fb == 0 && fa == 1) return launch_general_layouts<OpF8<0, 1>, BM, BN, AL>(la, lb, a, s);
    return launch_general_layouts<OpF8<1, 1>, BM, BN, AL>(la, lb, a, s);
  }
  if (fa == 0 && fb == 0) return launch_general_layouts<OpF8W<0, 0>, BM, BN, AL>(la, lb, a, s);
  if (fa == 0 && fb == 1) return launch_general_layouts<OpF8W<0, 1>, BM, BN, AL>(la, lb, a, s);
  if (fa == 1 && fb == 0) return launch_general_layouts<OpF8W<1, 0>, BM, BN, AL>(la, lb, a, s);
  return launch_general_layouts<OpF8W<1, 1>, BM, BN, AL>(la, lb, a, s);
}

}  // namespace mcg
