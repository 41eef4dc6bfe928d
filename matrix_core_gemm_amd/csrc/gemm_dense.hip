// gemm_dense.hip -- the general dense kernel with 128 x 128 tiles, split-K
// support kernels, and the choice of kernel and K split for a dense problem.
//
// Split K: when a problem has too few output tiles to occupy the 256 compute
// units (skinny shapes such as N <= 32, or few tiles with a long K), the K
// loop is cut into ranges multiplied by separate workgroups.  D (binary32 or
// int32) is zeroed first, every workgroup adds alpha times its partial sum
// into D with device-scope atomic adds, and when beta != 0 a last pass adds
// beta * C with one rounding.  C enters once, after all partial sums: adding
// it to the running sum first would round every later partial sum against
// |C|, which the accuracy bound does not allow for when |C| dominates.  The
// order of the atomic additions is not fixed, so float results may differ in
// the last bits from run to run (int32 sums wrap modulo 2^32 and are exact).
#include <algorithm>

#include "dense_general.hpp"
#include "gemm_kernels.hpp"

namespace mcg {

// D[m][n] = 0 for m < M, n < N (all-zero bits: +0.0f and int 0).  Grid:
// x covers N in blocks of 256, y strides over the rows.
__global__ __launch_bounds__(256) void splitk_zero_kernel(DenseArgs p) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= p.N) return;
  for (int64_t m = blockIdx.y; m < p.M; m += gridDim.y) ((int*)p.D)[m * p.ldc + n] = 0;
}

// D = D + beta * C with one rounding (fp32 fma), or in wrapping int32; run
// only when beta != 0.
template <bool INT>
__global__ __launch_bounds__(256) void splitk_finish_kernel(DenseArgs p) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= p.N) return;
  for (int64_t m = blockIdx.y; m < p.M; m += gridDim.y) {
    const int64_t off = m * p.ldc + n;
    if constexpr (INT) {
      int* D = (int*)p.D;
      D[off] = (int)((uint32_t)D[off] + (uint32_t)p.beta_i * (uint32_t)((const int*)p.C)[off]);
    } else {
      float* D = (float*)p.D;
      D[off] = __builtin_fmaf(p.beta, ((const float*)p.C)[off], D[off]);
    }
  }
}

static dim3 rows_grid(const DenseArgs& a) {
  return dim3((unsigned)((a.N + 255) / 256), (unsigned)(a.M < 4096 ? a.M : 4096));
}

// ------------------------------------------------------------------ plan

namespace {
constexpr int64_t FAST_MIN_TILES = 128;   // 256 x 256 tiles from which the fast kernel wins
// Split-K cost model of the 4-wave general kernels (MI355X, measured with
// bf16, fp8 and int8 over 256^2..2048^2 outputs and K up to 65536):
//   time(s) ~ rounds * (KT_US * ceil(nk / s) + ROUND_US) + ATOMIC_US * s * M * N + SPLIT_US [s > 1]
// with rounds = ceil(tiles * s / num_cu) workgroups per CU, KT_US per 128-byte
// K tile of a workgroup, ATOMIC_US per device-scope atomic add of D and
// SPLIT_US for zeroing D and the extra launches.
constexpr double KT_US = 1.0, ROUND_US = 3.0, ATOMIC_US = 1.4e-5, SPLIT_US = 5.0;
// The 128 x 128 form of the fast kernel (KERNEL_MID, one workgroup per CU):
// ceil(tiles / num_cu) * (MID_KT_US * nk + MID_ROUND_US), fitted over 100..256
// tiles and K up to 8192; taken when it beats the best general plan by MID_MARGIN.
constexpr double MID_KT_US = 0.5, MID_ROUND_US = 3.0, MID_MARGIN = 0.95;
// The streaming kernel is HBM-bound: split only when there are too few blocks
// to spread over the CUs (fewer than 128: splitting 64 blocks in two measured
// 1.2-1.5x faster on bf16 2048 x 16 x 16384 and 3072 x 16 x 8192), keeping 16 K
// tiles or more per split.
constexpr int64_t STREAM_MIN_BLOCKS = 128, STREAM_MIN_KT = 16, STREAM_MN_MIN_WIDE = 2048;
}  // namespace

DensePlan plan_dense(int dtA, int la, int lb, const DenseArgs& a, bool aligned, bool can_split, int num_cu) {
  const int64_t NUM_CU = num_cu > 0 ? num_cu : 256;
  const int64_t eb = (dtA == DT_BF16 || dtA == DT_F16) ? 2 : 1;
  const int64_t KE = KT_BYTES / eb;
  const int64_t nk = (a.K + KE - 1) / KE;
  auto cdiv = [](int64_t x, int64_t y) { return (x + y - 1) / y; };
  // number of K ranges for `tiles` workgroups of the general kernels, and the
  // modelled time of that plan
  auto plan_general = [&](int64_t tiles, double* time) -> int64_t {
    auto model = [&](int64_t ss) {  // ss >= 1
      const double rounds = (double)cdiv(tiles * ss, NUM_CU);
      return rounds * (KT_US * (double)cdiv(nk, ss) + ROUND_US) +
             ATOMIC_US * (double)ss * (double)a.M * (double)a.N + (ss > 1 ? SPLIT_US : 0.0);
    };
    int64_t best = 1;
    double best_t = model(1);
    if (can_split && nk >= 2) {
      for (int64_t s = 2; s <= nk / 2 + 1 && s <= 1024; s = s < 4 ? s + 1 : s * 2) {
        const int64_t ss = std::min(s, nk);
        const double t = model(ss);
        if (t < best_t) { best = ss; best_t = t; }
      }
    }
    // the model charges atomic adds to the unsplit plan too (it only ranks split
    // counts); the unsplit kernel stores D directly
    if (time) *time = best_t - (best == 1 ? ATOMIC_US * (double)a.M * (double)a.N : 0.0);
    return best;
  };
  auto splits_for = [&](int64_t tiles) { return plan_general(tiles, nullptr); };
  auto make = [&](int kernel, int64_t s) {
    DensePlan p{kernel, 1, (int)(nk > 0 ? nk : 1), 0};
    if (s > 1) {
      const int64_t kps = cdiv(nk, s);
      p.kt_per_split = (int)kps;
      p.splits = (int)cdiv(nk, kps);  // every range non-empty
    }
    return p;
  };

  if (fast_path_ok(dtA, la, lb, a, aligned) && cdiv(a.M, 256) * cdiv(a.N, 256) >= FAST_MIN_TILES)
    return make(KERNEL_FAST, 1);
  if (fast_path_ok(dtA, la, lb, a, aligned, 128)) {
    const int64_t tiles = cdiv(a.M, 128) * cdiv(a.N, 128);
    double t_general;
    plan_general(tiles, &t_general);
    const double t_mid = (double)cdiv(tiles, NUM_CU) * (MID_KT_US * (double)nk + MID_ROUND_US);
    if (t_mid < MID_MARGIN * t_general) return make(KERNEL_MID, 1);
  }
  // Skinny problems: the streaming kernel, except with an MN-contiguous wide
  // operand of fewer than STREAM_MN_MIN_WIDE rows, where the general kernel's
  // 128 x 32 / 32 x 128 tiles were faster (bf16 1024 x 16 x 3008: 13.2 against
  // 14.6-17.5 us)
  const bool wide_a = a.N <= 32 && a.N <= a.M;
  const int64_t wide = wide_a ? a.M : a.N;
  const bool wide_mn = (wide_a ? la : lb) == LAYOUT_MN;
  if (stream_path_ok(dtA, la, lb, a, aligned) && !(wide_mn && wide < STREAM_MN_MIN_WIDE)) {
    // 128-row blocks when that still gives most CUs a block, else 32-row blocks
    // (measured: more blocks beat wider ones below 16384 rows), except for an
    // MN-contiguous wide operand: its LDS rows are one k of the block's rows, so
    // only 128-row blocks fetch whole 128-byte lines.  Fewer than
    // STREAM_MIN_BLOCKS blocks are split along K (measured: 64 blocks unsplit ran
    // at half the HBM rate; 256 workgroups were slower than 128 at 16384 rows)
    const int bw = wide >= 64 * NUM_CU || wide_mn ? 128 : 32;
    const int64_t blocks = cdiv(wide, bw);
    int64_t s = 1;
    if (can_split && blocks < STREAM_MIN_BLOCKS)
      s = std::max<int64_t>(1, std::min(cdiv(STREAM_MIN_BLOCKS, blocks), nk / STREAM_MIN_KT));
    DensePlan pl = make(KERNEL_STREAM, s);
    pl.stream_bw = bw;
    return pl;
  }
  if (aligned && a.N <= 32 && a.N <= a.M) return make(KERNEL_SKINNY_N, splits_for(cdiv(a.M, 128)));
  if (aligned && a.M <= 32) return make(KERNEL_SKINNY_M, splits_for(cdiv(a.N, 128)));
  return make(KERNEL_GENERAL, splits_for(cdiv(a.M, 128) * cdiv(a.N, 128)));
}

// ------------------------------------------------------------------ launch

hipError_t launch_dense(int dtA, int dtB, int la, int lb, bool aligned, const DenseArgs& a0,
                        const DensePlan& plan, hipStream_t s) {
  DenseArgs a = a0;
  a.splits = plan.splits;
  a.kt_per_split = plan.kt_per_split;
  a.stream_bw = plan.stream_bw;
  const bool split = a.splits > 1;
  const bool is_int = dtA == DT_I8;
  // the launch limits of the kernel that follows are checked before D is
  // zeroed, so a rejected plan writes nothing
  if (a.splits < 1 || a.splits > 65535) return hipErrorInvalidValue;
  {
    const int64_t bm = plan.kernel == KERNEL_SKINNY_M ? 32 : 128, bn = plan.kernel == KERNEL_SKINNY_N ? 32 : 128;
    int64_t blocks = ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
    if (plan.kernel == KERNEL_STREAM) {
      const int64_t wide = a.N <= 32 && a.N <= a.M ? a.M : a.N;
      blocks = (wide + a.stream_bw - 1) / (a.stream_bw > 0 ? a.stream_bw : 1);
    }
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  }
  if (split) {
    if (a.out != OUT_32) return hipErrorInvalidValue;
    hipLaunchKernelGGL(splitk_zero_kernel, rows_grid(a), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  switch (plan.kernel) {
    case KERNEL_SKINNY_N: e = launch_skinny_n(dtA, dtB, la, lb, a, s); break;
    case KERNEL_SKINNY_M: e = launch_skinny_m(dtA, dtB, la, lb, a, s); break;
    case KERNEL_STREAM: e = launch_stream(dtA, dtB, la, lb, a, s); break;
    default:
      e = aligned ? launch_general<128, 128, true>(dtA, dtB, la, lb, a, s)
                  : launch_general<128, 128, false>(dtA, dtB, la, lb, a, s);
  }
  if (e != hipSuccess || !split || !a.use_c) return e;
  if (is_int) hipLaunchKernelGGL(splitk_finish_kernel<true>, rows_grid(a), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(splitk_finish_kernel<false>, rows_grid(a), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mcg
