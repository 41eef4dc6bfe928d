// api.cpp -- the C ABI declared in include/mcg.h: argument validation (pure host code,
// no HIP call before it has passed), the gfx950 check, and dispatch to the kernels.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/mcg.h"
#include "gemm_kernels.hpp"

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool is_float8(int dt) { return dt == MCG_FP8_E4M3 || dt == MCG_FP8_E5M2; }
bool is_in_dtype(int dt) { return dt >= MCG_BF16 && dt <= MCG_FP8_E5M2; }
// Output format of D (and C) for the kernels; 0 for binary32 / int32.
static int out_format(int dtypeD) {
  return dtypeD == MCG_BF16 ? mcg::OUT_BF16 : dtypeD == MCG_F16 ? mcg::OUT_F16 : mcg::OUT_32;
}
static bool float_out(int dtypeD) { return dtypeD == MCG_F32 || dtypeD == MCG_BF16 || dtypeD == MCG_F16; }

int elem_bytes(int dt) {
  switch (dt) {
    case MCG_BF16:
    case MCG_F16: return 2;
    case MCG_I8:
    case MCG_FP8_E4M3:
    case MCG_FP8_E5M2: return 1;
    case MCG_F32:
    case MCG_I32: return 4;
    case MCG_F64: return 8;
    default: return 0;
  }
}
bool aligned_to(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
bool valid_layout(int l) { return l == MCG_K_CONTIG || l == MCG_MN_CONTIG; }
bool int32_integral(double v) {
  return std::isfinite(v) && v == std::floor(v) && v >= -2147483648.0 && v <= 2147483647.0;
}

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other;
// and the device's compute-unit count (0 unknown).
std::atomic<int> g_arch_state[64];
std::atomic<int> g_num_cu[64];

constexpr int kDefaultCUs = 256;  // an MI355X's compute units

// Reads (once per device) the architecture name and compute-unit count.
int probe_device(int dev) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MCG_ERR_HIP;
  g_num_cu[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : kDefaultCUs,
                      std::memory_order_relaxed);
  g_arch_state[dev].store(std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2, std::memory_order_relaxed);
  return MCG_SUCCESS;
}

int check_arch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MCG_ERR_HIP;
  if (dev < 0 || dev >= 64) return MCG_ERR_UNSUPPORTED_ARCH;
  if (g_arch_state[dev].load(std::memory_order_relaxed) == 0) {
    const int st = probe_device(dev);
    if (st != MCG_SUCCESS) return st;
  }
  return g_arch_state[dev].load(std::memory_order_relaxed) == 1 ? MCG_SUCCESS : MCG_ERR_UNSUPPORTED_ARCH;
}

// Compute units of the current device, for the kernel planners; the MI355X
// count when no device is visible (host-only planning queries).
int current_num_cu() {
  int ndev = 0, dev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return kDefaultCUs;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefaultCUs;
  if (g_num_cu[dev].load(std::memory_order_relaxed) == 0 && probe_device(dev) != MCG_SUCCESS) return kDefaultCUs;
  return g_num_cu[dev].load(std::memory_order_relaxed);
}

// A float alpha/beta the kernels receive as fp32 must stay finite there.
bool finite_as_f32(double v) { return std::isfinite((float)v); }

int hip_status(hipError_t e) { return e == hipSuccess ? MCG_SUCCESS : MCG_ERR_HIP; }

}  // namespace

extern "C" {

// Validation of gemm_dense arguments; touches no device state.
int mcg_validate_dense(int dtypeA, int dtypeB, int layoutA, int layoutB, int64_t M, int64_t N,
                       int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, const void* D, int64_t ldc, int dtypeD, double alpha,
                       double beta, float scaleA, float scaleB) {
  if (dtypeA == MCG_F64 || dtypeB == MCG_F64) {
    if (dtypeA != dtypeB || dtypeD != MCG_F64) return MCG_ERR_UNSUPPORTED_DTYPE;
  } else if (!is_in_dtype(dtypeA) || !is_in_dtype(dtypeB)) {
    return MCG_ERR_UNSUPPORTED_DTYPE;
  }
  const bool f8 = is_float8(dtypeA) && is_float8(dtypeB);
  if (!f8 && dtypeA != dtypeB) return MCG_ERR_UNSUPPORTED_DTYPE;
  if (is_float8(dtypeA) != is_float8(dtypeB)) return MCG_ERR_UNSUPPORTED_DTYPE;
  const bool i8 = dtypeA == MCG_I8;
  const bool f64 = dtypeA == MCG_F64;
  if (i8 ? dtypeD != MCG_I32 : f64 ? dtypeD != MCG_F64 : !float_out(dtypeD)) return MCG_ERR_UNSUPPORTED_DTYPE;
  if (!valid_layout(layoutA) || !valid_layout(layoutB)) return MCG_ERR_UNSUPPORTED_DTYPE;
  if (M < 0 || N < 0 || K < 0) return MCG_ERR_INVALID_SIZE;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return MCG_ERR_INVALID_SIZE;
  if (M == 0 || N == 0) return MCG_SUCCESS;
  if (!D) return MCG_ERR_NULL_POINTER;
  if (K > 0 && (!A || !B)) return MCG_ERR_NULL_POINTER;
  if (beta != 0.0 && !C) return MCG_ERR_NULL_POINTER;
  const int64_t min_lda = layoutA == MCG_K_CONTIG ? K : M;
  const int64_t min_ldb = layoutB == MCG_K_CONTIG ? K : N;
  if (lda < (min_lda > 1 ? min_lda : 1) || ldb < (min_ldb > 1 ? min_ldb : 1) || ldc < N)
    return MCG_ERR_INVALID_LD;
  const int ebd = elem_bytes(dtypeD);
  if (!aligned_to(A, elem_bytes(dtypeA)) || !aligned_to(B, elem_bytes(dtypeB)) ||
      !aligned_to(D, ebd) || (C && !aligned_to(C, ebd)))
    return MCG_ERR_MISALIGNED;
  if (i8) {
    if (!int32_integral(alpha) || !int32_integral(beta)) return MCG_ERR_INVALID_VALUE;
  } else if (!std::isfinite(alpha) || !std::isfinite(beta)) {
    return MCG_ERR_INVALID_VALUE;
  }
  if (!f8 && (scaleA != 1.0f || scaleB != 1.0f)) return MCG_ERR_INVALID_VALUE;
  if (f8 && (!std::isfinite(scaleA) || !std::isfinite(scaleB))) return MCG_ERR_INVALID_VALUE;
  // the float epilogues take alpha*scaleA*scaleB and beta as fp32
  if (!i8 && !f64 && (!finite_as_f32(alpha * (double)scaleA * (double)scaleB) || !finite_as_f32(beta)))
    return MCG_ERR_INVALID_VALUE;
  return MCG_SUCCESS;
}

// 16-byte aligned operands whose rows are whole 16-byte chunks: the vector load paths.
static bool dense_aligned(int eb, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb) {
  return K == 0 || (aligned_to(A, 16) && aligned_to(B, 16) && (lda * eb) % 16 == 0 && (ldb * eb) % 16 == 0);
}

// Split K zeroes D and adds partial sums into it: only for binary32 / int32 D
// that is not also the C being read.
static bool can_split_k(const mcg::DenseArgs& a, const void* C, const void* D) {
  return a.out == mcg::OUT_32 && !(a.use_c && C == D);
}

static mcg::F64Args f64_args(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                             int64_t ldb, const void* C, void* D, int64_t ldc, double alpha, double beta) {
  mcg::F64Args a{};
  a.A = (const double*)A;
  a.B = (const double*)B;
  a.C = (const double*)C;
  a.D = (double*)D;
  a.M = M;
  a.N = N;
  a.K = K;
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.alpha = alpha;
  a.beta = beta;
  a.use_c = beta != 0.0;
  return a;
}

// The stream-K form of a pipelined plan: fills the sk_* fields of a, sets *tile
// (the tile size to launch) and returns the workspace bytes, or 0 for none.  A
// 128 x 128 plan that has no stream-K split of its own although its last round
// leaves CUs idle takes the 256 x 256 split instead when K is long (at least
// LONG_K_TILES K tiles of 128 bytes) and that split needs at most alt_cap bytes:
// a few 256 x 256 tiles cut along K then beat the 128 x 128 tiles whole
// (measured, bf16 1536^2 x 16384: 110 against 126 us, 134 against 169 us from a
// flushed cache; 2560^2 x 16384: 213 against 252 us; below about 256 K tiles the
// two are even, and with whole rounds of 128 x 128 tiles, as at 2048^2, the
// 128 x 128 tiles are faster while the operands stay in the caches).
constexpr int64_t LONG_K_TILES = 256;

static int64_t dense_streamk(int dtypeA, int layoutA, int layoutB, mcg::DenseArgs& a, bool aligned, int kernel,
                             int64_t alt_cap, int* tile) {
  const int ncu = current_num_cu();
  if (kernel == mcg::KERNEL_GENERAL) {
    // Few tiles and a long K, which the cost model without a workspace leaves
    // to the general kernel (with split K): the 128 x 128 form's stream-K split
    // when it has one and it fits alt_cap (measured, bf16 1024^2 x 16384: 50
    // against 120 us; 1024^2 x 32768: 79 against 176 us)
    a.dp_tiles = a.sk_tiles = a.sk_wgs = 0;
    if (!mcg::fast_path_ok(dtypeA, layoutA, layoutB, a, aligned, 128)) return 0;
    *tile = 128;
    const int64_t need = mcg::plan_streamk(dtypeA, a, ncu, 128);
    if (need > 0 && need <= alt_cap) return need;
    a.dp_tiles = a.sk_tiles = a.sk_wgs = 0;
    return 0;
  }
  if (kernel != mcg::KERNEL_FAST && kernel != mcg::KERNEL_MID) return 0;
  *tile = kernel == mcg::KERNEL_MID ? 128 : 256;
  const int64_t need = mcg::plan_streamk(dtypeA, a, ncu, *tile);
  if (need > 0 || kernel != mcg::KERNEL_MID) return need;
  const int64_t tiles128 = ((a.M + 127) / 128) * ((a.N + 127) / 128);
  if (tiles128 % ncu == 0 || a.K * elem_bytes(dtypeA) < LONG_K_TILES * 128 ||
      !mcg::fast_path_ok(dtypeA, layoutA, layoutB, a, aligned, 256))
    return 0;
  const int64_t alt = mcg::plan_streamk(dtypeA, a, ncu, 256);
  if (alt <= 0 || alt > alt_cap) {
    a.dp_tiles = a.sk_tiles = a.sk_wgs = 0;
    return 0;
  }
  *tile = 256;
  return alt;
}

// gemm_dense, gemm_dense_ws and gemm_dense_noalloc: ws (ws_bytes) is the
// caller's workspace, or null; use_static: take the stream-K slots from the
// library's static scratch, rejecting plans that need more than it holds.
static int dense_impl(int dtypeA, int dtypeB, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda, const void* B, int64_t ldb, const void* C, void* D,
                      int64_t ldc, int dtypeD, double alpha, double beta, float scaleA, float scaleB,
                      void* ws, int64_t ws_bytes, void* stream, bool use_static = false) {
  int st = mcg_validate_dense(dtypeA, dtypeB, layoutA, layoutB, M, N, K, A, lda, B, ldb, C, D, ldc,
                              dtypeD, alpha, beta, scaleA, scaleB);
  if (st != MCG_SUCCESS) return st;
  if (ws != nullptr && (ws_bytes < 0 || !aligned_to(ws, 16))) return ws_bytes < 0 ? MCG_ERR_INVALID_SIZE : MCG_ERR_MISALIGNED;
  if (M == 0 || N == 0) return st;
  st = check_arch();
  if (st != MCG_SUCCESS) return st;
  if (dtypeA == MCG_F64) {
    const mcg::F64Args a = f64_args(M, N, K, A, lda, B, ldb, C, D, ldc, alpha, beta);
    const mcg::F64Plan plan = mcg::plan_f64(a, !(a.use_c && C == D), current_num_cu());
    return hip_status(mcg::launch_f64(layoutA, layoutB, a, plan, (hipStream_t)stream));
  }

  const int eb = elem_bytes(dtypeA);
  mcg::DenseArgs a{};
  a.A = (const char*)A;
  a.B = (const char*)B;
  a.C = C;
  a.D = D;
  a.M = M;
  a.N = N;
  a.K = K;
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.alpha = (float)(alpha * (double)scaleA * (double)scaleB);
  a.beta = (float)beta;
  a.alpha_i = dtypeA == MCG_I8 ? (int)alpha : 0;
  a.beta_i = dtypeA == MCG_I8 ? (int)beta : 0;
  a.use_c = beta != 0.0;
  a.out = out_format(dtypeD);
  const int vb = 4 * elem_bytes(dtypeD);  // bytes of 4 consecutive C/D elements
  a.vec_cd = aligned_to(D, vb) && (!a.use_c || aligned_to(C, vb)) && ldc % 4 == 0;
  const bool aligned = dense_aligned(eb, K, A, lda, B, ldb);
  const mcg::DensePlan plan =
      mcg::plan_dense(dtypeA, layoutA, layoutB, a, aligned, can_split_k(a, C, D), current_num_cu());
  // the pipelined kernels, and few-tile problems of the general kernel, may
  // take a stream-K form with a workspace (dense_streamk)
  const bool pipelined = plan.kernel == mcg::KERNEL_FAST || plan.kernel == mcg::KERNEL_MID ||
                         plan.kernel == mcg::KERNEL_GENERAL;
  int tile = 0;
  if (pipelined && use_static) {
    const int64_t need =
        dense_streamk(dtypeA, layoutA, layoutB, a, aligned, plan.kernel, mcg::STATIC_SCRATCH_BYTES, &tile);
    if (need > mcg::STATIC_SCRATCH_BYTES) return MCG_ERR_SCRATCH_LIMIT;
    if (need > 0) {
      void* p = nullptr;
      const hipError_t e = mcg::static_scratch(&p);
      if (e != hipSuccess) return hip_status(e);
      a.ws = p;
      return hip_status(mcg::launch_fast_sk(dtypeA, dtypeB, layoutA, layoutB, a, (hipStream_t)stream, tile));
    }
  }
  if (pipelined && ws != nullptr) {
    const int64_t need = dense_streamk(dtypeA, layoutA, layoutB, a, aligned, plan.kernel, INT64_MAX, &tile);
    if (need > 0 && need <= ws_bytes) {
      a.ws = ws;
      return hip_status(mcg::launch_fast_sk(dtypeA, dtypeB, layoutA, layoutB, a, (hipStream_t)stream, tile));
    }
    a.dp_tiles = a.sk_tiles = a.sk_wgs = 0;
  }
  if (plan.kernel == mcg::KERNEL_FAST || plan.kernel == mcg::KERNEL_MID)
    return hip_status(mcg::launch_fast(dtypeA, dtypeB, layoutA, layoutB, a, (hipStream_t)stream,
                                       plan.kernel == mcg::KERNEL_MID ? 128 : 256));
  return hip_status(mcg::launch_dense(dtypeA, dtypeB, layoutA, layoutB, aligned, a, plan, (hipStream_t)stream));
}

int gemm_dense(int dtypeA, int dtypeB, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
               const void* A, int64_t lda, const void* B, int64_t ldb, const void* C, void* D,
               int64_t ldc, int dtypeD, double alpha, double beta, float scaleA, float scaleB,
               void* stream) {
  return dense_impl(dtypeA, dtypeB, layoutA, layoutB, M, N, K, A, lda, B, ldb, C, D, ldc, dtypeD, alpha, beta,
                    scaleA, scaleB, nullptr, 0, stream);
}

int gemm_dense_ws(int dtypeA, int dtypeB, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
                  const void* A, int64_t lda, const void* B, int64_t ldb, const void* C, void* D,
                  int64_t ldc, int dtypeD, double alpha, double beta, float scaleA, float scaleB,
                  void* workspace, int64_t workspace_bytes, void* stream) {
  return dense_impl(dtypeA, dtypeB, layoutA, layoutB, M, N, K, A, lda, B, ldb, C, D, ldc, dtypeD, alpha, beta,
                    scaleA, scaleB, workspace, workspace_bytes, stream);
}

int mcg_validate_sparse24(int dtypeA, int dtypeB, int layoutB, int64_t M, int64_t N, int64_t K,
                          const void* A_compressed, int64_t lda_c, const uint32_t* A_index,
                          int64_t ld_idx, const void* B, int64_t ldb, const void* C, const void* D,
                          int64_t ldc, int dtypeD, double alpha, double beta) {
  const bool fp8 = (dtypeA == MCG_FP8_E4M3 || dtypeA == MCG_FP8_E5M2) &&
                   (dtypeB == MCG_FP8_E4M3 || dtypeB == MCG_FP8_E5M2);
  const bool i8 = dtypeA == MCG_I8 && dtypeB == MCG_I8;
  if (!((dtypeA == MCG_BF16 && dtypeB == MCG_BF16) || (dtypeA == MCG_F16 && dtypeB == MCG_F16) || fp8 || i8))
    return MCG_ERR_UNSUPPORTED_DTYPE;
  if ((i8 ? dtypeD != MCG_I32 : !float_out(dtypeD)) || !valid_layout(layoutB)) return MCG_ERR_UNSUPPORTED_DTYPE;
  if (M < 0 || N < 0 || K < 0 || K % 4 != 0) return MCG_ERR_INVALID_SIZE;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return MCG_ERR_INVALID_SIZE;
  if (M == 0 || N == 0) return MCG_SUCCESS;
  if (!D) return MCG_ERR_NULL_POINTER;
  if (K > 0 && (!A_compressed || !A_index || !B)) return MCG_ERR_NULL_POINTER;
  if (beta != 0.0 && !C) return MCG_ERR_NULL_POINTER;
  const int64_t min_ldb = layoutB == MCG_K_CONTIG ? K : N;
  if (lda_c < (K / 2 > 1 ? K / 2 : 1) || ld_idx < ((K + 31) / 32 > 1 ? (K + 31) / 32 : 1) ||
      ldb < (min_ldb > 1 ? min_ldb : 1) || ldc < N)
    return MCG_ERR_INVALID_LD;
  const int ebd = elem_bytes(dtypeD), eb = elem_bytes(dtypeA);
  if (!aligned_to(A_compressed, eb) || !aligned_to(B, eb) || !aligned_to(A_index, 4) ||
      !aligned_to(D, ebd) || (C && !aligned_to(C, ebd)))
    return MCG_ERR_MISALIGNED;
  if (i8) {
    if (!int32_integral(alpha) || !int32_integral(beta)) return MCG_ERR_INVALID_VALUE;
  } else if (!finite_as_f32(alpha) || !finite_as_f32(beta)) {
    return MCG_ERR_INVALID_VALUE;  // non-finite, or beyond fp32's range
  }
  return MCG_SUCCESS;
}

// gemm_sparse24 and gemm_sparse24_ws: ws (ws_bytes) is the caller's workspace, or null.
static int sparse_impl(int dtypeA, int dtypeB, int layoutB, int64_t M, int64_t N, int64_t K,
                       const void* A_compressed, int64_t lda_c, const uint32_t* A_index, int64_t ld_idx,
                       const void* B, int64_t ldb, const void* C, void* D, int64_t ldc, int dtypeD,
                       double alpha, double beta, void* ws, int64_t ws_bytes, void* stream) {
  int st = mcg_validate_sparse24(dtypeA, dtypeB, layoutB, M, N, K, A_compressed, lda_c, A_index,
                                 ld_idx, B, ldb, C, D, ldc, dtypeD, alpha, beta);
  if (st != MCG_SUCCESS) return st;
  if (ws != nullptr && (ws_bytes < 0 || !aligned_to(ws, 16))) return ws_bytes < 0 ? MCG_ERR_INVALID_SIZE : MCG_ERR_MISALIGNED;
  if (M == 0 || N == 0) return st;
  st = check_arch();
  if (st != MCG_SUCCESS) return st;
  mcg::SparseArgs a{};
  a.Ac = (const char*)A_compressed;
  a.idx = A_index;
  a.B = (const char*)B;
  a.C = C;
  a.D = D;
  a.M = M;
  a.N = N;
  a.K = K;
  a.lda_c = lda_c;
  a.ld_idx = ld_idx;
  a.ldb = ldb;
  a.ldc = ldc;
  a.alpha = (float)alpha;
  a.beta = (float)beta;
  a.alpha_i = dtypeA == MCG_I8 ? (int)alpha : 0;
  a.beta_i = dtypeA == MCG_I8 ? (int)beta : 0;
  a.use_c = beta != 0.0;
  a.out = out_format(dtypeD);
  const int vb = 4 * elem_bytes(dtypeD);
  a.vec_cd = aligned_to(D, vb) && (!a.use_c || aligned_to(C, vb)) && ldc % 4 == 0;
  const int eb = elem_bytes(dtypeA);
  const bool aligned = K == 0 || (aligned_to(A_compressed, 16) && aligned_to(B, 16) &&
                                  aligned_to(A_index, 16) && (lda_c * eb) % 16 == 0 &&
                                  (ldb * eb) % 16 == 0 && (ld_idx * 4) % 16 == 0);
  if (mcg::sparse_fast_ok(dtypeA, layoutB, a)) {
    if (ws != nullptr) {
      const int64_t need = mcg::plan_sparse_streamk(dtypeA, a, current_num_cu());
      if (need > 0 && need <= ws_bytes) {
        a.ws = ws;
        return hip_status(mcg::launch_sparse_fast_sk(dtypeA, dtypeB, layoutB, a, (hipStream_t)stream));
      }
      a.dp_tiles = a.sk_tiles = a.sk_wgs = 0;
    }
    return hip_status(mcg::launch_sparse_fast(dtypeA, dtypeB, layoutB, a, (hipStream_t)stream));
  }
  return hip_status(mcg::launch_sparse(dtypeA, dtypeB, layoutB, aligned, a, (hipStream_t)stream));
}

int gemm_sparse24(int dtypeA, int dtypeB, int layoutB, int64_t M, int64_t N, int64_t K,
                  const void* A_compressed, int64_t lda_c, const uint32_t* A_index, int64_t ld_idx,
                  const void* B, int64_t ldb, const void* C, void* D, int64_t ldc, int dtypeD,
                  double alpha, double beta, void* stream) {
  return sparse_impl(dtypeA, dtypeB, layoutB, M, N, K, A_compressed, lda_c, A_index, ld_idx, B, ldb, C, D, ldc,
                     dtypeD, alpha, beta, nullptr, 0, stream);
}

int gemm_sparse24_ws(int dtypeA, int dtypeB, int layoutB, int64_t M, int64_t N, int64_t K,
                     const void* A_compressed, int64_t lda_c, const uint32_t* A_index, int64_t ld_idx,
                     const void* B, int64_t ldb, const void* C, void* D, int64_t ldc, int dtypeD,
                     double alpha, double beta, void* workspace, int64_t workspace_bytes, void* stream) {
  return sparse_impl(dtypeA, dtypeB, layoutB, M, N, K, A_compressed, lda_c, A_index, ld_idx, B, ldb, C, D, ldc,
                     dtypeD, alpha, beta, workspace, workspace_bytes, stream);
}

int mcg_validate_compress24(int dtype, int64_t M, int64_t K, const void* A, int64_t lda,
                            const void* A_compressed, int64_t lda_c, const uint32_t* A_index,
                            int64_t ld_idx) {
  if (!is_in_dtype(dtype)) return MCG_ERR_UNSUPPORTED_DTYPE;
  if (M < 0 || K < 0 || K % 4 != 0) return MCG_ERR_INVALID_SIZE;
  if (M == 0 || K == 0) return MCG_SUCCESS;
  if (!A || !A_compressed || !A_index) return MCG_ERR_NULL_POINTER;
  if (lda < K || lda_c < K / 2 || ld_idx < (K + 31) / 32) return MCG_ERR_INVALID_LD;
  const int eb = elem_bytes(dtype);
  if (!aligned_to(A, eb) || !aligned_to(A_compressed, eb) || !aligned_to(A_index, 4))
    return MCG_ERR_MISALIGNED;
  return MCG_SUCCESS;
}

int compress24(int dtype, int64_t M, int64_t K, const void* A, int64_t lda, void* A_compressed,
               int64_t lda_c, uint32_t* A_index, int64_t ld_idx, int32_t* d_violations,
               void* stream) {
  int st = mcg_validate_compress24(dtype, M, K, A, lda, A_compressed, lda_c, A_index, ld_idx);
  if (st != MCG_SUCCESS) return st;
  if (d_violations && !aligned_to(d_violations, 4)) return MCG_ERR_MISALIGNED;
  if ((M == 0 || K == 0) && !d_violations) return MCG_SUCCESS;
  st = check_arch();
  if (st != MCG_SUCCESS) return st;
  mcg::CompressArgs a{};
  a.A = (const char*)A;
  a.Ac = (char*)A_compressed;
  a.idx = A_index;
  a.violations = d_violations;
  a.M = M;
  a.K = K;
  a.lda = lda;
  a.lda_c = lda_c;
  a.ld_idx = ld_idx;
  return hip_status(mcg::launch_compress(dtype, a, (hipStream_t)stream));
}

int compress24_host(int dtype, int64_t M, int64_t K, const void* A, int64_t lda, void* A_compressed,
                    int64_t lda_c, uint32_t* A_index, int64_t ld_idx) {
  int st = mcg_validate_compress24(dtype, M, K, A, lda, A_compressed, lda_c, A_index, ld_idx);
  if (st != MCG_SUCCESS) return st;
  const int eb = elem_bytes(dtype);
  const int64_t ngroups = K / 4, nwords = (K + 31) / 32;
  int64_t bad = 0;
  for (int64_t i = 0; i < M; ++i) {
    const unsigned char* row = (const unsigned char*)A + i * lda * eb;
    unsigned char* out = (unsigned char*)A_compressed + i * lda_c * eb;
    for (int64_t w = 0; w < nwords; ++w) {
      uint32_t word = 0;
      for (int gi = 0; gi < 8 && w * 8 + gi < ngroups; ++gi) {
        const int64_t g = w * 8 + gi;
        int sel[4], nz = 0;
        for (int e = 0; e < 4; ++e) {
          uint32_t v = 0;
          std::memcpy(&v, row + (4 * g + e) * eb, eb);
          const bool isnz = dtype == MCG_I8 ? v != 0 : (eb == 2 ? (v & 0x7fffu) != 0 : (v & 0x7fu) != 0);
          if (isnz && nz < 4) sel[nz] = e;
          nz += isnz;
        }
        int p0 = 0, p1 = 1;
        if (nz > 2) {
          ++bad;
          std::memset(out + 2 * g * eb, 0, 2 * eb);
        } else {
          if (nz == 2) { p0 = sel[0]; p1 = sel[1]; }
          else if (nz == 1 && sel[0] != 0) { p0 = 0; p1 = sel[0]; }
          std::memcpy(out + 2 * g * eb, row + (4 * g + p0) * eb, eb);
          std::memcpy(out + (2 * g + 1) * eb, row + (4 * g + p1) * eb, eb);
        }
        word |= (uint32_t)(p0 | (p1 << 2)) << (4 * gi);
      }
      A_index[i * ld_idx + w] = word;
    }
  }
  return bad ? MCG_ERR_NOT_2_4_SPARSE : MCG_SUCCESS;
}

int decompress24_host(int dtype, int64_t M, int64_t K, const void* A_compressed, int64_t lda_c,
                      const uint32_t* A_index, int64_t ld_idx, void* A, int64_t lda) {
  int st = mcg_validate_compress24(dtype, M, K, A, lda, A_compressed, lda_c, A_index, ld_idx);
  if (st != MCG_SUCCESS) return st;
  const int eb = elem_bytes(dtype);
  const int64_t ngroups = K / 4;
  auto code = [&](int64_t i, int64_t g) { return (A_index[i * ld_idx + g / 8] >> (4 * (g % 8))) & 0xfu; };
  // every used code must name two ascending positions; nothing is written otherwise
  for (int64_t i = 0; i < M; ++i)
    for (int64_t g = 0; g < ngroups; ++g)
      if ((code(i, g) & 3u) >= (code(i, g) >> 2)) return MCG_ERR_INVALID_INDEX;
  for (int64_t i = 0; i < M; ++i) {
    const unsigned char* in = (const unsigned char*)A_compressed + i * lda_c * eb;
    unsigned char* row = (unsigned char*)A + i * lda * eb;
    for (int64_t g = 0; g < ngroups; ++g) {
      const uint32_t c = code(i, g);
      std::memset(row + 4 * g * eb, 0, 4 * eb);
      std::memcpy(row + (4 * g + (c & 3u)) * eb, in + 2 * g * eb, eb);
      std::memcpy(row + (4 * g + (c >> 2)) * eb, in + (2 * g + 1) * eb, eb);
    }
  }
  return MCG_SUCCESS;
}

static mcg::DensePlan dense_plan(int dtypeA, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
                                 const void* A, int64_t lda, const void* B, int64_t ldb, bool can_split) {
  const int eb = elem_bytes(dtypeA);
  mcg::DenseArgs a{};
  a.A = (const char*)A;
  a.B = (const char*)B;
  a.M = M;
  a.N = N;
  a.K = K;
  a.lda = lda;
  a.ldb = ldb;
  return mcg::plan_dense(dtypeA, layoutA, layoutB, a, dense_aligned(eb, K, A, lda, B, ldb), can_split,
                         current_num_cu());
}

int mcg_dense_path(int dtypeA, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K, const void* A,
                   int64_t lda, const void* B, int64_t ldb) {
  if (dtypeA == MCG_F64) return mcg::KERNEL_F64;
  if (dtypeA < MCG_BF16 || dtypeA > MCG_FP8_E5M2) return 0;
  return dense_plan(dtypeA, layoutA, layoutB, M, N, K, A, lda, B, ldb, true).kernel;
}

int gemm_dense_noalloc(int dtypeA, int dtypeB, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t lda, const void* B, int64_t ldb, const void* C, void* D,
                       int64_t ldc, int dtypeD, double alpha, double beta, float scaleA, float scaleB,
                       void* stream) {
  return dense_impl(dtypeA, dtypeB, layoutA, layoutB, M, N, K, A, lda, B, ldb, C, D, ldc, dtypeD, alpha, beta,
                    scaleA, scaleB, nullptr, 0, stream, true);
}

int64_t mcg_dense_noalloc_scratch_bytes(void) { return mcg::STATIC_SCRATCH_BYTES; }

int64_t mcg_dense_workspace_bytes(int dtypeA, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
                                  const void* A, int64_t lda, const void* B, int64_t ldb) {
  if (dtypeA < MCG_BF16 || dtypeA > MCG_FP8_E5M2 || M <= 0 || N <= 0 || K <= 0) return 0;
  const int kernel = dense_plan(dtypeA, layoutA, layoutB, M, N, K, A, lda, B, ldb, true).kernel;
  if (kernel != mcg::KERNEL_FAST && kernel != mcg::KERNEL_MID && kernel != mcg::KERNEL_GENERAL) return 0;
  mcg::DenseArgs a{};
  a.A = (const char*)A;
  a.B = (const char*)B;
  a.M = M;
  a.N = N;
  a.K = K;
  a.lda = lda;
  a.ldb = ldb;
  int tile = 0;
  return dense_streamk(dtypeA, layoutA, layoutB, a, dense_aligned(elem_bytes(dtypeA), K, A, lda, B, ldb), kernel,
                       INT64_MAX, &tile);
}

int mcg_dense_splits(int dtypeA, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K, const void* A,
                     int64_t lda, const void* B, int64_t ldb, const void* C, const void* D, int dtypeD,
                     double beta) {
  if (dtypeA == MCG_F64) {
    const mcg::F64Args a = f64_args(M, N, K, A, lda, B, ldb, C, (void*)D, N, 1.0, beta);
    return mcg::plan_f64(a, dtypeD == MCG_F64 && !(beta != 0.0 && C == D), current_num_cu()).splits;
  }
  if (dtypeA < MCG_BF16 || dtypeA > MCG_FP8_E5M2) return 1;
  const bool can_split = (dtypeD == MCG_F32 || dtypeD == MCG_I32) && !(beta != 0.0 && C == D);
  return dense_plan(dtypeA, layoutA, layoutB, M, N, K, A, lda, B, ldb, can_split).splits;
}

int64_t mcg_sparse24_workspace_bytes(int dtypeA, int layoutB, int64_t M, int64_t N, int64_t K,
                                     const void* A_compressed, int64_t lda_c, const uint32_t* A_index,
                                     int64_t ld_idx, const void* B, int64_t ldb) {
  if (dtypeA < MCG_BF16 || dtypeA > MCG_FP8_E5M2 || M <= 0 || N <= 0 || K <= 0) return 0;
  if (mcg_sparse24_path(dtypeA, layoutB, M, N, K, A_compressed, lda_c, A_index, ld_idx, B, ldb) != 1) return 0;
  mcg::SparseArgs a{};
  a.M = M;
  a.N = N;
  a.K = K;
  return mcg::plan_sparse_streamk(dtypeA, a, current_num_cu());
}

int mcg_sparse24_path(int dtypeA, int layoutB, int64_t M, int64_t N, int64_t K, const void* A_compressed,
                      int64_t lda_c, const uint32_t* A_index, int64_t ld_idx, const void* B, int64_t ldb) {
  if (dtypeA < MCG_BF16 || dtypeA > MCG_FP8_E5M2) return 0;
  mcg::SparseArgs a{};
  a.Ac = (const char*)A_compressed;
  a.idx = A_index;
  a.B = (const char*)B;
  a.M = M;
  a.N = N;
  a.K = K;
  a.lda_c = lda_c;
  a.ld_idx = ld_idx;
  a.ldb = ldb;
  return mcg::sparse_fast_ok(dtypeA, layoutB, a) ? 1 : 0;
}

const char* mcg_status_string(int status) {
  switch (status) {
    case MCG_SUCCESS: return "success";
    case MCG_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MCG_ERR_INVALID_SIZE: return "invalid size";
    case MCG_ERR_INVALID_LD: return "leading dimension below its minimum";
    case MCG_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype or layout combination";
    case MCG_ERR_MISALIGNED: return "pointer not aligned to its element size";
    case MCG_ERR_NOT_2_4_SPARSE: return "a group of four holds more than two non-zeros";
    case MCG_ERR_INVALID_INDEX: return "malformed 2:4 index";
    case MCG_ERR_UNSUPPORTED_ARCH: return "current device is not gfx950";
    case MCG_ERR_HIP: return "HIP runtime error";
    case MCG_ERR_INVALID_VALUE: return "alpha, beta or scale not usable for this dtype";
    case MCG_ERR_SCRATCH_LIMIT: return "the stream-K plan needs more than the library's static scratch";
    default: return "unknown status";
  }
}

int mcg_mfma_eval_k(int dtype, int shape) { return mcg::mfma_eval_k(dtype == MCG_F64 ? mcg::DT_F64 : dtype, shape); }

int mcg_mfma_eval(int dtype, int shape, int64_t n, const void* a, const void* b, const void* c, void* d,
                  void* stream) {
  const int k = mcg::mfma_eval_k(dtype == MCG_F64 ? mcg::DT_F64 : dtype, shape);
  if (k == 0) return MCG_ERR_UNSUPPORTED_DTYPE;
  if (n < 0 || n > ((int64_t)1 << 31)) return MCG_ERR_INVALID_SIZE;
  if (n == 0) return MCG_SUCCESS;
  if (!a || !b || !c || !d) return MCG_ERR_NULL_POINTER;
  const int acc_bytes = dtype == MCG_F64 ? 8 : 4;
  if (!aligned_to(a, elem_bytes(dtype)) || !aligned_to(b, elem_bytes(dtype)) || !aligned_to(c, acc_bytes) ||
      !aligned_to(d, acc_bytes))
    return MCG_ERR_MISALIGNED;
  int st = check_arch();
  if (st != MCG_SUCCESS) return st;
  return hip_status(
      mcg::launch_mfma_eval(dtype == MCG_F64 ? mcg::DT_F64 : dtype, shape, a, b, c, d, n, (hipStream_t)stream));
}

int mcg_mfma_probe(int dtypeA, int dtypeB, int sparse, const void* a, const void* b, const void* idx,
                   int64_t instr_per_wave, int num_wg, float* sink, int64_t* clocks, void* stream) {
  if (dtypeA < 0 || dtypeA > MCG_FP8_E5M2 || dtypeB < 0 || dtypeB > MCG_FP8_E5M2 ||
      !mcg::mfma_probe_supported(dtypeA, dtypeB, sparse))
    return MCG_ERR_UNSUPPORTED_DTYPE;
  if (instr_per_wave <= 0 || instr_per_wave % 16 != 0 || instr_per_wave > ((int64_t)1 << 24) || num_wg <= 0 ||
      num_wg > 65536)
    return MCG_ERR_INVALID_SIZE;
  if (!a || !b || !sink || !clocks || (sparse && !idx)) return MCG_ERR_NULL_POINTER;
  if (!aligned_to(a, 16) || !aligned_to(b, 16) || (sparse && !aligned_to(idx, 16)) || !aligned_to(sink, 4) ||
      !aligned_to(clocks, 8))
    return MCG_ERR_MISALIGNED;
  int st = check_arch();
  if (st != MCG_SUCCESS) return st;
  return hip_status(mcg::launch_mfma_probe(dtypeA, dtypeB, sparse, a, b, sparse ? idx : nullptr, instr_per_wave,
                                           num_wg, sink, clocks, (hipStream_t)stream));
}

int mcg_version(void) { return kVersion; }

}  // extern "C"
