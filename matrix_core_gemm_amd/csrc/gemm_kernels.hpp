// gemm_kernels.hpp -- kernel argument blocks and launchers shared by the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcg {
// Format of C and D: binary32 (int32 for int8 inputs), bfloat16 or binary16.
enum : int { OUT_32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

struct DenseArgs {
  const char* A;
  const char* B;
  const void* C;
  void* D;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;  // elements
  float alpha, beta;      // float paths: alpha already includes scaleA*scaleB
  int alpha_i, beta_i;    // int8 path
  int use_c;              // beta != 0: C is read
  int vec_cd;             // 4 consecutive C/D elements can be moved as one vector (aligned, ldc % 4 == 0)
  int out;                // OUT_32 (binary32 / int32), OUT_BF16 or OUT_F16: format of C and D
  int splits;             // K ranges multiplied by separate workgroups (1: no split)
  int kt_per_split;       // K tiles per range
  int stream_bw;          // streaming kernel: rows of the wide operand per workgroup
  int tiles_m, tiles_n;   // filled by the launcher
  // stream-K form of the 256 x 256 kernel (sk_tiles > 0): the first dp_tiles
  // tiles of the grouped tile order are whole-tile workgroups; the K iterations
  // of the last sk_tiles tiles are cut into consecutive ranges of sk_iters over
  // sk_wgs workgroups.  Pieces of a tile that are not the whole tile leave their
  // partial sums in ws (one 256 x 256 binary32 / int32 slot per piece), which a
  // second kernel adds up in piece order before the epilogue.  sk_period: the
  // number of ranges after which a range boundary meets a tile boundary again.
  int dp_tiles, sk_tiles, sk_wgs;
  int64_t sk_iters, sk_period;
  void* ws;
};

// Kernel chosen for a dense problem (also reported by mcg_dense_path).
enum : int {
  KERNEL_GENERAL = 0,   // 128 x 128 tiles, 4 waves, register-staged LDS double buffer
  KERNEL_FAST = 1,      // 256 x 256 tiles, 8 waves, LDS-DMA ring (large problems)
  KERNEL_SKINNY_N = 2,  // general kernel with 128 x 32 tiles (N <= 32)
  KERNEL_SKINNY_M = 3,  // general kernel with 32 x 128 tiles (M <= 32)
  KERNEL_STREAM = 4,    // streaming kernel for N <= 32 or M <= 32 (K-contiguous, aligned)
  KERNEL_F64 = 5,       // binary64 kernel (128 x 128 tiles on the 16x16x4 FP64 instruction)
  KERNEL_MID = 6        // the KERNEL_FAST design with 128 x 128 tiles (too few 256 x 256 tiles)
};

struct DensePlan {
  int kernel;
  int splits;        // >1: K split over grid.y, partial sums added into D
  int kt_per_split;  // K tiles of 128 bytes per split
  int stream_bw;     // KERNEL_STREAM: 32, 64 or 128 rows of the wide operand per workgroup
};

struct SparseArgs {
  const char* Ac;       // compressed values, M x K/2
  const uint32_t* idx;  // index words, M x ceil(K/32)
  const char* B;
  const void* C;
  void* D;
  int64_t M, N, K;               // dense K
  int64_t lda_c, ld_idx, ldb, ldc;
  float alpha, beta;    // float paths (fp8: alpha carries the dequantisation scales)
  int alpha_i, beta_i;  // int8 path
  int use_c, vec_cd;
  int out;  // OUT_32 (binary32 / int32), OUT_BF16 or OUT_F16: format of C and D
  int tiles_m, tiles_n;
  // stream-K form of the 256 x 256 sparse kernel, as in DenseArgs; pieces are
  // counted in kept-value stages (128 dense k of 16-bit, 256 of 8-bit values)
  int dp_tiles, sk_tiles, sk_wgs;
  int64_t sk_iters, sk_period;
  void* ws;
};

// binary64 GEMM (DGEMM); DT_F64 continues the input codes of arch_gfx950.hpp
constexpr int DT_F64 = 7;
struct F64Args {
  const double* A;
  const double* B;
  const double* C;
  double* D;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;  // elements
  double alpha, beta;
  int use_c;              // beta != 0: C is read
  int kt_per_split;       // K tiles of 16 per workgroup range (filled by the launcher)
  int dma_mode;           // HBM -> LDS DMA: 0 none, 1 16-byte, 2 4-byte (filled by the launcher)
  int tiles_m, tiles_n;   // filled by the launcher
};

struct F64Plan {
  int splits;        // >1: K split over grid.y, partial sums added into D with atomics
  int kt_per_split;  // K tiles of 16 per range
};

// Split-K cost model of the binary64 kernel (microseconds; gfx950, up to two resident
// 128 x 128 workgroups per CU; fitted on 256 CUs to forced-split timings from 1024^3 to
// 256 x 256 x 65536).
constexpr int64_t F64_SPLIT_MIN_KT = 16;  // at least 256 K values per range
constexpr double F64_KT_ALONE_US = 2.05;  // one K tile (16) of a workgroup alone on its CU
constexpr double F64_KT_SHARED_US = 3.4;  // the same with two workgroups sharing the CU
constexpr double F64_ATOMIC_US = 7e-6;    // per atomic add of a partial sum (overlaps compute)
constexpr double F64_SPLIT_US = 5.0;      // zeroing D and the extra launch

// can_split: D is not C with beta != 0; num_cu: the device's compute units.
F64Plan plan_f64(const F64Args& a, bool can_split, int num_cu);
hipError_t launch_f64(int layoutA, int layoutB, const F64Args& a, const F64Plan& plan, hipStream_t s);

struct CompressArgs {
  const char* A;
  char* Ac;
  uint32_t* idx;
  int32_t* violations;  // may be null
  int64_t M, K, lda, lda_c, ld_idx;
};

// fp8 inputs: the native f8f6f4 instruction sums each group of eight products
// keeping only about 13 bits below the group's largest product (measured on
// gfx950), then accumulates groups with about 24 bits.  Its worst-case error is
// then below 2^-10 * S + (K/8) * 2^-22 * S (S = sum |a b|), which is inside the
// accuracy bound 4 * 2^-24 * (K + 2) * S once 7K/8 >= 4096.  Below this K the
// fp8 operands are widened exactly to bf16 and multiplied on the bf16 path.
constexpr int64_t FP8_NATIVE_MIN_K = 6144;

// Kernel and K split for a dense problem.  can_split: D is binary32/int32 and
// is not C (split K zeroes D first and adds the partial sums into it);
// num_cu: the device's compute units.
DensePlan plan_dense(int dtA, int layoutA, int layoutB, const DenseArgs& a, bool aligned, bool can_split,
                     int num_cu);

// Enqueue the kernels; arguments were validated by the caller.
hipError_t launch_dense(int dtA, int dtB, int layoutA, int layoutB, bool aligned, const DenseArgs& a,
                        const DensePlan& plan, hipStream_t s);
// The general kernel with skinny tiles (aligned operands only), one per translation unit.
hipError_t launch_skinny_n(int dtA, int dtB, int layoutA, int layoutB, const DenseArgs& a, hipStream_t s);
hipError_t launch_skinny_m(int dtA, int dtB, int layoutA, int layoutB, const DenseArgs& a, hipStream_t s);
bool stream_path_ok(int dtA, int layoutA, int layoutB, const DenseArgs& a, bool aligned);
hipError_t launch_stream(int dtA, int dtB, int layoutA, int layoutB, const DenseArgs& a, hipStream_t s);
// tile: 256 (KERNEL_FAST) or 128 (KERNEL_MID)
bool fast_path_ok(int dtA, int layoutA, int layoutB, const DenseArgs& a, bool aligned, int tile = 256);
hipError_t launch_fast(int dtA, int dtB, int layoutA, int layoutB, const DenseArgs& a, hipStream_t s, int tile = 256);
hipError_t launch_fast_mid(int dtA, int dtB, int layoutA, int layoutB, const DenseArgs& a, hipStream_t s);
// Stream-K plan for a problem on the pipelined kernel with tile x tile tiles (256,
// or 128 for its mid-size form): fills the sk_* and dp_tiles fields of a and
// returns the workspace bytes it needs, or 0 (and sk_tiles = 0) when the plan
// would not be faster than whole tiles.
int64_t plan_streamk(int dtA, DenseArgs& a, int num_cu, int tile = 256);
hipError_t launch_fast_sk(int dtA, int dtB, int layoutA, int layoutB, const DenseArgs& a, hipStream_t s,
                          int tile = 256);
hipError_t launch_fast_mid_sk(int dtA, int dtB, int layoutA, int layoutB, const DenseArgs& a, hipStream_t s);
// The fixup of a stream-K launch with 256 x 256 slots: a carries the plan, the
// epilogue arguments and the workspace; nk counts the pieces' K units per tile.
hipError_t launch_streamk_fixup(const DenseArgs& a, int64_t nk, bool int_acc, hipStream_t s);
// Stream-K plan of the 256 x 256 sparse kernel (fills the sk_* and dp_tiles
// fields of a), and its launch; workspace bytes as plan_streamk.
int64_t plan_sparse_streamk(int dtA, SparseArgs& a, int num_cu);
hipError_t launch_sparse_fast_sk(int dtA, int dtB, int layoutB, const SparseArgs& a, hipStream_t s);
// The library's static stream-K scratch: STATIC_SCRATCH_BYTES per device; its
// device address for the current device (looked up on the first call there).
constexpr int64_t STATIC_SCRATCH_BYTES = (int64_t)32 << 20;
hipError_t static_scratch(void** ptr);
hipError_t launch_sparse(int dtA, int dtB, int layoutB, bool aligned, const SparseArgs& a, hipStream_t s);
bool sparse_fast_ok(int dtA, int layoutB, const SparseArgs& a);
hipError_t launch_sparse_fast(int dtA, int dtB, int layoutB, const SparseArgs& a, hipStream_t s);
hipError_t launch_compress(int dtype, const CompressArgs& a, hipStream_t s);
int mfma_eval_k(int dt, int shape);
hipError_t launch_mfma_eval(int dt, int shape, const void* a, const void* b, const void* c, void* d,
                            int64_t n, hipStream_t s);
// Matrix-core rate probe (mfma_probe.hip): the GEMM kernels' instructions on
// fragments loaded once from a, b (and idx for 2:4), instr_per_wave (a multiple
// of 16) per wavefront, num_wg workgroups of 512 threads.
bool mfma_probe_supported(int dtA, int dtB, int sparse);
hipError_t launch_mfma_probe(int dtA, int dtB, int sparse, const void* a, const void* b, const void* idx,
                             int64_t instr_per_wave, int num_wg, float* sink, int64_t* clocks, hipStream_t s);

}  // namespace mcg
