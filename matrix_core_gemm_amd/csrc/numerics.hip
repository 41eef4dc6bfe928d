// numerics.hip -- one matrix-core instruction per test vector, for numerical
// characterisation of gfx950 MFMA.
//
// "Accurate Models of AMD Matrix Cores" (Section 2, Eq. (1); Section 3)
// characterises a matrix core by the single output element
//     d = sum_{l=1..k} a_l b_l + c
// of one instruction, fed with targeted and with randomised test vectors.
// mcg_mfma_eval runs exactly that on gfx950 (and on the FP64 instructions, "CDNA3
// dense MFMA builtins", FP64-accumulate builtins): test vector t places a[t*k ..]
// in row 0 of the instruction's A operand, b[t*k ..] in column 0 of its B
// operand and c[t] in element (0, 0) of its accumulator input (everything
// else zero) and returns element (0, 0) of the result.  Element l of a test
// vector goes to operand slot l, slots numbered in register order: lane group
// g (lane / 16 for the 16x16 shapes, lane / 32 for 32x32) holds slots
// [g * E, (g + 1) * E) in the order of its register bytes, E being the
// elements one lane holds (8 for bf16/f16, 32 for fp8).  The GEMM kernels
// feed K to these slots in their own (consistent) order.
// One wavefront per test vector.
#include "arch_gfx950.hpp"
#include "gemm_kernels.hpp"

namespace mcg {
namespace numerics {

// KIND: 0 bf16, 1 f16, 2 fp8 E4M3, 3 fp8 E5M2; SHAPE: 16 or 32
template <int KIND, int SHAPE>
struct Instr {
  static constexpr bool F8 = KIND >= 2;
  static constexpr int K = F8 ? (SHAPE == 16 ? 128 : 64) : (SHAPE == 16 ? 32 : 16);
  static constexpr int EB = F8 ? 1 : 2;
  static constexpr int ROWS = SHAPE;
  // slot of byte j (0 <= j < lane bytes) of lane group g's fragment
  __device__ static __forceinline__ int kpos(int g, int j) {
    if constexpr (!F8) return 8 * g + j / 2;
    else return 32 * g + j;
  }
  static constexpr int LANE_BYTES = F8 ? 32 : 16;
};

template <int KIND, int SHAPE>
__global__ __launch_bounds__(256) void mfma_eval_kernel(const unsigned char* a, const unsigned char* b,
                                                        const float* c, float* d, int64_t n) {
  using I = Instr<KIND, SHAPE>;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;  // whole wavefronts leave together
  const int g = lane / I::ROWS;
  const bool first = (lane % I::ROWS) == 0;  // row 0 of A / column 0 of B
  unsigned char fa[32] = {}, fb[32] = {};
  if (first) {
    for (int j = 0; j < I::LANE_BYTES; ++j) {
      const int k = I::kpos(g, j);
      const int byte = I::F8 ? 0 : (j & 1);
      fa[j] = a[(t * I::K + k) * I::EB + byte];
      fb[j] = b[(t * I::K + k) * I::EB + byte];
    }
  }
  float out;
  if constexpr (SHAPE == 16) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (lane == 0) acc[0] = c[t];
    if constexpr (!I::F8) {
      i32x4 pa, pb;
      __builtin_memcpy(&pa, fa, 16);
      __builtin_memcpy(&pb, fb, 16);
      if constexpr (KIND == 0)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bit_cast<bf16x8>(pa), bit_cast<bf16x8>(pb), acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bit_cast<f16x8>(pa), bit_cast<f16x8>(pb), acc, 0, 0, 0);
    } else {
      i32x8 pa, pb;
      __builtin_memcpy(&pa, fa, 32);
      __builtin_memcpy(&pb, fb, 32);
      constexpr int F = KIND == 2 ? 0 : 1;
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pa, pb, acc, F, F, 0, 0, 0, 0);
    }
    out = acc[0];
  } else {
    typedef float f32x16_t __attribute__((ext_vector_type(16)));
    f32x16_t acc = {};
    if (lane == 0) acc[0] = c[t];
    if constexpr (!I::F8) {
      i32x4 pa, pb;
      __builtin_memcpy(&pa, fa, 16);
      __builtin_memcpy(&pb, fb, 16);
      if constexpr (KIND == 0)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bit_cast<bf16x8>(pa), bit_cast<bf16x8>(pb), acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(bit_cast<f16x8>(pa), bit_cast<f16x8>(pb), acc, 0, 0, 0);
    } else {
      i32x8 pa, pb;
      __builtin_memcpy(&pa, fa, 32);
      __builtin_memcpy(&pb, fb, 32);
      constexpr int F = KIND == 2 ? 0 : 1;
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, pb, acc, F, F, 0, 0, 0, 0);
    }
    out = acc[0];
  }
  if (lane == 0) d[t] = out;
}

// Binary64: SHAPE 16 is v_mfma_f64_16x16x4_f64, SHAPE 4 block 0 of v_mfma_f64_4x4x4_4b_f64.
// Row 0 of A (block 0) and column 0 of B sit in lanes 16k (K index k = 0..3) for both, and
// result element (0, 0) in lane 0, register 0.
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_eval_f64_kernel(const double* a, const double* b, const double* c,
                                                            double* d, int64_t n) {
  typedef double f64x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;  // whole wavefronts leave together
  double av = 0.0, bv = 0.0;
  if ((lane & 15) == 0) {
    av = a[t * 4 + (lane >> 4)];
    bv = b[t * 4 + (lane >> 4)];
  }
  double out;
  if constexpr (SHAPE == 16) {
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
    if (lane == 0) acc[0] = c[t];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
    out = acc[0];
  } else {
    double acc = lane == 0 ? c[t] : 0.0;
    out = __builtin_amdgcn_mfma_f64_4x4x4f64(av, bv, acc, 0, 0, 0);
  }
  if (lane == 0) d[t] = out;
}

template <int KIND>
static hipError_t launch_kind(int shape, const void* a, const void* b, const float* c, float* d, int64_t n,
                              hipStream_t s) {
  const int64_t blocks = (n + 3) / 4;
  if (shape == 16)
    hipLaunchKernelGGL((mfma_eval_kernel<KIND, 16>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const unsigned char*)a, (const unsigned char*)b, c, d, n);
  else
    hipLaunchKernelGGL((mfma_eval_kernel<KIND, 32>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const unsigned char*)a, (const unsigned char*)b, c, d, n);
  return hipGetLastError();
}

}  // namespace numerics

int mfma_eval_k(int dt, int shape) {
  if (dt == DT_F64) return shape == 16 || shape == 4 ? 4 : 0;
  const bool f8 = dt == DT_E4M3 || dt == DT_E5M2;
  if ((dt < DT_BF16 || dt > DT_E5M2) || dt == DT_I8 || (shape != 16 && shape != 32)) return 0;
  return f8 ? (shape == 16 ? 128 : 64) : (shape == 16 ? 32 : 16);
}

hipError_t launch_mfma_eval(int dt, int shape, const void* a, const void* b, const void* c, void* d,
                            int64_t n, hipStream_t s) {
  using namespace numerics;
  if (n <= 0) return hipSuccess;
  if (dt == DT_F64) {
    const dim3 grid((unsigned)((n + 3) / 4));
    if (shape == 16)
      hipLaunchKernelGGL(mfma_eval_f64_kernel<16>, grid, dim3(256), 0, s, (const double*)a, (const double*)b,
                         (const double*)c, (double*)d, n);
    else
      hipLaunchKernelGGL(mfma_eval_f64_kernel<4>, grid, dim3(256), 0, s, (const double*)a, (const double*)b,
                         (const double*)c, (double*)d, n);
    return hipGetLastError();
  }
  const float* cf = (const float*)c;
  float* df = (float*)d;
  if (dt == DT_BF16) return launch_kind<0>(shape, a, b, cf, df, n, s);
  if (dt == DT_F16) return launch_kind<1>(shape, a, b, cf, df, n, s);
  if (dt == DT_E4M3) return launch_kind<2>(shape, a, b, cf, df, n, s);
  return launch_kind<3>(shape, a, b, cf, df, n, s);
}

}  // namespace mcg
