// sparse_ops.hpp -- the gfx950 2:4 sparse matrix instructions as operation types
// (kept values of A, dense B, one index register), shared by the 256 x 256 2:4
// kernel and the matrix-core rate probe.  Instruction semantics: "RDNA4 sparse
// WMMA builtins", Structured sparsity (2:4 pattern) and Common parameters;
// the operand layouts are measured ones (see gemm_sparse_fast.hip).
#pragma once
#include "fast_tiles.hpp"

namespace mcg {
namespace fast {

struct Sp32BF16 {
  static constexpr int EB = 2;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x16;
  __device__ static __forceinline__ void mma(acc_t& c, const i32x4& a, const i32x8& b, int idx) {
    c = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(bit_cast<bf16x8>(a), bit_cast<bf16x16>(b), c, idx, 0, 0);
  }
};
struct Sp32F16 {
  static constexpr int EB = 2;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x16;
  __device__ static __forceinline__ void mma(acc_t& c, const i32x4& a, const i32x8& b, int idx) {
    c = __builtin_amdgcn_smfmac_f32_32x32x32_f16(bit_cast<f16x8>(a), bit_cast<f16x16>(b), c, idx, 0, 0);
  }
};
struct Sp32I8 {
  static constexpr int EB = 1;
  static constexpr bool INT_ACC = true;
  using acc_t = i32x16;
  __device__ static __forceinline__ void mma(acc_t& c, const i32x4& a, const i32x8& b, int idx) {
    c = __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c, idx, 0, 0);
  }
};
// native fp8: FA / FB = formats of A / B (0 E4M3, 1 E5M2)
template <int FA, int FB>
struct Sp32F8 {
  static constexpr int EB = 1;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x16;
  __device__ static __forceinline__ void mma(acc_t& c, const i32x4& a, const i32x8& b, int idx) {
    if constexpr (FA == 0 && FB == 0) c = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a, b, c, idx, 0, 0);
    else if constexpr (FA == 0 && FB == 1) c = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_bf8(a, b, c, idx, 0, 0);
    else if constexpr (FA == 1 && FB == 0) c = __builtin_amdgcn_smfmac_f32_32x32x64_bf8_fp8(a, b, c, idx, 0, 0);
    else c = __builtin_amdgcn_smfmac_f32_32x32x64_bf8_bf8(a, b, c, idx, 0, 0);
  }
};

}  // namespace fast
}  // namespace mcg
