// arch_gfx950.hpp -- gfx950 (CDNA4) matrix-core instruction wrappers and fragment layouts.
//
// One MFMA instruction computes one K-step of a small output tile across the 64
// lanes of a wavefront ("CDNA3 dense MFMA builtins", Naming convention and
// Accumulator layout).  The pages document the CDNA3 (gfx942) layouts; the
// gfx950 layouts below were measured on an MI355X with one-hot operands and are
// re-checked end to end by the one-hot GEMM tests:
//
//  Dense 16x16xK (bf16/f16 K=32, i8 K=64, f8f6f4 K=128), wave64:
//    operand P (the instruction's "A"): lane l holds row (l & 15),
//    operand Q (the instruction's "B"): lane l holds column (l & 15),
//    and both hold the K run selected by lane group g = l >> 4; the K positions
//    of element e of lane group g are the same function for P and Q, so any
//    consistent K order of the two fragments gives the same product.
//    Output: lane l, register r holds out[4*(l >> 4) + r][l & 15]
//    (the single-block case of the 16x16 accumulator layout).
//
//  Sparse 16x16x64 (smfmac bf16/f16; 2:4 on P, dense K = 64):
//    P (compressed, 8 values per lane): lane l holds row (l & 15); lane group
//    g = l >> 4 covers dense K 16g..16g+15 as four groups of four; compressed
//    values 2n, 2n+1 belong to group n and sit at the positions given by the
//    4-bit code n of the index (p0 = code & 3, p1 = code >> 2).  The index
//    VGPR holds two 16-bit halves of four codes; the abid modifier selects
//    the half (0: bits 0..15).
//    Q (dense, 16 values per lane): lane l holds column (l & 15); elements
//    0..7 are dense K 8g..8g+7 and elements 8..15 are K 32+8g..32+8g+7.
//    Output: same as the dense 16x16 layout.
//
//  Transposing LDS reads (per 16-lane group; lane L supplies an 8-byte address):
//    ds_read_b64_tr_b16: output lane t, element e (0..3) = 16-bit element (t & 3)
//      of the 8 bytes addressed by lane 4e + (t >> 2).
//    ds_read_b64_tr_b8 : output lane t, element e (0..7) = byte (t & 7) of the
//      8 bytes addressed by lane 2e + (t >> 3).
//
// frag_layout.hpp holds these maps as functions, (lane, register) <-> (i, j,
// block), together with the 32x32 and FP64 layouts; every epilogue uses them.
//
// fp8 operands use the OCP encodings (measured: code 0x7E of E4M3 is 448); the
// f8f6f4 instruction takes the A/B formats in its cbsz/blgp fields
// (0 = E4M3, 1 = E5M2) and, with zero scale operands, computes plain products.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "frag_layout.hpp"
#include "gemm_kernels.hpp"

namespace mcg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <class T, class S>
__device__ __forceinline__ T bit_cast(const S& s) {
  static_assert(sizeof(T) == sizeof(S), "bit_cast size mismatch");
  T t;
  __builtin_memcpy(&t, &s, sizeof(T));
  return t;
}

// Element-type codes, identical in value to the public mcg_dtype enum.
enum : int { DT_BF16 = 0, DT_F16 = 1, DT_I8 = 2, DT_E4M3 = 3, DT_E5M2 = 4 };

// f8f6f4 format field values
__host__ __device__ constexpr int f8fmt(int dt) { return dt == DT_E5M2 ? 1 : 0; }

// ------------------------------------------------------------------ dense ops
// Every op multiplies a 16x16 output tile by one K-step.  STEPS is the number
// of K-steps in a 128-byte K tile.  mma(p, q, acc): acc += P.Q with P/Q in the
// layout described above.  frag_a / frag_b read the A (instruction Q) and B
// (instruction P) fragments of K-step s from LDS through a FragReader R.

struct DirectFrags {
  template <class R>
  __device__ static __forceinline__ typename R::frag_t frag_a(const __attribute__((address_space(3))) char* t,
                                                               int rb, int s, int lane) {
    return R::read(t, rb, s, lane);
  }
  template <class R>
  __device__ static __forceinline__ typename R::frag_t frag_b(const __attribute__((address_space(3))) char* t,
                                                               int rb, int s, int lane) {
    return R::read(t, rb, s, lane);
  }
};

struct OpBF16 : DirectFrags {
  static constexpr int ELEM_BYTES = 2, LANE_BYTES = 16, K_STEP = 32, STEPS = 2;
  static constexpr bool INT_ACC = false;
  using frag_t = i32x4;
  using acc_t = f32x4;
  __device__ static __forceinline__ acc_t mma(frag_t p, frag_t q, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bit_cast<bf16x8>(p), bit_cast<bf16x8>(q), c, 0, 0, 0);
  }
};

struct OpF16 : DirectFrags {
  static constexpr int ELEM_BYTES = 2, LANE_BYTES = 16, K_STEP = 32, STEPS = 2;
  static constexpr bool INT_ACC = false;
  using frag_t = i32x4;
  using acc_t = f32x4;
  __device__ static __forceinline__ acc_t mma(frag_t p, frag_t q, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bit_cast<f16x8>(p), bit_cast<f16x8>(q), c, 0, 0, 0);
  }
};

struct OpI8 : DirectFrags {
  static constexpr int ELEM_BYTES = 1, LANE_BYTES = 16, K_STEP = 64, STEPS = 2;
  static constexpr bool INT_ACC = true;
  using frag_t = i32x4;
  using acc_t = i32x4;
  __device__ static __forceinline__ acc_t mma(frag_t p, frag_t q, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(p, q, c, 0, 0, 0);
  }
};

// Native fp8: FP = format of operand P (the B tensor), FQ = format of Q (A tensor);
// 0 = E4M3, 1 = E5M2.
template <int FP, int FQ>
struct OpF8 : DirectFrags {
  static constexpr int ELEM_BYTES = 1, LANE_BYTES = 32, K_STEP = 128, STEPS = 1;
  static constexpr bool INT_ACC = false;
  using frag_t = i32x8;
  using acc_t = f32x4;
  __device__ static __forceinline__ acc_t mma(frag_t p, frag_t q, acc_t c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(p, q, c, FP, FQ, 0, 0, 0, 0);
  }
};

// Eight fp8 codes (two dwords) -> eight bf16 values, exactly: the hardware
// conversion to fp32 is exact for every finite fp8 value, and an fp32 that
// came from fp8 has at most 4 significant bits, so its upper 16 bits are the
// bf16 encoding of the same value.
template <int FMT>
__device__ __forceinline__ i32x4 fp8x8_to_bf16x8(i32x2 v) {
  i32x4 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 lo, hi;
    if constexpr (FMT == 0) {
      lo = __builtin_amdgcn_cvt_pk_f32_fp8(v[w], false);
      hi = __builtin_amdgcn_cvt_pk_f32_fp8(v[w], true);
    } else {
      lo = __builtin_amdgcn_cvt_pk_f32_bf8(v[w], false);
      hi = __builtin_amdgcn_cvt_pk_f32_bf8(v[w], true);
    }
    // select the upper halves: result = (hi16(y) << 16) | hi16(x)
    r[2 * w] = (int)__builtin_amdgcn_perm(bit_cast<uint32_t>(lo.y), bit_cast<uint32_t>(lo.x), 0x07060302u);
    r[2 * w + 1] = (int)__builtin_amdgcn_perm(bit_cast<uint32_t>(hi.y), bit_cast<uint32_t>(hi.x), 0x07060302u);
  }
  return r;
}

// Widened fp8: the fp8 tiles are staged in LDS as fp8, each lane reads eight
// consecutive K values per K-step, converts them exactly to bf16 and issues the
// bf16 instruction (full fp32-class accumulation).  FA/FB = formats of the A/B
// tensors.  K-step s of lane group g covers tile K bytes [32s + 8g, +8).
template <int FA, int FB>
struct OpF8W {
  static constexpr int ELEM_BYTES = 1, LANE_BYTES = 8, K_STEP = 32, STEPS = 4;
  static constexpr bool INT_ACC = false;
  using frag_t = i32x4;
  using acc_t = f32x4;
  template <class R>
  __device__ static __forceinline__ frag_t frag_a(const __attribute__((address_space(3))) char* t, int rb,
                                                  int s, int lane) {
    return fp8x8_to_bf16x8<FA>(R::run8(t, rb, 32 * s + 8 * (lane >> 4), lane));
  }
  template <class R>
  __device__ static __forceinline__ frag_t frag_b(const __attribute__((address_space(3))) char* t, int rb,
                                                  int s, int lane) {
    return fp8x8_to_bf16x8<FB>(R::run8(t, rb, 32 * s + 8 * (lane >> 4), lane));
  }
  __device__ static __forceinline__ acc_t mma(frag_t p, frag_t q, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bit_cast<bf16x8>(p), bit_cast<bf16x8>(q), c, 0, 0, 0);
  }
};


// ------------------------------------------------------------ LDS primitives
// ----------------------------------------------------- output conversions
// Output formats of the float epilogues (OUT_32, OUT_BF16, OUT_F16) are
// declared with the kernel argument blocks; C is read in the output format.

// binary32 -> bfloat16 bits, round to nearest, ties to even (adding 0x7fff plus
// the lowest kept bit carries exactly when the dropped half is above the
// midpoint, or at it with an odd kept part); overflow gives infinity; a NaN
// stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  const uint32_t u = bit_cast<uint32_t>(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// binary32 -> binary16 bits by the hardware conversion (round to nearest even,
// gradual underflow, overflow to infinity in the default mode).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  return bit_cast<uint16_t>((_Float16)x);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return bit_cast<float>(h << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)bit_cast<_Float16>((uint16_t)h);
}
__device__ __forceinline__ uint32_t to_out_bits(int out, float x) {
  return out == OUT_BF16 ? f32_to_bf16_bits(x) : f32_to_f16_bits(x);
}
__device__ __forceinline__ float from_out_bits(int out, uint32_t h) {
  return out == OUT_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
}

// D[off] = alpha * v + beta * C[off] (C read only when use_c), with C and D in
// the output format `out`; the fp32 result is rounded once to a 16-bit format.
__device__ __forceinline__ void combine_store(const void* C, void* D, int64_t off, float v, float alpha,
                                              float beta, bool use_c, int out) {
  if (out == OUT_32) {
    const float c = use_c ? ((const float*)C)[off] : 0.f;
    ((float*)D)[off] = use_c ? __builtin_fmaf(alpha, v, beta * c) : alpha * v;
  } else {
    const float c = use_c ? from_out_bits(out, ((const uint16_t*)C)[off]) : 0.f;
    ((uint16_t*)D)[off] = (uint16_t)to_out_bits(out, use_c ? __builtin_fmaf(alpha, v, beta * c) : alpha * v);
  }
}

// operand storage order along K: K-contiguous (A row-major, B column-major) or
// MN-contiguous (A column-major, B row-major)
enum : int { LAYOUT_K = 0, LAYOUT_MN = 1 };

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ i32x4 lds_read_b128(const lds_char* base, int off) {
  return *(const __attribute__((address_space(3))) i32x4*)(base + off);
}
__device__ __forceinline__ void lds_write_b128(lds_char* base, int off, i32x4 v) {
  *(__attribute__((address_space(3))) i32x4*)(base + off) = v;
}
__device__ __forceinline__ i32x2 lds_read_tr16(const lds_char* base, int off) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<lds_char*>(base) + off));
  return bit_cast<i32x2>(v);
}
__device__ __forceinline__ i32x2 lds_read_tr8(const lds_char* base, int off) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(const_cast<lds_char*>(base) + off));
}

// Transposing LDS reads in inline asm: four 8-byte reads per address a[n], at byte
// offsets 0, O1, O2, O3 from it, in one block that waits for all of them
// (lgkmcnt(0)) before it ends, so that no read is still in flight once the
// compiler owns the output registers.  The compiler precedes its own
// transposing-read builtins with a wait for all of the wavefront's outstanding
// buffer_load ... lds transfers (it cannot tell which LDS bytes those write),
// which drains a kernel's prefetch ring at every K tile; these reads are ordered
// against the transfers by the kernel's own vmcnt waits and barriers, as its
// ordinary LDS reads are.  Issue the ordinary LDS reads of the same phase before
// the block: its wait then covers them too.
#define MCG_TR_X1(OP)                                                   \
  asm volatile(                                                         \
      OP " %0, %4\n\t"                                                  \
      OP " %1, %4 offset:%c5\n\t"                                       \
      OP " %2, %4 offset:%c6\n\t"                                       \
      OP " %3, %4 offset:%c7\n\t"                                       \
      "s_waitcnt lgkmcnt(0)"                                            \
      : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[0][2]), "=&v"(r[0][3])  \
      : "v"(a[0]), "i"(O1), "i"(O2), "i"(O3)                            \
      : "memory")
#define MCG_TR_X2(OP)                                                    \
  asm volatile(                                                          \
      OP " %0, %8\n\t"                                                   \
      OP " %1, %8 offset:%c10\n\t"                                       \
      OP " %2, %8 offset:%c11\n\t"                                       \
      OP " %3, %8 offset:%c12\n\t"                                       \
      OP " %4, %9\n\t"                                                   \
      OP " %5, %9 offset:%c10\n\t"                                       \
      OP " %6, %9 offset:%c11\n\t"                                       \
      OP " %7, %9 offset:%c12\n\t"                                       \
      "s_waitcnt lgkmcnt(0)"                                             \
      : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[0][2]), "=&v"(r[0][3]),  \
        "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[1][2]), "=&v"(r[1][3])   \
      : "v"(a[0]), "v"(a[1]), "i"(O1), "i"(O2), "i"(O3)                  \
      : "memory")
#define MCG_TR_X4(OP)                                                          \
  asm volatile(                                                                \
      OP " %0, %16\n\t"                                                        \
      OP " %1, %16 offset:%c20\n\t"                                            \
      OP " %2, %16 offset:%c21\n\t"                                            \
      OP " %3, %16 offset:%c22\n\t"                                            \
      OP " %4, %17\n\t"                                                        \
      OP " %5, %17 offset:%c20\n\t"                                            \
      OP " %6, %17 offset:%c21\n\t"                                            \
      OP " %7, %17 offset:%c22\n\t"                                            \
      OP " %8, %18\n\t"                                                        \
      OP " %9, %18 offset:%c20\n\t"                                            \
      OP " %10, %18 offset:%c21\n\t"                                           \
      OP " %11, %18 offset:%c22\n\t"                                           \
      OP " %12, %19\n\t"                                                       \
      OP " %13, %19 offset:%c20\n\t"                                           \
      OP " %14, %19 offset:%c21\n\t"                                           \
      OP " %15, %19 offset:%c22\n\t"                                           \
      "s_waitcnt lgkmcnt(0)"                                                   \
      : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[0][2]), "=&v"(r[0][3]),        \
        "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[1][2]), "=&v"(r[1][3]),        \
        "=&v"(r[2][0]), "=&v"(r[2][1]), "=&v"(r[2][2]), "=&v"(r[2][3]),        \
        "=&v"(r[3][0]), "=&v"(r[3][1]), "=&v"(r[3][2]), "=&v"(r[3][3])         \
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(O1), "i"(O2), "i"(O3)  \
      : "memory")
#define MCG_TR_X6(OP)                                                                                \
  asm volatile(                                                                                      \
      OP " %0, %24\n\t"                                                                              \
      OP " %1, %24 offset:%c30\n\t"                                                                  \
      OP " %2, %24 offset:%c31\n\t"                                                                  \
      OP " %3, %24 offset:%c32\n\t"                                                                  \
      OP " %4, %25\n\t"                                                                              \
      OP " %5, %25 offset:%c30\n\t"                                                                  \
      OP " %6, %25 offset:%c31\n\t"                                                                  \
      OP " %7, %25 offset:%c32\n\t"                                                                  \
      OP " %8, %26\n\t"                                                                              \
      OP " %9, %26 offset:%c30\n\t"                                                                  \
      OP " %10, %26 offset:%c31\n\t"                                                                 \
      OP " %11, %26 offset:%c32\n\t"                                                                 \
      OP " %12, %27\n\t"                                                                             \
      OP " %13, %27 offset:%c30\n\t"                                                                 \
      OP " %14, %27 offset:%c31\n\t"                                                                 \
      OP " %15, %27 offset:%c32\n\t"                                                                 \
      OP " %16, %28\n\t"                                                                             \
      OP " %17, %28 offset:%c30\n\t"                                                                 \
      OP " %18, %28 offset:%c31\n\t"                                                                 \
      OP " %19, %28 offset:%c32\n\t"                                                                 \
      OP " %20, %29\n\t"                                                                             \
      OP " %21, %29 offset:%c30\n\t"                                                                 \
      OP " %22, %29 offset:%c31\n\t"                                                                 \
      OP " %23, %29 offset:%c32\n\t"                                                                 \
      "s_waitcnt lgkmcnt(0)"                                                                         \
      : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[0][2]), "=&v"(r[0][3]),                              \
        "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[1][2]), "=&v"(r[1][3]),                              \
        "=&v"(r[2][0]), "=&v"(r[2][1]), "=&v"(r[2][2]), "=&v"(r[2][3]),                              \
        "=&v"(r[3][0]), "=&v"(r[3][1]), "=&v"(r[3][2]), "=&v"(r[3][3]),                              \
        "=&v"(r[4][0]), "=&v"(r[4][1]), "=&v"(r[4][2]), "=&v"(r[4][3]),                              \
        "=&v"(r[5][0]), "=&v"(r[5][1]), "=&v"(r[5][2]), "=&v"(r[5][3])                               \
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "i"(O1), "i"(O2), "i"(O3)  \
      : "memory")
#define MCG_TR_P1(OP)                   \
  asm volatile(                         \
      OP " %0, %2\n\t"                  \
      OP " %1, %2 offset:%c3\n\t"       \
      "s_waitcnt lgkmcnt(0)"            \
      : "=&v"(r[0][0]), "=&v"(r[0][1])  \
      : "v"(a[0]), "i"(O1)              \
      : "memory")
#define MCG_TR_P2(OP)                    \
  asm volatile(                          \
      OP " %0, %4\n\t"                   \
      OP " %1, %4 offset:%c6\n\t"        \
      OP " %2, %5\n\t"                   \
      OP " %3, %5 offset:%c6\n\t"        \
      "s_waitcnt lgkmcnt(0)"             \
      : "=&v"(r[0][0]), "=&v"(r[0][1]),  \
        "=&v"(r[1][0]), "=&v"(r[1][1])   \
      : "v"(a[0]), "v"(a[1]), "i"(O1)    \
      : "memory")

template <int EB, int O1, int O2, int O3, int N>
__device__ __forceinline__ void lds_read_tr_x4(const uint32_t (&a)[N], i32x2 (&r)[N][4]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 6, "1, 2, 4 or 6 addresses");
  static_assert(O1 > 0 && O2 > O1 && O3 > O2 && O3 < 65536, "ds offsets");
  if constexpr (EB == 2 && N == 1) MCG_TR_X1("ds_read_b64_tr_b16");
  else if constexpr (EB == 2 && N == 2) MCG_TR_X2("ds_read_b64_tr_b16");
  else if constexpr (EB == 2 && N == 4) MCG_TR_X4("ds_read_b64_tr_b16");
  else if constexpr (EB == 2) MCG_TR_X6("ds_read_b64_tr_b16");
  else if constexpr (N == 1) MCG_TR_X1("ds_read_b64_tr_b8");
  else if constexpr (N == 2) MCG_TR_X2("ds_read_b64_tr_b8");
  else if constexpr (N == 4) MCG_TR_X4("ds_read_b64_tr_b8");
  else MCG_TR_X6("ds_read_b64_tr_b8");
}
// The same with two reads per address, at byte offsets 0 and O1.
template <int EB, int O1, int N>
__device__ __forceinline__ void lds_read_tr_x2(const uint32_t (&a)[N], i32x2 (&r)[N][2]) {
  static_assert(N == 1 || N == 2, "1 or 2 addresses");
  static_assert(O1 > 0 && O1 < 65536, "ds offset");
  if constexpr (EB == 2 && N == 1) MCG_TR_P1("ds_read_b64_tr_b16");
  else if constexpr (EB == 2) MCG_TR_P2("ds_read_b64_tr_b16");
  else if constexpr (N == 1) MCG_TR_P1("ds_read_b64_tr_b8");
  else MCG_TR_P2("ds_read_b64_tr_b8");
}
#undef MCG_TR_X1
#undef MCG_TR_X2
#undef MCG_TR_X4
#undef MCG_TR_X6
#undef MCG_TR_P1
#undef MCG_TR_P2

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) { return (uint32_t)(uintptr_t)p; }

}  // namespace mcg
