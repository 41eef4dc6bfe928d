// mfma_probe.hip -- the matrix cores' sustained rate on given operand bits.
//
// A measurement aid for the GEMM kernels' roofline, not part of any GEMM: the
// published peaks ("CDNA3 dense MFMA builtins", Instruction throughput: flops
// per instruction times instructions per cycle times the peak clock) hold only
// at the peak clock, and on gfx950 the clock under full matrix-core load
// depends on the operand bits (measured: all-zero operands keep it at about
// 2.4 GHz; N(0,1) bf16 operands bring it down to about 1.6-1.7 GHz).  The
// probe runs the GEMM kernels' instructions, in their arrangement (one
// workgroup of 8 wavefronts per CU, two per SIMD, all of the LDS reserved,
// the two wavefronts of a SIMD alternating between barriers), on fragments
// loaded once from the caller's operand bytes, with no other memory traffic.
// Its rate is then the ceiling that data movement cannot raise for those bits.
//
// Per wavefront and phase: 16 instructions over a 4 x 2 grid of 32 x 32
// accumulators (the 256 x 256 kernels' wavefront tile), two per accumulator.
#include "fast_tiles.hpp"
#include "gemm_kernels.hpp"
#include "sparse_ops.hpp"

namespace mcg {
namespace probe {

using namespace fast;

template <class Op>
struct Frags {
  typename Op::frag_t a[4], b[2];
};

template <class Op, bool SPARSE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_probe_kernel(const char* a, const char* b, const char* idx, int phases, float* sink, int64_t* clocks) {
  __shared__ char reserve[160 * 1024];  // one workgroup per CU, as the pipelined GEMM kernels run
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  // this lane's 64-byte window; every fragment lies in [0, 65536) of a, b and idx
  const int base = (int)((blockIdx.x * 4096u) & 32767u) + (wave * 64 + lane) * 64;
  using acc_t = typename Op::acc_t;
  acc_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = acc_t{};
  auto ld16 = [&](const char* p, int off) { return *(const i32x4*)(p + base + off); };
  auto ld32 = [&](const char* p, int off) {
    const i32x4 x = ld16(p, off), y = ld16(p, off + 16);
    return i32x8{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
  };
  // fragments: A (kept values for 2:4) 4 x 16 or 32 bytes, B 2 x 16 or 32 bytes, index words 4 x 4 bytes
  i32x4 fa16[4];
  i32x8 fa32[4], fb32[2];
  i32x4 fb16[2];
  int fi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa16[i] = ld16(a, 16 * i);
    fa32[i] = ld32(a, 32 * i);
    fi[i] = SPARSE ? *(const int*)(idx + base + 4 * i) : 0;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    fb16[j] = ld16(b, 16 * j);
    fb32[j] = ld32(b, 32 * j);
  }
  // reading the reservation keeps it allocated; the value is never used otherwise
  if (((volatile char*)reserve)[tid] == 0x5a && phases < 0) sink[0] = 0.f;

  auto phase = [&]() {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (SPARSE) {
            Op::mma(acc[i][j], fa16[i], fb32[j], fi[i]);
          } else if constexpr (Op::LANE_BYTES == 32) {
            Op::mma(acc[i][j], fb32[j], fa32[i]);
          } else {
            Op::mma(acc[i][j], fb16[j], fa16[i]);
          }
        }
  };
  __builtin_amdgcn_s_barrier();
  const int64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  // group 0 multiplies in even slots, group 1 in odd slots; slots end at barriers
  if (grp == 1) __builtin_amdgcn_s_barrier();
  for (int t = 0; t < phases; ++t) {
    __builtin_amdgcn_sched_barrier(0);
    phase();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_barrier();
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();
  const int64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += (float)acc[i][j][e];
  sink[blockIdx.x * 512 + tid] = s;
}

template <class Op, bool SPARSE>
static hipError_t launch(const void* a, const void* b, const void* idx, int phases, int num_wg, float* sink,
                         int64_t* clocks, hipStream_t s) {
  hipLaunchKernelGGL((mfma_probe_kernel<Op, SPARSE>), dim3((unsigned)num_wg), dim3(512), 0, s, (const char*)a,
                     (const char*)b, (const char*)idx, phases, sink, clocks);
  return hipGetLastError();
}

}  // namespace probe

bool mfma_probe_supported(int dtA, int dtB, int sparse) {
  const bool f8a = dtA == DT_E4M3 || dtA == DT_E5M2, f8b = dtB == DT_E4M3 || dtB == DT_E5M2;
  if (dtA == DT_BF16 || dtA == DT_F16 || dtA == DT_I8) return dtB == dtA && (sparse == 0 || sparse == 1);
  return f8a && f8b && (sparse == 0 || sparse == 1);
}

hipError_t launch_mfma_probe(int dtA, int dtB, int sparse, const void* a, const void* b, const void* idx,
                             int64_t instr_per_wave, int num_wg, float* sink, int64_t* clocks, hipStream_t s) {
  using namespace fast;
  const int phases = (int)(instr_per_wave / 16);
  const int fa = dtA == DT_E5M2 ? 1 : 0, fb = dtB == DT_E5M2 ? 1 : 0;
  if (sparse) {
    if (dtA == DT_BF16) return probe::launch<Sp32BF16, true>(a, b, idx, phases, num_wg, sink, clocks, s);
    if (dtA == DT_F16) return probe::launch<Sp32F16, true>(a, b, idx, phases, num_wg, sink, clocks, s);
    if (dtA == DT_I8) return probe::launch<Sp32I8, true>(a, b, idx, phases, num_wg, sink, clocks, s);
    if (fa == 0 && fb == 0) return probe::launch<Sp32F8<0, 0>, true>(a, b, idx, phases, num_wg, sink, clocks, s);
    if (fa == 0 && fb == 1) return probe::launch<Sp32F8<0, 1>, true>(a, b, idx, phases, num_wg, sink, clocks, s);
    if (fa == 1 && fb == 0) return probe::launch<Sp32F8<1, 0>, true>(a, b, idx, phases, num_wg, sink, clocks, s);
    return probe::launch<Sp32F8<1, 1>, true>(a, b, idx, phases, num_wg, sink, clocks, s);
  }
  if (dtA == DT_BF16) return probe::launch<BF16, false>(a, b, idx, phases, num_wg, sink, clocks, s);
  if (dtA == DT_F16) return probe::launch<F16, false>(a, b, idx, phases, num_wg, sink, clocks, s);
  if (dtA == DT_I8) return probe::launch<I8, false>(a, b, idx, phases, num_wg, sink, clocks, s);
  // F8<FP, FQ>: FP = format of the first operand (B), FQ = of the second (A)
  if (fb == 0 && fa == 0) return probe::launch<F8<0, 0>, false>(a, b, idx, phases, num_wg, sink, clocks, s);
  if (fb == 1 && fa == 0) return probe::launch<F8<1, 0>, false>(a, b, idx, phases, num_wg, sink, clocks, s);
  if (fb == 0 && fa == 1) return probe::launch<F8<0, 1>, false>(a, b, idx, phases, num_wg, sink, clocks, s);
  return probe::launch<F8<1, 1>, false>(a, b, idx, phases, num_wg, sink, clocks, s);
}

}  // namespace mcg
