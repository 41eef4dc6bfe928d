// gemm_sparse_fast.hip -- 256 x 256 pipelined 2:4 sparse GEMM on the gfx950
// sparse matrix cores (the fast path of gemm_sparse24 for aligned problems of
// at least 256 x 256 with K a multiple of 16).
//
// The operation and the operand format are those of the general sparse kernel
// (the 2:4 model of "RDNA4 sparse WMMA builtins", Structured sparsity (2:4
// pattern) and Common parameters: two kept values per group of four along K,
// ascending, and a 2-bit position per kept value).  The mapping onto CDNA4:
//   - smfmac_f32_32x32x32_{bf16,f16}: 32 x 32 outputs and 32 dense k per
//     instruction, twice the dense instruction's work in about the same issue
//     time.  Measured operand layout: lane group g = lane >> 5 of the sparse
//     operand holds the 8 kept values of dense k [16g, 16g + 16) of its row;
//     lane group g of the dense operand holds k [8g, 8g + 8) and
//     [16 + 8g, 24 + 8g) of its column; the lane's index register holds, in
//     the 16-bit half that the instruction's abid selects, one 4-bit code per
//     group of four (code n for kept values 2n and 2n + 1).  The canonical
//     index word of a row and 32 dense k therefore serves both lane groups
//     directly: group g uses bits [16g, 16g + 16).
//   - 256 x 256 output tile per workgroup of 8 wavefronts, two per SIMD, each
//     owning 128 x 64 outputs = 4 x 2 instructions of 32 x 32.
//   - LDS: kept values in stages of 128 dense k (128 bytes = one cache line
//     per row) together with their index words (16 bytes per row), 2 stages of
//     36 KiB; B in stages of 64 dense k (one 128-byte line per column), 2
//     stages of 32 KiB.  All filled by buffer_load ... lds.
//   - ping-pong schedule as in the dense kernel: the two wavefronts of a SIMD
//     alternate between multiplying one 64-k step (16 instructions) and a
//     memory phase (fragment reads of the next step and DMA issues); wavefronts
//     0-3 issue the B loads, wavefronts 4-7 the kept values and index words.
//   - the sparse operand must be the instruction's first operand, so a lane's
//     output registers hold four consecutive rows of one column: the epilogue
//     stores one 4-byte value per register (each store instruction writes two
//     128-byte row segments).
#include "fast_tiles.hpp"
#include "gemm_kernels.hpp"

namespace mcg {
namespace fast {

constexpr int SP_KA = 128;               // dense k per stage of kept values (128 bytes per row)
constexpr int SP_KB = 64;                // dense k per stage of B (128 bytes per column)
constexpr int SP_BM = 256, SP_BN = 256;
constexpr int SP_THREADS = 512;
constexpr int SP_A_STAGE = 32768 + 4096;  // kept values + index words of 256 rows
constexpr int SP_B_STAGE = 32768;

struct Sp32BF16 {
  __device__ static __forceinline__ void mma(f32x16& c, const i32x4& a, const i32x8& b, int idx) {
    c = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(bit_cast<bf16x8>(a), bit_cast<bf16x16>(b), c, idx, 0, 0);
  }
};
struct Sp32F16 {
  __device__ static __forceinline__ void mma(f32x16& c, const i32x4& a, const i32x8& b, int idx) {
    c = __builtin_amdgcn_smfmac_f32_32x32x32_f16(bit_cast<f16x8>(a), bit_cast<f16x16>(b), c, idx, 0, 0);
  }
};


template <class Op, int LB>
__global__ __launch_bounds__(SP_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_sparse_fast_kernel(SparseArgs p) {
  constexpr int WTM = 4, WTN = 2;
  using RA = Reader<2, LAYOUT_K, SP_BM, 128>;
  using RB = Reader<2, LB, SP_BN, 128>;
  using LdA = LineLoader<2, LAYOUT_K, SP_BM, 128>;
  using LdB = LineLoader<2, LB, SP_BN, 128>;
  static_assert(Geom<2, LAYOUT_K, SP_BM, 128>::BYTES == 32768 && Geom<2, LB, SP_BN, 128>::BYTES == 32768, "");
  static_assert(LdA::INSTR == 8 && LdB::INSTR == 8, "8 loads per wave and stage");

  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * SP_A_STAGE + 2 * SP_B_STAGE];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: multiplies in even slots, loads B; 1: odd slots, loads A and index
  const int q = wave & 3;
  const int rbA = (q >> 1) * 128, rbB = (q & 1) * 128 + grp * 64;
  const int g = lane >> 5;
  int tm, tn;
  tile_coords<4>(p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * SP_BM, n0 = (int64_t)tn * SP_BN;
  const int64_t rows = min(p.M - m0, (int64_t)SP_BM);
  const int64_t Kc = p.K / 2;  // kept values per row
  const int nwords = (int)((p.K + 31) / 32);
  const int nu = (int)((p.K + SP_KB - 1) / SP_KB);   // 64-k steps

  auto stA = [&](int T) { return smem + (T & 1) * SP_A_STAGE; };
  auto stI = [&](int T) { return smem + (T & 1) * SP_A_STAGE + 32768; };
  auto stB = [&](int u) { return smem + 2 * SP_A_STAGE + (u & 1) * SP_B_STAGE; };

  LdA la;
  LdB lb;
  __amdgpu_buffer_rsrc_t rs_idx;
  uint32_t off_idx[4];
  int word_idx[4];
  if (grp) {
    la.init(p.Ac + m0 * p.lda_c * 2, (uint32_t)(rows * p.lda_c * 2), p.lda_c, Kc, q, lane);
    rs_idx = make_rsrc((const char*)(p.idx + m0 * p.ld_idx), (uint32_t)(rows * p.ld_idx * 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // 4-byte loads: lane -> (row, word) of a 16-byte index row
      const int e = i * 256 + q * 64 + lane;
      word_idx[i] = e & 3;
      off_idx[i] = (uint32_t)((e >> 2) * p.ld_idx * 4 + (e & 3) * 4);
    }
  } else {
    if constexpr (LB == LAYOUT_K)
      lb.init(p.B + n0 * p.ldb * 2, (uint32_t)(min(p.N - n0, (int64_t)SP_BN) * p.ldb * 2), p.ldb, p.K, q, lane);
    else
      lb.init(p.B + n0 * 2, (uint32_t)((p.K * p.ldb - n0) * 2), p.ldb, p.K, q, lane);
  }
  // kept values and index words of stage T (group 1, all 8 + 4 loads per wave)
  auto issueA = [&](int T) {
    la.issue(stA(T), T, 0, 8, q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = T * 4 + word_idx[i] < nwords ? off_idx[i] + (uint32_t)T * 16u : BUF_OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_idx, (__attribute__((address_space(3))) void*)(stI(T) + (i * 256 + q * 64) * 4), 4, o, 0, 0, 0);
    }
  };
  auto issueB = [&](int u) { lb.issue(stB(u), u, 0, 8, q); };  // group 0, all 8 loads per wave

  f32x16 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = f32x16{};

  i32x4 fa[2][WTM];
  i32x8 fb[2][WTN];
  int fi[2][WTM];
  // fragments of 64-k step u = 2T + h: instruction s covers dense k [64h + 32s, +32) of stage T
  auto read_frags = [&](int u) {
    const int T = u >> 1, h = u & 1;
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const int row = rbA + 32 * i + (lane & 31);
      const i32x2 w = *(const __attribute__((address_space(3))) i32x2*)(stI(T) + row * 16 + 8 * h);
      fi[0][i] = (int)((uint32_t)w.x >> (16 * g));
      fi[1][i] = (int)((uint32_t)w.y >> (16 * g));
#pragma unroll
      for (int s = 0; s < 2; ++s) fa[s][i] = RA::read16k(stA(T), rbA + 32 * i, 64 * h + 32 * s + 16 * g, lane);
    }
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const i32x4 lo = RB::read16k(stB(u), rbB + 32 * j, 64 * s + 16 * g, lane);
        const i32x4 hi = RB::read16k(stB(u), rbB + 32 * j, 64 * s + 32 + 16 * g, lane);
        fb[s][j] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
  };
  auto multiply = [&]() {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j) Op::mma(acc[i][j], fa[s][i], fb[s][j], fi[s][i]);
  };

  // Steps u (64 dense k).  Group 0 reads step u in slot 2u - 1 and multiplies
  // it in slot 2u; group 1 reads it in slot 2u and multiplies it in slot
  // 2u + 1; slots are separated by workgroup barriers.  B stage u % 2 is last
  // read in slot 2u; group 0 refills it with B(u + 2) in slot 2u + 1 and waits
  // for it at the end of slot 2u + 2.  Kept-value stage T % 2 is last read in
  // slot 4T + 2; group 1 refills it with stage T + 2 in slot 4T + 4 and waits
  // for it at the end of slot 4T + 6.  Loads of stages past K read nothing
  // and fill their stage with zeros.
  if (grp == 0) issueB(0);
  else issueA(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  barrier_lds();
  if (grp == 0) {
    for (int u = 0; u < nu; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      read_frags(u);  // slot 2u - 1
      issueB(u + 1);
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      multiply();  // slot 2u
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // B(u + 1)
      barrier_lds();
    }
  } else {
    barrier_lds();  // slot -1
    for (int u = 0; u < nu; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      read_frags(u);  // slot 2u
      if ((u & 1) == 0) issueA((u >> 1) + 1);
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // kept values of stage (u >> 1) + 1
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      multiply();  // slot 2u + 1
      __builtin_amdgcn_sched_barrier(0);
      if (u + 1 < nu) barrier_lds();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS DMA outstanding at exit

  // epilogue: block (i, j), register r holds D[m][n] with
  // m = m0 + rbA + 32 i + 8 (r / 4) + 4 (lane >> 5) + r % 4, n = n0 + rbB + 32 j + (lane & 31)
  const float* C = (const float*)p.C;
  float* D = (float*)p.D;
  const bool interior = m0 + SP_BM <= p.M && n0 + SP_BN <= p.N;
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int64_t n = n0 + rbB + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + rbA + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (!interior && (m >= p.M || n >= p.N)) continue;
        const float v = acc[i][j][r];
        D[m * p.ldc + n] = p.use_c ? __builtin_fmaf(p.alpha, v, p.beta * C[m * p.ldc + n]) : p.alpha * v;
      }
    }
}

template <class Op, int LB>
static hipError_t launch_sparse_fast_one(const SparseArgs& a0, hipStream_t s) {
  SparseArgs a = a0;
  a.tiles_m = (int)((a.M + SP_BM - 1) / SP_BM);
  a.tiles_n = (int)((a.N + SP_BN - 1) / SP_BN);
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_sparse_fast_kernel<Op, LB>), dim3((unsigned)blocks), dim3(SP_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace fast

bool sparse_fast_ok(int layoutB, const SparseArgs& a) {
  // 16-byte chunks of kept values (8 values = 16 dense k) and of B (8 k) never
  // straddle the end of K when K % 16 == 0; index words are fetched 4 bytes at a time
  auto al = [](const void* q, int64_t n) { return ((uintptr_t)q % (uintptr_t)n) == 0; };
  const bool aligned = al(a.Ac, 16) && al(a.B, 16) && al(a.idx, 4) && (a.lda_c * 2) % 16 == 0 &&
                       (a.ldb * 2) % 16 == 0;
  if (!aligned || a.K == 0 || a.K % 16 != 0) return false;
  if (a.M < fast::SP_BM || a.N < fast::SP_BN) return false;
  // every buffer window (and offset into it) must stay below 2 GiB;
  // MN-contiguous B offsets advance by whole stages, up to NST stages past K
  const int64_t lim = (int64_t)1 << 31;
  const int64_t kpad = 3 * (int64_t)fast::SP_KB;
  const int64_t wa = (int64_t)fast::SP_BM * a.lda_c * 2;
  const int64_t wi = (int64_t)fast::SP_BM * a.ld_idx * 4;
  const int64_t wb = layoutB == LAYOUT_K ? (int64_t)fast::SP_BN * a.ldb * 2 : (a.K + kpad) * a.ldb * 2;
  const int64_t tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  return wa < lim && wi < lim && wb < lim && tiles <= 0x7fffffff;
}

hipError_t launch_sparse_fast(int dt, int layoutB, const SparseArgs& a, hipStream_t s) {
  using namespace fast;
  if (dt == DT_BF16)
    return layoutB == LAYOUT_K ? launch_sparse_fast_one<Sp32BF16, LAYOUT_K>(a, s)
                               : launch_sparse_fast_one<Sp32BF16, LAYOUT_MN>(a, s);
  return layoutB == LAYOUT_K ? launch_sparse_fast_one<Sp32F16, LAYOUT_K>(a, s)
                             : launch_sparse_fast_one<Sp32F16, LAYOUT_MN>(a, s);
}

}  // namespace mcg
