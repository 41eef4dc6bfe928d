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
constexpr int SP_BH_STAGE = 16384;        // one column half of B, 64 dense k

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


// HBM -> LDS loader of one column half of the B tile.  Half c holds the
// tile's columns [64c, 64c + 64) and [128 + 64c, 192 + 64c), the columns that
// the wavefronts of group c read, as 128 LDS rows of 64 dense k (K-contiguous
// B) or as 128 columns of each of 64 k rows (MN-contiguous B).  Same fetch
// pattern as LineLoader (whole 128-byte lines for K-contiguous rows); the
// second 64 columns are reached by an extra uniform jump (K-contiguous: for
// instructions 2 and 3) or a per-lane offset (MN-contiguous: chunks 8..15).
template <int LB>
struct BHalfLoader {
  using G = Geom<2, LB, 128, 128>;
  static constexpr int INSTR = G::CHUNKS / (64 * NW);
  static_assert(INSTR == 4, "4 loads per wave and half stage");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff, istride, jump, kstride;
  int klim;

  __device__ __forceinline__ void init(const char* B, int64_t n0, int c, int64_t N, int64_t K, int64_t ldb,
                                       int wave, int lane) {
    const int q = wave * 64 + lane;
    const int r = q / G::CPR, pc = q % G::CPR;
    const int lc = pc ^ swz<2, LB, G::CPR>(r);
    const int64_t col0 = n0 + 64 * c;
    if constexpr (LB == LAYOUT_K) {
      const int64_t rows = min(N - n0, (int64_t)256) - 64 * c;  // tile columns from col0 to the end of N
      rsrc = make_rsrc(B + col0 * ldb * 2, (uint32_t)(rows > 0 ? rows * ldb * 2 : 0));
      voff = (uint32_t)(r * ldb * 2 + lc * 16);
      istride = __builtin_amdgcn_readfirstlane((uint32_t)(32 * ldb * 2));
      jump = __builtin_amdgcn_readfirstlane((uint32_t)(64 * ldb * 2));
      kstride = 128;
      const int64_t left = K - (int64_t)lc * 8;
      klim = left <= 0 ? 0 : (int)((left + 63) / 64);
    } else {
      rsrc = make_rsrc(B + col0 * 2, (uint32_t)((K * ldb - col0) * 2));
      voff = (uint32_t)(r * ldb * 2 + lc * 16 + (lc >= 8 ? 128 : 0));
      istride = __builtin_amdgcn_readfirstlane((uint32_t)(16 * ldb * 2));
      jump = 0;
      kstride = __builtin_amdgcn_readfirstlane((uint32_t)(64 * ldb * 2));
      klim = 0x7fffffff;  // rows past K lie outside the buffer window
    }
  }

  __device__ __forceinline__ void issue(lds_char* dst, int u, int wave) const {
    const uint32_t v = u < klim ? voff + (uint32_t)u * kstride : BUF_OOB;
#pragma unroll
    for (int i = 0; i < INSTR; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(dst + (i * NW + wave) * 1024), 16,
          v + (uint32_t)i * istride + (i >= INSTR / 2 ? jump : 0u), 0, 0, 0);
  }
};

template <class Op, int LB>
__global__ __launch_bounds__(SP_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_sparse_fast_kernel(SparseArgs p) {
  constexpr int WTM = 4, WTN = 2;
  using RA = Reader<2, LAYOUT_K, SP_BM, 128>;
  using RB = Reader<2, LB, 128, 128>;
  using LdA = LineLoader<2, LAYOUT_K, SP_BM, 128>;
  static_assert(Geom<2, LAYOUT_K, SP_BM, 128>::BYTES == 32768 && Geom<2, LB, 128, 128>::BYTES == SP_BH_STAGE, "");
  static_assert(LdA::INSTR == 8, "8 loads per wave and kept-value stage");

  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * SP_A_STAGE + 4 * SP_BH_STAGE];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: multiplies in even slots; 1: odd slots
  const int q = wave & 3;
  const int rbA = (q >> 1) * 128, rbB = (q & 1) * 128 + grp * 64;  // tile coordinates
  const int rbBh = (q & 1) * 64;                                    // row in this group's B half
  const int g = lane >> 5;
  int tm, tn;
  tile_coords<4>(p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * SP_BM, n0 = (int64_t)tn * SP_BN;
  const int64_t rows = min(p.M - m0, (int64_t)SP_BM);
  const int64_t Kc = p.K / 2;  // kept values per row
  const int nwords = (int)((p.K + 31) / 32);
  const int nT = (int)((p.K + SP_KA - 1) / SP_KA);  // kept-value stages; 2 steps of 64 dense k each

  auto stA = [&](int T) { return smem + (T & 1) * SP_A_STAGE; };
  auto stI = [&](int T) { return smem + (T & 1) * SP_A_STAGE + 32768; };
  // B half c of step u
  auto stBh = [&](int c, int u) { return smem + 2 * SP_A_STAGE + (2 * c + (u & 1)) * SP_BH_STAGE; };

  // every wave loads half of the kept values (instructions 4 grp .. 4 grp + 3)
  // and the other group's half of B; group 0 also loads the index words
  LdA la;
  la.init(p.Ac + m0 * p.lda_c * 2, (uint32_t)(rows * p.lda_c * 2), p.lda_c, Kc, q, lane);
  BHalfLoader<LB> lb;
  lb.init(p.B, n0, 1 - grp, p.N, p.K, p.ldb, q, lane);
  __amdgpu_buffer_rsrc_t rs_idx;
  uint32_t off_idx[4];
  int word_idx[4];
  rs_idx = make_rsrc((const char*)(p.idx + m0 * p.ld_idx), (uint32_t)(rows * p.ld_idx * 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // 4-byte loads: lane -> (row, word) of a 16-byte index row
    const int e = i * 256 + q * 64 + lane;
    word_idx[i] = e & 3;
    off_idx[i] = (uint32_t)((e >> 2) * p.ld_idx * 4 + (e & 3) * 4);
  }
  auto issueA = [&](int T) { la.issue(stA(T), T, 4 * grp, 4, q); };
  auto issueI = [&](int T) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = T * 4 + word_idx[i] < nwords ? off_idx[i] + (uint32_t)T * 16u : BUF_OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_idx, (__attribute__((address_space(3))) void*)(stI(T) + (i * 256 + q * 64) * 4), 4, o, 0, 0, 0);
    }
  };
  auto issueB = [&](int u) { lb.issue(stBh(1 - grp, u), u, q); };  // the other group's half

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
        const i32x4 lo = RB::read16k(stBh(grp, u), rbBh + 32 * j, 64 * s + 16 * g, lane);
        const i32x4 hi = RB::read16k(stBh(grp, u), rbBh + 32 * j, 64 * s + 32 + 16 * g, lane);
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

  // Steps u (64 dense k), two per kept-value stage T.  Group 0 reads step u in
  // slot 2u - 1 and multiplies it in slot 2u; group 1 reads it in slot 2u and
  // multiplies it in slot 2u + 1; slots are separated by workgroup barriers.
  // B half c of step u is read only by group c, so it is free as soon as
  // group c has read it, and the other group refills it in its next memory
  // phase: group 0 loads group 1's half of B(u + 1) in slot 2u - 1, group 1
  // loads group 0's half of B(u + 2) in slot 2u; each has 3 slots in flight.
  // Kept-value stage T (and its index words) is last read in slot 4T + 2;
  // group 0 loads its half of stage T + 2 and the index words in slot 4T + 3,
  // group 1 the other half in slot 4T + 4.  Every wave waits for its loads at
  // the end of its memory phases, just early enough for their first reader.
  // Loads past K read nothing and fill their stage with zeros (an odd number
  // of steps is padded with one such zero step).
  if (grp == 0) {
    issueB(0);
    issueA(0);
    issueI(0);
  } else {
    issueB(0);
    issueB(1);
    issueA(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  barrier_lds();
  if (grp == 0) {
    for (int T = 0; T < nT; ++T) {
      const int u = 2 * T;
      __builtin_amdgcn_sched_barrier(0);
      read_frags(u);  // slot 4T - 1
      issueB(u + 1);
      issueA(T + 1);
      issueI(T + 1);
      asm volatile("s_waitcnt vmcnt(12)" ::: "memory");  // group 1's half of B(u)
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      multiply();  // slot 4T
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      read_frags(u + 1);  // slot 4T + 1
      issueB(u + 2);
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // B(u + 1) half, kept values and index of T + 1
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      multiply();  // slot 4T + 2
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds();
    }
  } else {
    barrier_lds();  // slot -1
    for (int T = 0; T < nT; ++T) {
      const int u = 2 * T;
      __builtin_amdgcn_sched_barrier(0);
      read_frags(u);  // slot 4T
      issueB(u + 2);
      issueA(T + 1);
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // group 0's half of B(u + 1)
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      multiply();  // slot 4T + 1
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      read_frags(u + 1);  // slot 4T + 2
      issueB(u + 3);
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // B(u + 2) half, kept values of T + 1
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      multiply();  // slot 4T + 3
      __builtin_amdgcn_sched_barrier(0);
      if (T + 1 < nT) barrier_lds();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS DMA outstanding at exit

  // epilogue: block (i, j), register r holds D[m][n] with
  // m = m0 + rbA + 32 i + 8 (r / 4) + 4 (lane >> 5) + r % 4, n = n0 + rbB + 32 j + (lane & 31)
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
        combine_store(p.C, p.D, m * p.ldc + n, acc[i][j][r], p.alpha, p.beta, p.use_c, p.out);
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
  const int64_t kpad = 4 * (int64_t)fast::SP_KB;
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
