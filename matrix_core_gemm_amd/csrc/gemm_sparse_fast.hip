// gemm_sparse_fast.hip -- 256 x 256 pipelined 2:4 sparse GEMM on the gfx950
// sparse matrix cores (the fast path of gemm_sparse24 for aligned problems of
// at least 256 x 256 with K a multiple of 16).
//
// The operation and the operand format are those of the general sparse kernel
// (the 2:4 model of "RDNA4 sparse WMMA builtins", Structured sparsity (2:4
// pattern) and Common parameters: two kept values per group of four along K,
// ascending, and a 2-bit position per kept value).  The mapping onto CDNA4:
//   - smfmac_f32_32x32x32_{bf16,f16}: 32 x 32 outputs and 32 dense k per
//     instruction, twice the dense instruction's work in the same issue time.
//     Measured operand layout: lane group g = lane >> 5 of the sparse operand
//     holds the 8 kept values of dense k [16g, 16g + 16) of its row; lane
//     group g of the dense operand holds k [8g, 8g + 8) and [16 + 8g, 24 + 8g)
//     of its column; the lane's index register holds, in the 16-bit half that
//     the instruction's abid selects, one 4-bit code per group of four (code n
//     for kept values 2n and 2n + 1).  The canonical index word of a row and 32
//     dense k therefore serves both lane groups directly: group g uses bits
//     [16g, 16g + 16).
//   - 256 x 256 output tile per workgroup of 4 wavefronts (one per SIMD), each
//     owning 128 x 128 = 4 x 4 instructions of 32 x 32.
//   - one stage = 32 dense k: kept values 256 rows x 32 bytes, B 256 x 64
//     bytes, index 256 rows x 4 bytes (25 KiB); a ring of 6 stages; every
//     stage is filled by buffer_load ... lds (16 bytes per lane for values and
//     B, 4 bytes per lane for the index), issued 5 stages ahead.
//   - per stage: half of the instructions run before the workgroup barrier;
//     after it the next stage's fragments are read while the other half runs.
//   - the sparse operand must be the instruction's first operand, so a lane's
//     output registers hold four consecutive rows of one column: the epilogue
//     stores one 4-byte value per register (each store instruction writes two
//     128-byte row segments).
#include "fast_tiles.hpp"
#include "gemm_kernels.hpp"

namespace mcg {
namespace fast {

constexpr int SP_KD = 32;                 // dense k per stage
constexpr int SP_KTB_A = SP_KD / 2 * 2;   // bytes of kept values per row and stage (16 x 16-bit)
constexpr int SP_KTB_B = SP_KD * 2;       // bytes of B per column and stage
constexpr int SP_NST = 6;                 // LDS stages
constexpr int SP_BM = 256, SP_BN = 256;

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

__device__ __forceinline__ uint32_t lds_read_b32(const lds_char* base, int off) {
  return *(const __attribute__((address_space(3))) uint32_t*)(base + off);
}

template <class Op, int LB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_sparse_fast_kernel(SparseArgs p) {
  constexpr int WT = 4;
  using GA = Geom<2, LAYOUT_K, SP_BM, SP_KTB_A>;
  using GB = Geom<2, LB, SP_BN, SP_KTB_B>;
  using RA = Reader<2, LAYOUT_K, SP_BM, SP_KTB_A>;
  using RB = Reader<2, LB, SP_BN, SP_KTB_B>;
  using LDA = Loader<2, LAYOUT_K, SP_BM, SP_KTB_A>;
  using LDB = Loader<2, LB, SP_BN, SP_KTB_B>;
  constexpr int IDX_BYTES = SP_BM * 4;
  constexpr int STAGE = GA::BYTES + GB::BYTES + IDX_BYTES;
  static_assert(LDA::INSTR + LDB::INSTR + 1 == 7, "vmcnt bookkeeping assumes 7 loads per wave per stage");
  static_assert(IDX_BYTES == NW * 64 * 4, "one 4-byte index load per lane and stage");
  static_assert(STAGE % 1024 == 0 && SP_NST * STAGE <= 160 * 1024, "LDS ring");

  __shared__ __attribute__((aligned(1024))) char smem_raw[SP_NST * STAGE];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords<4>(p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * SP_BM, n0 = (int64_t)tn * SP_BN;
  const int64_t rows = min(p.M - m0, (int64_t)SP_BM);

  LDA la;
  LDB lb;
  la.init(p.Ac + m0 * p.lda_c * 2, (uint32_t)(rows * p.lda_c * 2), p.lda_c, wave, lane);
  if constexpr (LB == LAYOUT_K)
    lb.init(p.B + n0 * p.ldb * 2, (uint32_t)(min(p.N - n0, (int64_t)SP_BN) * p.ldb * 2), p.ldb, wave, lane);
  else
    lb.init(p.B + n0 * 2, (uint32_t)((p.K * p.ldb - n0) * 2), p.ldb, wave, lane);
  // index: lane (wave, lane) fetches the word of row 64 * wave + lane
  const __amdgpu_buffer_rsrc_t rs_idx =
      make_rsrc((const char*)(p.idx + m0 * p.ld_idx), (uint32_t)(rows * p.ld_idx * 4));
  const uint32_t off_idx = (uint32_t)((64 * wave + lane) * p.ld_idx * 4);

  const int64_t Kc = p.K / 2;  // kept values per row
  const int nk = (int)((p.K + SP_KD - 1) / SP_KD);
  auto stA = [&](int kt) { return smem + (kt % SP_NST) * STAGE; };
  auto stB = [&](int kt) { return smem + (kt % SP_NST) * STAGE + GA::BYTES; };
  auto stI = [&](int kt) { return smem + (kt % SP_NST) * STAGE + GA::BYTES + GB::BYTES; };
  auto issue = [&](int kt) {
    la.issue(stA(kt), kt, Kc, wave);
    lb.issue(stB(kt), kt, p.K, wave);
    const uint32_t o = kt < nk ? off_idx + (uint32_t)kt * 4u : BUF_OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs_idx, (__attribute__((address_space(3))) void*)(stI(kt) + wave * 256), 4, o, 0, 0, 0);
  };

  f32x16 acc[WT][WT];
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j) acc[i][j] = f32x16{};

  const int rbA = wm * (SP_BM / 2), rbB = wn * (SP_BN / 2);
  const int g = lane >> 5;
  const int ishift = 16 * g;
  struct Frags {
    i32x4 a[WT];
    i32x8 b[WT];
    int idx[WT];
  };
  auto read_frags = [&](Frags& f, int kt) {
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      f.a[i] = RA::read16k(stA(kt), rbA + 32 * i, 16 * g, lane);
      f.idx[i] = (int)(lds_read_b32(stI(kt), (rbA + 32 * i + (lane & 31)) * 4) >> ishift);
    }
#pragma unroll
    for (int j = 0; j < WT; ++j) {
      const i32x4 lo = RB::read16k(stB(kt), rbB + 32 * j, 16 * g, lane);
      const i32x4 hi = RB::read16k(stB(kt), rbB + 32 * j, 32 + 16 * g, lane);
      f.b[j] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  };

  // Prologue: stages 0 .. NST-1.  Loads of stages at or beyond nk read nothing
  // (every offset is out of range) and fill their stage with zeros, so every
  // iteration issues the same 7 loads per wave and the number of loads in
  // flight at each wait is constant.
#pragma unroll
  for (int kt = 0; kt < SP_NST; ++kt) issue(kt);
  asm volatile("s_waitcnt vmcnt(35)" ::: "memory");  // stage 0 has landed
  barrier_lds();

  // Per stage kt (its fragments already requested into `cur`):
  //   multiply rows 0-1 of the wave's blocks
  //   wait for stage kt+1, barrier (every wave has finished reading stage kt)
  //   read stage kt+1 into `nxt` | refill stage kt with stage kt+NST | multiply rows 2-3
  auto step = [&](Frags& cur, Frags& nxt, int kt) {
#pragma unroll
    for (int i = 0; i < WT / 2; ++i)
#pragma unroll
      for (int j = 0; j < WT; ++j) Op::mma(acc[i][j], cur.a[i], cur.b[j], cur.idx[i]);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(28)" ::: "memory");  // stage kt+1 has landed
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(nxt, kt + 1);
    issue(kt + SP_NST);
#pragma unroll
    for (int i = WT / 2; i < WT; ++i)
#pragma unroll
      for (int j = 0; j < WT; ++j) Op::mma(acc[i][j], cur.a[i], cur.b[j], cur.idx[i]);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  Frags f0, f1;
  read_frags(f0, 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(f0, f1, kt);
    step(f1, f0, kt + 1);
  }
  if (kt < nk) step(f0, f1, kt);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS DMA outstanding at exit

  // epilogue: block (i, j), register r holds D[m][n] with
  // m = m0 + rbA + 32 i + 8 (r / 4) + 4 (lane >> 5) + r % 4, n = n0 + rbB + 32 j + (lane & 31)
  const float* C = (const float*)p.C;
  float* D = (float*)p.D;
  const bool interior = m0 + SP_BM <= p.M && n0 + SP_BN <= p.N;
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j) {
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
  hipLaunchKernelGGL((gemm_sparse_fast_kernel<Op, LB>), dim3((unsigned)blocks), dim3(256), 0, s, a);
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
  const int64_t kpad = (int64_t)fast::SP_NST * fast::SP_KD;
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
