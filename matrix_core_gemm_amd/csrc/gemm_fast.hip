// gemm_fast.hip -- large-tile, deeply pipelined dense MFMA GEMM for gfx950 (the fast path of
// gemm_dense for aligned problems of at least 256 x 256).
//
// Same operation as gemm_dense.hip (the matrix fused multiply-add of "Accurate
// Models of AMD Matrix Cores", Section 2, Eq. (1), tiled over K as in "CDNA3
// dense MFMA builtins", Using MFMA builtins as a compute policy); what differs
// is the mapping onto CDNA4:
//   - 256 x 256 output tile per workgroup of 4 wavefronts (one per SIMD); each
//     wavefront owns a 128 x 128 sub-tile = 4 x 4 instructions of 32 x 32
//     (all 256 accumulator registers of its lanes), so each operand fragment
//     read from LDS feeds 4 instructions.
//   - K is staged in tiles of 64 bytes per row (32 bf16 / 64 8-bit values) in
//     a ring of 5 LDS stages of 32 KiB (A and B); HBM -> LDS uses
//     buffer_load ... lds (16 bytes per lane, no VGPRs), issued 3 K tiles ahead
//     of use.  The XOR swizzle of the LDS rows is folded into the global
//     address each lane loads; lanes whose chunk lies outside the matrix get
//     an out-of-range offset and the buffer unit writes zeros.
//   - the instructions of a K tile are split in two halves around the
//     workgroup barrier; for 16-byte fragments (bf16, f16, int8) the next K
//     tile's first-half fragments are read from LDS while the second half
//     executes (two 32-VGPR fragment sets).
//   - epilogue: for interior tiles, straight-line code reads C in four batches
//     of 16 vector loads per lane (so the loads overlap) and stores
//     D = alpha * acc + beta * C (16 bytes per lane per
//     row segment, thanks to issuing each instruction with the B fragment as its
//     first operand); edge tiles use per-element bounds.
//   - the 8 XCDs receive workgroups round-robin; the tile sequence is permuted
//     so that the workgroups resident on one XCD cover a compact block of tiles.
// LDS swizzles were chosen by measuring SQ_LDS_BANK_CONFLICT for the exact
// access patterns on an MI355X (all conflict-free):
//   K-contiguous rows (64 bytes, 4 chunks): chunk ^= (row / 4) mod 4;
//   MN-contiguous 16-bit rows (transposing 16-bit reads): chunk ^= 4 * (row mod 4);
//   MN-contiguous 8-bit rows (transposing 8-bit reads): chunk ^= 2 * (row mod 8).
// Preconditions (checked on the host): 16-byte aligned operands, K * elem_bytes
// and ld * elem_bytes multiples of 16, M, N >= 256, and each workgroup's
// operand window below 2 GiB (32-bit buffer offsets).
#include "fast_tiles.hpp"
#include "gemm_kernels.hpp"

namespace mcg {
namespace fast {

constexpr int KTB = 64;  // bytes of K per LDS row and stage
constexpr int NST = 5;   // LDS stages
constexpr int BM = 256, BN = 256;


// ------------------------------------------------------------- 32x32 ops
// P (first operand) = B fragment, Q = A fragment.  Lane group g = lane >> 5 of
// a 32-row fragment owns the tile K bytes [32g, 32g + 32) of its row (gathered
// by transposing reads when the operand is MN-contiguous).  Ops with
// SUBSTEPS == 2 consume them as two 16-byte halves (sub-step s = bytes
// [32g + 16s, +16)), one instruction each; SUBSTEPS == 1 ops take all 32 bytes
// in one instruction.  Output lane l, register r holds
// out[8*(r/4) + 4*(l/32) + r%4][l % 32] (the 32 x 32 accumulator layout).

struct BF16 {
  static constexpr int EB = 2, SUBSTEPS = 2;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x16;
  using frag_t = i32x4;
  __device__ static __forceinline__ void mma(acc_t& c, const frag_t& p, const frag_t& q) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bit_cast<bf16x8>(p), bit_cast<bf16x8>(q), c, 0, 0, 0);
  }
};
struct F16 {
  static constexpr int EB = 2, SUBSTEPS = 2;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x16;
  using frag_t = i32x4;
  __device__ static __forceinline__ void mma(acc_t& c, const frag_t& p, const frag_t& q) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(bit_cast<f16x8>(p), bit_cast<f16x8>(q), c, 0, 0, 0);
  }
};
struct I8 {
  static constexpr int EB = 1, SUBSTEPS = 2;
  static constexpr bool INT_ACC = true;
  using acc_t = i32x16;
  using frag_t = i32x4;
  __device__ static __forceinline__ void mma(acc_t& c, const frag_t& p, const frag_t& q) {
    c = __builtin_amdgcn_mfma_i32_32x32x32_i8(p, q, c, 0, 0, 0);
  }
};
// native fp8: FP = format of P (B tensor), FQ = format of Q (A tensor)
template <int FP, int FQ>
struct F8 {
  static constexpr int EB = 1, SUBSTEPS = 1;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x16;
  using frag_t = i32x8;
  __device__ static __forceinline__ void mma(acc_t& c, const frag_t& p, const frag_t& q) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(p, q, c, FP, FQ, 0, 0, 0, 0);
  }
};
// fp8 widened exactly to bf16 (K below the native-fp8 threshold): FA/FB = formats
// of A/B; a 16-byte sub-step holds 16 fp8 values = two bf16 instructions.
template <int FA, int FB>
struct F8W {
  static constexpr int EB = 1, SUBSTEPS = 2;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x16;
  using frag_t = i32x4;
  __device__ static __forceinline__ void mma(acc_t& c, const frag_t& p, const frag_t& q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const i32x4 pb = fp8x8_to_bf16x8<FB>(i32x2{p[2 * h], p[2 * h + 1]});
      const i32x4 qb = fp8x8_to_bf16x8<FA>(i32x2{q[2 * h], q[2 * h + 1]});
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bit_cast<bf16x8>(pb), bit_cast<bf16x8>(qb), c, 0, 0, 0);
    }
  }
};

template <class Op, int LA, int LB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fast_kernel(DenseArgs p) {
  constexpr int EB = Op::EB;
  constexpr int WT = 4;  // 32 x 32 instruction tiles per wave along m and n
  using GA = Geom<EB, LA, BM, KTB>;
  using GB = Geom<EB, LB, BN, KTB>;
  using RA = Reader<EB, LA, BM, KTB>;
  using RB = Reader<EB, LB, BN, KTB>;
  using acc_t = typename Op::acc_t;
  using v4 = typename std::conditional<Op::INT_ACC, i32x4, f32x4>::type;
  using s1 = typename std::conditional<Op::INT_ACC, int, float>::type;
  constexpr int STAGE = GA::BYTES + GB::BYTES;
  constexpr int PER_TILE = Loader<EB, LA, BM, KTB>::INSTR + Loader<EB, LB, BN, KTB>::INSTR;  // loads per wave
  static_assert(PER_TILE == 8, "vmcnt bookkeeping assumes 8 loads per wave per K tile");

  __shared__ __attribute__((aligned(1024))) char smem_raw[NST * STAGE];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  tile_coords<4>(p.tiles_m, p.tiles_n, tm, tn);  // XCD-aware, grouped tile order
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  Loader<EB, LA, BM, KTB> la;
  Loader<EB, LB, BN, KTB> lb;
  if constexpr (LA == LAYOUT_K)
    la.init(p.A + m0 * p.lda * EB, (uint32_t)(min(p.M - m0, (int64_t)BM) * p.lda * EB), p.lda, wave, lane);
  else
    la.init(p.A + m0 * EB, (uint32_t)((p.K * p.lda - m0) * EB), p.lda, wave, lane);
  if constexpr (LB == LAYOUT_K)
    lb.init(p.B + n0 * p.ldb * EB, (uint32_t)(min(p.N - n0, (int64_t)BN) * p.ldb * EB), p.ldb, wave, lane);
  else
    lb.init(p.B + n0 * EB, (uint32_t)((p.K * p.ldb - n0) * EB), p.ldb, wave, lane);

  acc_t acc[WT][WT];
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j) acc[i][j] = acc_t{};

  const int nk = (int)((p.K + KTB / EB - 1) / (KTB / EB));
  const int rbA = wm * (BM / 2), rbB = wn * (BN / 2);
  auto stA = [&](int kt) { return smem + (kt % NST) * STAGE; };
  auto stB = [&](int kt) { return smem + (kt % NST) * STAGE + GA::BYTES; };

  // Prologue: K tiles 0 .. NST-2.  Loads of tiles at or beyond nk read nothing
  // (every lane's offset is out of range) and fill their stage with zeros, so
  // the loop below issues the same 8 loads per wave in every iteration and the
  // number of loads still in flight at each wait is constant.
#pragma unroll
  for (int kt = 0; kt < NST - 1; ++kt) {
    la.issue(stA(kt), kt, p.K, wave);
    lb.issue(stB(kt), kt, p.K, wave);
  }
  asm volatile("s_waitcnt vmcnt(24)" ::: "memory");  // tile 0 has landed
  barrier_lds();

  if constexpr (Op::SUBSTEPS == 2) {
    // f0 holds sub-step 0 of the current tile, f1 sub-step 1.  Per tile:
    //   read sub-step 1 | multiply sub-step 0       (interleaved 1 read : 2 mfma)
    //   wait for tile kt+1, barrier
    //   refill the stage of tile kt-1 with tile kt+NST-1 | read the next tile's
    //   sub-step 0 | multiply sub-step 1           (interleaved 1 load : 1 mfma : 1 read : 1 mfma)
    i32x4 fa0[WT], fb0[WT], fa1[WT], fb1[WT];
#pragma unroll
    for (int i = 0; i < WT; ++i) fa0[i] = RA::read16(stA(0), rbA + 32 * i, 0, lane);
#pragma unroll
    for (int j = 0; j < WT; ++j) fb0[j] = RB::read16(stB(0), rbB + 32 * j, 0, lane);
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int i = 0; i < WT; ++i) fa1[i] = RA::read16(stA(kt), rbA + 32 * i, 1, lane);
#pragma unroll
      for (int j = 0; j < WT; ++j) fb1[j] = RB::read16(stB(kt), rbB + 32 * j, 1, lane);
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int j = 0; j < WT; ++j) Op::mma(acc[i][j], fb0[j], fa0[i]);
#pragma unroll
      for (int r = 0; r < 2 * WT; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMA
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the first half before the barrier
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // tile kt+1 has landed
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      // next tile's sub-step 0 is read before the new DMA loads are issued, so
      // no LDS read has to wait for in-flight DMA writes it cannot alias
#pragma unroll
      for (int i = 0; i < WT; ++i) fa0[i] = RA::read16(stA(kt + 1), rbA + 32 * i, 0, lane);
#pragma unroll
      for (int j = 0; j < WT; ++j) fb0[j] = RB::read16(stB(kt + 1), rbB + 32 * j, 0, lane);
      la.issue(stA(kt + NST - 1), kt + NST - 1, p.K, wave);
      lb.issue(stB(kt + NST - 1), kt + NST - 1, p.K, wave);
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int j = 0; j < WT; ++j) Op::mma(acc[i][j], fb1[j], fa1[i]);
#pragma unroll
      for (int r = 0; r < 2 * WT; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
      }
#pragma unroll
      for (int r = 0; r < 2 * WT; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);  // buffer load -> LDS
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // one instruction per 32-byte fragment: a single fragment set; the first
    // half of the tile's instructions runs before the barrier, the next tile's
    // fragments are read after the second half.
    i32x8 fa[WT], fb[WT];
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int i = 0; i < WT; ++i) fa[i] = RA::read32(stA(kt), rbA + 32 * i, lane);
#pragma unroll
      for (int j = 0; j < WT; ++j) fb[j] = RB::read32(stB(kt), rbB + 32 * j, lane);
#pragma unroll
      for (int i = 0; i < WT / 2; ++i)
#pragma unroll
        for (int j = 0; j < WT; ++j) Op::mma(acc[i][j], fb[j], fa[i]);
      __builtin_amdgcn_sched_barrier(0);  // keep the first half before the barrier
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // tile kt+1 has landed
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      la.issue(stA(kt + NST - 1), kt + NST - 1, p.K, wave);
      lb.issue(stB(kt + NST - 1), kt + NST - 1, p.K, wave);
#pragma unroll
      for (int i = WT / 2; i < WT; ++i)
#pragma unroll
        for (int j = 0; j < WT; ++j) Op::mma(acc[i][j], fb[j], fa[i]);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);  // buffer load -> LDS
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS DMA outstanding at exit

  // epilogue: tile (i, j), register group q: lane holds D[m][n .. n+3] with
  // m = m0 + rbA + 32 i + (lane & 31), n = n0 + rbB + 32 j + 8 q + 4 (lane >> 5)
  const bool vec_ok = p.vec_cd;
  const s1* C = (const s1*)p.C;
  s1* D = (s1*)p.D;
  auto combine = [&](const acc_t& a, int q, const v4& c, bool use_c) {
    v4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (Op::INT_ACC)
        o[r] = (int)((uint32_t)p.alpha_i * (uint32_t)a[4 * q + r] +
                     (use_c ? (uint32_t)p.beta_i * (uint32_t)c[r] : 0u));
      else
        o[r] = use_c ? __builtin_fmaf(p.alpha, a[4 * q + r], p.beta * c[r]) : p.alpha * a[4 * q + r];
    }
    return o;
  };
  if (vec_ok && m0 + BM <= p.M && n0 + BN <= p.N) {
    // interior tile: straight-line code, C read in four batches of 16 vector
    // loads per lane (issued back to back)
    const s1* Cb = C + (m0 + rbA + (lane & 31)) * p.ldc + n0 + rbB + 4 * (lane >> 5);
    s1* Db = D + (m0 + rbA + (lane & 31)) * p.ldc + n0 + rbB + 4 * (lane >> 5);
    if (p.use_c) {
#pragma unroll
      for (int i = 0; i < WT; ++i) {
        v4 cbuf[WT][4];
#pragma unroll
        for (int j = 0; j < WT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            cbuf[j][q] = *(const v4*)(Cb + (32 * i) * p.ldc + 32 * j + 8 * q);
#pragma unroll
        for (int j = 0; j < WT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(v4*)(Db + (32 * i) * p.ldc + 32 * j + 8 * q) = combine(acc[i][j], q, cbuf[j][q], true);
      }
    } else {
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int j = 0; j < WT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(v4*)(Db + (32 * i) * p.ldc + 32 * j + 8 * q) = combine(acc[i][j], q, v4{}, false);
    }
  } else {
    // edge tile: per-element bounds
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      const int64_t m = m0 + rbA + 32 * i + (lane & 31);
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < WT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = n0 + rbB + 32 * j + 8 * q + 4 * (lane >> 5);
          if (n >= p.N) continue;
          const bool full = vec_ok && n + 4 <= p.N;
          v4 c = {};
          if (p.use_c) {
            if (full) c = *(const v4*)(C + m * p.ldc + n);
            else
              for (int r = 0; r < 4; ++r)
                if (n + r < p.N) c[r] = C[m * p.ldc + n + r];
          }
          const v4 o = combine(acc[i][j], q, c, p.use_c);
          if (full) {
            *(v4*)(D + m * p.ldc + n) = o;
          } else {
            for (int r = 0; r < 4; ++r)
              if (n + r < p.N) D[m * p.ldc + n + r] = o[r];
          }
        }
    }
  }
}

template <class Op, int LA, int LB>
static hipError_t launch_one(const DenseArgs& a0, hipStream_t s) {
  DenseArgs a = a0;
  a.tiles_m = (int)((a.M + BM - 1) / BM);
  a.tiles_n = (int)((a.N + BN - 1) / BN);
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_fast_kernel<Op, LA, LB>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class Op>
static hipError_t launch_layouts(int la, int lb, const DenseArgs& a, hipStream_t s) {
  if (la == 0 && lb == 0) return launch_one<Op, 0, 0>(a, s);
  if (la == 0 && lb == 1) return launch_one<Op, 0, 1>(a, s);
  if (la == 1 && lb == 0) return launch_one<Op, 1, 0>(a, s);
  return launch_one<Op, 1, 1>(a, s);
}

}  // namespace fast

bool fast_path_ok(int dtA, int la, int lb, const DenseArgs& a, bool aligned) {
  const int64_t eb = (dtA == DT_BF16 || dtA == DT_F16) ? 2 : 1;
  if (!aligned || a.K == 0 || (a.K * eb) % 16 != 0) return false;
  if (a.M < 256 || a.N < 256) return false;  // small problems: the 128 x 128 kernel fills the chip better
  // every buffer window (and offset into it) must stay below 2 GiB
  const int64_t lim = (int64_t)1 << 31;
  // MN-contiguous offsets advance by whole K tiles, up to NST tiles past the end of K
  const int64_t kpad = fast::NST * fast::KTB / eb;
  const int64_t wa = la == 0 ? 256 * a.lda * eb : (a.K + kpad) * a.lda * eb;
  const int64_t wb = lb == 0 ? 256 * a.ldb * eb : (a.K + kpad) * a.ldb * eb;
  return wa < lim && wb < lim;
}

hipError_t launch_fast(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s) {
  using namespace fast;
  if (dtA == DT_BF16) return launch_layouts<BF16>(la, lb, a, s);
  if (dtA == DT_F16) return launch_layouts<F16>(la, lb, a, s);
  if (dtA == DT_I8) return launch_layouts<I8>(la, lb, a, s);
  const int fa = f8fmt(dtA), fb = f8fmt(dtB);
  if (a.K >= FP8_NATIVE_MIN_K) {
    if (fb == 0 && fa == 0) return launch_layouts<F8<0, 0>>(la, lb, a, s);
    if (fb == 1 && fa == 0) return launch_layouts<F8<1, 0>>(la, lb, a, s);
    if (fb == 0 && fa == 1) return launch_layouts<F8<0, 1>>(la, lb, a, s);
    return launch_layouts<F8<1, 1>>(la, lb, a, s);
  }
  if (fa == 0 && fb == 0) return launch_layouts<F8W<0, 0>>(la, lb, a, s);
  if (fa == 0 && fb == 1) return launch_layouts<F8W<0, 1>>(la, lb, a, s);
  if (fa == 1 && fb == 0) return launch_layouts<F8W<1, 0>>(la, lb, a, s);
  return launch_layouts<F8W<1, 1>>(la, lb, a, s);
}

}  // namespace mcg
