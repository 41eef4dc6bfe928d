// gemm_sparse_fast.hip -- 256 x 256 pipelined 2:4 sparse GEMM on the gfx950
// sparse matrix cores (the fast path of gemm_sparse24 for aligned problems of
// at least 256 x 256 with K * elem_bytes a multiple of 32; fp8 from K = 6144).
//
// The operation and the operand format are those of the general sparse kernel
// (the 2:4 model of "RDNA4 sparse WMMA builtins", Structured sparsity (2:4
// pattern) and Common parameters: two kept values per group of four along K,
// ascending, and a 2-bit position per kept value).  The mapping onto CDNA4:
//   - 32 x 32 outputs per instruction: smfmac_f32_32x32x32_{bf16,f16} (32
//     dense k) and smfmac_{i32_32x32x64_i8, f32_32x32x64_<fp8|bf8>_<fp8|bf8>}
//     (64 dense k), twice the dense instruction's work in about the same issue
//     time.  Measured operand layouts, the same in bytes for both widths: lane
//     group g = lane >> 5 of the sparse operand holds the 16 kept bytes of
//     dense k [16g, 16g + 16) (16-bit) or [32g, 32g + 32) (8-bit) of its row;
//     lane group g of the dense operand holds bytes [16g, 16g + 16) and
//     [32 + 16g, 48 + 16g) of its column's 64 bytes; the lane's index register
//     holds one 4-bit code per group of four (code n for kept values 2n and
//     2n + 1): for 16-bit elements in the 16-bit half that abid selects, so
//     group g uses bits [16g, 16g + 16) of the canonical word of 32 dense k,
//     for 8-bit elements the whole register, so group g uses the canonical
//     word g of the instruction's 64 dense k.
//   - 256 x 256 output tile per workgroup of 8 wavefronts, two per SIMD, each
//     owning 128 x 64 outputs = 4 x 2 instructions of 32 x 32.
//   - LDS: kept values in stages of 128 bytes per row (one cache line: 128
//     dense k of 16-bit or 256 of 8-bit elements), 2 stages; their index words
//     (16 or 32 bytes per row and stage) in blocks of 64 bytes per row (4 or 2
//     stages), fetched as 64 contiguous bytes per row by 4 lanes, 2 blocks, with
//     the row's 16-byte chunks rotated by row / 4 so that the 16 rows one LDS
//     cycle serves fall in different banks; B in stages of 128 bytes per column
//     (64 or 128 dense k), 2 stages per column half.  160 KiB, all filled by
//     buffer_load ... lds.
//   - ping-pong schedule as in the dense kernel: the two wavefronts of a SIMD
//     alternate between multiplying one step (16 instructions) and a memory
//     phase (fragment reads of the next step and DMA issues); each group of
//     wavefronts loads the other group's half of B, half of the kept values,
//     and group 0 the index words.
//   - the sparse operand must be the instruction's first operand, so a lane's
//     output registers hold four consecutive rows of one column: the epilogue
//     stores one 4-byte value per register (each store instruction writes two
//     128-byte row segments).
#include "fast_tiles.hpp"
#include "frag_layout.hpp"
#include "gemm_kernels.hpp"
#include "sparse_ops.hpp"

namespace mcg {
namespace fast {

constexpr int SP_BM = 256, SP_BN = 256;
constexpr int SP_THREADS = 512;
constexpr int SP_BH_STAGE = 16384;  // one column half of B: 128 columns x 128 bytes

// Per element width EB: a kept-value stage holds 128 bytes per row (KA dense k),
// whose index words take IWB bytes per row; a B stage holds 128 bytes per
// column (KB dense k); one instruction takes 32 kept bytes and 64 B bytes of each
// row / column.  Index words move in blocks of 64 bytes per row (SPB kept-value
// stages), so that 4 lanes fetch one row's 64 contiguous bytes.
template <int EB>
struct SpGeom {
  static constexpr int KA = 256 / EB;            // dense k per kept-value stage
  static constexpr int KB = 128 / EB;            // dense k per B stage
  static constexpr int IWB = KA / 32 * 4;        // index bytes per row and stage
  static constexpr int A_STAGE = SP_BM * 128;    // kept values
  static constexpr int SPB = 64 / IWB;           // kept-value stages per index block
  static constexpr int I_BLOCK = SP_BM * 64;     // one index block in LDS
};

// HBM -> LDS loader of one column half of the B tile.  Half c holds the
// tile's columns [64c, 64c + 64) and [128 + 64c, 192 + 64c), the columns that
// the wavefronts of group c read, as 128 LDS rows of 64 dense k (K-contiguous
// B) or as 128 columns of each of 64 k rows (MN-contiguous B).  Same fetch
// pattern as LineLoader (whole 128-byte lines for K-contiguous rows); the
// second 64 columns are reached by an extra uniform jump (K-contiguous: for
// instructions 2 and 3) or a per-lane offset (MN-contiguous: chunks 8..15).
template <int EB, int LB>
struct BHalfLoader {
  using G = Geom<EB, LB, 128, 128>;
  static constexpr int INSTR = G::CHUNKS / (64 * NW);
  static constexpr int EPC = 16 / EB;  // elements per 16-byte chunk
  static_assert(INSTR == 4, "4 loads per wave and half stage");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff, istride, jump, kstride;
  int klim;

  __device__ __forceinline__ void init(const char* B, int64_t n0, int c, int64_t N, int64_t K, int64_t ldb,
                                       int wave, int lane) {
    const int q = wave * 64 + lane;
    const int r = q / G::CPR, pc = q % G::CPR;
    const int lc = pc ^ swz<EB, LB, G::CPR>(r);
    const int64_t col0 = n0 + 64 * c;
    if constexpr (LB == LAYOUT_K) {
      const int64_t rows = min(N - n0, (int64_t)256) - 64 * c;  // tile columns from col0 to the end of N
      rsrc = make_rsrc(B + col0 * ldb * EB, (uint32_t)(rows > 0 ? rows * ldb * EB : 0));
      voff = (uint32_t)(r * ldb * EB + lc * 16);
      istride = __builtin_amdgcn_readfirstlane((uint32_t)(32 * ldb * EB));
      jump = __builtin_amdgcn_readfirstlane((uint32_t)(64 * ldb * EB));
      kstride = 128;
      const int64_t left = K - (int64_t)lc * EPC;
      klim = left <= 0 ? 0 : (int)((left + SpGeom<EB>::KB - 1) / SpGeom<EB>::KB);
    } else {
      // an LDS row holds columns [0, 64) then [128, 192) of the half: chunks
      // past the first 64 columns jump over the other group's 64
      rsrc = make_rsrc(B + col0 * EB, (uint32_t)((K * ldb - col0) * EB));
      voff = (uint32_t)(r * ldb * EB + lc * 16 + (lc >= 4 * EB ? 64 * EB : 0));
      istride = __builtin_amdgcn_readfirstlane((uint32_t)(NW * 64 / G::CPR * ldb * EB));  // k rows per instruction
      jump = 0;
      kstride = __builtin_amdgcn_readfirstlane((uint32_t)(SpGeom<EB>::KB * ldb * EB));
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

// SK: the stream-K form, whose workgroups each take a range of the kept-value
// stages of the tiles after the first dp_tiles (which a launch of the whole-tile
// form covers); see gemm_fast_sk.hip.
template <class Op, int LB, bool SK = false>
__global__ __launch_bounds__(SP_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_sparse_fast_kernel(SparseArgs p) {
  constexpr int WTM = 4, WTN = 2;
  constexpr int EB = Op::EB;
  using SG = SpGeom<EB>;
  constexpr int A_STAGE = SG::A_STAGE, IWB = SG::IWB, SPB = SG::SPB, I_BLOCK = SG::I_BLOCK;
  constexpr int II = SP_BM * IWB / (1024 * NW);  // 16-byte index loads per wave of group 0 and stage
  using RA = Reader<EB, LAYOUT_K, SP_BM, 128>;
  using RB = Reader<EB, LB, 128, 128>;
  using LdA = LineLoader<EB, LAYOUT_K, SP_BM, 128>;
  using acc_t = typename Op::acc_t;
  static_assert(Geom<EB, LAYOUT_K, SP_BM, 128>::BYTES == 32768 && Geom<EB, LB, 128, 128>::BYTES == SP_BH_STAGE, "");
  static_assert(LdA::INSTR == 8, "8 loads per wave and kept-value stage");
  static_assert(II == 1 || II == 2, "index loads per stage");
  static_assert(II * NW * SPB == I_BLOCK / 1024, "a block's loads, one part per stage");

  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * A_STAGE + 4 * SP_BH_STAGE + 2 * I_BLOCK];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: multiplies in even slots; 1: odd slots
  const int q = wave & 3;
  const int rbA = (q >> 1) * 128, rbB = (q & 1) * 128 + grp * 64;  // tile coordinates
  const int rbBh = (q & 1) * 64;                                    // row in this group's B half
  const int g = lane >> 5;
  const int nT_all = (int)((p.K + SG::KA - 1) / SG::KA);  // kept-value stages of the problem

  // One piece of work: kept-value stages [Tb, Tb + nT) of output tile (tm, tn),
  // whose epilogue writes to d.
  auto work = [&](int tm, int tn, int Tb, int nT, const EpiDst& d) {
  const int64_t m0 = (int64_t)tm * SP_BM, n0 = (int64_t)tn * SP_BN;
  const int64_t rows = min(p.M - m0, (int64_t)SP_BM);
  const int64_t Kc = p.K / 2;  // kept values per row
  const int nwords = (int)((p.K + 31) / 32);

  auto stA = [&](int T) { return smem + (T & 1) * A_STAGE; };
  // B half c of step u
  auto stBh = [&](int c, int u) { return smem + 2 * A_STAGE + (2 * c + (u & 1)) * SP_BH_STAGE; };
  // index block b (kept-value stages [SPB b, SPB b + SPB) of the problem)
  auto stIB = [&](int b) { return smem + 2 * A_STAGE + 4 * SP_BH_STAGE + (b & 1) * I_BLOCK; };

  // every wave loads half of the kept values (instructions 4 grp .. 4 grp + 3)
  // and the other group's half of B; group 0 also loads the index words
  LdA la;
  la.init(p.Ac + m0 * p.lda_c * EB, (uint32_t)(rows * p.lda_c * EB), p.lda_c, Kc, q, lane);
  BHalfLoader<EB, LB> lb;
  lb.init(p.B, n0, 1 - grp, p.N, p.K, p.ldb, q, lane);
  // Index words: block b holds words [16 b, 16 b + 16) of each of the tile's rows,
  // 64 bytes per row, in 16 load instructions of 16 rows (4 lanes per row, 16 bytes
  // each).  LDS row r of a block keeps its 16-byte chunk c (the words of stage
  // SPB b + c / CPR) at position (c + r / 4) mod 4, so that the 16 rows that one
  // LDS cycle of 16-byte reads serves fall in 16 different bank groups; the
  // rotation is applied on the global side (lane l of an instruction, at
  // position l mod 4 of row l / 4, fetches the chunk that belongs there).  Group 0
  // loads part t = S mod SPB of block S / SPB + 1 while stage S is current
  // (instructions t 16 / SPB + II q + i of wave q), so a block is complete two
  // slots before its first stage is read; the first block of a piece, and the
  // parts of the next block that belong to stages before the piece, are loaded
  // with the first stage.
  constexpr int CPR = IWB / 16;  // 16-byte chunks per row and stage
  const __amdgpu_buffer_rsrc_t rs_idx =
      make_rsrc((const char*)(p.idx + m0 * p.ld_idx), (uint32_t)(rows * p.ld_idx * 4));
  const int ilr = lane >> 2;                    // row within an instruction's 16
  const int ichunk = ((lane & 3) - (ilr >> 2)) & 3;  // chunk this lane fetches
  const uint32_t ioff = (uint32_t)(ilr * p.ld_idx * 4 + ichunk * 16);
  const uint32_t istride = (uint32_t)(16 * p.ld_idx * 4);  // bytes per instruction (16 rows)
  auto issueIpart = [&](int b, int t) {
#pragma unroll
    for (int i = 0; i < II; ++i) {
      const int k = t * (16 / SPB) + II * q + i;
      // chunks that start past the last index word read zeros; a chunk that
      // straddles it reads the row's next words, which only cover groups past K
      // (their kept values are zero)
      const uint32_t o = 16 * b + 4 * ichunk < nwords ? ioff + (uint32_t)k * istride + (uint32_t)(64 * b) : BUF_OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_idx, (__attribute__((address_space(3))) void*)(stIB(b) + k * 1024), 16, o, 0, 0, 0);
    }
  };
  auto issueA = [&](int T) { la.issue(stA(T), Tb + T, 4 * grp, 4, q); };
  // while kept-value stage T of the piece is current: the next block's part
  auto issueI = [&](int T) {
    const int S = Tb + T;
    issueIpart(S / SPB + 1, S % SPB);
  };
  auto issueB = [&](int u) { lb.issue(stBh(1 - grp, u), 2 * Tb + u, q); };  // the other group's half

  acc_t acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = acc_t{};

  i32x4 fa[2][WTM];
  i32x8 fb[2][WTN];
  int fi[2][WTM];
  int fi_next[2][WTM];  // 16-bit: the second step's codes, from the first step's read of the stage's record
  // fragments of step u = 2T + h (KB dense k): instruction s covers kept bytes
  // [64h + 32s, +32) of stage T and B bytes [64s, +64) of step u.  Index codes:
  // 16-bit elements use half g of word 2h + s (32 dense k per instruction),
  // 8-bit elements word 4h + 2s + g (64 dense k per instruction).
  // this lane's index row rbA + (lane & 31) of a block (rows 32 i further add 32 i 64
  // bytes; their rotation is the same, 32 i / 4 being a multiple of 4)
  const int ibase = (rbA + (lane & 31)) * 64;
  const int irot = (lane & 31) >> 2;
  auto read_frags = [&](int u) {
    const int T = u >> 1, h = u & 1;
    const int S = Tb + T;
    // the stage's chunk (8-bit: the step's) in its block, at its rotated position
    const int c = (S % SPB) * CPR + (CPR == 2 ? h : 0);
    const lds_char* ib = stIB(S / SPB) + ibase + (((c + irot) & 3) << 4);
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      if constexpr (EB == 2 && !SK) {
        // one 16-byte record per row and stage: words 0, 1 for the first step,
        // 2, 3 for the second, which keeps them from this read (the stream-K form
        // reads it in both steps: the 8 more registers made it spill)
        if (h == 0) {
          const i32x4 w = *(const __attribute__((address_space(3))) i32x4*)(ib + 32 * i * 64);
          fi[0][i] = (int)((uint32_t)w.x >> (16 * g));
          fi[1][i] = (int)((uint32_t)w.y >> (16 * g));
          fi_next[0][i] = (int)((uint32_t)w.z >> (16 * g));
          fi_next[1][i] = (int)((uint32_t)w.w >> (16 * g));
        } else {
          fi[0][i] = fi_next[0][i];
          fi[1][i] = fi_next[1][i];
        }
      } else if constexpr (EB == 2) {
        const i32x4 w = *(const __attribute__((address_space(3))) i32x4*)(ib + 32 * i * 64);
        fi[0][i] = (int)((uint32_t)(h ? w.z : w.x) >> (16 * g));
        fi[1][i] = (int)((uint32_t)(h ? w.w : w.y) >> (16 * g));
      } else {
        const i32x4 w = *(const __attribute__((address_space(3))) i32x4*)(ib + 32 * i * 64);
        fi[0][i] = g ? w.y : w.x;
        fi[1][i] = g ? w.w : w.z;
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) fa[s][i] = RA::read16k(stA(T), rbA + 32 * i, 64 * h + 32 * s + 16 * g, lane);
    }
    if constexpr (LB == LAYOUT_K) {
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const i32x4 lo = RB::read16k(stBh(grp, u), rbBh + 32 * j, 64 * s + 16 * g, lane);
          const i32x4 hi = RB::read16k(stBh(grp, u), rbBh + 32 * j, 64 * s + 32 + 16 * g, lane);
          fb[s][j] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
    } else {
      // transposing reads in one inline-asm block, after the ordinary reads above
      // (lds_read_tr_x4): per block j and step s, the reads of lo lie at rows r and
      // r + 4 (16-bit) or r + 8 (8-bit), those of hi 16 or 32 rows further
      constexpr int TRW = 128 * EB;  // bytes per LDS row (one k) of a B half
      constexpr int O1 = EB == 2 ? 4 * TRW : 8 * TRW, O2 = EB == 2 ? 16 * TRW : 32 * TRW;
      uint32_t ad[2 * WTN];
      i32x2 r[2 * WTN][4];
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s) ad[2 * j + s] = RB::mn_addr(stBh(grp, u), rbBh + 32 * j, 64 * s + 16 * g, lane);
      lds_read_tr_x4<EB, O1, O2, O1 + O2>(ad, r);
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const i32x2(&q)[4] = r[2 * j + s];
          fb[s][j] = i32x8{q[0].x, q[0].y, q[1].x, q[1].y, q[2].x, q[2].y, q[3].x, q[3].y};
        }
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
  // Kept-value stage T is last read in slot 4T + 2; group 0 loads its half of
  // stage T + 2 and a part of the next index block in slot 4T + 3, group 1 the
  // other half in slot 4T + 4.  Every wave waits for its loads at
  // the end of its memory phases, just early enough for their first reader.
  // Loads past K read nothing and fill their stage with zeros (an odd number
  // of steps is padded with one such zero step).
  if (grp == 0) {
    issueB(0);
    issueA(0);
    // the piece's first index block, and the parts of the next one that belong
    // to stages before the piece (the loop loads the rest)
    const int b0 = Tb / SPB, p0 = Tb % SPB;
    for (int t = 0; t < SPB; ++t) issueIpart(b0, t);
    for (int t = 0; t < p0; ++t) issueIpart(b0 + 1, t);
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
      issueI(T);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(8 + II) : "memory");  // group 1's half of B(u)
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

  // epilogue: the sparse (A) fragment is the instruction's first operand, so
  // element (i', j') of its 32 x 32 accumulator layout is D[m][n] with m = i',
  // n = j' within the block: block (i, j), register r holds
  // D[em0 + rbA + 32 i + i'][en0 + rbB + 32 j + j'], (i', j') = ACC::coord(lane, r)
  using ACC = frag::Acc<frag::ACC_32x32>;
  const int64_t em0 = d.m0, en0 = d.n0;  // the tile's first element in the destination (D, or a workspace slot)
  const bool interior = em0 + SP_BM <= d.M && en0 + SP_BN <= d.N;
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int64_t n = en0 + rbB + 32 * j + ACC::coord(lane, 0).j;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = em0 + rbA + 32 * i + ACC::coord(lane, r).i;
        if (!interior && (m >= d.M || n >= d.N)) continue;
        const int64_t off = m * d.ld + n;
        if constexpr (Op::INT_ACC) {
          const uint32_t c = d.use_c ? (uint32_t)((const int*)d.C)[off] : 0u;
          ((int*)d.D)[off] = (int)((uint32_t)d.alpha_i * (uint32_t)acc[i][j][r] + (uint32_t)d.beta_i * c);
        } else {
          combine_store(d.C, d.D, off, acc[i][j][r], d.alpha, d.beta, d.use_c, d.out);
        }
      }
    }
  };  // work

  if constexpr (!SK) {
    // XCD-aware, grouped tile order over all tiles, or over the first dp_tiles
    // tiles when the rest are left to the stream-K form
    int tm, tn;
    tile_coords_of<4>(blockIdx.x, p.dp_tiles > 0 ? p.dp_tiles : p.tiles_m * p.tiles_n, p.tiles_m, p.tiles_n, tm, tn);
    work(tm, tn, 0, nT_all,
         EpiDst{p.D, p.C, p.ldc, p.M, p.N, (int64_t)tm * SP_BM, (int64_t)tn * SP_BN, p.alpha, p.beta, p.alpha_i,
                p.beta_i, p.use_c, p.vec_cd, p.out});
  } else {
    // Workgroup w takes kept-value stages [w L, (w + 1) L) of the tiles after the
    // first dp_tiles, numbered tile by tile; a piece that is a whole tile is
    // stored to D, any other piece stores its raw sums to its own workspace slot.
    const int64_t w = blockIdx.x;
    const int64_t L = p.sk_iters;
    int64_t it = w * L;
    const int64_t end = min(it + L, (int64_t)p.sk_tiles * nT_all);
    int64_t piece = sk_first_piece(w, L, nT_all, p.sk_period);
    for (int pc = 0; it < end; ++pc) {
      const int64_t x = it / nT_all;
      const int Tbeg = (int)(it - x * nT_all);
      const int Tcnt = (int)min((int64_t)(nT_all - Tbeg), end - it);
      int tm, tn;
      {
        int m, n;
        grouped_tile<4>(p.dp_tiles + (int)x, p.tiles_m, p.tiles_n, m, n);
        tm = __builtin_amdgcn_readfirstlane(m);
        tn = __builtin_amdgcn_readfirstlane(n);
      }
      if (pc > 0) barrier_lds();  // the previous piece is done with the LDS
      const bool whole = Tbeg == 0 && Tcnt == nT_all;
      const EpiDst d = whole ? EpiDst{p.D, p.C, p.ldc, p.M, p.N, (int64_t)tm * SP_BM, (int64_t)tn * SP_BN, p.alpha,
                                      p.beta, p.alpha_i, p.beta_i, p.use_c, p.vec_cd, p.out}
                             : EpiDst{(char*)p.ws + piece * (int64_t)(SP_BM * SP_BN * 4), nullptr, SP_BN, SP_BM,
                                      SP_BN, 0, 0, 1.0f, 0.0f, 1, 0, 0, 1, OUT_32};
      work(tm, tn, Tbeg, Tcnt, d);
      it += Tcnt;
      ++piece;
    }
  }
}

template <class Op, int LB, bool SK = false>
static hipError_t launch_sparse_fast_one(const SparseArgs& a0, hipStream_t s) {
  SparseArgs a = a0;
  a.tiles_m = (int)((a.M + SP_BM - 1) / SP_BM);
  a.tiles_n = (int)((a.N + SP_BN - 1) / SP_BN);
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  if (tiles <= 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (!SK || a.dp_tiles > 0) {  // whole tiles: every tile, or the first dp_tiles
    hipLaunchKernelGGL((gemm_sparse_fast_kernel<Op, LB, false>), dim3((unsigned)(SK ? a.dp_tiles : tiles)),
                       dim3(SP_THREADS), 0, s, a);
    e = hipGetLastError();
  }
  if constexpr (SK) {
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_sparse_fast_kernel<Op, LB, true>), dim3((unsigned)a.sk_wgs), dim3(SP_THREADS), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the fixup of the dense form, on the sparse launch's epilogue arguments
    DenseArgs f{};
    f.C = a.C;
    f.D = a.D;
    f.M = a.M;
    f.N = a.N;
    f.ldc = a.ldc;
    f.alpha = a.alpha;
    f.beta = a.beta;
    f.alpha_i = a.alpha_i;
    f.beta_i = a.beta_i;
    f.use_c = a.use_c;
    f.vec_cd = a.vec_cd;
    f.out = a.out;
    f.tiles_m = a.tiles_m;
    f.tiles_n = a.tiles_n;
    f.dp_tiles = a.dp_tiles;
    f.sk_tiles = a.sk_tiles;
    f.sk_wgs = a.sk_wgs;
    f.sk_iters = a.sk_iters;
    f.sk_period = a.sk_period;
    f.ws = a.ws;
    const int64_t nT = (a.K + SpGeom<Op::EB>::KA - 1) / SpGeom<Op::EB>::KA;
    e = launch_streamk_fixup(f, nT, Op::INT_ACC, s);
  }
  return e;
}

}  // namespace fast

bool sparse_fast_ok(int dtA, int layoutB, const SparseArgs& a) {
  const int64_t eb = (dtA == DT_BF16 || dtA == DT_F16) ? 2 : 1;
  // 16-byte chunks of kept values (16 / eb values = 32 / eb dense k) and of B
  // never straddle the end of K when K * eb % 32 == 0; index words are fetched
  // 16 bytes at a time from 4-byte aligned rows (a chunk that runs past a row's
  // last word reads codes only for groups past K, whose kept values are zero).
  // Native fp8 only from the accuracy threshold on (below
  // it fp8 is widened to bf16 by the general kernel).
  auto al = [](const void* q, int64_t n) { return ((uintptr_t)q % (uintptr_t)n) == 0; };
  const bool aligned = al(a.Ac, 16) && al(a.B, 16) && al(a.idx, 4) && (a.lda_c * eb) % 16 == 0 &&
                       (a.ldb * eb) % 16 == 0;
  if (!aligned || a.K == 0 || (a.K * eb) % 32 != 0) return false;
  if ((dtA == DT_E4M3 || dtA == DT_E5M2) && a.K < FP8_NATIVE_MIN_K) return false;
  if (a.M < fast::SP_BM || a.N < fast::SP_BN) return false;
  // every buffer window (and offset into it) must stay below 2 GiB;
  // MN-contiguous B offsets advance by whole stages, up to 4 stages past K
  const int64_t lim = (int64_t)1 << 31;
  const int64_t kpad = 4 * 128 / eb;
  const int64_t wa = (int64_t)fast::SP_BM * a.lda_c * eb;
  const int64_t wi = (int64_t)fast::SP_BM * a.ld_idx * 4;
  const int64_t wb = layoutB == LAYOUT_K ? (int64_t)fast::SP_BN * a.ldb * eb : (a.K + kpad) * a.ldb * eb;
  const int64_t tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  return wa < lim && wi < lim && wb < lim && tiles <= 0x7fffffff;
}

template <class Op, bool SK>
static hipError_t launch_sparse_fast_layouts(int layoutB, const SparseArgs& a, hipStream_t s) {
  return layoutB == LAYOUT_K ? fast::launch_sparse_fast_one<Op, LAYOUT_K, SK>(a, s)
                             : fast::launch_sparse_fast_one<Op, LAYOUT_MN, SK>(a, s);
}

template <bool SK>
static hipError_t launch_sparse_fast_sk_or_not(int dtA, int dtB, int layoutB, const SparseArgs& a, hipStream_t s) {
  using namespace fast;
  if (dtA == DT_BF16) return launch_sparse_fast_layouts<Sp32BF16, SK>(layoutB, a, s);
  if (dtA == DT_F16) return launch_sparse_fast_layouts<Sp32F16, SK>(layoutB, a, s);
  if (dtA == DT_I8) return launch_sparse_fast_layouts<Sp32I8, SK>(layoutB, a, s);
  const int fa = f8fmt(dtA), fb = f8fmt(dtB);
  if (fa == 0 && fb == 0) return launch_sparse_fast_layouts<Sp32F8<0, 0>, SK>(layoutB, a, s);
  if (fa == 0 && fb == 1) return launch_sparse_fast_layouts<Sp32F8<0, 1>, SK>(layoutB, a, s);
  if (fa == 1 && fb == 0) return launch_sparse_fast_layouts<Sp32F8<1, 0>, SK>(layoutB, a, s);
  return launch_sparse_fast_layouts<Sp32F8<1, 1>, SK>(layoutB, a, s);
}

hipError_t launch_sparse_fast(int dtA, int dtB, int layoutB, const SparseArgs& a, hipStream_t s) {
  return launch_sparse_fast_sk_or_not<false>(dtA, dtB, layoutB, a, s);
}

hipError_t launch_sparse_fast_sk(int dtA, int dtB, int layoutB, const SparseArgs& a, hipStream_t s) {
  if (a.sk_tiles <= 0 || a.ws == nullptr) return hipErrorInvalidValue;
  return launch_sparse_fast_sk_or_not<true>(dtA, dtB, layoutB, a, s);
}

}  // namespace mcg
