// gemm_fast_kernel.hpp -- the pipelined dense MFMA kernel template, shared by the
// translation units that instantiate its two tile sizes (gemm_fast.hip: 256 x 256 and the
// host-side choice; gemm_fast_mid.hip: 128 x 128).  It is the fast path of gemm_dense
// for aligned problems of at least 256 x 256, and in its 128 x 128 form for aligned
// problems with too few 256 x 256 tiles to fill the chip.
//
// Same operation as gemm_dense.hip (the matrix fused multiply-add of "Accurate
// Models of AMD Matrix Cores", Section 2, Eq. (1), tiled over K as in "CDNA3
// dense MFMA builtins", Using MFMA builtins as a compute policy); what differs
// is the mapping onto CDNA4:
//   - 256 x 256 output tile per workgroup of 8 wavefronts, two per SIMD
//     (wavefronts w and w + 4 share a SIMD, measured).  Each wavefront owns a
//     128 x 64 sub-tile = 4 x 2 instructions of 32 x 32 (128 accumulator
//     registers per lane).
//   - K is staged in tiles of 128 bytes per row (64 bf16 / 128 8-bit values),
//     so that every 8 lanes of a load fetch one whole 128-byte line: twice the
//     bytes per outstanding L1 miss of a 64-byte tile, which measured as the
//     limit of the HBM -> LDS stream.  A has 2 LDS stages and B 3 (32 KiB each,
//     160 KiB), filled by buffer_load ... lds (16 bytes per lane, no VGPRs).
//     The XOR swizzle of the LDS rows is folded into the global address each
//     lane loads; chunks outside the matrix get an out-of-range offset and the
//     buffer unit writes zeros.
//   - ping-pong schedule: the two wavefronts of a SIMD alternate between a
//     multiply phase (only matrix instructions, on fragments already in
//     registers) and a memory phase (LDS -> register reads of the next half K
//     tile's fragments and 4 DMA issues per wave), separated by workgroup
//     barriers, so that one of them keeps the SIMD's matrix core busy while
//     the other waits on memory.
//   - epilogue: a lane's accumulators hold 4 consecutive columns of one row
//     (each instruction is issued with the B fragment as its first operand).
//     Interior tiles pass each wavefront's 32 x 64 blocks through LDS, so that 16
//     lanes read C and write D = alpha * acc + beta * C along one row segment
//     (whole lines: storing from the accumulator layout wrote 32 rows x 16 or 32
//     bytes per instruction, and the fixed cost of the launch was twice that of a
//     line-wise store); edge tiles use per-element bounds.
//   - the 8 XCDs receive workgroups round-robin; the tile sequence is permuted
//     so that the workgroups resident on one XCD cover a compact block of tiles.
//   - 128 x 128 form: the two wavefronts of a SIMD cover the same 64 x 64
//     quadrant and split every K tile (one half each), so a phase holds 8
//     instructions and a K tile 2 barriers; 4 stages of A and of B (16 KiB each)
//     with a prefetch distance of 3 tiles; at the end each wave hands its partner
//     the 32-row block the partner stores, through LDS.  128 KiB of LDS: one
//     workgroup per CU.  The host takes it for problems with too few 256 x 256
//     tiles when its cost model puts it ahead of the general kernel.
// Preconditions (checked on the host): 16-byte aligned operands, K * elem_bytes
// and ld * elem_bytes multiples of 16, M, N >= the tile size, and each workgroup's
// operand window below 2 GiB (32-bit buffer offsets).
#pragma once
#include "fast_tiles.hpp"
#include "frag_layout.hpp"
#include "gemm_kernels.hpp"

namespace mcg {
namespace fast {

constexpr int KTB = 128;     // bytes of K per LDS row and stage: one 128-byte line per row
constexpr int NSA = 2;       // LDS stages of A
constexpr int NSB = 3;       // LDS stages of B
constexpr int THREADS = 512;

// TB: output tile TB x TB (256, or 128 for problems with too few 256 x 256 tiles to
// fill the chip); each wavefront owns (TB / 2) x (TB / 4) outputs.  SK: the
// stream-K form, whose workgroups each take a range of the K
// iterations of the tiles after the first dp_tiles, which a launch of the
// whole-tile form covers.
template <class Op, int LA, int LB, int TB, bool SK = false>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_fast_kernel(DenseArgs p) {
  constexpr int BM = TB, BN = TB;
  constexpr int SB = TB * KTB;          // bytes of one operand stage
  constexpr int EB = Op::EB;
  constexpr int LB16 = Op::LANE_BYTES;  // bytes of K per lane and instruction (16 or 32)
  constexpr int S = 64 / (2 * LB16);    // instructions per block and half K tile
  // KS (128 x 128 tiles): the two wavefronts of a SIMD cover the same 64 x 64 quadrant
  // and split every K tile, each multiplying one half; otherwise each covers half of
  // the quadrant's columns over all of K
  constexpr bool KS = TB == 128;
  constexpr int WTM = TB / 64, WTN = KS ? 2 : TB / 128;  // 32 x 32 instruction tiles per wave
  // KS: prefetch distance KPD for both operands (KPD + 1 stages each, 128 KiB of LDS;
  // measured 3-15% faster than distance 2 over 1024..3072-row outputs, distance 4 slower)
  constexpr int KPD = 3;
  constexpr int NA = KS ? KPD + 1 : NSA;  // LDS stages of A
  constexpr int NB = KS ? KPD + 1 : NSB;  // LDS stages of B
  using GA = Geom<EB, LA, BM, KTB>;
  using GB = Geom<EB, LB, BN, KTB>;
  using RA = Reader<EB, LA, BM, KTB>;
  using RB = Reader<EB, LB, BN, KTB>;
  using LdA = LineLoader<EB, LA, BM, KTB>;
  using LdB = LineLoader<EB, LB, BN, KTB>;
  using acc_t = typename Op::acc_t;
  using frag_t = typename Op::frag_t;
  using v4 = typename std::conditional<Op::INT_ACC, i32x4, f32x4>::type;
  using s1 = typename std::conditional<Op::INT_ACC, int, float>::type;
  static_assert(TB == 256 || TB == 128, "tile");
  static_assert(GA::BYTES == SB && GB::BYTES == SB, "one stage size for both operands");
  constexpr int LH = LdA::INSTR / 2;  // loads per wave, operand and half stage (one group's share)
  static_assert(LdA::INSTR == LdB::INSTR && (LH == 4 || LH == 2), "vmcnt bookkeeping");

  __shared__ __attribute__((aligned(1024))) char smem_raw[(NA + NB) * SB];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: multiplies in even slots; 1: in odd slots
  const int q = wave & 3;     // wavefronts q and q + 4 share a SIMD and a quadrant of the tile
  const int rbA = (q >> 1) * (TB / 2), rbB = (q & 1) * (TB / 2) + (KS ? 0 : grp * (TB / 4));
  const int g = lane >> 5;

  const int nk_all = (int)((p.K + KTB / EB - 1) / (KTB / EB));  // K tiles of the problem

  // One piece of work: K tiles [kb, kb + nk) of output tile (tm, tn), whose
  // epilogue writes to d.
  auto work = [&](int tm, int tn, int kb, int nk, const EpiDst& d) {
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  LdA la;
  LdB lb;
  if constexpr (LA == LAYOUT_K)
    la.init(p.A + m0 * p.lda * EB, (uint32_t)(min(p.M - m0, (int64_t)BM) * p.lda * EB), p.lda, p.K, q, lane);
  else
    la.init(p.A + m0 * EB, (uint32_t)((p.K * p.lda - m0) * EB), p.lda, p.K, q, lane);
  if constexpr (LB == LAYOUT_K)
    lb.init(p.B + n0 * p.ldb * EB, (uint32_t)(min(p.N - n0, (int64_t)BN) * p.ldb * EB), p.ldb, p.K, q, lane);
  else
    lb.init(p.B + n0 * EB, (uint32_t)((p.K * p.ldb - n0) * EB), p.ldb, p.K, q, lane);

  acc_t acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = acc_t{};

  auto stA = [&](int kt) { return smem + (KS ? kt % NA : kt & 1) * SB; };
  auto stB = [&](int kt) { return smem + NA * SB + (kt % NB) * SB; };
  // this group's half (LH of the 2 LH load instructions per wave) of operand X of K tile kt
  const int ihalf = LH * grp;
  auto issueA = [&](int kt) { la.issue(stA(kt), kb + kt, ihalf, LH, q); };
  auto issueB = [&](int kt) { lb.issue(stB(kt), kb + kt, ihalf, LH, q); };

  frag_t fa[S][WTM], fb[S][WTN];
  // fragments of half h (K bytes [64h, 64h + 64) of each row) of K tile kt;
  // instruction s of the half takes lane group g's bytes [64h + 2 LB16 s + LB16 g, +LB16).
  // K-contiguous operands take ordinary LDS reads; MN-contiguous ones take their
  // transposing reads in inline-asm blocks (lds_read_tr_x4), issued after the
  // ordinary reads.  A lane's 4 transposing reads of a 32-row block lie TR_O1,
  // TR_O2, TR_O3 bytes after the first: the second read of a 16-byte part is 4
  // (16-bit) or 8 (8-bit) rows further, the next part 16 or 32 rows.
  constexpr int TRW = TB * EB;  // bytes per LDS row (one k) of an MN-contiguous tile
  constexpr int TR_O1 = EB == 2 ? 4 * TRW : 8 * TRW;
  constexpr int TR_O2 = (LB16 == 32 || EB == 2) ? 16 * TRW : 32 * TRW;
  constexpr int TR_O3 = TR_O2 + TR_O1;
  constexpr int NTA = LA == LAYOUT_MN ? WTM : 0, NTB = LB == LAYOUT_MN ? WTN : 0;
  auto unpack = [&](const i32x2 (&r)[4], frag_t& f0, frag_t& f1) {
    if constexpr (LB16 == 16) {
      f0 = frag_t{r[0].x, r[0].y, r[1].x, r[1].y};
      f1 = frag_t{r[2].x, r[2].y, r[3].x, r[3].y};
    } else {
      f0 = frag_t{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
    }
  };
  auto read_frags = [&](int kt, int h) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int kb = 64 * h + 2 * LB16 * s + LB16 * g;
      if constexpr (LA == LAYOUT_K) {
#pragma unroll
        for (int i = 0; i < WTM; ++i) {
          if constexpr (LB16 == 16) {
            fa[s][i] = RA::read16k(stA(kt), rbA + 32 * i, kb, lane);
          } else {
            const i32x4 x = RA::read16k(stA(kt), rbA + 32 * i, kb, lane);
            const i32x4 y = RA::read16k(stA(kt), rbA + 32 * i, kb + 16, lane);
            fa[s][i] = frag_t{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
          }
        }
      }
      if constexpr (LB == LAYOUT_K) {
#pragma unroll
        for (int j = 0; j < WTN; ++j) {
          if constexpr (LB16 == 16) {
            fb[s][j] = RB::read16k(stB(kt), rbB + 32 * j, kb, lane);
          } else {
            const i32x4 x = RB::read16k(stB(kt), rbB + 32 * j, kb, lane);
            const i32x4 y = RB::read16k(stB(kt), rbB + 32 * j, kb + 16, lane);
            fb[s][j] = frag_t{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
          }
        }
      }
    }
    if constexpr (NTA + NTB > 0) {
      const int kb0 = 64 * h + LB16 * g;
      uint32_t ad[NTA + NTB];  // one block: 2, 4 or 6 addresses
      i32x2 r[NTA + NTB][4];
      if constexpr (NTA > 0)
#pragma unroll
        for (int i = 0; i < NTA; ++i) ad[i] = RA::mn_addr(stA(kt), rbA + 32 * i, kb0, lane);
      if constexpr (NTB > 0)
#pragma unroll
        for (int j = 0; j < NTB; ++j) ad[NTA + j] = RB::mn_addr(stB(kt), rbB + 32 * j, kb0, lane);
      lds_read_tr_x4<EB, TR_O1, TR_O2, TR_O3>(ad, r);
#pragma unroll
      for (int i = 0; i < NTA; ++i) unpack(r[i], fa[0][i], fa[S - 1][i]);
#pragma unroll
      for (int j = 0; j < NTB; ++j) unpack(r[NTA + j], fb[0][j], fb[S - 1][j]);
    }
  };
  auto multiply = [&]() {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j) Op::mma(acc[i][j], fb[s][j], fa[s][i]);
  };
  // Memory phase of half tile (t, H): this group's DMA half and the fragment
  // reads.  The DMA targets another stage than the reads, so it goes first (more
  // time in flight), except with both operands MN-contiguous, where the reads go
  // first (measured: 1-2% faster there and 18% less HBM traffic at bf16 8192^3,
  // 1-2% slower with one MN-contiguous operand).
  auto mem = [&](auto hc, int t) {
    if constexpr (LA == LAYOUT_MN && LB == LAYOUT_MN) read_frags(t, decltype(hc)::value);
    if constexpr (decltype(hc)::value == 0) issueA(t + 1);
    else issueB(t + 2);
    if constexpr (!(LA == LAYOUT_MN && LB == LAYOUT_MN)) read_frags(t, decltype(hc)::value);
  };

  // Half tiles u = 2t + h.  Group 0 reads half u in slot 2u - 1 and multiplies
  // it in slot 2u; group 1 reads it in slot 2u and multiplies it in slot
  // 2u + 1; slots are separated by workgroup barriers.  K tile t (A stage
  // t % 2, B stage t % 3) is last read in slot 4t + 2 and first needed in slot
  // 4t + 3 (= 4(t+1) - 1 for tile t + 1).  DMA halves, 4 instructions per wave
  // in every memory phase:
  //   slot 4t     (group 1): second half of A(t+1)  -> A stage of tile t-1, free since slot 4t-1
  //   slot 4t + 1 (group 0): first half of B(t+2)   -> B stage of tile t-1
  //   slot 4t + 2 (group 1): second half of B(t+2)
  //   slot 4t + 3 (group 0): first half of A(t+2)   -> A stage of tile t, free since slot 4t+3
  // At the end of slot 4t + 2 each wave waits until only its newest LH loads
  // (its half of B(t+2)) are in flight, so tile t+1 is complete from slot 4t+3.
  // DMA of tiles at or beyond nk read nothing and fill their stage with zeros.
  if constexpr (KS) {
    // Group g reads half g of K tile t in slot 2t - 1 + g and multiplies it in the
    // next slot.  Each memory phase issues this wave's shares of A(t+KPD) and
    // B(t+KPD) into the stages of tile t-1 (stage index mod KPD + 1; last read in
    // slot 2t - 2); at the end of slot 2t each wave waits until only the loads of
    // tiles t+2 .. t+KPD ((KPD - 1) 2 LH) are in flight, so tile t+1 is complete
    // from slot 2t + 1.
#pragma unroll
    for (int t0 = 0; t0 < KPD; ++t0) {
      issueA(t0);
      issueB(t0);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((KPD - 1) * 2 * LH) : "memory");  // own shares of tile 0
    barrier_lds();
    if (grp == 0) {
      for (int t = 0; t < nk; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        issueA(t + KPD);
        issueB(t + KPD);
        read_frags(t, 0);  // slot 2t - 1
        barrier_lds();
        __builtin_amdgcn_sched_barrier(0);
        multiply();  // slot 2t
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((KPD - 1) * 2 * LH) : "memory");  // own shares of tile t+1
        barrier_lds();
      }
    } else {
      barrier_lds();  // slot -1
      for (int t = 0; t < nk; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        issueA(t + KPD);
        issueB(t + KPD);
        read_frags(t, 1);  // slot 2t
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((KPD - 1) * 2 * LH) : "memory");  // own shares of tile t+1
        barrier_lds();
        __builtin_amdgcn_sched_barrier(0);
        multiply();  // slot 2t + 1
        __builtin_amdgcn_sched_barrier(0);
        if (t + 1 < nk) barrier_lds();
      }
    }
  } else {
  issueB(0);
  issueA(0);
  issueB(1);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LH) : "memory");  // own shares of tile 0 have landed
  barrier_lds();
  // The two half tiles of a K tile are written out (no run-time choice between
  // the A and B loads, whose buffer descriptors then stay in scalar registers).
  if (grp == 0) {
    for (int t = 0; t < nk; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      mem(std::integral_constant<int, 0>{}, t);  // slot 4t - 1
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      multiply();  // slot 4t
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      mem(std::integral_constant<int, 1>{}, t);  // slot 4t + 1
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      multiply();  // slot 4t + 2
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LH) : "memory");  // own shares of tile t+1
      barrier_lds();
    }
  } else {
    barrier_lds();  // slot -1
    for (int t = 0; t < nk; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      mem(std::integral_constant<int, 0>{}, t);  // slot 4t
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      multiply();  // slot 4t + 1
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      mem(std::integral_constant<int, 1>{}, t);  // slot 4t + 2
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LH) : "memory");  // own shares of tile t+1
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      multiply();  // slot 4t + 3
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < nk) barrier_lds();
    }
  }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS DMA outstanding at exit
  if constexpr (KS) {
    // Sum the two K halves: wave w hands its partner (w ^ 4) the 32-row block
    // i = 1 - grp, which the partner stores, through 8 KiB of LDS per wave.
    using e1 = typename std::conditional<Op::INT_ACC, int, float>::type;
    typedef __attribute__((address_space(3))) e1 lds_e1;
    barrier_lds();  // all LDS DMA has landed; no fragment reads remain
    lds_e1* mine = (lds_e1*)(smem + wave * 8192);
    const lds_e1* theirs = (const lds_e1*)(smem + (wave ^ 4) * 8192);
    auto put = [&](const acc_t (&blk)[WTN]) {
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(j * 16 + r) * 64 + lane] = blk[j][r];
    };
    auto add = [&](acc_t (&blk)[WTN]) {
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (Op::INT_ACC)
            blk[j][r] = (int)((uint32_t)blk[j][r] + (uint32_t)theirs[(j * 16 + r) * 64 + lane]);
          else
            blk[j][r] += theirs[(j * 16 + r) * 64 + lane];
        }
    };
    if (grp == 0) put(acc[1]);
    else put(acc[0]);
    barrier_lds();
    if (grp == 0) add(acc[0]);
    else add(acc[1]);
  }

  // epilogue: each instruction multiplied (B fragment) x (A fragment), so element
  // (i', j') of its 32 x 32 accumulator layout is D[m][n] with m = j' and n = i'
  // within the block: block (i, j), register 4 r4 + r of a lane holds
  // D[em0 + rbA + 32 i + j'][en0 + rbB + 32 j + i' + r], (i', j') = ACC::coord(lane, 4 r4),
  // i.e. 4 consecutive columns of one row per register group r4; (em0, en0) is the
  // tile's first element in the destination (D, or a workspace slot)
  using ACC = frag::Acc<frag::ACC_32x32>;
  const int64_t em0 = d.m0, en0 = d.n0;
  const int acc_m = ACC::coord(lane, 0).j;  // m within a block
  auto acc_n = [&](int r4) { return ACC::coord(lane, 4 * r4).i; };  // first n of register group r4
  const bool vec_ok = d.vec;
  const s1* C = (const s1*)d.C;
  s1* D = (s1*)d.D;
  if constexpr (Op::INT_ACC) {
    // wrapping alpha * acc, in place (keeps the products out of the C batches)
    if (d.alpha_i != 1) {
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = (int)((uint32_t)d.alpha_i * (uint32_t)acc[i][j][r]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  auto combine = [&](const acc_t& a, int r4, const v4& c, bool use_c) {
    v4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (Op::INT_ACC)
        o[r] = (int)((uint32_t)a[4 * r4 + r] + (use_c ? (uint32_t)d.beta_i * (uint32_t)c[r] : 0u));
      else
        o[r] = use_c ? __builtin_fmaf(d.alpha, a[4 * r4 + r], d.beta * c[r]) : d.alpha * a[4 * r4 + r];
    }
    return o;
  };
  if (vec_ok && em0 + BM <= d.M && en0 + BN <= d.N) {
    // Interior tile.  Each wavefront passes the 32 x 64 block of its row group i
    // (KS: the one block it stores) through LDS (8 KiB; two buffers for the 256 x 256
    // form, one for the 128 x 128 form), so that 16 lanes then read C and write D
    // along one row segment (256 bytes of binary32 / int32, 128 of 16-bit values):
    // whole lines per store instruction instead of 32 rows x 16 or 32 bytes.
    // Chunk ch (16 bytes) of staging row r sits at ch ^ (r & 15): the writes (32
    // rows at one chunk) and the reads (4 rows x 16 chunks) are free of bank conflicts.
    // all LDS DMA has landed (vmcnt(0) above) and no fragment reads remain; KS: the
    // partner has read the block this wave handed it, in the same LDS
    barrier_lds();
    typedef __attribute__((address_space(3))) v4 lds_v4;
    lds_char* wbuf = smem + wave * (KS ? 8192 : 16384);
    const int wr = lane & 31, rr = lane >> 4, cc = lane & 15;
    const int64_t col = en0 + rbB + 4 * cc;
    const int out = d.out;
    auto combine4 = [&](const v4& a, const v4& c) {
      v4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (Op::INT_ACC)
          o[r] = (int)((uint32_t)a[r] + (d.use_c ? (uint32_t)d.beta_i * (uint32_t)c[r] : 0u));
        else
          o[r] = d.use_c ? __builtin_fmaf(d.alpha, a[r], d.beta * c[r]) : d.alpha * a[r];
      }
      return o;
    };
    // The passes over the row blocks, for binary32 / int32 (O16 false) or 16-bit
    // (O16 true) C and D.  Each pass's C rows are loaded one pass ahead: pass i + 1's
    // loads go out once pass i has staged its accumulators (whose registers they
    // reuse), so their latency overlaps pass i's staging, reads and stores; the first
    // pass's loads go out before any staging.  C is read once, so its loads are
    // non-temporal (they keep the operand panels in the caches: measured 0.75-0.9%
    // faster at 8192^3 with an N(0,1) C, bit-identical).
    auto passes = [&](auto o16) {
      constexpr bool O16 = decltype(o16)::value;
      using cvec = typename std::conditional<O16, i32x2, v4>::type;
      cvec cn[8];
      auto load_c = [&](int i) {
        const int64_t rb = (em0 + rbA + 32 * i + rr) * d.ld + col;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if constexpr (O16)
            cn[t] = __builtin_nontemporal_load((const i32x2*)((const uint16_t*)d.C + rb + 4 * t * d.ld));
          else
            cn[t] = __builtin_nontemporal_load((const v4*)(C + rb + 4 * t * d.ld));
        }
      };
      if (d.use_c) load_c(KS ? grp : 0);
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (KS && i != grp) continue;  // the partner wave stores this row block
        lds_char* buf = wbuf + (KS ? 0 : (i & 1) * 8192);
        const int64_t rbase = (em0 + rbA + 32 * i + rr) * d.ld + col;  // row 4t further: + 4t ldc
        cvec cv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) cv[t] = cn[t];
#pragma unroll
        for (int j = 0; j < WTN; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int ch = (32 * j + acc_n(r4)) / 4;  // 16-byte chunk of the wavefront's 64 columns
            v4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = acc[i][j][4 * r4 + r];
            *(lds_v4*)(buf + wr * 256 + ((ch ^ (wr & 15)) << 4)) = x;
          }
        if (!KS && i + 1 < WTM && d.use_c) load_c(i + 1);
        // the reads below take other lanes' values: wait for the writes
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        v4 a[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int row = 4 * t + rr;
          a[t] = *(const lds_v4*)(buf + row * 256 + ((cc ^ (row & 15)) << 4));
        }
        if constexpr (O16) {
          uint16_t* D16 = (uint16_t*)d.D;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            v4 c = {};
            if (d.use_c) {  // (16-bit D only with binary32 accumulators)
              c[0] = from_out_bits(out, (uint32_t)cv[t].x & 0xffffu);
              c[1] = from_out_bits(out, (uint32_t)cv[t].x >> 16);
              c[2] = from_out_bits(out, (uint32_t)cv[t].y & 0xffffu);
              c[3] = from_out_bits(out, (uint32_t)cv[t].y >> 16);
            }
            const v4 o = combine4(a[t], c);
            *(i32x2*)(D16 + rbase + 4 * t * d.ld) =
                i32x2{(int)(to_out_bits(out, o[0]) | (to_out_bits(out, o[1]) << 16)),
                      (int)(to_out_bits(out, o[2]) | (to_out_bits(out, o[3]) << 16))};
          }
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) *(v4*)(D + rbase + 4 * t * d.ld) = combine4(a[t], d.use_c ? cv[t] : v4{});
        }
      }
    };
    if constexpr (!Op::INT_ACC) {
      if (out != OUT_32) {
        passes(std::true_type{});
        return;
      }
    }
    passes(std::false_type{});
    return;
  }
  if constexpr (!Op::INT_ACC) {
    if (d.out != OUT_32) {
      // bfloat16 / binary16 C and D: 4 consecutive elements = 8 bytes per lane
      // and row segment; the fp32 result is rounded once to the output format
      const int out = d.out;
      const uint16_t* C16 = (const uint16_t*)d.C;
      uint16_t* D16 = (uint16_t*)d.D;
      auto unpack = [&](const i32x2 w) {
        return v4{from_out_bits(out, (uint32_t)w.x & 0xffffu), from_out_bits(out, (uint32_t)w.x >> 16),
                  from_out_bits(out, (uint32_t)w.y & 0xffffu), from_out_bits(out, (uint32_t)w.y >> 16)};
      };
      auto pack = [&](const v4& o) {
        return i32x2{(int)(to_out_bits(out, o[0]) | (to_out_bits(out, o[1]) << 16)),
                     (int)(to_out_bits(out, o[2]) | (to_out_bits(out, o[3]) << 16))};
      };
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (KS && i != grp) continue;  // the partner wave stores this row block
        const int64_t m = em0 + rbA + 32 * i + acc_m;
        if (m >= d.M) continue;
#pragma unroll
        for (int j = 0; j < WTN; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int64_t n = en0 + rbB + 32 * j + acc_n(r4);
            if (n >= d.N) continue;
            const int64_t off = m * d.ld + n;
            const bool full = vec_ok && n + 4 <= d.N;
            v4 c = {};
            if (d.use_c) {
              if (full) c = unpack(*(const i32x2*)(C16 + off));
              else
                for (int r = 0; r < 4; ++r)
                  if (n + r < d.N) c[r] = from_out_bits(out, C16[off + r]);
            }
            const v4 o = combine(acc[i][j], r4, c, d.use_c);
            if (full) {
              *(i32x2*)(D16 + off) = pack(o);
            } else {
              for (int r = 0; r < 4; ++r)
                if (n + r < d.N) D16[off + r] = (uint16_t)to_out_bits(out, o[r]);
            }
          }
      }
      return;
    }
  }
  {
    // edge tile: per-element bounds
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      if (KS && i != grp) continue;  // the partner wave stores this row block
      const int64_t m = em0 + rbA + 32 * i + acc_m;
      if (m >= d.M) continue;
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int64_t n = en0 + rbB + 32 * j + acc_n(r4);
          if (n >= d.N) continue;
          const bool full = vec_ok && n + 4 <= d.N;
          v4 c = {};
          if (d.use_c) {
            if (full) c = *(const v4*)(C + m * d.ld + n);
            else
              for (int r = 0; r < 4; ++r)
                if (n + r < d.N) c[r] = C[m * d.ld + n + r];
          }
          const v4 o = combine(acc[i][j], r4, c, d.use_c);
          if (full) {
            *(v4*)(D + m * d.ld + n) = o;
          } else {
            for (int r = 0; r < 4; ++r)
              if (n + r < d.N) D[m * d.ld + n + r] = o[r];
          }
        }
    }
  }
  };  // work

  if constexpr (!SK) {
    // XCD-aware, grouped tile order over all tiles, or over the first dp_tiles
    // tiles when the rest are left to the stream-K form
    int tm, tn;
    tile_coords_of<4>(blockIdx.x, p.dp_tiles > 0 ? p.dp_tiles : p.tiles_m * p.tiles_n, p.tiles_m, p.tiles_n, tm, tn);
    work(tm, tn, 0, nk_all,
         EpiDst{p.D, p.C, p.ldc, p.M, p.N, (int64_t)tm * BM, (int64_t)tn * BN, p.alpha, p.beta, p.alpha_i,
                p.beta_i, p.use_c, p.vec_cd, p.out});
  } else {
    // Workgroup w takes K iterations [w L, (w + 1) L) of the tiles after the
    // first dp_tiles (which a whole-tile launch covers), numbered tile by tile:
    // one or two pieces.  A piece that is a whole tile is stored to D; any other
    // piece stores its raw sums (alpha 1, no C) to its own workspace slot.
    const int64_t w = blockIdx.x;
    const int64_t L = p.sk_iters;
    int64_t it = w * L;
    const int64_t end = min(it + L, (int64_t)p.sk_tiles * nk_all);
    int64_t piece = sk_first_piece(w, L, nk_all, p.sk_period);
    for (int pc = 0; it < end; ++pc) {
      const int64_t x = it / nk_all;
      const int kbeg = (int)(it - x * nk_all);
      const int kcnt = (int)min((int64_t)(nk_all - kbeg), end - it);
      int tm, tn;
      {
        int m, n;
        grouped_tile<4>(p.dp_tiles + (int)x, p.tiles_m, p.tiles_n, m, n);
        tm = __builtin_amdgcn_readfirstlane(m);
        tn = __builtin_amdgcn_readfirstlane(n);
      }
      if (pc > 0) barrier_lds();  // the previous piece's epilogue is done with the LDS
      const bool whole = kbeg == 0 && kcnt == nk_all;
      const EpiDst d = whole ? EpiDst{p.D, p.C, p.ldc, p.M, p.N, (int64_t)tm * BM, (int64_t)tn * BN, p.alpha,
                                      p.beta, p.alpha_i, p.beta_i, p.use_c, p.vec_cd, p.out}
                             : EpiDst{(char*)p.ws + piece * (int64_t)(TB * TB * 4), nullptr, TB, TB, TB, 0, 0,
                                      1.0f, 0.0f, 1, 0, 0, 1, OUT_32};
      work(tm, tn, kbeg, kcnt, d);
      it += kcnt;
      ++piece;
    }
  }
}

// Stream-K fixup: for each remainder tile cut into more than one piece, add the
// pieces' partial sums in piece order (ascending K) and apply the epilogue
// D = alpha * sum + beta * C of the whole-tile path (binary32 fma, or wrapping
// int32), rounding once to a 16-bit D.  Grid (sk_tiles, TB * TB / 1024), 256
// threads: one 16-byte group of 4 columns per thread, consecutive threads along a
// row; up to FIX_BATCH pieces are loaded before they are added, so that the
// loads overlap.
constexpr int FIX_BATCH = 8;
template <bool INT, int TB>
__global__ __launch_bounds__(256) void streamk_fixup_kernel(DenseArgs p, int64_t nk) {
  const int64_t x = blockIdx.x, L = p.sk_iters;
  const int64_t w0 = x * nk / L, w1 = ((x + 1) * nk - 1) / L;  // workgroups with a piece of tile x
  if (w0 == w1) return;  // one piece: the whole tile, stored by its workgroup
  const int64_t first = sk_first_piece(w0, L, nk, p.sk_period) + (x - w0 * L / nk);
  const int npieces = (int)(w1 - w0 + 1);
  int tm, tn;
  grouped_tile<4>(p.dp_tiles + (int)x, p.tiles_m, p.tiles_n, tm, tn);
  const int idx = blockIdx.y * 256 + threadIdx.x;  // 16-byte group of the row-major tile
  const int r = idx / (TB / 4), c = 4 * (idx % (TB / 4));
  const int64_t m = (int64_t)tm * TB + r, n = (int64_t)tn * TB + c;
  if (m >= p.M || n >= p.N) return;
  using e1 = typename std::conditional<INT, int, float>::type;
  using v4 = typename std::conditional<INT, i32x4, f32x4>::type;
  const char* src = (const char*)p.ws + first * (int64_t)(TB * TB * 4) + (int64_t)idx * 16;
  auto slot = [&](int q) { return *(const v4*)(src + (int64_t)q * (TB * TB * 4)); };
  v4 acc = slot(0);
  for (int q0 = 1; q0 < npieces; q0 += FIX_BATCH) {
    v4 t[FIX_BATCH];
#pragma unroll
    for (int u = 0; u < FIX_BATCH; ++u)
      if (q0 + u < npieces) t[u] = slot(q0 + u);
#pragma unroll
    for (int u = 0; u < FIX_BATCH; ++u)
      if (q0 + u < npieces) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (INT) acc[e] = (int)((uint32_t)acc[e] + (uint32_t)t[u][e]);
          else acc[e] += t[u][e];
        }
      }
  }
  const int64_t doff = m * p.ldc + n;
  const bool full = p.vec_cd && n + 4 <= p.N;
  e1 o[4];
  if constexpr (INT) {
    const int* C = (const int*)p.C;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t cv = p.use_c && n + e < p.N ? (uint32_t)C[doff + e] : 0u;
      o[e] = (int)((uint32_t)p.alpha_i * (uint32_t)acc[e] + (uint32_t)p.beta_i * cv);
    }
    if (full) {
      *(i32x4*)((int*)p.D + doff) = i32x4{o[0], o[1], o[2], o[3]};
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < p.N) ((int*)p.D)[doff + e] = o[e];
    }
  } else if (p.out == OUT_32) {
    const float* C = (const float*)p.C;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = p.use_c && n + e < p.N ? __builtin_fmaf(p.alpha, acc[e], p.beta * C[doff + e]) : p.alpha * acc[e];
    if (full) {
      *(f32x4*)((float*)p.D + doff) = f32x4{o[0], o[1], o[2], o[3]};
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < p.N) ((float*)p.D)[doff + e] = o[e];
    }
  } else {
    const uint16_t* C16 = (const uint16_t*)p.C;
    uint16_t* D16 = (uint16_t*)p.D;
    for (int e = 0; e < 4; ++e) {
      if (n + e >= p.N) continue;
      const float v = p.use_c ? __builtin_fmaf(p.alpha, acc[e], p.beta * from_out_bits(p.out, C16[doff + e]))
                              : p.alpha * acc[e];
      D16[doff + e] = (uint16_t)to_out_bits(p.out, v);
    }
  }
}

template <class Op, int LA, int LB, int TB, bool SK = false>
hipError_t launch_one(const DenseArgs& a0, hipStream_t s) {
  DenseArgs a = a0;
  a.tiles_m = (int)((a.M + TB - 1) / TB);
  a.tiles_n = (int)((a.N + TB - 1) / TB);
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  if (tiles <= 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (!SK || a.dp_tiles > 0) {  // whole tiles: every tile, or the first dp_tiles
    hipLaunchKernelGGL((gemm_fast_kernel<Op, LA, LB, TB, false>), dim3((unsigned)(SK ? a.dp_tiles : tiles)),
                       dim3(THREADS), 0, s, a);
    e = hipGetLastError();
  }
  if constexpr (SK) {
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_fast_kernel<Op, LA, LB, TB, true>), dim3((unsigned)a.sk_wgs), dim3(THREADS), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nk = (a.K + KTB / Op::EB - 1) / (KTB / Op::EB);
    hipLaunchKernelGGL((streamk_fixup_kernel<Op::INT_ACC, TB>), dim3((unsigned)a.sk_tiles, TB * TB / 1024), dim3(256), 0, s,
                       a, nk);
    e = hipGetLastError();
  }
  return e;
}

template <class Op, int TB, bool SK = false>
hipError_t launch_layouts_tb(int la, int lb, const DenseArgs& a, hipStream_t s) {
  if (la == 0 && lb == 0) return launch_one<Op, 0, 0, TB, SK>(a, s);
  if (la == 0 && lb == 1) return launch_one<Op, 0, 1, TB, SK>(a, s);
  if (la == 1 && lb == 0) return launch_one<Op, 1, 0, TB, SK>(a, s);
  return launch_one<Op, 1, 1, TB, SK>(a, s);
}

// Operation-type dispatch for tile size TB (one translation unit per TB and form).
template <int TB, bool SK = false>
hipError_t launch_fast_tb(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s) {
  if (dtA == DT_BF16) return launch_layouts_tb<BF16, TB, SK>(la, lb, a, s);
  if (dtA == DT_F16) return launch_layouts_tb<F16, TB, SK>(la, lb, a, s);
  if (dtA == DT_I8) return launch_layouts_tb<I8, TB, SK>(la, lb, a, s);
  const int fa = f8fmt(dtA), fb = f8fmt(dtB);
  if (a.K >= FP8_NATIVE_MIN_K) {
    if (fb == 0 && fa == 0) return launch_layouts_tb<F8<0, 0>, TB, SK>(la, lb, a, s);
    if (fb == 1 && fa == 0) return launch_layouts_tb<F8<1, 0>, TB, SK>(la, lb, a, s);
    if (fb == 0 && fa == 1) return launch_layouts_tb<F8<0, 1>, TB, SK>(la, lb, a, s);
    return launch_layouts_tb<F8<1, 1>, TB, SK>(la, lb, a, s);
  }
  if (fa == 0 && fb == 0) return launch_layouts_tb<F8W<0, 0>, TB, SK>(la, lb, a, s);
  if (fa == 0 && fb == 1) return launch_layouts_tb<F8W<0, 1>, TB, SK>(la, lb, a, s);
  if (fa == 1 && fb == 0) return launch_layouts_tb<F8W<1, 0>, TB, SK>(la, lb, a, s);
  return launch_layouts_tb<F8W<1, 1>, TB, SK>(la, lb, a, s);
}

}  // namespace fast
}  // namespace mcg
