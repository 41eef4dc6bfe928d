// gemm_f64.hip -- binary64 GEMM (DGEMM) on the FP64 matrix instructions of gfx950.
//
// D = alpha * (A . B) + beta * C for binary64 A, B, C and D, accumulated in binary64
// by the FP64-accumulate matrix instructions ("CDNA3 dense MFMA builtins",
// FP64-accumulate builtins; the accumulator layouts of the 4x4 FP64 tile shape).
//
// Instruction.  v_mfma_f64_16x16x4_f64 (one 16 x 16 x 4 block; 64 cycles) runs at
// 78.0 TFLOP/s over the chip in a register-only loop (measured, 99% of the peak),
// against 73-75 for the four-block 4x4x4 one, and reads a quarter of the operand
// bytes per flop.  The compiler's default form keeps MFMA accumulators in AGPRs and
// copies them to and from VGPRs around loops (about 49 TFLOP/s for the same loop);
// this file is built with the VGPR form.  Operand and result lanes (measured; D as
// the pages' 16 x 16 FP64 layout): A[i][k] in lane i + 16k, B[k][j] in lane j + 16k,
// D[i][j] in lane 16 (i mod 4) + j, register pair i / 4.
//
// Tiling.  128 x 128 output tiles, 4 waves of 64 x 64 (4 x 4 instructions per K
// index group), K in tiles of 16, two LDS stages of 32 KiB; two workgroups share
// a CU, so each SIMD holds waves of two workgroups whose barriers and tile starts
// do not coincide and one keeps the matrix core busy while the other waits.  Lane
// group g (lane >> 4) owns K = 4g .. 4g + 3 of each tile and reads them as two
// pairs (h = 0, 1); the two instructions fed by pair h take the K index sets
// {4g + 2h} and {4g + 2h + 1}, consistently for A and B.
//
// LDS images.  A K-contiguous operand keeps one row of A (column of B) per 128
// bytes, 16-byte chunk c of row r at position c ^ s(r), s(r) = bits 1..3 of r with
// bit 1 flipped when bits 2 and 3 of r differ.  A 16-byte read is served 16 lanes per
// cycle, lanes {0-3, 12-15, 20-27} together (equal lane bit 5, equal parity of lane
// bits 2..4); such a set reads 16 rows of two lane groups at chunks c and c ^ 2, and s
// sends them to 16 different 16-byte bank slots (rows of either parity sit in different
// halves of 256 bytes; 0 bank-conflict cycles, against 4 per read for plain bits 1..3).
// Pairs are read with one 16-byte read.  An MN-contiguous operand keeps one K per 1 KiB row
// (16 lanes read 128 consecutive bytes); pairs are read as two 8-byte values 1 KiB
// apart.
//
// Loads.  The FP64 matrix instructions leave no issue slots to vector ALU work
// (the pages' throughput table lists no co-execution for them), so the steady
// state keeps both registers and vector arithmetic out of the loads: K tiles move
// HBM -> LDS by buffer_load ... lds (16 bytes per lane, 1 KiB per wave instruction)
// from a scalar descriptor at the tile's corner, with fixed per-lane offsets, into
// the stage the previous tile is not using; the swizzle is applied on the global
// side (each lane fetches the chunk that belongs at its LDS position).  In the last
// tiles of M or N, lanes whose rows lie past the matrix fetch a valid row instead
// (those rows only feed outputs that are not stored).  A K tile that crosses the end
// of K is loaded element by element with bounds checks (zeros outside) and stored
// with ds_write; so are the last tile of an MN-contiguous operand whose valid width is
// odd (a 16-byte pair would cross the edge) and every tile of operands with very large
// leading dimensions.  Operands whose rows are not 16-byte aligned (odd leading
// dimensions) load with 4-byte DMA into the same LDS images, edge tiles included.
//
// Split K (few output tiles, long K): grid.y ranges of K tiles; the ranges add
// alpha * partial into a zeroed D with binary64 atomic adds, and beta * C is added
// afterwards (D must not be C then).
#include "arch_gfx950.hpp"
#include "fast_tiles.hpp"
#include "gemm_kernels.hpp"

#include <type_traits>

namespace mcg {
namespace f64 {

constexpr int BM = 128, BN = 128, BK = 16, THREADS = 256, NWAVE = 4;
constexpr int WM = 64, WN = 64;            // wave tile
constexpr int FM = WM / 16, FN = WN / 16;  // instructions per K index group: FM x FN
constexpr int OP_BYTES = BM * BK * 8;      // 16 KiB: one operand's tile
constexpr int STAGE = 2 * OP_BYTES;        // A then B
constexpr int DMA_I = OP_BYTES / 1024 / NWAVE;  // 1 KiB DMA instructions per wave and operand
constexpr int PT = BM * BK / THREADS;      // elements of each operand per thread in the checked path
static_assert(BM == BN, "one loader geometry serves both operands");
static_assert(PT * THREADS == BM * BK, "checked loader covers the tile");
static_assert(DMA_I * NWAVE * 1024 == OP_BYTES, "whole DMA instructions");

typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzle of K-contiguous row r (t = bits 1..3 of r): t with bit 1 flipped when
// bits 2 and 3 of r differ.  A 16-byte LDS read is served 16 lanes per cycle, and the
// lanes served together are those with equal lane bit 5 and equal parity of lane bits
// 2..4 (measured with SQ_LDS_BANK_CONFLICT on two-lane patterns); such a set holds, for
// the two lane groups g = 2G and 2G + 1 it spans, rows of opposite parity of bits 2..3,
// read at chunks c and c ^ 2.  The flip sends its 16 lanes to 16 different 16-byte bank
// slots; plain t would pair them up (2-way conflicts on every fragment read).
__device__ __forceinline__ int kswz(int r) { return ((r >> 1) ^ ((((r >> 2) ^ (r >> 3)) & 1) << 1)) & 7; }

// LDS byte offset of element (r, k) of an operand tile (r: row of A / column of B).
template <int LAY>
__device__ __forceinline__ int lds_elem(int r, int k) {
  if constexpr (LAY == 0) return r * 128 + (((k >> 1) ^ kswz(r)) & 7) * 16 + (k & 1) * 8;
  else return k * 1024 + r * 8;
}

// One operand's tiles.  LAY 0 (K-contiguous): element (r, k) at X[r * ld + k];
// LAY 1 (MN-contiguous): at X[k * ld + r].
template <int LAY>
struct Operand {
  const double* X;
  int64_t ld, rows, K, r0;
  // DMA: wave w, instruction i fills LDS bytes [(4i + w) KiB, +1 KiB) of the tile.
  //   LAY 0: rows 32i + 8w + (l >> 3); lane l's LDS position l & 7 takes global chunk
  //          (l & 7) ^ kswz(row) of that row
  //   LAY 1: K row 4i + w; lane l takes values 2l, 2l + 1 of it
  // Rows past the edge of the matrix (last tiles of M or N) fetch the last valid row
  // (LAY 0) or the tile's first pair (LAY 1) instead: they only feed rows (columns)
  // of D that are not stored.
  uint32_t voff[DMA_I];  // per lane and instruction (LAY 1: instruction 0 only)
  uint32_t soff;         // LAY 1: per wave, instruction 0
  uint32_t istr;         // LAY 1: per instruction
  // 4-byte DMA (rows without 16-byte alignment; interior tiles): wave w, instruction i
  // fills LDS bytes [256 (4i + w), +256) of the tile.
  //   LAY 0: rows 8i + 2w + (l >> 5) (two 128-byte rows); lane l's dword l & 3 of LDS
  //          chunk position (l >> 2) & 7 takes the same dword of global chunk
  //          ((l >> 2) & 7) ^ kswz(row), which depends on i only through its parity
  //          (bits 1..3 of the row are those of 8 (i & 1) + 2w)
  //   LAY 1: K row i (4 x 256 bytes); lane l takes dword l of quarter w
  uint32_t voff4[2];

  __device__ __forceinline__ void init(const double* X_, int64_t ld_, int64_t r0_, int64_t rows_, int64_t K_,
                                       int w, int lane) {
    X = X_;
    ld = ld_;
    rows = rows_;
    K = K_;
    r0 = r0_;
    if constexpr (LAY == 0) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int q = (lane >> 2) & 7;
        voff4[par] = (uint32_t)((2 * w + (lane >> 5)) * ld * 8 + (q ^ kswz(8 * par + 2 * w)) * 16 + (lane & 3) * 4);
      }
    } else {
      voff4[0] = voff4[1] = (uint32_t)(w * 256 + lane * 4);
    }
    const int64_t valid = rows - r0;  // rows of this tile inside the matrix (>= 1)
    if constexpr (LAY == 0) {
#pragma unroll
      for (int i = 0; i < DMA_I; ++i) {
        const int row = 32 * i + 8 * w + (lane >> 3);
        const int64_t src = row < valid ? row : valid - 1;
        const int c = (lane & 7) ^ kswz(row);
        voff[i] = (uint32_t)(src * ld * 8 + c * 16);
      }
      soff = 0;
      istr = 0;
    } else {
      voff[0] = (uint32_t)(2 * lane + 1 < valid ? lane * 16 : 0);
      soff = __builtin_amdgcn_readfirstlane((uint32_t)(w * ld * 8));
      istr = __builtin_amdgcn_readfirstlane((uint32_t)(4 * ld * 8));
    }
  }
  // K tile starting at k0, inside the rows and K.
  __device__ __forceinline__ void dma(char* dst, int64_t k0, int w) const {
    const char* corner = (const char*)(X + (LAY == 0 ? r0 * ld + k0 : k0 * ld + r0));
    const __amdgpu_buffer_rsrc_t rs = fast::make_rsrc(corner, 0xFFFFFFFFu);
    typedef __attribute__((address_space(3))) char lds_c;
    lds_c* base = (lds_c*)(lds_void*)(dst + w * 1024);
    uint32_t so = soff, lo = 0;
#pragma unroll
    for (int i = 0; i < DMA_I; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + lo), 16, voff[LAY == 0 ? i : 0], so, 0, 0);
      so += istr;
      lo += NWAVE * 1024;
      asm volatile("" : "+s"(so), "+s"(lo));
    }
  }
  // The same with 4-byte DMA: any 4-byte aligned rows, tile inside the rows and K.
  __device__ __forceinline__ void dma4(char* dst, int64_t k0, int w) const {
    const char* corner = (const char*)(X + (LAY == 0 ? r0 * ld + k0 : k0 * ld + r0));
    const __amdgpu_buffer_rsrc_t rs = fast::make_rsrc(corner, 0xFFFFFFFFu);
    // running scalar global and LDS offsets: two registers, not 16 hoisted constants each
    const uint32_t step = __builtin_amdgcn_readfirstlane((uint32_t)(LAY == 0 ? 8 * ld * 8 : ld * 8));
    typedef __attribute__((address_space(3))) char lds_c;
    lds_c* base = (lds_c*)(lds_void*)(dst + w * 256);
    uint32_t so = 0, lo = 0;
#pragma unroll
    for (int i = 0; i < 4 * DMA_I; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + lo), 4, voff4[i & 1], so, 0, 0);
      so += step;
      lo += NWAVE * 256;
      asm volatile("" : "+s"(so), "+s"(lo));
    }
  }
  // 4-byte DMA of a tile that crosses the edge of the rows: lanes whose rows lie past
  // the matrix fetch the last valid row (LAY 0; offsets computed per instruction) or
  // the tile's first element (LAY 1); those rows only feed outputs that are not stored.
  __device__ __forceinline__ void dma4_edge(char* dst, int64_t k0, int w, int lane) const {
    const char* corner = (const char*)(X + (LAY == 0 ? r0 * ld + k0 : k0 * ld + r0));
    const __amdgpu_buffer_rsrc_t rs = fast::make_rsrc(corner, 0xFFFFFFFFu);
    const int valid = (int)(rows - r0 < BM ? rows - r0 : BM);
    typedef __attribute__((address_space(3))) char lds_c;
    lds_c* base = (lds_c*)(lds_void*)(dst + w * 256);
    const uint32_t lane1 = (uint32_t)((32 * w + (lane >> 1)) < valid ? w * 256 + lane * 4 : (lane & 1) * 4);
    const uint32_t step = __builtin_amdgcn_readfirstlane((uint32_t)(ld * 8));
    // LAY 0: the chunk term for the two parities of i, and the row as a running value
    // (recomputed per instruction rather than 16 offsets hoisted out of the K loop)
    const uint32_t cterm[2] = {(uint32_t)(((((lane >> 2) & 7) ^ kswz(2 * w)) * 16) + (lane & 3) * 4),
                               (uint32_t)(((((lane >> 2) & 7) ^ kswz(8 + 2 * w)) * 16) + (lane & 3) * 4)};
    int row = 2 * w + (lane >> 5);
    uint32_t so = 0, lo = 0;
#pragma unroll
    for (int i = 0; i < 4 * DMA_I; ++i) {
      uint32_t vo;
      if constexpr (LAY == 0) {
        const int src = row < valid ? row : valid - 1;
        vo = (uint32_t)src * step + cterm[i & 1];
        row += 8;
        asm volatile("" : "+v"(row));
      } else {
        vo = lane1;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + lo), 4, vo, LAY == 0 ? 0u : so, 0, 0);
      so += step;
      lo += NWAVE * 256;
      asm volatile("" : "+s"(so), "+s"(lo));
    }
  }
  // Any K tile: element by element, zeros outside the rows and K, stored with ds_write.
  // Element p of thread t: LAY 0 (r, k) = ((t >> 4) + 16 p, t & 15); LAY 1 (t & 127, (t >> 7) + 2 p).
  __device__ __forceinline__ void checked(char* dst, int64_t k0, int tid) const {
    double v[PT];
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int r = LAY == 0 ? (tid >> 4) + 16 * p : tid & 127;
      const int k = LAY == 0 ? tid & 15 : (tid >> 7) + 2 * p;
      const int64_t gr = r0 + r, gk = k0 + k;
      v[p] = (gr < rows && gk < K) ? X[LAY == 0 ? gr * ld + gk : gk * ld + gr] : 0.0;
    }
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int r = LAY == 0 ? (tid >> 4) + 16 * p : tid & 127;
      const int k = LAY == 0 ? tid & 15 : (tid >> 7) + 2 * p;
      *(double*)(dst + lds_elem<LAY>(r, k)) = v[p];
    }
  }
};

// Fragment reads of one operand for pair h: lane row (column) rb, then groups of 16
// rows (columns).  For LAY 0 the swizzle term of group q depends on q mod VAR.
template <int LAY, int N, int STRIDE>
struct Frags {
  static constexpr int VAR = LAY == 0 && STRIDE < 16 ? 16 / STRIDE : 1;
  int base[2][VAR];
  __device__ __forceinline__ void init(int rb, int g) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < VAR; ++v) {
        const int r = rb + v * STRIDE;
        base[h][v] = LAY == 0 ? rb * 128 + (((2 * g + h) ^ kswz(r)) & 7) * 16 : (4 * g + 2 * h) * 1024 + rb * 8;
      }
  }
  // groups [Q0, Q0 + NQ)
  template <int Q0, int NQ>
  __device__ __forceinline__ void read(const char* op, int h, f64x2 (&x)[NQ]) const {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int q = Q0 + j;
      if constexpr (LAY == 0) {
        x[j] = *(const f64x2*)(op + base[h][q % VAR] + q * STRIDE * 128);
      } else {
        const char* a = op + base[h][0] + q * STRIDE * 8;
        x[j][0] = *(const double*)a;
        x[j][1] = *(const double*)(a + 1024);
      }
    }
  }
};

template <int LA, int LB>
__global__ __launch_bounds__(THREADS, 2) void dgemm_kernel(F64Args p) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];
  int tm, tn;
  fast::tile_coords<8>(p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (w & 1) * WM, wn = (w >> 1) * WN;
  static_assert(2 * WM == BM && 2 * WN == BN, "2 x 2 waves");

  // K range of this workgroup (grid.y > 1: split K)
  const int64_t nk_all = (p.K + BK - 1) / BK;
  const int64_t kt0 = (int64_t)blockIdx.y * p.kt_per_split;
  const int64_t nk = nk_all - kt0 < p.kt_per_split ? nk_all - kt0 : p.kt_per_split;
  const int64_t kbeg = kt0 * BK;

  Operand<LA> oa;
  Operand<LB> ob;
  oa.init(p.A, p.lda, m0, p.M, p.K, w, lane);
  ob.init(p.B, p.ldb, n0, p.N, p.K, w, lane);
  const int g = lane >> 4;
  Frags<LA, FM, 16> fa;
  Frags<LB, FN, 16> fb;
  fa.init(wm + (lane & 15), g);
  fb.init(wn + (lane & 15), g);

  typedef double f64x4 __attribute__((ext_vector_type(4)));
  f64x4 acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int c = 0; c < FN; ++c) acc[f][c] = (f64x4){0.0, 0.0, 0.0, 0.0};

  // fragments of pair h of the tile in stage st, and the 2 x FM x FN instructions they feed
  auto read = [&](const char* st, int h, f64x2 (&a)[FM], f64x2 (&b)[FN]) {
    fa.template read<0, FM>(st, h, a);
    fb.template read<0, FN>(st + OP_BYTES, h, b);
  };
  auto mma = [&](const f64x2 (&a)[FM], const f64x2 (&b)[FN]) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int c = 0; c < FN; ++c)
          acc[f][c] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[f][e], b[c][e], acc[f][c], 0, 0, 0);
  };
  auto compute = [&](const char* st) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f64x2 a[FM], b[FN];
      read(st, h, a, b);
      mma(a, b);
    }
  };
  auto checked = [&](char* st, int64_t k0) __attribute__((always_inline)) {
    oa.checked(st, k0, tid);
    ob.checked(st + OP_BYTES, k0, tid);
  };

  // 16-byte DMA unless an MN-contiguous operand's last tile ends inside a 16-byte pair;
  // 4-byte DMA for interior tiles of operands whose rows are not 16-byte aligned
  const bool pairs_a = LA == 0 || m0 + BM <= p.M || ((p.M - m0) & 1) == 0;
  const bool pairs_b = LB == 0 || n0 + BN <= p.N || ((p.N - n0) & 1) == 0;
  const bool dword = p.dma_mode == 2;
  const bool inside_a = m0 + BM <= p.M, inside_b = n0 + BN <= p.N;
  // The DMA loop, instantiated twice: EDGE for tiles of 4-byte DMA operands that cross
  // the edge of M or N (per-instruction clamped offsets), and once for all other DMA
  // tiles, so that the edge arithmetic holds no registers in the common loop.
  auto dma_loop = [&](auto edge_tag) __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    // DMA for the K tiles inside K; a K tile crossing the end of K (the last one of the
    // last range) follows the loop, loaded by the checked path
    const int64_t kfull = (p.K - kbeg) / BK;
    const int64_t nfull = kfull < nk ? kfull : nk;
    auto dma = [&](char* st, int64_t t) __attribute__((always_inline)) {
      if constexpr (EDGE) {
        if (inside_a) oa.dma4(st, kbeg + t * BK, w);
        else oa.dma4_edge(st, kbeg + t * BK, w, lane);
        if (inside_b) ob.dma4(st + OP_BYTES, kbeg + t * BK, w);
        else ob.dma4_edge(st + OP_BYTES, kbeg + t * BK, w, lane);
      } else if (dword) {
        oa.dma4(st, kbeg + t * BK, w);
        ob.dma4(st + OP_BYTES, kbeg + t * BK, w);
      } else {
        oa.dma(st, kbeg + t * BK, w);
        ob.dma(st + OP_BYTES, kbeg + t * BK, w);
      }
    };
    // the DMA writes of a wave are complete once its vmcnt drains; the barrier then
    // publishes the stage to every wave
    auto publish = [&]() __attribute__((always_inline)) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    // Fragments are read one pair ahead of the instructions that use them: pair 1 of a
    // tile before pair 0 is multiplied, and pair 0 of the next tile right after the
    // barrier that publishes it, before pair 1 of this tile is multiplied; so no
    // instruction waits for LDS.
    f64x2 a0[FM], b0[FN], a1[FM], b1[FN];
    auto step = [&](auto stage, int64_t t) __attribute__((always_inline)) {
      constexpr int S = decltype(stage)::value;
      const char* st = lds + S * STAGE;
      if (t + 1 < nfull) dma(lds + (1 - S) * STAGE, t + 1);
      read(st, 1, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      mma(a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      publish();
      if (t + 1 < nfull) read(lds + (1 - S) * STAGE, 0, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mma(a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    };
    if (nfull > 0) {
      dma(lds, 0);
      publish();
      read(lds, 0, a0, b0);
    }
    for (int64_t t = 0; t < nfull; t += 2) {
      step(std::integral_constant<int, 0>(), t);
      if (t + 1 < nfull) step(std::integral_constant<int, 1>(), t + 1);
    }
    if (nfull < nk) {
      char* st = lds + (nfull & 1) * STAGE;  // last read before the previous barrier
      checked(st, kbeg + nfull * BK);
      __syncthreads();
      compute(st);
    }
  };
  if (dword && !(inside_a && inside_b)) {
    dma_loop(std::true_type{});
  } else if ((p.dma_mode == 1 && pairs_a && pairs_b) || dword) {
    dma_loop(std::false_type{});
  } else {
    // misaligned operands or odd edges: one stage, checked loads
    for (int64_t t = 0; t < nk; ++t) {
      checked(lds, kbeg + t * BK);
      __syncthreads();
      compute(lds);
      __syncthreads();
    }
  }

  // result register pair r of a lane: element ACC::coord(lane, r) of each 16 x 16
  // piece (row 4r + lane / 16, column lane mod 16: the FP64 16 x 16 layout)
  using ACC = frag::Acc<frag::ACC_16x16_F64>;
  double* D = p.D;
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + wm + 16 * f + ACC::coord(lane, r).i;
      if (row >= p.M) continue;
#pragma unroll
      for (int c = 0; c < FN; ++c) {
        const int64_t col = n0 + wn + 16 * c + ACC::coord(lane, r).j;
        if (col >= p.N) continue;
        const int64_t off = row * p.ldc + col;
        if (gridDim.y > 1) {
          atomicAdd(D + off, p.alpha * acc[f][c][r]);
        } else {
          double v = p.alpha * acc[f][c][r];
          if (p.use_c) v = __builtin_fma(p.beta, p.C[off], v);
          D[off] = v;
        }
      }
    }
}

// Split K, before the partial sums: D = 0 over M x N.
__global__ __launch_bounds__(256) void zero_kernel(F64Args p) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= p.N) return;
  for (int64_t m = blockIdx.y; m < p.M; m += gridDim.y) p.D[m * p.ldc + n] = 0.0;
}

// Split K, after the partial sums (only when beta != 0): D = beta * C + D, one rounding.
__global__ __launch_bounds__(256) void finish_kernel(F64Args p) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= p.N) return;
  for (int64_t m = blockIdx.y; m < p.M; m += gridDim.y) {
    const int64_t off = m * p.ldc + n;
    p.D[off] = __builtin_fma(p.beta, p.C[off], p.D[off]);
  }
}

template <int LA, int LB>
static void launch_tiles(const F64Args& a, int splits, hipStream_t s) {
  hipLaunchKernelGGL((dgemm_kernel<LA, LB>), dim3((unsigned)(a.tiles_m * a.tiles_n), (unsigned)splits), dim3(THREADS),
                     0, s, a);
}

// DMA paths: every offset of a tile from its corner in 32 bits, at most (127 ld + 15) * 8
// (K-contiguous) or (15 ld + 127) * 8 (MN-contiguous), plus 16 bytes; the 16-byte
// path also needs 16-byte aligned rows (base and even leading dimension).
static bool f64_offsets32(int lay, int64_t ld) {
  const int64_t span = lay == 0 ? (127 * ld + 15) * 8 : (15 * ld + 127) * 8;
  return span + 16 < ((int64_t)0xFFFFFFFF);
}
static bool f64_rows16(const double* X, int64_t ld) { return ((uintptr_t)X % 16) == 0 && ld % 2 == 0; }

}  // namespace f64

F64Plan plan_f64(const F64Args& a, bool can_split, int num_cu) {
  using namespace f64;
  F64Plan plan{1, (int)((a.K + BK - 1) / BK)};
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const int64_t nk = (a.K + BK - 1) / BK;
  const int64_t slots = 2 * (int64_t)num_cu;
  if (!can_split || nk < 2 * F64_SPLIT_MIN_KT || tiles >= 4 * slots) return plan;
  // Estimated time of S ranges: full waves of resident workgroups (two per CU), then the
  // last wave, whose workgroups run alone on their CUs when there are at most 256 of
  // them; plus the atomic adds of the partial sums and the extra launches.
  auto cost = [&](int64_t S) __attribute__((always_inline)) {
    const int64_t per = (nk + S - 1) / S;
    const int64_t wgs = tiles * S;
    const int64_t rounds = (wgs + slots - 1) / slots;
    const int64_t last = wgs - (rounds - 1) * slots;
    double t = (double)(rounds - 1) * (double)per * F64_KT_SHARED_US +
               (double)per * (last <= (int64_t)num_cu ? F64_KT_ALONE_US : F64_KT_SHARED_US);
    if (S > 1) t += F64_ATOMIC_US * (double)S * (double)a.M * (double)a.N + F64_SPLIT_US;
    return t;
  };
  int64_t best = 1;
  double best_t = cost(1);
  for (int64_t S = 2; S <= nk / F64_SPLIT_MIN_KT && tiles * S <= 4 * slots; ++S) {
    const double t = cost(S);
    if (t < best_t) {
      best_t = t;
      best = S;
    }
  }
  const int64_t per = (nk + best - 1) / best;
  plan.splits = (int)((nk + per - 1) / per);  // no empty range
  plan.kt_per_split = (int)per;
  return plan;
}

hipError_t launch_f64(int la, int lb, const F64Args& a0, const F64Plan& plan, hipStream_t s) {
  using namespace f64;
  F64Args a = a0;
  a.tiles_m = (int)((a.M + BM - 1) / BM);
  a.tiles_n = (int)((a.N + BN - 1) / BN);
  a.kt_per_split = plan.kt_per_split;
  const bool off32 = f64_offsets32(la, a.lda) && f64_offsets32(lb, a.ldb);
  a.dma_mode = a.K == 0 || (off32 && f64_rows16(a.A, a.lda) && f64_rows16(a.B, a.ldb)) ? 1 : off32 ? 2 : 0;
  const dim3 rows_grid((unsigned)((a.N + 255) / 256), (unsigned)(a.M < 4096 ? a.M : 4096));
  if (plan.splits > 1) {
    hipLaunchKernelGGL(zero_kernel, rows_grid, dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (la == 0 && lb == 0) launch_tiles<0, 0>(a, plan.splits, s);
  else if (la == 0) launch_tiles<0, 1>(a, plan.splits, s);
  else if (lb == 0) launch_tiles<1, 0>(a, plan.splits, s);
  else launch_tiles<1, 1>(a, plan.splits, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1 || !a.use_c) return e;
  hipLaunchKernelGGL(finish_kernel, rows_grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mcg
