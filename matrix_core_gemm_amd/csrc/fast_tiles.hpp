// fast_tiles.hpp -- LDS tile geometry, HBM -> LDS loaders and LDS -> VGPR
// fragment readers shared by the 256 x 256 dense and 2:4 sparse kernels.
//
// A tile holds, for one stage, KTB bytes of K of ROWS_MN rows (M rows of A or
// N columns of B).  K-contiguous operands keep one LDS row per matrix row
// (KTB bytes); MN-contiguous operands keep one LDS row per k (ROWS_MN
// elements).  Rows are split in 16-byte chunks whose order is XOR-swizzled
// per row so that the fragment reads are free of LDS bank conflicts (measured
// with SQ_LDS_BANK_CONFLICT on gfx950 for exactly these access patterns):
//   K-contiguous rows of CPR chunks: chunk ^= (row / (16 / CPR)) mod CPR
//     (16 consecutive rows of one chunk land in 16 distinct 16-byte slots of
//     the 256 bytes the 64 banks serve per cycle);
//   MN-contiguous 16-bit rows (transposing 16-bit reads): chunk ^= 4 * (row mod 4);
//   MN-contiguous 8-bit rows (transposing 8-bit reads): chunk ^= 2 * (row mod 8).
// The swizzle is applied on the global side: each lane of a buffer_load ... lds
// instruction fetches the global chunk that belongs at its (fixed) LDS slot.
#pragma once
#include "arch_gfx950.hpp"
#include "tile_order.hpp"

namespace mcg {
namespace fast {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int NW = 4;                      // wavefronts per workgroup
constexpr uint32_t BUF_OOB = 0x80000000u;  // buffer offset past every window: the load returns zeros

template <int EB, int LAYOUT, int ROWS_MN, int KTB>
struct Geom {
  static constexpr int R = LAYOUT == LAYOUT_K ? ROWS_MN : KTB / EB;  // LDS rows
  static constexpr int W = LAYOUT == LAYOUT_K ? KTB : ROWS_MN * EB;  // bytes per row
  static constexpr int CPR = W / 16;
  static constexpr int CHUNKS = R * CPR;
  static constexpr int BYTES = R * W;
};

template <int EB, int LAYOUT, int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (LAYOUT == LAYOUT_K) {
    static_assert(CPR == 2 || CPR == 4 || CPR == 8, "K-contiguous rows of 32, 64 or 128 bytes");
    constexpr int SH = CPR == 2 ? 3 : CPR == 4 ? 2 : 1;  // log2(16 / CPR)
    return (row >> SH) & (CPR - 1);
  }
  else if constexpr (EB == 2) return (4 * (row & 3)) & (CPR - 1);
  else return (2 * (row & 7)) & (CPR - 1);
}

// Buffer resource over [base, base + bytes) built from wave-uniform values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)n, 0x00020000);
}

// HBM -> LDS loader of one operand tile: wave w, instruction i of a stage
// writes LDS bytes [(i * NW + w) * 1024, +1024) of that stage's tile.  K is
// counted in elements of this operand.
template <int EB, int LAYOUT, int ROWS_MN, int KTB>
struct Loader {
  using G = Geom<EB, LAYOUT, ROWS_MN, KTB>;
  static constexpr int INSTR = G::CHUNKS / (64 * NW);
  static_assert(G::CHUNKS % (64 * NW) == 0, "tile must split into whole wave instructions");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[INSTR];
  int kpos[INSTR];
  uint32_t kstride;

  __device__ __forceinline__ void init(const char* base, uint32_t bytes, int64_t ld, int wave, int lane) {
    rsrc = make_rsrc(base, bytes);
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int q = (i * NW + wave) * 64 + lane;
      const int r = q / G::CPR, pc = q % G::CPR;
      const int lc = pc ^ swz<EB, LAYOUT, G::CPR>(r);
      off[i] = (uint32_t)(r * ld * EB + lc * 16);
      kpos[i] = LAYOUT == LAYOUT_K ? lc * (16 / EB) : r;
    }
    kstride = LAYOUT == LAYOUT_K ? (uint32_t)KTB : (uint32_t)(KTB / EB * ld * EB);
  }

  __device__ __forceinline__ void issue(lds_char* dst, int kt, int64_t K, int wave) const {
    const int64_t k0 = (int64_t)kt * (KTB / EB);
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      uint32_t o = off[i] + (uint32_t)kt * kstride;
      if constexpr (LAYOUT == LAYOUT_K) o = (k0 + kpos[i] < K) ? o : BUF_OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(dst + (i * NW + wave) * 1024), 16, o, 0, 0, 0);
    }
  }
};

// HBM -> LDS loader with one lane offset and uniform strides.  The chunk a
// lane fetches is the same in every instruction of a stage up to a whole
// number of swizzle periods of rows, so instruction i only adds i * istride
// and K tile kt adds kt * kstride.  Every offset is passed as the per-lane
// (range-checked) buffer offset, so rows past M / N and k past K read zeros.
// For K-contiguous rows of 128 bytes every 8 lanes fetch one whole 128-byte
// line of a row.
template <int EB, int LAYOUT, int ROWS_MN, int KTB>
struct LineLoader {
  using G = Geom<EB, LAYOUT, ROWS_MN, KTB>;
  static constexpr int INSTR = G::CHUNKS / (64 * NW);   // per wave and stage
  static constexpr int ROWS_PER_I = NW * 64 / G::CPR;   // LDS rows advanced per instruction
  static_assert(G::CHUNKS % (64 * NW) == 0, "tile must split into whole wave instructions");
  static_assert(LAYOUT != LAYOUT_K || ROWS_PER_I % 16 == 0, "swizzle period (16 rows) per instruction");
  static_assert(LAYOUT == LAYOUT_K || ROWS_PER_I % (EB == 2 ? 4 : 8) == 0, "swizzle period per instruction");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff;     // lane offset of instruction 0, K tile 0
  int klim;          // K-contiguous: K tiles kt < klim hold this lane's chunk inside K
  uint32_t istride;  // bytes between consecutive instructions
  uint32_t kstride;  // bytes per K tile

  __device__ __forceinline__ void init(const char* base, uint32_t bytes, int64_t ld, int64_t K, int wave,
                                       int lane) {
    rsrc = make_rsrc(base, bytes);
    const int q = wave * 64 + lane;
    const int r = q / G::CPR, pc = q % G::CPR;
    const int lc = pc ^ swz<EB, LAYOUT, G::CPR>(r);
    voff = (uint32_t)(r * ld * EB + lc * 16);
    istride = __builtin_amdgcn_readfirstlane((uint32_t)(ROWS_PER_I * ld * EB));
    kstride = __builtin_amdgcn_readfirstlane(LAYOUT == LAYOUT_K ? (uint32_t)KTB : (uint32_t)(KTB / EB * ld * EB));
    if constexpr (LAYOUT == LAYOUT_K) {
      const int64_t left = K - (int64_t)lc * (16 / EB);  // k values from this chunk to the end of K
      klim = left <= 0 ? 0 : (int)((left + KTB / EB - 1) / (KTB / EB));
    } else {
      klim = 0x7fffffff;  // MN-contiguous: rows past K lie outside the buffer window
    }
  }

  // instructions [i0, i0 + n) of K tile kt into stage `dst`.  The out-of-range
  // offset plus i * istride cannot wrap: every window is below 2 GiB.
  __device__ __forceinline__ void issue(lds_char* dst, int kt, int i0, int n, int wave) const {
    issue_if(dst, kt, i0, n, wave, true);
  }
  // the same; when !live the instructions read nothing and fill the stage with zeros.
  // AUX: the loads' cache-policy bits (2: non-temporal, for data read once)
  template <int AUX = 0>
  __device__ __forceinline__ void issue_if(lds_char* dst, int kt, int i0, int n, int wave, bool live) const {
    const uint32_t v = live && kt < klim ? voff + (uint32_t)kt * kstride : BUF_OOB;
#pragma unroll
    for (int i = i0; i < i0 + n; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(dst + (i * NW + wave) * 1024), 16,
          v + (uint32_t)i * istride, 0, 0, AUX);
  }
};

// LDS -> VGPR fragments of the 32 rows [rb, rb + 32) of a tile.  Lane group
// g = lane >> 5 reads 16 bytes of K starting at byte kb (chosen by the caller
// per lane group); MN-contiguous tiles gather them with transposing reads.
template <int EB, int LAYOUT, int ROWS_MN, int KTB>
struct Reader {
  using G = Geom<EB, LAYOUT, ROWS_MN, KTB>;
  __device__ static __forceinline__ int addr(int row, int byte) {
    const int c = byte >> 4;
    return row * G::W + ((c ^ swz<EB, LAYOUT, G::CPR>(row)) << 4) + (byte & 15);
  }
  __device__ static __forceinline__ i32x4 read16k(const lds_char* tile, int rb, int kb, int lane) {
    if constexpr (LAYOUT == LAYOUT_K) {
      return lds_read_b128(tile, addr(rb + (lane & 31), kb));
    } else if constexpr (EB == 2) {
      // 8 k values = 2 transposed reads of 4 k rows; sub-group (lane >> 4) & 1
      // serves the second 16 columns of the 32-row block
      const int L = lane & 15;
      const int col = rb + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
      const int row = kb / 2 + (L >> 2);
      const i32x2 lo = lds_read_tr16(tile, addr(row, 2 * col));
      const i32x2 hi = lds_read_tr16(tile, addr(row + 4, 2 * col));
      return i32x4{lo.x, lo.y, hi.x, hi.y};
    } else {
      // 16 k values = 2 transposed reads of 8 k rows
      const int L = lane & 15;
      const int col = rb + 16 * ((lane >> 4) & 1) + 8 * (L & 1);
      const int row = kb + (L >> 1);
      const i32x2 lo = lds_read_tr8(tile, addr(row, col));
      const i32x2 hi = lds_read_tr8(tile, addr(row + 8, col));
      return i32x4{lo.x, lo.y, hi.x, hi.y};
    }
  }
  // MN-contiguous tiles: LDS byte address of the first of the transposing reads
  // read16k makes for block rb and K bytes kb; the reads of kb + 32 (16-bit) or
  // kb + 16, kb + 32 (8-bit) lie whole rows further, in rows of the same swizzle
  __device__ static __forceinline__ uint32_t mn_addr(const lds_char* tile, int rb, int kb, int lane) {
    static_assert(LAYOUT == LAYOUT_MN, "transposing reads");
    const int L = lane & 15;
    if constexpr (EB == 2) {
      const int col = rb + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
      return lds_addr(tile + addr(kb / 2 + (L >> 2), 2 * col));
    } else {
      const int col = rb + 16 * ((lane >> 4) & 1) + 8 * (L & 1);
      return lds_addr(tile + addr(kb + (L >> 1), col));
    }
  }
  // dense 32x32 instructions: lane group g owns tile K bytes [32g, 32g + 32);
  // sub-step s is its half [32g + 16s, +16)
  __device__ static __forceinline__ i32x4 read16(const lds_char* tile, int rb, int s, int lane) {
    return read16k(tile, rb, 32 * (lane >> 5) + 16 * s, lane);
  }
  __device__ static __forceinline__ i32x8 read32(const lds_char* tile, int rb, int lane) {
    const i32x4 a = read16(tile, rb, 0, lane), b = read16(tile, rb, 1, lane);
    return i32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  }
};

// ------------------------------------------------------------- 32x32 ops
// P (first operand) = B fragment, Q = A fragment.  One instruction takes
// LANE_BYTES bytes of K per lane; lane group g = lane >> 5 of a 32-row
// fragment holds the g-th LANE_BYTES-byte part of the instruction's K range
// (gathered by transposing reads when the operand is MN-contiguous); A and B
// use the same assignment, so any consistent choice is valid.  Output lane l,
// register r holds out[8*(r/4) + 4*(l/32) + r%4][l % 32] (the 32 x 32
// accumulator layout).

struct BF16 {
  static constexpr int EB = 2, LANE_BYTES = 16;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x16;
  using frag_t = i32x4;
  __device__ static __forceinline__ void mma(acc_t& c, const frag_t& p, const frag_t& q) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bit_cast<bf16x8>(p), bit_cast<bf16x8>(q), c, 0, 0, 0);
  }
};
struct F16 {
  static constexpr int EB = 2, LANE_BYTES = 16;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x16;
  using frag_t = i32x4;
  __device__ static __forceinline__ void mma(acc_t& c, const frag_t& p, const frag_t& q) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(bit_cast<f16x8>(p), bit_cast<f16x8>(q), c, 0, 0, 0);
  }
};
struct I8 {
  static constexpr int EB = 1, LANE_BYTES = 16;
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
  static constexpr int EB = 1, LANE_BYTES = 32;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x16;
  using frag_t = i32x8;
  __device__ static __forceinline__ void mma(acc_t& c, const frag_t& p, const frag_t& q) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(p, q, c, FP, FQ, 0, 0, 0, 0);
  }
};
// fp8 widened exactly to bf16 (K below the native-fp8 threshold): FA/FB = formats
// of A/B; 16 bytes per lane hold 16 fp8 values = two bf16 instructions.
template <int FA, int FB>
struct F8W {
  static constexpr int EB = 1, LANE_BYTES = 16;
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

__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup bid of nwg whole-tile workgroups -> output tile.  Workgroups are
// dispatched round-robin over the 8 XCDs; the sequence is permuted so that the
// workgroups of one XCD take consecutive logical tiles, which concurrently
// resident workgroups then share in their XCD's L2.
template <int GROUP>
__device__ __forceinline__ void tile_coords_of(int bid, int nwg, int tiles_m, int tiles_n, int& tm, int& tn) {
  int pid = bid;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  int m, n;
  grouped_tile<GROUP>(pid, tiles_m, tiles_n, m, n);
  tm = __builtin_amdgcn_readfirstlane(m);
  tn = __builtin_amdgcn_readfirstlane(n);
}

template <int GROUP>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  tile_coords_of<GROUP>(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
}

}  // namespace fast
}  // namespace mcg
