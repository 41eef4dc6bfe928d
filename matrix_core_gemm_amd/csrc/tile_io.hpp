// tile_io.hpp -- HBM -> LDS staging and LDS -> VGPR fragment reads for the GEMM kernels.
//
// A K-tile of an operand always holds 128 bytes of K per output row/column
// (64 bf16/f16 values or 128 8-bit values).  In LDS it is stored in the
// operand's own storage order:
//   K-contiguous : one LDS row per output row (m or n), 128 bytes of K each;
//   MN-contiguous: one LDS row per k, (rows of the tile) * elem_bytes each.
// Rows are split into 16-byte chunks and the chunk index is XOR-swizzled with
// a function of the row so that the fragment reads of a wavefront hit distinct
// LDS banks (see the per-layout swizzle functions).
#pragma once
#include "arch_gfx950.hpp"

namespace mcg {

constexpr int KT_BYTES = 128;  // bytes of K per tile row


// KTB: bytes of K per tile row (128 for the dense kernels).
template <int EB, int LAYOUT, int ROWS_MN, int KTB = KT_BYTES>
struct TileGeom {
  static constexpr int R = LAYOUT == LAYOUT_K ? ROWS_MN : KTB / EB;  // LDS rows
  static constexpr int W = LAYOUT == LAYOUT_K ? KTB : ROWS_MN * EB;  // bytes per row
  static constexpr int CPR = W / 16;                                      // chunks per row
  static constexpr int CHUNKS = R * CPR;
  static constexpr int BYTES = R * W;
  static_assert(W % 16 == 0, "tile rows must be whole 16-byte chunks");
};

// Swizzle of the 16-byte chunk index within an LDS row.
//  LDS on gfx950 has 64 four-byte banks; measured: an 8-byte read (plain or
//  transposing) serves lanes 0-31 and 32-63 in one cycle each when their
//  addresses fall in distinct banks, and a 16-byte read of 16 rows x 128 bytes
//  at one logical chunk per lane group is conflict-free when the chunk is
//  XOR-ed with (row / 2) mod 8 (but not with (row ^ row/8) mod 8).
//  K-contiguous rows: 8-chunk rows XOR with (r / 2) mod 8, so 16 consecutive
//  rows land on 16 distinct 16-byte slots modulo 256 bytes; 16-chunk rows XOR
//  with r mod 16.
//  MN-contiguous rows read with ds_read_b64_tr_b16 (4 rows x 2 chunks per 16
//  lanes) or ds_read_b64_tr_b8 (8 rows x 1 chunk per 16 lanes): XOR with the
//  row's position inside that group, plus a half-row flip between the groups
//  that share a 256-byte bank window.
template <int EB, int LAYOUT, int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (LAYOUT == LAYOUT_K) {
    if constexpr (CPR == 8) return (row >> 1) & 7;
    else return row & (CPR - 1);
  } else if constexpr (EB == 2) {
    int f = 2 * (row & 3) | (8 * ((row >> 3) & 1));
    return f & (CPR - 1);
  } else {
    int f = (row & 7) | (8 * ((row >> 4) & 1));
    return f & (CPR - 1);
  }
}

// Global -> registers -> LDS staging of one operand tile by NT threads.
// The tile covers storage rows [row0, row0 + R) and contiguous elements
// [col0, col0 + W/EB) of a matrix with leading dimension ld (elements); rows at
// or beyond rlim and elements at or beyond clim read as zero.  ONCE: every
// element is read by one workgroup only (the wide operand of a skinny problem),
// so the 16-byte loads are non-temporal.
template <int EB, int LAYOUT, int ROWS_MN, int NT, bool ALIGNED, int KTB = KT_BYTES, bool ONCE = false>
struct TileLoader {
  using G = TileGeom<EB, LAYOUT, ROWS_MN, KTB>;
  static constexpr int PER_THREAD = G::CHUNKS / NT;
  static_assert(G::CHUNKS % NT == 0, "tile chunks must divide evenly among threads");
  static constexpr int EPC = 16 / EB;  // elements per chunk

  i32x4 regs[PER_THREAD];

  __device__ __forceinline__ void load(const char* base, int64_t ld, int64_t row0, int64_t col0,
                                       int64_t rlim, int64_t clim, int tid) {
#pragma unroll
    for (int t = 0; t < PER_THREAD; ++t) {
      const int q = tid + t * NT;
      const int r = q / G::CPR, cc = q % G::CPR;
      const int64_t gr = row0 + r, gc = col0 + (int64_t)cc * EPC;
      const char* p = base + (gr * ld + gc) * EB;
      if (ALIGNED && gr < rlim && gc + EPC <= clim) {
        regs[t] = ONCE ? __builtin_nontemporal_load((const i32x4*)p) : *(const i32x4*)p;
      } else {
        union { i32x4 v; char b[16]; } u;
        u.v = i32x4{0, 0, 0, 0};
        if (gr < rlim) {
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            if (gc + e < clim) {
              if constexpr (EB == 2) {
                const uint16_t h = *(const uint16_t*)(p + 2 * e);
                u.b[2 * e] = (char)(h & 0xff);
                u.b[2 * e + 1] = (char)(h >> 8);
              } else {
                u.b[e] = p[e];
              }
            }
          }
        }
        regs[t] = u.v;
      }
    }
  }

  __device__ __forceinline__ void store(lds_char* tile, int tid) const {
#pragma unroll
    for (int t = 0; t < PER_THREAD; ++t) {
      const int q = tid + t * NT;
      const int r = q / G::CPR, cc = q % G::CPR;
      lds_write_b128(tile, r * G::W + ((cc ^ swz<EB, LAYOUT, G::CPR>(r)) * 16), regs[t]);
    }
  }
};

// Fragment of 16 output rows (or columns) [rb, rb + 16) for K-step s of the
// tile, in the operand layout of the 16x16 instructions (lane l -> row l & 15,
// lane group g = l >> 4 -> its K run).  K positions per lane group:
//   16-byte fragments (bf16/f16 K-step 32, i8 K-step 64): tile bytes
//     [16*(4s + g), +16);
//   32-byte fragments (fp8 K-step 128): tile bytes [16g, +16) then [64 + 16g, +16).
template <int EB, int LANE_BYTES, int LAYOUT, int ROWS_MN, int KTB = KT_BYTES>
struct FragReader {
  using G = TileGeom<EB, LAYOUT, ROWS_MN, KTB>;
  using frag_t = typename std::conditional<LANE_BYTES == 16, i32x4, i32x8>::type;

  // byte offset (in K) of the 16-byte K run h (0 or 1) of lane group g, step s
  __device__ static __forceinline__ int kbyte(int s, int g, int h) {
    if constexpr (LANE_BYTES == 16) return 16 * (4 * s + g);
    else return h == 0 ? 16 * g : 64 + 16 * g;
  }

  // 16 bytes of K starting at K byte kb (multiple of 16) for row rb + (lane & 15)
  __device__ static __forceinline__ i32x4 run16(const lds_char* tile, int rb, int kb, int lane) {
    if constexpr (LAYOUT == LAYOUT_K) {
      const int r = rb + (lane & 15);
      const int c = kb >> 4;
      return lds_read_b128(tile, r * G::W + ((c ^ swz<EB, LAYOUT, G::CPR>(r)) * 16));
    } else if constexpr (EB == 2) {
      // 8 values of K = two transposed reads of 4 k-rows each
      const int L = lane & 15;
      const int k0 = kb >> 1;  // element index of K
      const int mb = rb;       // first output row (element index along the row)
      i32x2 lo, hi;
      {
        const int row = k0 + (L >> 2);
        const int byte = (mb + 4 * (L & 3)) * 2;
        const int c = byte >> 4, w = byte & 15;
        lo = lds_read_tr16(tile, row * G::W + ((c ^ swz<EB, LAYOUT, G::CPR>(row)) * 16) + w);
      }
      {
        const int row = k0 + 4 + (L >> 2);
        const int byte = (mb + 4 * (L & 3)) * 2;
        const int c = byte >> 4, w = byte & 15;
        hi = lds_read_tr16(tile, row * G::W + ((c ^ swz<EB, LAYOUT, G::CPR>(row)) * 16) + w);
      }
      return i32x4{lo.x, lo.y, hi.x, hi.y};
    } else {
      // 16 values of K = two transposed reads of 8 k-rows each
      const int L = lane & 15;
      const int k0 = kb;
      const int mb = rb;
      i32x2 lo, hi;
      {
        const int row = k0 + (L >> 1);
        const int byte = mb + 8 * (L & 1);
        const int c = byte >> 4, w = byte & 15;
        lo = lds_read_tr8(tile, row * G::W + ((c ^ swz<EB, LAYOUT, G::CPR>(row)) * 16) + w);
      }
      {
        const int row = k0 + 8 + (L >> 1);
        const int byte = mb + 8 * (L & 1);
        const int c = byte >> 4, w = byte & 15;
        hi = lds_read_tr8(tile, row * G::W + ((c ^ swz<EB, LAYOUT, G::CPR>(row)) * 16) + w);
      }
      return i32x4{lo.x, lo.y, hi.x, hi.y};
    }
  }

  // 8 bytes of K starting at K byte kb (multiple of 8) for row rb + (lane & 15);
  // 8-bit elements only.
  __device__ static __forceinline__ i32x2 run8(const lds_char* tile, int rb, int kb, int lane) {
    static_assert(EB == 1, "8-byte K runs are used for 8-bit elements");
    if constexpr (LAYOUT == LAYOUT_K) {
      const int r = rb + (lane & 15);
      const int c = kb >> 4;
      return *(const __attribute__((address_space(3))) i32x2*)(
          tile + r * G::W + ((c ^ swz<EB, LAYOUT, G::CPR>(r)) * 16) + (kb & 8));
    } else {
      const int L = lane & 15;
      const int row = kb + (L >> 1);
      const int byte = rb + 8 * (L & 1);
      const int c = byte >> 4, w = byte & 15;
      return lds_read_tr8(tile, row * G::W + ((c ^ swz<EB, LAYOUT, G::CPR>(row)) * 16) + w);
    }
  }

  __device__ static __forceinline__ frag_t read(const lds_char* tile, int rb, int s, int lane) {
    const int g = lane >> 4;
    if constexpr (LANE_BYTES == 16) {
      return run16(tile, rb, kbyte(s, g, 0), lane);
    } else {
      const i32x4 a = run16(tile, rb, kbyte(s, g, 0), lane);
      const i32x4 b = run16(tile, rb, kbyte(s, g, 1), lane);
      return i32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    }
  }
};

}  // namespace mcg
