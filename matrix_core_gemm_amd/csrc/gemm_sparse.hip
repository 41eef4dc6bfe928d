// gemm_sparse.hip -- 2:4 structured-sparse GEMM on the sparse matrix cores (SMFMAC) and the
// device 2:4 compressor.
//
// The sparse operand follows the 2:4 model of "RDNA4 sparse WMMA builtins"
// (Structured sparsity (2:4 pattern): in every group of four along K at most two
// values are non-zero; only those are stored, halving A's storage and
// bandwidth; an index of 2-bit positions tells the hardware where each stored
// value sits; Common parameters: the index operand packs the positions of all
// values a lane holds into one 32-bit register).  The same model is provided on
// CDNA by SMFMAC, the wave64 sparse MFMA named on that page's introduction.
//
// Index layout in memory (the library's canonical form): group g of row i has
// the 4-bit code p0 | p1 << 2 at bits 4*(g % 8) of word g/8.  On gfx950 the
// sparse instructions read, per lane, the codes of the groups its kept values
// belong to, nibble n for kept values 2n and 2n+1 (measured): a lane of the
// 16-bit instructions (8 kept values, 4 groups) uses one 16-bit half of a
// canonical word, a lane of the 8-bit instructions (16 kept values, 8 groups)
// a whole word.  So a lane's index is a slice of one canonical word and needs
// no re-packing.
//
// Sparse kernel structure: as the dense kernel (256 threads, 2 x 2 waves,
// double-buffered LDS), with K tiles of KD dense k (128 for 16-bit, 256 for
// 8-bit elements): kept values 128 bytes per row, index KD / 32 words per row,
// B 256 bytes of K per column.  The sparse operand must be the instruction's
// first operand, so output lanes hold four consecutive rows of one column of D.
#include "gemm_kernels.hpp"
#include "tile_io.hpp"

namespace mcg {

// Replace every all-zero 4-bit code with 0b0100 (positions 0 and 1).  Zero codes
// only occur past the end of K (padding) where all values are zero; this keeps
// every code the instruction sees a valid 2:4 selection.
__device__ __forceinline__ uint32_t fix_zero_codes(uint32_t w) {
  uint32_t t = w | (w >> 1);
  t |= t >> 2;
  const uint32_t zero = (~t) & 0x11111111u;
  return w | (zero << 2);
}

// ---------------------------------------------------------------- 16x16 ops
// Per instruction s of a tile, lane l serves row / column l & 15 and lane
// group g = l >> 4 (measured layouts):
//   16-bit (16x16x64): kept values of dense k [16g, 16g + 16) of the
//     instruction's 64 (8 values, kept bytes [32s... see frag_a]); B k
//     [8g, 8g + 8) and [32 + 8g, 40 + 8g); codes in half g % 2 of word 2s + g / 2.
//   8-bit (16x16x128): kept values of dense k [32g, 32g + 32) (16 values); B
//     k [16g, 16g + 16) and [64 + 16g, 80 + 16g); codes in word 4s + g.
// In bytes both read 16 kept bytes at 16 (4s + g) and B bytes at 128s + 16g
// and 128s + 64 + 16g.
template <int EB_>
struct SpTile {
  static constexpr int EB = EB_;
  static constexpr int KD = 256 / EB_;  // dense k per LDS tile
  static constexpr int IW = KD / 32;    // index words per row and tile
};

template <class R>
__device__ __forceinline__ i32x8 sp_b_bytes(const lds_char* t, int rb, int s, int g, int lane) {
  const i32x4 lo = R::run16(t, rb, 128 * s + 16 * g, lane);
  const i32x4 hi = R::run16(t, rb, 128 * s + 64 + 16 * g, lane);
  return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

template <bool F16>
struct SpH : SpTile<2> {  // bfloat16 / binary16
  static constexpr int K_STEP = 64;  // dense k per instruction
  static constexpr bool INT_ACC = false;
  using acc_t = f32x4;
  using frag_a_t = i32x4;
  template <class R>
  __device__ static __forceinline__ i32x4 frag_a(const lds_char* t, int rb, int s, int lane) {
    return R::run16(t, rb, 16 * (4 * s + (lane >> 4)), lane);
  }
  template <class R>
  __device__ static __forceinline__ i32x8 frag_b(const lds_char* t, int rb, int s, int lane) {
    return sp_b_bytes<R>(t, rb, s, lane >> 4, lane);
  }
  __device__ static __forceinline__ int frag_i(const lds_char* ti, int row, int s, int lane) {
    const int g = lane >> 4;
    const uint32_t w = *(const __attribute__((address_space(3))) uint32_t*)(ti + row * 4 * IW + 4 * (2 * s + (g >> 1)));
    return (int)(fix_zero_codes(w >> (16 * (g & 1))) & 0xffffu);
  }
  __device__ static __forceinline__ acc_t mma(i32x4 a, i32x8 b, acc_t c, int idx) {
    if constexpr (F16)
      return __builtin_amdgcn_smfmac_f32_16x16x64_f16(bit_cast<f16x8>(a), bit_cast<f16x16>(b), c, idx, 0, 0);
    else
      return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(bit_cast<bf16x8>(a), bit_cast<bf16x16>(b), c, idx, 0, 0);
  }
};

// 8-bit: KIND 0 int8, 1 native fp8 (FA / FB = formats of A / B: 0 E4M3, 1 E5M2)
template <int KIND, int FA = 0, int FB = 0>
struct Sp8 : SpTile<1> {
  static constexpr int K_STEP = 128;
  static constexpr bool INT_ACC = KIND == 0;
  using acc_t = typename std::conditional<KIND == 0, i32x4, f32x4>::type;
  template <class R>
  __device__ static __forceinline__ i32x4 frag_a(const lds_char* t, int rb, int s, int lane) {
    return R::run16(t, rb, 16 * (4 * s + (lane >> 4)), lane);
  }
  template <class R>
  __device__ static __forceinline__ i32x8 frag_b(const lds_char* t, int rb, int s, int lane) {
    return sp_b_bytes<R>(t, rb, s, lane >> 4, lane);
  }
  __device__ static __forceinline__ int frag_i(const lds_char* ti, int row, int s, int lane) {
    const uint32_t w = *(const __attribute__((address_space(3))) uint32_t*)(ti + row * 4 * IW + 4 * (4 * s + (lane >> 4)));
    return (int)fix_zero_codes(w);
  }
  __device__ static __forceinline__ acc_t mma(i32x4 a, i32x8 b, acc_t c, int idx) {
    if constexpr (KIND == 0) return __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, c, idx, 0, 0);
    else if constexpr (FA == 0 && FB == 0) return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, c, idx, 0, 0);
    else if constexpr (FA == 0 && FB == 1) return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_bf8(a, b, c, idx, 0, 0);
    else if constexpr (FA == 1 && FB == 0) return __builtin_amdgcn_smfmac_f32_16x16x128_bf8_fp8(a, b, c, idx, 0, 0);
    else return __builtin_amdgcn_smfmac_f32_16x16x128_bf8_bf8(a, b, c, idx, 0, 0);
  }
};

// fp8 widened exactly to bfloat16 and multiplied by the bfloat16 instruction
// (K below the native-fp8 threshold): the 8-bit tiles of Sp8, read in the
// 16-bit instruction's k assignment 8 bytes at a time and converted.
template <int FA, int FB>
struct Sp8W : SpTile<1> {
  static constexpr int K_STEP = 64;
  static constexpr bool INT_ACC = false;
  using acc_t = f32x4;
  template <class R>
  __device__ static __forceinline__ i32x4 frag_a(const lds_char* t, int rb, int s, int lane) {
    return fp8x8_to_bf16x8<FA>(R::run8(t, rb, 32 * s + 8 * (lane >> 4), lane));
  }
  template <class R>
  __device__ static __forceinline__ i32x8 frag_b(const lds_char* t, int rb, int s, int lane) {
    const int g = lane >> 4;
    const i32x4 lo = fp8x8_to_bf16x8<FB>(R::run8(t, rb, 64 * s + 8 * g, lane));
    const i32x4 hi = fp8x8_to_bf16x8<FB>(R::run8(t, rb, 64 * s + 32 + 8 * g, lane));
    return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
  __device__ static __forceinline__ int frag_i(const lds_char* ti, int row, int s, int lane) {
    const int g = lane >> 4;
    const uint32_t w = *(const __attribute__((address_space(3))) uint32_t*)(ti + row * 4 * IW + 4 * (2 * s + (g >> 1)));
    return (int)(fix_zero_codes(w >> (16 * (g & 1))) & 0xffffu);
  }
  __device__ static __forceinline__ acc_t mma(i32x4 a, i32x8 b, acc_t c, int idx) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(bit_cast<bf16x8>(a), bit_cast<bf16x16>(b), c, idx, 0, 0);
  }
};

template <class Op, int LB, int BM, int BN, bool ALIGNED>
__global__ __launch_bounds__(256) void gemm_sparse_kernel(SparseArgs p) {
  constexpr int NT = 256;
  constexpr int EB = Op::EB;
  constexpr int KD = Op::KD;            // dense K per tile
  constexpr int IW = Op::IW;            // index words per row and tile
  constexpr int KTB_A = KD / 2 * EB;    // 128 bytes of kept values per row
  constexpr int KTB_B = KD * EB;        // 256 bytes of dense K per column
  constexpr int STEPS = KD / Op::K_STEP;
  constexpr int WTM = BM / 2 / 16, WTN = BN / 2 / 16;
  using GA = TileGeom<EB, LAYOUT_K, BM, KTB_A>;
  using GB = TileGeom<EB, LB, BN, KTB_B>;
  using RA = FragReader<EB, 16, LAYOUT_K, BM, KTB_A>;
  using RB = FragReader<EB, 16, LB, BN, KTB_B>;
  using acc_t = typename Op::acc_t;
  constexpr int IDX_BYTES = BM * 4 * IW;
  static_assert(KTB_A == 128 && KTB_B == 256 && IW % 4 == 0, "tile geometry");

  __shared__ __attribute__((aligned(16))) char smem_raw[2 * (GA::BYTES + GB::BYTES + IDX_BYTES)];
  lds_char* smem = (lds_char*)smem_raw;
  constexpr int STAGE = GA::BYTES + GB::BYTES + IDX_BYTES;
  lds_char* ldsA[2] = {smem, smem + STAGE};
  lds_char* ldsB[2] = {smem + GA::BYTES, smem + STAGE + GA::BYTES};
  lds_char* ldsI[2] = {smem + GA::BYTES + GB::BYTES, smem + STAGE + GA::BYTES + GB::BYTES};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int pid = blockIdx.x;
  const int group = 8;
  const int tiles_in_group = group * p.tiles_n;
  const int gid = pid / tiles_in_group;
  const int first_m = gid * group;
  const int gsize = min(p.tiles_m - first_m, group);
  const int tm = first_m + (pid % tiles_in_group) % gsize;
  const int tn = (pid % tiles_in_group) / gsize;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int nk = (int)((p.K + KD - 1) / KD);
  const int64_t Kc = p.K / 2;             // kept values per row
  const int64_t nwords = (p.K + 31) / 32; // index words per row

  TileLoader<EB, LAYOUT_K, BM, NT, ALIGNED, KTB_A> la;
  TileLoader<EB, LB, BN, NT, ALIGNED, KTB_B> lb;
  i32x4 ireg[IW / 4];  // threads < BM: the index words of one row
  auto load_tiles = [&](int kt) {
    const int64_t k0 = (int64_t)kt * KD;
    la.load(p.Ac, p.lda_c, m0, k0 / 2, p.M, Kc, tid);
    if constexpr (LB == LAYOUT_K) lb.load(p.B, p.ldb, n0, k0, p.N, p.K, tid);
    else lb.load(p.B, p.ldb, k0, n0, p.K, p.N, tid);
    if (tid < BM) {
      const int64_t row = m0 + tid, w0 = k0 / 32;
      const uint32_t* src = p.idx + row * p.ld_idx + w0;
#pragma unroll
      for (int v = 0; v < IW / 4; ++v) {
        if (ALIGNED && row < p.M && w0 + 4 * v + 4 <= nwords) {
          ireg[v] = *(const i32x4*)(src + 4 * v);
        } else {
          ireg[v] = i32x4{0, 0, 0, 0};
          if (row < p.M)
            for (int e = 0; e < 4; ++e)
              if (w0 + 4 * v + e < nwords) ireg[v][e] = (int)src[4 * v + e];
        }
      }
    }
  };
  auto store_tiles = [&](int buf) {
    la.store(ldsA[buf], tid);
    lb.store(ldsB[buf], tid);
    if (tid < BM)
#pragma unroll
      for (int v = 0; v < IW / 4; ++v) lds_write_b128(ldsI[buf], tid * 4 * IW + 16 * v, ireg[v]);
  };

  acc_t acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  if (nk > 0) {
    load_tiles(0);
    store_tiles(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles(kt + 1);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      i32x4 fa[WTM];
      int fi[WTM];
      i32x8 fb[WTN];
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        const int rb = wm * (BM / 2) + i * 16;
        fa[i] = Op::template frag_a<RA>(ldsA[cur], rb, s, lane);
        fi[i] = Op::frag_i(ldsI[cur], rb + (lane & 15), s, lane);
      }
#pragma unroll
      for (int j = 0; j < WTN; ++j) fb[j] = Op::template frag_b<RB>(ldsB[cur], wn * (BN / 2) + j * 16, s, lane);
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j) acc[i][j] = Op::mma(fa[i], fb[j], acc[i][j], fi[i]);
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // epilogue: the sparse (A) fragment is the instruction's first operand, so
  // element (i', j') of its 16 x 16 accumulator layout is D[m][n] with m = i',
  // n = j' within the block, (i', j') = ACC::coord(lane, r): 4 consecutive rows
  // of one column per lane
  using ACC = frag::Acc<frag::ACC_16x16>;
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int64_t n = n0 + wn * (BN / 2) + j * 16 + ACC::coord(lane, 0).j;
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * (BM / 2) + i * 16 + ACC::coord(lane, r).i;
        if (m >= p.M) continue;
        const int64_t off = m * p.ldc + n;
        if constexpr (Op::INT_ACC) {
          const uint32_t c = p.use_c ? (uint32_t)((const int*)p.C)[off] : 0u;
          ((int*)p.D)[off] = (int)((uint32_t)p.alpha_i * (uint32_t)acc[i][j][r] + (uint32_t)p.beta_i * c);
        } else {
          combine_store(p.C, p.D, off, acc[i][j][r], p.alpha, p.beta, p.use_c, p.out);
        }
      }
    }
  }
}

template <class Op, int LB, bool AL>
static hipError_t launch_sparse_one(const SparseArgs& a0, hipStream_t s) {
  constexpr int BM = 128, BN = 128;
  SparseArgs a = a0;
  a.tiles_m = (int)((a.M + BM - 1) / BM);
  a.tiles_n = (int)((a.N + BN - 1) / BN);
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_sparse_kernel<Op, LB, BM, BN, AL>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class Op>
static hipError_t launch_sparse_layouts(int lb, bool aligned, const SparseArgs& a, hipStream_t s) {
  if (lb == LAYOUT_K)
    return aligned ? launch_sparse_one<Op, LAYOUT_K, true>(a, s) : launch_sparse_one<Op, LAYOUT_K, false>(a, s);
  return aligned ? launch_sparse_one<Op, LAYOUT_MN, true>(a, s) : launch_sparse_one<Op, LAYOUT_MN, false>(a, s);
}

hipError_t launch_sparse(int dtA, int dtB, int lb, bool aligned, const SparseArgs& a, hipStream_t s) {
  if (dtA == DT_BF16) return launch_sparse_layouts<SpH<false>>(lb, aligned, a, s);
  if (dtA == DT_F16) return launch_sparse_layouts<SpH<true>>(lb, aligned, a, s);
  if (dtA == DT_I8) return launch_sparse_layouts<Sp8<0>>(lb, aligned, a, s);
  const int fa = f8fmt(dtA), fb = f8fmt(dtB);
  if (a.K >= FP8_NATIVE_MIN_K) {
    if (fa == 0 && fb == 0) return launch_sparse_layouts<Sp8<1, 0, 0>>(lb, aligned, a, s);
    if (fa == 0 && fb == 1) return launch_sparse_layouts<Sp8<1, 0, 1>>(lb, aligned, a, s);
    if (fa == 1 && fb == 0) return launch_sparse_layouts<Sp8<1, 1, 0>>(lb, aligned, a, s);
    return launch_sparse_layouts<Sp8<1, 1, 1>>(lb, aligned, a, s);
  }
  if (fa == 0 && fb == 0) return launch_sparse_layouts<Sp8W<0, 0>>(lb, aligned, a, s);
  if (fa == 0 && fb == 1) return launch_sparse_layouts<Sp8W<0, 1>>(lb, aligned, a, s);
  if (fa == 1 && fb == 0) return launch_sparse_layouts<Sp8W<1, 0>>(lb, aligned, a, s);
  return launch_sparse_layouts<Sp8W<1, 1>>(lb, aligned, a, s);
}

// ------------------------------------------------------------- compressor
// One thread per (row, index word): reads the 32 dense values of 8 groups,
// keeps the non-zeros of each group (ascending; padded with the lowest free
// positions), writes the kept values and the word of codes.  +0 and -0 count
// as zero and NaN as non-zero.  A group with more than two non-zeros is
// counted and written as two zeros with code 0b0100.

template <int EB>
__device__ __forceinline__ bool nonzero_code(uint32_t v) {
  if constexpr (EB == 2) return (v & 0x7fffu) != 0;
  else return (v & 0x7fu) != 0;
}

template <int EB, bool INT8>
__global__ __launch_bounds__(256) void compress24_kernel(CompressArgs p) {
  const int64_t nwords = (p.K + 31) / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= p.M * nwords) return;
  const int64_t row = t / nwords, w = t % nwords;
  const int64_t g0 = w * 8;
  const int64_t ngroups = p.K / 4;
  const char* src = p.A + (row * p.lda + g0 * 4) * EB;
  char* dst = p.Ac + (row * p.lda_c + g0 * 2) * EB;
  uint32_t word = 0;
  int bad = 0;
  for (int gi = 0; gi < 8; ++gi) {
    if (g0 + gi >= ngroups) break;
    uint32_t v[4];
    for (int e = 0; e < 4; ++e) {
      if constexpr (EB == 2) v[e] = *(const uint16_t*)(src + (gi * 4 + e) * 2);
      else v[e] = (uint8_t)src[gi * 4 + e];
    }
    int pos[4], nz = 0;
    for (int e = 0; e < 4; ++e) {
      const bool isnz = INT8 ? (v[e] != 0) : nonzero_code<EB>(v[e]);
      if (isnz) pos[nz++ & 3] = e;
    }
    int p0, p1;
    uint32_t k0, k1;
    if (nz > 2) {
      ++bad;
      p0 = 0; p1 = 1; k0 = 0; k1 = 0;
    } else {
      if (nz == 0) { p0 = 0; p1 = 1; }
      else if (nz == 1) {
        if (pos[0] == 0) { p0 = 0; p1 = 1; }
        else { p0 = 0; p1 = pos[0]; }
      } else { p0 = pos[0]; p1 = pos[1]; }
      k0 = v[p0]; k1 = v[p1];
    }
    word |= (uint32_t)(p0 | (p1 << 2)) << (4 * gi);
    if constexpr (EB == 2) {
      *(uint16_t*)(dst + (gi * 2) * 2) = (uint16_t)k0;
      *(uint16_t*)(dst + (gi * 2 + 1) * 2) = (uint16_t)k1;
    } else {
      dst[gi * 2] = (char)k0;
      dst[gi * 2 + 1] = (char)k1;
    }
  }
  p.idx[row * p.ld_idx + w] = word;
  if (bad && p.violations) atomicAdd(p.violations, bad);
}

// One 16-byte chunk of a row (G = 2 groups of 16-bit or 4 groups of 8-bit
// values): its 4-bit codes (group gi at bits 4 gi) and its kept values (8 bytes),
// by the selection rule of compress24_kernel; bad counts groups with more than
// two non-zeros.
template <int EB, bool INT8>
__device__ __forceinline__ void compress_chunk(const i32x4& v, uint32_t& code, uint64_t& kept, int& bad) {
  constexpr int G = 16 / (4 * EB);
  code = 0;
  kept = 0;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    uint32_t x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int el = 4 * gi + e;
      if constexpr (EB == 2) x[e] = ((uint32_t)v[el >> 1] >> (16 * (el & 1))) & 0xFFFFu;
      else x[e] = ((uint32_t)v[el >> 2] >> (8 * (el & 3))) & 0xFFu;
    }
    int pos[4], nz = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool isnz = INT8 ? (x[e] != 0) : nonzero_code<EB>(x[e]);
      if (isnz) pos[nz++ & 3] = e;
    }
    int p0, p1;
    uint32_t k0, k1;
    if (nz > 2) {
      ++bad;
      p0 = 0; p1 = 1; k0 = 0; k1 = 0;
    } else {
      if (nz == 0) { p0 = 0; p1 = 1; }
      else if (nz == 1) {
        if (pos[0] == 0) { p0 = 0; p1 = 1; }
        else { p0 = 0; p1 = pos[0]; }
      } else { p0 = pos[0]; p1 = pos[1]; }
      k0 = x[p0]; k1 = x[p1];
    }
    code |= (uint32_t)(p0 | (p1 << 2)) << (4 * gi);
    kept |= (uint64_t)k0 << (2 * gi * 8 * EB);
    kept |= (uint64_t)k1 << ((2 * gi + 1) * 8 * EB);
  }
}

// Vector forms for aligned rows (K * elem_bytes a multiple of 16).  Chunk
// slots past the end of a row (a partial last index word) give zero codes and
// store no values.  Grid: x covers a row in blocks of 256 lanes, y strides over
// the rows.  Same selection rule as compress24_kernel.  Measured on MI355X at
// 8192^2, against one lane per chunk with 1- or 2-byte code stores: 16-bit
// elements gain nothing cold and 0-5% warm from the shuffled words; 8-bit
// elements gain 9% cold and warm with one lane per word (a lane per word on
// 16-bit elements lost 7% cold: each load instruction then covers a quarter of
// every line it touches).
//
// 16-bit elements: one lane per 16-byte chunk (2 groups), consecutive lanes on
// consecutive chunks, so every 16-byte load and 8-byte store of a wavefront
// covers 1 KiB or 512 bytes of contiguous memory.  The 4 lanes of one index word
// combine their codes with lane shuffles and the first stores the word.  Each
// lane takes the same chunk of VR consecutive rows, all loads first, and the
// dense input is read once, with non-temporal loads.  Measured at 8192^2 bf16
// against one row per lane and ordinary loads (bit-identical): 1.18-1.23x faster
// with L2 and MALL flushed first (the usual case: a matrix compressed once), 4-6%
// slower when the same input is compressed again while it sits in the MALL (4
// rows per lane: a little faster flushed, 9% slower cached).
constexpr int VR = 2;
template <int EB, bool INT8>
__global__ __launch_bounds__(256) void compress24_vec_kernel(CompressArgs p) {
  constexpr int CH = 32 * EB / 16;  // chunks per index word
  constexpr int G = 16 / (4 * EB);  // groups per chunk
  const int64_t nwords = (p.K + 31) / 32;
  const int64_t nchunks = p.K * EB / 16;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;  // chunk slot; blocks start at a word boundary
  const int sub = threadIdx.x % CH;                            // chunk of its word
  int bad = 0;
  for (int64_t r0 = (int64_t)blockIdx.y * VR; r0 < p.M; r0 += (int64_t)gridDim.y * VR) {
    i32x4 v[VR];
#pragma unroll
    for (int r = 0; r < VR; ++r)
      v[r] = c < nchunks && r0 + r < p.M
                 ? __builtin_nontemporal_load((const i32x4*)(p.A + (r0 + r) * p.lda * EB + c * 16))
                 : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int64_t row = r0 + r;
      if (row >= p.M) break;
      uint32_t code = 0;
      uint64_t kept = 0;
      if (c < nchunks) {
        compress_chunk<EB, INT8>(v[r], code, kept, bad);
        *(uint64_t*)(p.Ac + row * p.lda_c * EB + c * 8) = kept;
      }
      uint32_t word = code << (4 * G * sub);
#pragma unroll
      for (int d = 1; d < CH; d <<= 1) word |= (uint32_t)__shfl_xor((int)word, d, CH);
      if (sub == 0 && c / CH < nwords) p.idx[row * p.ld_idx + c / CH] = word;
    }
  }
  if (bad && p.violations) atomicAdd(p.violations, bad);
}

// 8-bit elements: one lane per index word of a row (2 chunks of 4 groups),
// consecutive lanes on consecutive words: two 16-byte loads and one 16-byte
// store of kept values per lane (8-byte stores when the destination rows are not
// 16-byte aligned), and the word stored whole.  Non-temporal loads (the input is
// read once): int8 and E4M3 8192^2 1.08-1.15x faster with L2 and MALL flushed
// first, 4-6% slower when compressed again from the MALL; more rows per lane
// measured slower here.
template <bool INT8>
__global__ __launch_bounds__(256) void compress24_word8_kernel(CompressArgs p, int a16) {
  const int64_t nwords = (p.K + 31) / 32;
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= nwords) return;
  const int64_t nchunks = p.K / 16;
  const int64_t c0 = 2 * w;
  int bad = 0;
  for (int64_t row = blockIdx.y; row < p.M; row += gridDim.y) {
    const char* src = p.A + row * p.lda + c0 * 16;
    char* dst = p.Ac + row * p.lda_c + c0 * 8;
    i32x4 v[2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
      v[k] = c0 + k < nchunks ? __builtin_nontemporal_load((const i32x4*)(src + 16 * k)) : i32x4{0, 0, 0, 0};
    uint32_t word = 0;
    uint64_t kept[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t code;
      compress_chunk<1, INT8>(v[k], code, kept[k], bad);
      if (c0 + k < nchunks) word |= code << (16 * k);
    }
    if (a16 && c0 + 2 <= nchunks) {
      *(i32x4*)dst = i32x4{(int)(uint32_t)kept[0], (int)(uint32_t)(kept[0] >> 32), (int)(uint32_t)kept[1],
                           (int)(uint32_t)(kept[1] >> 32)};
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (c0 + k < nchunks) *(uint64_t*)(dst + 8 * k) = kept[k];
    }
    p.idx[row * p.ld_idx + w] = word;
  }
  if (bad && p.violations) atomicAdd(p.violations, bad);
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

hipError_t launch_compress(int dtype, const CompressArgs& a, hipStream_t s) {
  if (a.violations) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, s, a.violations);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nwords = (a.K + 31) / 32;
  const int eb = (dtype == DT_BF16 || dtype == DT_F16) ? 2 : 1;
  const bool vec = (a.K * eb) % 16 == 0 && (uintptr_t)a.A % 16 == 0 && (a.lda * eb) % 16 == 0 &&
                   (uintptr_t)a.Ac % 8 == 0 && (a.lda_c * eb) % 8 == 0;
  if (vec) {
    if (a.M <= 0 || nwords <= 0) return hipSuccess;
    const unsigned rows = (unsigned)(a.M < 65535 ? a.M : 65535);
    if (eb == 2) {
      const int64_t ry = (a.M + VR - 1) / VR;  // row blocks of VR rows
      const int64_t slots = nwords * 4;  // chunk slots per row (whole index words)
      if ((slots + 255) / 256 > 0x7fffffff) return hipErrorInvalidValue;
      hipLaunchKernelGGL((compress24_vec_kernel<2, false>),
                         dim3((unsigned)((slots + 255) / 256), (unsigned)(ry < 65535 ? ry : 65535)), dim3(256), 0, s, a);
      return hipGetLastError();
    }
    if ((nwords + 255) / 256 > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((nwords + 255) / 256), rows);
    const int a16 = (uintptr_t)a.Ac % 16 == 0 && a.lda_c % 16 == 0;
    if (dtype == DT_I8) hipLaunchKernelGGL((compress24_word8_kernel<true>), grid, dim3(256), 0, s, a, a16);
    else hipLaunchKernelGGL((compress24_word8_kernel<false>), grid, dim3(256), 0, s, a, a16);
    return hipGetLastError();
  }
  const int64_t threads = a.M * nwords;
  if (threads <= 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (dtype == DT_BF16 || dtype == DT_F16)
    hipLaunchKernelGGL((compress24_kernel<2, false>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  else if (dtype == DT_I8)
    hipLaunchKernelGGL((compress24_kernel<1, true>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((compress24_kernel<1, false>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mcg
