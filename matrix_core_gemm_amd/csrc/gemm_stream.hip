// gemm_stream.hip -- streaming dense MFMA kernel for skinny problems (N <= 32
// or M <= 32) on gfx950.
//
// Same operation as the other dense kernels (the matrix fused multiply-add of
// "Accurate Models of AMD Matrix Cores", Section 2, Eq. (1), tiled over K as in
// "CDNA3 dense MFMA builtins", Using MFMA builtins as a compute policy).  When
// one output dimension is small the product is bound by reading the large
// operand once from HBM, so the kernel is built around that stream:
//   - the "wide" operand (A when N is small, B when M is small) is cut into
//     blocks of BW = 32, 64 or 128 rows (M rows of A / N columns of B), one
//     per workgroup of 4 wavefronts, BW chosen so that every CU gets a block;
//     the "narrow" operand has at most 32 rows, zero-filled past M or N, and
//     is shared by every workgroup through L2;
//   - either operand may be K- or MN-contiguous (an MN-contiguous tile keeps one
//     LDS row per k and is gathered with transposing reads);
//   - K is staged in tiles of 128 bytes per row through a ring of LDS stages
//     (144 KiB, one workgroup per CU) filled by buffer_load ... lds (whole
//     128-byte lines per 8 lanes, no VGPRs); all but one stage are in flight
//     while one is multiplied, which is what keeps HBM busy;
//   - the wide block is multiplied in 32-row blocks by the 32 narrow rows with
//     32 x 32 MFMA instructions (one accumulator tile per wavefront); the
//     4 / (BW / 32) wavefronts of a block take alternate instructions of each
//     K tile and their sums are added through LDS at the end, in a fixed order;
//   - split K (grid.y > 1) as in the general kernel: alpha times the partial
//     sums is added into a zeroed D with device-scope atomic adds, and beta * C
//     by a last pass; otherwise the epilogue computes D = alpha*acc + beta*C
//     itself in every output format.
// Preconditions (checked on the host): 16-byte aligned operands, K * elem_bytes
// and ld * elem_bytes multiples of 16, and every operand window below 2 GiB
// (32-bit buffer offsets).
#include "fast_tiles.hpp"
#include "gemm_kernels.hpp"

namespace mcg {
namespace stream {

using namespace fast;

constexpr int KTB = 128;      // bytes of K per LDS row and stage
constexpr int NR = 32;        // narrow rows
constexpr int THREADS = 256;  // 4 wavefronts (fast::NW)
constexpr int LDS_RING = 147456;  // bytes of LDS ring per workgroup (one workgroup per CU)
constexpr int AUX_NT = 2;         // buffer cache-policy bit: non-temporal (gfx950)

static_assert(THREADS == 64 * NW, "loaders assume NW wavefronts");

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Stages of the LDS ring for a wide block of BW rows.
template <int EB, int BW>
constexpr int ring_stages() {
  return LDS_RING / ((BW + NR) * KTB);
}

// One instruction's fragment of a 32-row block of a stage: K-contiguous tiles
// take ordinary LDS reads; MN-contiguous ones (W bytes per LDS row) take their
// transposing reads from one inline-asm block that waits for its own reads
// (lds_read_tr_x2 / lds_read_tr_x4): the read16k reads of kb lie at rows r and
// r + 4 (16-bit) or r + 8 (8-bit), those of kb + 16 (32-byte lanes) 16 and 24
// rows after r.
template <class Op, class Rd, int LAYOUT, int W>
struct StreamFrag {
  using frag_t = typename Op::frag_t;
  static constexpr int EB = Op::EB, LB16 = Op::LANE_BYTES;
  static __device__ __forceinline__ frag_t read(const lds_char* tile, int rb, int kb, int lane) {
    if constexpr (LAYOUT == LAYOUT_K) {
      if constexpr (LB16 == 16) {
        return Rd::read16k(tile, rb, kb, lane);
      } else {
        const i32x4 x = Rd::read16k(tile, rb, kb, lane), y = Rd::read16k(tile, rb, kb + 16, lane);
        return frag_t{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
      }
    } else {
      const uint32_t ad[1] = {Rd::mn_addr(tile, rb, kb, lane)};
      if constexpr (LB16 == 16) {
        i32x2 r[1][2];
        lds_read_tr_x2<EB, (EB == 2 ? 4 : 8) * W>(ad, r);
        return frag_t{r[0][0].x, r[0][0].y, r[0][1].x, r[0][1].y};
      } else {
        static_assert(EB == 1, "32-byte lanes: 8-bit operands");
        i32x2 r[1][4];
        lds_read_tr_x4<EB, 8 * W, 16 * W, 24 * W>(ad, r);
        return frag_t{r[0][0].x, r[0][0].y, r[0][1].x, r[0][1].y, r[0][2].x, r[0][2].y, r[0][3].x, r[0][3].y};
      }
    }
  }
};

template <class Op, int LA, int LB, bool WIDE_A, int BW>
__global__ __launch_bounds__(THREADS) void gemm_stream_kernel(DenseArgs p) {
  constexpr int EB = Op::EB;
  constexpr int LB16 = Op::LANE_BYTES;         // bytes of K per lane and instruction (16 or 32)
  constexpr int SPS = KTB / (2 * LB16);        // instructions per stage
  constexpr int RBLK = BW / 32;                // 32-row blocks of the wide operand
  constexpr int KG = NW / RBLK;                // wavefronts sharing one block, splitting K
  constexpr int NS = ring_stages<EB, BW>();
  constexpr int RA_ROWS = WIDE_A ? BW : NR, RB_ROWS = WIDE_A ? NR : BW;
  using GA = Geom<EB, LA, RA_ROWS, KTB>;
  using GB = Geom<EB, LB, RB_ROWS, KTB>;
  using LdA = LineLoader<EB, LA, RA_ROWS, KTB>;
  using LdB = LineLoader<EB, LB, RB_ROWS, KTB>;
  using RdA = Reader<EB, LA, RA_ROWS, KTB>;
  using RdB = Reader<EB, LB, RB_ROWS, KTB>;
  using acc_t = typename Op::acc_t;
  using frag_t = typename Op::frag_t;
  constexpr int STAGE = GA::BYTES + GB::BYTES;
  constexpr int IPS = LdA::INSTR + LdB::INSTR;  // DMA instructions per wave and stage
  static_assert(NS * STAGE <= LDS_RING && NS >= 3, "ring");
  static_assert((NS - 2) * IPS < 64, "vmcnt counts at most 63 instructions");
  static_assert(RBLK * KG == NW, "wave arrangement");

  __shared__ __attribute__((aligned(1024))) char smem_raw[NS * STAGE];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int blk = wave % RBLK, kg = wave / RBLK;  // 32-row block and K group of this wave

  const int64_t w0 = (int64_t)blockIdx.x * BW;  // first wide row of this workgroup
  const int64_t m0 = WIDE_A ? w0 : 0, n0 = WIDE_A ? 0 : w0;
  const int rbA = WIDE_A ? 32 * blk : 0, rbB = WIDE_A ? 0 : 32 * blk;

  LdA la;
  LdB lb;
  if constexpr (LA == LAYOUT_K)
    la.init(p.A + m0 * p.lda * EB, (uint32_t)(min(p.M - m0, (int64_t)RA_ROWS) * p.lda * EB), p.lda, p.K, wave, lane);
  else
    la.init(p.A + m0 * EB, (uint32_t)((p.K * p.lda - m0) * EB), p.lda, p.K, wave, lane);
  if constexpr (LB == LAYOUT_K)
    lb.init(p.B + n0 * p.ldb * EB, (uint32_t)(min(p.N - n0, (int64_t)RB_ROWS) * p.ldb * EB), p.ldb, p.K, wave, lane);
  else
    lb.init(p.B + n0 * EB, (uint32_t)((p.K * p.ldb - n0) * EB), p.ldb, p.K, wave, lane);

  // this workgroup's K tiles: [kt0, kt0 + nkl)
  const int nk_all = (int)((p.K + KTB / EB - 1) / (KTB / EB));
  const int kt0 = (int)blockIdx.y * p.kt_per_split;
  const int nkl = min(nk_all - kt0, p.kt_per_split);

  // Workgroups start their walk over K at evenly spread tiles (step t takes
  // K tile kt0 + (t + rot) mod nkl), so that at any moment they read different
  // tiles of the narrow operand rather than all the same few L2 lines.
  const int rot = nkl > 0 ? (int)(((int64_t)blockIdx.x * nkl) / gridDim.x) : 0;
  auto stage = [&](int t) { return smem + (t % NS) * STAGE; };
  // step t into its stage; steps past the range are issued as zero fills so
  // that every wave always has the same number of loads in flight
  auto issue = [&](int t) {
    const bool live = t < nkl;
    int kt = t + rot;
    kt = kt0 + (kt >= nkl ? kt - nkl : kt);
    // the wide operand is read once: non-temporal, so that its lines do not
    // displace the narrow operand, which every workgroup reads, from the caches
    la.template issue_if<WIDE_A ? AUX_NT : 0>(stage(t), kt, 0, LdA::INSTR, wave, live);
    lb.template issue_if<WIDE_A ? 0 : AUX_NT>(stage(t) + GA::BYTES, kt, 0, LdB::INSTR, wave, live);
  };

  acc_t acc{};
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) issue(t);
  for (int t = 0; t < nkl; ++t) {
    wait_vmcnt<(NS - 2) * IPS>();  // this wave's part of tile t has landed
    barrier_lds();                 // ... and every wave's; stage of tile t - 1 is free
    issue(t + NS - 1);
    const lds_char* sA = stage(t);
    const lds_char* sB = sA + GA::BYTES;
    // instruction s of the stage goes to K group (t * SPS + s) mod KG
#pragma unroll
    for (int s = 0; s < SPS; ++s) {
      if (KG > 1 && (t * SPS + s) % KG != kg) continue;
      const int kb = 2 * LB16 * s + LB16 * g;  // lane group g's K bytes of instruction s
      // a K-contiguous operand's ordinary reads go before the other's asm block,
      // whose wait then covers them
      frag_t fa, fb;
      if constexpr (LA == LAYOUT_K || LB == LAYOUT_MN) {
        fa = StreamFrag<Op, RdA, LA, RA_ROWS * EB>::read(sA, rbA, kb, lane);
        fb = StreamFrag<Op, RdB, LB, RB_ROWS * EB>::read(sB, rbB, kb, lane);
      } else {
        fb = StreamFrag<Op, RdB, LB, RB_ROWS * EB>::read(sB, rbB, kb, lane);
        fa = StreamFrag<Op, RdA, LA, RA_ROWS * EB>::read(sA, rbA, kb, lane);
      }
      Op::mma(acc, fb, fa);
    }
  }
  wait_vmcnt<0>();  // no LDS DMA outstanding at exit

  if constexpr (KG > 1) {
    // sum the K groups' accumulators of each block in LDS, in K-group order
    barrier_lds();  // every wave is done with the ring
    if (kg > 0) {
      lds_char* slot = smem + ((kg - 1) * RBLK + blk) * 4096;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        lds_write_b128(slot, (r4 * 64 + lane) * 16,
                       i32x4{bit_cast<int>(acc[4 * r4]), bit_cast<int>(acc[4 * r4 + 1]),
                             bit_cast<int>(acc[4 * r4 + 2]), bit_cast<int>(acc[4 * r4 + 3])});
    }
    barrier_lds();
    if (kg > 0) return;
#pragma unroll
    for (int q = 1; q < KG; ++q) {
      const lds_char* slot = smem + ((q - 1) * RBLK + blk) * 4096;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const i32x4 v = lds_read_b128(slot, (r4 * 64 + lane) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (Op::INT_ACC) acc[4 * r4 + e] = (int)((uint32_t)acc[4 * r4 + e] + (uint32_t)v[e]);
          else acc[4 * r4 + e] += bit_cast<float>(v[e]);
        }
      }
    }
  }

  // epilogue: the instruction multiplied (B fragment) x (A fragment), so element
  // (i', j') of its 32 x 32 accumulator layout is D[m][n] with m = j', n = i':
  // register 4 r4 + e of the lane holds D[m][nb + 8 r4 + e] with (i', j') =
  // ACC::coord(lane, 4 r4) = (nb - n0 - rbB + 8 r4, m - m0 - rbA)
  using ACC = frag::Acc<frag::ACC_32x32>;
  const int64_t m = m0 + rbA + ACC::coord(lane, 0).j;
  if (m >= p.M) return;
  const int64_t nb = n0 + rbB + ACC::coord(lane, 0).i;
  if (gridDim.y > 1) {
    // split K: add alpha * partial sum into the zeroed D
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t n = nb + 8 * r4 + e;
        if (n >= p.N) continue;
        if constexpr (Op::INT_ACC)
          atomicAdd((int*)p.D + m * p.ldc + n, (int)((uint32_t)p.alpha_i * (uint32_t)acc[4 * r4 + e]));
        else
          atomicAdd((float*)p.D + m * p.ldc + n, p.alpha * acc[4 * r4 + e]);
      }
    return;
  }
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const int64_t n = nb + 8 * r4;
    if (n >= p.N) continue;
    const int64_t off = m * p.ldc + n;
    const bool full = p.vec_cd && n + 4 <= p.N;
    if constexpr (Op::INT_ACC) {
      const int* C = (const int*)p.C;
      int* D = (int*)p.D;
      i32x4 c = {0, 0, 0, 0};
      if (p.use_c) {
        if (full) c = *(const i32x4*)(C + off);
        else
          for (int e = 0; e < 4; ++e) if (n + e < p.N) c[e] = C[off + e];
      }
      i32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (int)((uint32_t)p.alpha_i * (uint32_t)acc[4 * r4 + e] + (uint32_t)p.beta_i * (uint32_t)c[e]);
      if (full) *(i32x4*)(D + off) = o;
      else
        for (int e = 0; e < 4; ++e) if (n + e < p.N) D[off + e] = o[e];
    } else if (p.out == OUT_32 && full) {
      const float* C = (const float*)p.C;
      const f32x4 c = p.use_c ? *(const f32x4*)(C + off) : f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = p.use_c ? __builtin_fmaf(p.alpha, acc[4 * r4 + e], p.beta * c[e]) : p.alpha * acc[4 * r4 + e];
      *(f32x4*)((float*)p.D + off) = o;
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < p.N) combine_store(p.C, p.D, off + e, acc[4 * r4 + e], p.alpha, p.beta, p.use_c, p.out);
    }
  }
}

template <class Op, int LA, int LB, bool WIDE_A>
static hipError_t launch_one(const DenseArgs& a, hipStream_t s) {
  const int64_t wide = WIDE_A ? a.M : a.N;
  const int bw = a.stream_bw;
  const int64_t blocks = (wide + bw - 1) / bw;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff || a.splits < 1 || a.splits > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks, (unsigned)a.splits);
  if (bw == 128) hipLaunchKernelGGL((gemm_stream_kernel<Op, LA, LB, WIDE_A, 128>), grid, dim3(THREADS), 0, s, a);
  else if (bw == 64) hipLaunchKernelGGL((gemm_stream_kernel<Op, LA, LB, WIDE_A, 64>), grid, dim3(THREADS), 0, s, a);
  else if (bw == 32) hipLaunchKernelGGL((gemm_stream_kernel<Op, LA, LB, WIDE_A, 32>), grid, dim3(THREADS), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <class Op, bool WIDE_A>
static hipError_t launch_layouts(int la, int lb, const DenseArgs& a, hipStream_t s) {
  if (la == LAYOUT_K && lb == LAYOUT_K) return launch_one<Op, LAYOUT_K, LAYOUT_K, WIDE_A>(a, s);
  if (la == LAYOUT_K) return launch_one<Op, LAYOUT_K, LAYOUT_MN, WIDE_A>(a, s);
  if (lb == LAYOUT_K) return launch_one<Op, LAYOUT_MN, LAYOUT_K, WIDE_A>(a, s);
  return launch_one<Op, LAYOUT_MN, LAYOUT_MN, WIDE_A>(a, s);
}

template <bool WIDE_A>
static hipError_t launch_ops(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s) {
  if (dtA == DT_BF16) return launch_layouts<BF16, WIDE_A>(la, lb, a, s);
  if (dtA == DT_F16) return launch_layouts<F16, WIDE_A>(la, lb, a, s);
  if (dtA == DT_I8) return launch_layouts<I8, WIDE_A>(la, lb, a, s);
  const int fa = f8fmt(dtA), fb = f8fmt(dtB);
  if (a.K >= FP8_NATIVE_MIN_K) {
    // P = B fragment, Q = A fragment: the P format is B's.
    if (fb == 0 && fa == 0) return launch_layouts<F8<0, 0>, WIDE_A>(la, lb, a, s);
    if (fb == 1 && fa == 0) return launch_layouts<F8<1, 0>, WIDE_A>(la, lb, a, s);
    if (fb == 0 && fa == 1) return launch_layouts<F8<0, 1>, WIDE_A>(la, lb, a, s);
    return launch_layouts<F8<1, 1>, WIDE_A>(la, lb, a, s);
  }
  if (fa == 0 && fb == 0) return launch_layouts<F8W<0, 0>, WIDE_A>(la, lb, a, s);
  if (fa == 0 && fb == 1) return launch_layouts<F8W<0, 1>, WIDE_A>(la, lb, a, s);
  if (fa == 1 && fb == 0) return launch_layouts<F8W<1, 0>, WIDE_A>(la, lb, a, s);
  return launch_layouts<F8W<1, 1>, WIDE_A>(la, lb, a, s);
}

}  // namespace stream

bool stream_path_ok(int dtA, int la, int lb, const DenseArgs& a, bool aligned) {
  const int64_t eb = (dtA == DT_BF16 || dtA == DT_F16) ? 2 : 1;
  if (!aligned || a.K == 0 || (a.K * eb) % 16 != 0) return false;
  if (a.N > stream::NR && a.M > stream::NR) return false;
  // buffer windows and every offset into them (K tiles up to one past the end
  // of K, out-of-range offsets up to 2^31 + window) below 2 GiB
  const int64_t lim = (int64_t)1 << 31;
  const int64_t kpad = stream::KTB / eb;
  const int64_t ra = a.N <= stream::NR && a.N <= a.M ? 128 : stream::NR;  // rows of A per block (at most)
  const int64_t rb = ra == 128 ? stream::NR : 128;
  const int64_t wa = la == 0 ? ra * a.lda * eb : (a.K + kpad) * a.lda * eb;
  const int64_t wb = lb == 0 ? rb * a.ldb * eb : (a.K + kpad) * a.ldb * eb;
  return wa < lim && wb < lim;
}

hipError_t launch_stream(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s) {
  const bool wide_a = a.N <= stream::NR && a.N <= a.M;
  return wide_a ? stream::launch_ops<true>(dtA, dtB, la, lb, a, s)
                : stream::launch_ops<false>(dtA, dtB, la, lb, a, s);
}

}  // namespace mcg
