// gemm_fast_sk.hip -- stream-K form of the pipelined kernel (gemm_fast_kernel.hpp):
// the 256 x 256 instances and the plan of both tile sizes (the 128 x 128
// instances are in gemm_fast_mid_sk.hip).
//
// A problem whose number of 256 x 256 tiles is not a multiple of the number of
// compute units leaves most CUs idle in its last round of tiles (7168^3: 784
// tiles = 3 rounds of 256 and a round of 16).  The stream-K form runs the whole
// rounds as one launch of the whole-tile kernel, then spreads the K iterations
// of the remaining tiles evenly over all CUs in a second launch: workgroup w
// takes the consecutive K tiles [w L, (w + 1) L) of the remainder, numbered tile
// by tile (the kernel handles ranges that cross a tile boundary; the plan picks
// L so that each range is one piece of one tile).  (Running both parts in one launch
// measured slower: the loop over pieces costs the whole-tile rounds registers
// and about 6-8% of their speed.)  A
// piece that is not a whole tile writes its raw sums to a workspace slot; a
// second, elementwise kernel then adds each tile's pieces in piece order (K
// ascending, so the result does not depend on timing) and applies the epilogue.
// No workgroup waits for another and nothing is added atomically.
#include <algorithm>
#include <mutex>
#include <numeric>

#include "gemm_fast_kernel.hpp"

namespace mcg {

namespace {
// Cost model (one workgroup per CU): a K tile of a whole round takes at least
// KT_US (the 256 x 256 form: int8 / fp8; bf16 takes about 1.6 us at 8192^3; the
// 128 x 128 form about half), each piece writes and the fixup reads one slot of
// tile^2 binary32 values (PIECE_US for 256 KiB), and the fixup launch with its
// fixed latency costs SK_FIXED_US.  Stream-K is taken when the K tiles it saves in
// the last round outweigh its own cost.
constexpr double SK_KT_US_256 = 0.75, SK_KT_US_128 = 0.4, SK_PIECE_US_256 = 0.1, SK_FIXED_US = 8.0;
// the 256 x 256 sparse kernel: a kept-value stage of a whole round takes at least
// SK_STAGE_US_SPARSE (bf16 about 2.4 us at 8192^3, 8-bit about 2.9)
constexpr double SK_STAGE_US_SPARSE = 1.5;
constexpr int64_t SK_MIN_ITERS = 4;  // K tiles per workgroup range at least
}  // namespace

// The plan for T tiles of tile x tile outputs with nk K units each (K tiles of
// 128 bytes, or kept-value stages), kt_us per K unit of a whole round: fills the
// sk_* and dp_tiles fields and returns the workspace bytes, or 0.
template <class Args>
static int64_t plan_core(Args& a, int64_t T, int64_t nk, int num_cu, int tile, double kt_us, int64_t min_iters) {
  a.dp_tiles = a.sk_tiles = a.sk_wgs = 0;
  a.sk_iters = 0;
  a.sk_period = 1;
  const int64_t G = num_cu > 0 ? num_cu : 256;
  const int64_t R = T % G;
  if (R == 0 || nk < 2 * min_iters) return 0;
  // Each remainder tile is cut into s equal pieces, s the largest divisor of nk
  // with R s <= G and at least min_iters K units per piece, so that every
  // workgroup takes exactly one piece and the workgroups of one XCD (taken
  // round-robin) walk the same K range of neighbouring tiles and share their
  // panels in L2.  (Ranges that cross tile boundaries balance the CUs better but
  // give every workgroup its own K offset: measured slower than whole tiles.)
  int64_t sp = 0;
  for (int64_t c = std::min(G / R, nk / min_iters); c >= 2; --c)
    if (nk % c == 0) {
      sp = c;
      break;
    }
  if (sp < 2) return 0;
  const int64_t L = nk / sp;
  const int64_t wgs = R * sp;
  const int64_t pieces = wgs;
  const int64_t slot = (int64_t)tile * tile * 4;
  const double saved = (double)(nk - L) * kt_us;
  const double cost = (double)pieces * SK_PIECE_US_256 * (double)slot / (256.0 * 256 * 4) + SK_FIXED_US;
  if (saved <= cost || T - R + wgs > 0x7fffffff) return 0;
  a.dp_tiles = (int)(T - R);
  a.sk_tiles = (int)R;
  a.sk_wgs = (int)wgs;
  a.sk_iters = L;
  a.sk_period = nk / std::gcd(L, nk);
  return pieces * slot;
}

int64_t plan_streamk(int dtA, DenseArgs& a, int num_cu, int tile) {
  if (tile != 256 && tile != 128) {
    a.dp_tiles = a.sk_tiles = a.sk_wgs = 0;
    return 0;
  }
  const int64_t eb = (dtA == DT_BF16 || dtA == DT_F16) ? 2 : 1;
  const int64_t nk = (a.K * eb + fast::KTB - 1) / fast::KTB;
  const int64_t T = ((a.M + tile - 1) / tile) * ((a.N + tile - 1) / tile);
  return plan_core(a, T, nk, num_cu, tile, tile == 256 ? SK_KT_US_256 : SK_KT_US_128, SK_MIN_ITERS);
}

int64_t plan_sparse_streamk(int dtA, SparseArgs& a, int num_cu) {
  const int64_t eb = (dtA == DT_BF16 || dtA == DT_F16) ? 2 : 1;
  const int64_t nT = (a.K * eb + 255) / 256;  // kept-value stages of 128 bytes of kept values per row
  const int64_t T = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  return plan_core(a, T, nT, num_cu, 256, SK_STAGE_US_SPARSE, 2);
}

hipError_t launch_streamk_fixup(const DenseArgs& a, int64_t nk, bool int_acc, hipStream_t s) {
  if (int_acc)
    hipLaunchKernelGGL((fast::streamk_fixup_kernel<true, 256>), dim3((unsigned)a.sk_tiles, 64), dim3(256), 0, s, a, nk);
  else
    hipLaunchKernelGGL((fast::streamk_fixup_kernel<false, 256>), dim3((unsigned)a.sk_tiles, 64), dim3(256), 0, s, a, nk);
  return hipGetLastError();
}

hipError_t launch_fast_sk(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s, int tile) {
  if (a.sk_tiles <= 0 || a.ws == nullptr) return hipErrorInvalidValue;
  if (tile == 128) return launch_fast_mid_sk(dtA, dtB, la, lb, a, s);
  return fast::launch_fast_tb<256, true>(dtA, dtB, la, lb, a, s);
}

// ------------------------------------------------------------ static scratch
// Stream-K slots for callers that cannot allocate (gemm_dense_noalloc): a
// file-scope device array of STATIC_SCRATCH_BYTES, one copy per GPU, held until
// the process ends.  Host code never passes the array's name to a kernel: its
// device address is looked up once per device with that device current and
// kept, and only that address is used.  Every call on a GPU shares that GPU's
// copy; calls that overlap on one GPU race.  Nothing in it needs to start at
// zero (each slot is written whole before it is read).
static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mcg
