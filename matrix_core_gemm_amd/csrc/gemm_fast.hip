// gemm_fast.hip -- the 256 x 256 instances of the pipelined dense kernel
// (gemm_fast_kernel.hpp) and the host side of both tile sizes: the precondition
// check and the launch.
#include "gemm_fast_kernel.hpp"

namespace mcg {

bool fast_path_ok(int dtA, int la, int lb, const DenseArgs& a, bool aligned, int tile) {
  const int64_t eb = (dtA == DT_BF16 || dtA == DT_F16) ? 2 : 1;
  if (tile != 256 && tile != 128) return false;
  if (!aligned || a.K == 0 || (a.K * eb) % 16 != 0) return false;
  if (a.M < tile || a.N < tile) return false;  // smaller problems: the general kernel fills the chip better
  // every buffer window (and offset into it) must stay below 2 GiB
  const int64_t lim = (int64_t)1 << 31;
  // MN-contiguous offsets advance by whole K tiles, up to NST tiles past the end of K
  const int64_t kpad = 4 * fast::KTB / eb;
  const int64_t wa = la == 0 ? tile * a.lda * eb : (a.K + kpad) * a.lda * eb;
  const int64_t wb = lb == 0 ? tile * a.ldb * eb : (a.K + kpad) * a.ldb * eb;
  return wa < lim && wb < lim;
}

hipError_t launch_fast(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s, int tile) {
  if (tile == 128) return launch_fast_mid(dtA, dtB, la, lb, a, s);
  return fast::launch_fast_tb<256>(dtA, dtB, la, lb, a, s);
}

}  // namespace mcg
