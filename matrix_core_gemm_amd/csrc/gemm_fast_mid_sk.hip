// gemm_fast_mid_sk.hip -- the stream-K instances of the 128 x 128 form of the
// pipelined kernel (gemm_fast_kernel.hpp), in their own translation unit so that
// they compile in parallel with the 256 x 256 ones.
#include "gemm_fast_kernel.hpp"

namespace mcg {

hipError_t launch_fast_mid_sk(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s) {
  return fast::launch_fast_tb<128, true>(dtA, dtB, la, lb, a, s);
}

}  // namespace mcg
