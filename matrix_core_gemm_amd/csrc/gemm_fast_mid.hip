// gemm_fast_mid.hip -- the 128 x 128 instances of the pipelined dense kernel
// (gemm_fast_kernel.hpp), in their own translation unit so that both tile sizes
// compile in parallel.
#include "gemm_fast_kernel.hpp"

namespace mcg {

hipError_t launch_fast_mid(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s) {
  return fast::launch_fast_tb<128>(dtA, dtB, la, lb, a, s);
}

}  // namespace mcg
