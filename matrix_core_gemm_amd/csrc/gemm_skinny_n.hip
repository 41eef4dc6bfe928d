// gemm_skinny_n.hip -- the general dense kernel instantiated with 128 x 32
// output tiles for skinny problems (N <= 32: 128 x 32 tiles), aligned operands only.
// A translation unit of its own so that the instantiations compile in parallel.
#include "dense_general.hpp"

namespace mcg {

hipError_t launch_skinny_n(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s) {
  return launch_general<128, 32, true>(dtA, dtB, la, lb, a, s);
}

}  // namespace mcg
