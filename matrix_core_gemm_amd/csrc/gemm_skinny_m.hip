// gemm_skinny_m.hip -- the general dense kernel instantiated with 32 x 128
// output tiles for skinny problems (M <= 32: 32 x 128 tiles), aligned operands only.
// A translation unit of its own so that the instantiations compile in parallel.
#include "dense_general.hpp"

namespace mcg {

hipError_t launch_skinny_m(int dtA, int dtB, int la, int lb, const DenseArgs& a, hipStream_t s) {
  return launch_general<32, 128, true>(dtA, dtB, la, lb, a, s);
}

}  // namespace mcg
