// Host-side dump of the fragment-layout module (csrc/frag_layout.hpp) for the
// CPU tests: every (lane, register) -> (i, j, block) and (i, j, block) ->
// (lane, register) of each accumulator shape, and the operand maps.  Only the
// module's constexpr functions run here; nothing touches a device.
#include <cstdio>

#include "frag_layout.hpp"

using namespace mcg::frag;

template <int SHAPE>
static void dump_acc(const char* name) {
  using A = Acc<SHAPE>;
  const int regs = A::REGS;
  for (int l = 0; l < 64; ++l)
    for (int r = 0; r < regs; ++r) {
      const Coord c = A::coord(l, r);
      std::printf("coord %s %d %d %d %d %d\n", name, l, r, c.i, c.j, c.b);
    }
  for (int b = 0; b < A::MAX_BLOCKS; ++b)
    for (int i = 0; i < A::R; ++i)
      for (int j = 0; j < A::C; ++j) {
        const Slot s = A::slot(i, j, b);
        std::printf("slot %s %d %d %d %d %d\n", name, i, j, b, s.lane, s.reg);
      }
}

template <int S, int E>
static void dump_dense(const char* name) {
  using D = DenseOperand<S, E>;
  for (int l = 0; l < 64; ++l)
    for (int e = 0; e < E; ++e) {
      const Slot s = D::slot(D::row(l), D::k(l, e));
      std::printf("dense %s %d %d %d %d %d %d\n", name, l, e, D::row(l), D::k(l, e), s.lane, s.reg);
    }
}

template <int S, int EB>
static void dump_sparse(const char* name) {
  using P = SparseOperands<S, EB>;
  std::printf("sparse_geom %s %d %d %d %d %d\n", name, P::K, P::KEPT, P::EBD, P::CODES, P::GROUPS);
  for (int l = 0; l < 64; ++l) {
    for (int e = 0; e < P::KEPT; ++e) std::printf("sparse_a %s %d %d %d %d\n", name, l, e, P::row(l), P::group(l, e));
    for (int e = 0; e < P::EBD; ++e) std::printf("sparse_b %s %d %d %d %d\n", name, l, e, P::col(l), P::dense_k(l, e));
  }
}

int main() {
  dump_acc<ACC_32x32>("32x32");
  dump_acc<ACC_16x16>("16x16");
  dump_acc<ACC_4x4>("4x4");
  dump_acc<ACC_16x16_F64>("16x16_f64");
  dump_acc<ACC_4x4_F64>("4x4_f64");
  dump_dense<32, 8>("32x32x16_bf16");
  dump_dense<16, 8>("16x16x32_bf16");
  dump_dense<32, 16>("32x32x32_i8");
  dump_dense<16, 16>("16x16x64_i8");
  dump_dense<32, 32>("32x32x64_f8");
  dump_dense<16, 32>("16x16x128_f8");
  dump_sparse<32, 2>("32x32x32_16bit");
  dump_sparse<32, 1>("32x32x64_8bit");
  dump_sparse<16, 2>("16x16x64_16bit");
  dump_sparse<16, 1>("16x16x128_8bit");
  return 0;
}
