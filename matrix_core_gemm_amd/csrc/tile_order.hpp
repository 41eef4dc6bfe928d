// tile_order.hpp -- the order in which the pipelined kernels take output tiles,
// the numbering of stream-K pieces, and where a piece's epilogue writes.  Plain
// integer functions for host and device: the kernels, their launchers and the
// host-side tests use the same code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcg {
namespace fast {

// Logical tile index pid -> (tm, tn): tiles are ordered in groups of GROUP tile
// rows, column-major inside a group, so that consecutive logical tiles share A
// and B panels.
template <int GROUP>
__host__ __device__ inline void grouped_tile(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int tiles_in_group = GROUP * tiles_n;
  const int gid = pid / tiles_in_group;
  const int first_m = gid * GROUP;
  const int gsize = tiles_m - first_m < GROUP ? tiles_m - first_m : GROUP;
  tm = first_m + (pid % tiles_in_group) % gsize;
  tn = (pid % tiles_in_group) / gsize;
}

// Index of stream-K workgroup w's first piece in the sequence of all pieces
// (workgroup by workgroup, tile by tile): the workgroups before w cover w ranges
// of L K tiles, and every tile boundary strictly inside one of them adds a piece;
// a range boundary falls on a tile boundary every P ranges.
__host__ __device__ inline int64_t sk_first_piece(int64_t w, int64_t L, int64_t nk, int64_t P) {
  return w == 0 ? 0 : w + (w * L - 1) / nk - (w - 1) / P;
}

// Where an epilogue writes: D = alpha * acc + beta * C for the tile whose first
// element is (m0, n0) of an M x N matrix with leading dimension ld (elements).
struct EpiDst {
  void* D;
  const void* C;
  int64_t ld, M, N, m0, n0;
  float alpha, beta;
  int alpha_i, beta_i, use_c, vec, out;
};

}  // namespace fast
}  // namespace mcg
