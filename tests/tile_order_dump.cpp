// Host-side dump of the tile-order functions (csrc/tile_order.hpp) for the CPU
// tests: the grouped tile order of a few grids, and the first-piece index of
// every stream-K workgroup for a few range lengths.  Nothing touches a device.
#include <cstdio>

#include "tile_order.hpp"

using namespace mcg::fast;

int main() {
  const int grids[][2] = {{1, 1}, {3, 5}, {4, 4}, {7, 3}, {28, 28}, {16, 19}, {9, 1}, {1, 9}};
  for (const auto& g : grids)
    for (int pid = 0; pid < g[0] * g[1]; ++pid) {
      int tm, tn;
      grouped_tile<4>(pid, g[0], g[1], tm, tn);
      std::printf("tile %d %d %d %d %d\n", g[0], g[1], pid, tm, tn);
    }
  // (tiles, nk, L): every workgroup's first piece, P = nk / gcd(L, nk)
  const long long cases[][3] = {{16, 112, 7}, {64, 96, 24}, {48, 64, 12}, {144, 80, 45}, {3, 10, 4},
                                {5, 7, 3}, {1, 9, 4}, {40, 33, 5}, {7, 64, 64}, {100, 17, 6}};
  for (const auto& c : cases) {
    long long a = c[1], b = c[2];
    while (b) { const long long t = a % b; a = b; b = t; }
    const long long P = c[1] / a;
    const long long wgs = (c[0] * c[1] + c[2] - 1) / c[2];
    for (long long w = 0; w <= wgs - 1; ++w)
      std::printf("piece %lld %lld %lld %lld %lld\n", c[0], c[1], c[2], w, (long long)sk_first_piece(w, c[2], c[1], P));
  }
  return 0;
}
