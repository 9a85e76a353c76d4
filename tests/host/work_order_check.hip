// Host-side check of the forward's balanced work order (balanced_unit_rank in
// evo_kernels.h): over many grid shapes, every work unit gets exactly one rank,
// every workgroup of a unit the same rank, and the two unit slots that share a
// CU (local slots j and j + per / 2 of one XCD's range) ranks that sum to the
// last rank.  Exit status 0 when all hold.
#include <cstdio>
#include <vector>

#include "evo_kernels.h"

int main() {
  long shapes = 0;
  for (int unit = 1; unit <= 64; ++unit) {
    for (int upx = 2; upx <= 64; upx += 2) {
      const int per = upx * unit, grid = 8 * per, total = grid / unit;
      std::vector<int> seen(total, 0);
      for (int lg = 0; lg < grid; ++lg) {
        const int r = evo::balanced_unit_rank(lg, per, unit, total);
        if (r < 0 || r >= total) {
          std::printf("rank out of range: unit %d, units per XCD %d, workgroup %d, rank %d\n", unit, upx, lg, r);
          return 1;
        }
        if (r != evo::balanced_unit_rank(lg - lg % unit, per, unit, total)) {
          std::printf("a unit's workgroups differ in rank: unit %d, units per XCD %d\n", unit, upx);
          return 1;
        }
        if (lg % unit == 0) seen[r]++;
      }
      for (int r = 0; r < total; ++r)
        if (seen[r] != 1) {
          std::printf("rank %d taken %d times: unit %d, units per XCD %d\n", r, seen[r], unit, upx);
          return 1;
        }
      for (int x = 0; x < 8; ++x)
        for (int j = 0; j < per / 2; j += unit) {
          const int a = evo::balanced_unit_rank(x * per + j, per, unit, total);
          const int b = evo::balanced_unit_rank(x * per + j + per / 2, per, unit, total);
          if (a + b != total - 1) {
            std::printf("CU pair not complementary: unit %d, units per XCD %d, XCD %d, slot %d\n", unit, upx, x, j);
            return 1;
          }
        }
      ++shapes;
    }
  }
  std::printf("ok: %ld grid shapes\n", shapes);
  return 0;
}
