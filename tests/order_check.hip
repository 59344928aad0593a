// Host check of the workgroup orders in common.hpp: for every grid size up to
// 6000 and every grouping used, xcd_order and xcd_order_cu must map the
// workgroup ids 0..W-1 onto 0..W-1 one to one (a missed id would leave a tile
// of outputs unwritten).  Built with hipcc; runs on the host only.
#include <cstdio>
#include <vector>

#include "common.hpp"

int main() {
  for (int W = 1; W <= 6000; ++W) {
    for (int R = 0; R <= 4; ++R) {  // R = 0: xcd_order itself
      std::vector<int> seen(W, 0);
      for (int L = 0; L < W; ++L) {
        const int l = R ? ssd::xcd_order_cu(L, W, R) : ssd::xcd_order(L, W);
        if (l < 0 || l >= W || seen[l]++) {
          std::printf("W=%d R=%d: id %d maps to %d, not a permutation\n", W, R, L, l);
          return 1;
        }
      }
    }
  }
  std::printf("ok\n");
  return 0;
}
