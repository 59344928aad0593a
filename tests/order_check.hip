// Host check of two index maps in common.hpp.  For every grid size up to 6000
// and every grouping used, xcd_order and xcd_order_cu must map the workgroup ids
// 0..W-1 onto 0..W-1 one to one (a missed id would leave a tile of outputs
// unwritten).  For every chunk size, the fragment order of C.B^T (cbf_off) must
// be a permutation of the Q x Q elements, and the 16-byte piece that lane
// (q, r) loads of block (R, S) (cbf_piece) must hold exactly the elements
// (16R + r, 32S + 8q + e), e = 0..7, in order: the producers store by cbf_piece,
// the element readers address by cbf_off.  Built with hipcc; runs on the host.
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
  for (int Q : {64, 128, 256}) {
    std::vector<int> seen(Q * Q, 0);
    for (int i = 0; i < Q; ++i)
      for (int j = 0; j < Q; ++j) {
        const uint32_t o = ssd::cbf_off(i, j, Q);
        if (o >= (uint32_t)(Q * Q) || seen[o]++) {
          std::printf("Q=%d: element (%d, %d) at %u, not a permutation\n", Q, i, j, o);
          return 1;
        }
      }
    for (int R = 0; R < Q / 16; ++R)
      for (int S = 0; S < Q / 32; ++S)
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 8; ++e) {
            const int q = lane >> 4, r = lane & 15;
            const uint32_t piece = ssd::cbf_piece(R, S, lane, Q);
            if (piece % 16 || piece / 2 + e != ssd::cbf_off(16 * R + r, 32 * S + 8 * q + e, Q)) {
              std::printf("Q=%d: block (%d, %d) lane %d element %d disagrees\n", Q, R, S, lane, e);
              return 1;
            }
          }
  }
  std::printf("ok\n");
  return 0;
}
