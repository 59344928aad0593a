// Host-only check of the workspace layout (csrc/layout.hpp), built and run by
// tests/test_layout.py with the host compiler: for a spread of problem shapes,
// every region is 256-byte aligned, regions follow each other without overlap,
// each is exactly the size that its element type and its (chunk, head, ...)
// extent give, and the saved-context regions that ssd_bwd reads sit where
// ssd_fwd writes them.  Prints "ok" or the first failure and exits non-zero.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "layout.hpp"

using namespace ssd;

static int fails = 0;
#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      std::printf("FAIL %s:%d: ", __FILE__, __LINE__);  \
      std::printf(__VA_ARGS__);                         \
      std::printf("\n");                                \
      if (++fails > 10) std::exit(1);                   \
    }                                                   \
  } while (0)

struct Reg {
  const char* name;
  size_t off, bytes;
};

static void check_regions(const std::vector<Reg>& r, size_t end, const LayoutDims& d) {
  size_t o = 0;
  for (const Reg& g : r) {
    CHECK(g.off % 256 == 0, "%s at %zu not aligned (nck %lld)", g.name, g.off, (long long)d.nck);
    CHECK(g.off == o, "%s at %zu, expected %zu (nck %lld)", g.name, g.off, o, (long long)d.nck);
    o = g.off + lay_up(g.bytes);
  }
  CHECK(end == o, "end %zu, expected %zu", end, o);
}

int main() {
  const int Ps[] = {16, 32, 64, 128}, Ns[] = {16, 32, 64, 128}, Qs[] = {64, 128, 256};
  for (int packed = 0; packed < 2; ++packed)
    for (int bf = 0; bf < 2; ++bf)
      for (int P : Ps)
        for (int N : Ns)
          for (int Q : Qs)
            for (long long nck : {0LL, 1LL, 3LL, 64LL, 517LL}) {
              // bf16 io below 32-wide headdim or dstate runs the fp32 matrix-core kernels
              const bool wide = bf && (P < 32 || N < 32);
              LayoutDims d{nck, 64, P, N, 8, Q, packed ? 5 : 2, packed != 0, bf != 0, wide};
              const size_t st = (size_t)nck * 64 * P * N, tok = (size_t)nck * 64 * Q, ch = (size_t)nck * 64;
              const size_t io = bf ? 2 : 4;               // io tensors: C.B^T
              const bool bk = bf && !wide;                 // the bf16 kernels run
              const size_t pas = bk ? 2 : 4;               // passed states and their adjoints
              const FwdLayout f = fwd_layout(d);
              std::vector<Reg> fr = {
                  {"chunk table", f.tab, packed ? (size_t)nck * 16 : 0},
                  {"sequence offsets", f.seq_off, packed ? (size_t)(d.nseq + 1) * 4 : 0},
                  {"delta", f.delta, tok * sizeof(float)},
                  {"acs", f.acs, tok * sizeof(float)},
                  {"decay", f.decay, ch * sizeof(float)},
                  // written by the chunk-state kernel, read by the scan: fp32 on both sides
                  {"chunk states T", f.T, st * sizeof(ChunkStateT)},
                  {"passed states H", f.Hp, st * pas},
                  {"C.B^T", f.CB, (size_t)nck * 8 * Q * Q * io},
                  {"chained flags", f.sync, nck ? (size_t)(kChainSyncWords + nck * 64) * 4 : 0},
              };
              check_regions(fr, f.end, d);
              const BwdLayout b = bwd_layout(d);
              CHECK(b.f.end == f.end && b.f.T == f.T && b.f.Hp == f.Hp && b.f.CB == f.CB && b.f.delta == f.delta,
                    "the backward's saved-context offsets differ from the forward's");
              const size_t cb = bk ? (size_t)nck * 8 * Q * Q * 2 : 0;
              const size_t tiles = bk ? (size_t)nck * 64 * (Q / 64) * Q * 4 : 0;
              std::vector<Reg> br = fr;
              br.insert(br.end(), {
                  {"C.B^T transposed", b.CBt, cb},
                  {"head-summed dCB", b.dCBg, (size_t)nck * 8 * Q * Q * (bk ? 2 : 4)},
                  {"R partials", b.Rp, tiles},
                  {"K partials", b.Kp, tiles},
                  // written by the adjoint-state kernel, read by the reverse scan: fp32 on both sides
                  {"adjoint chunk states U", b.U, st * sizeof(ChunkStateT)},
                  {"adjoint passed states dE", b.dE, st * pas},
                  {"direct ddelta", b.ddd, tok * 4},
                  {"K + s", b.Ks, tok * 4},
                  {"r + R", b.rR, tok * 4},
                  {"last term", b.last, ch * 4},
                  {"dD partials", b.dDp, ch * 4},
                  {"dA partials", b.dAp, ch * 4},
                  {"d_dt_bias partials", b.dbp, ch * 4},
              });
              check_regions(br, b.end, d);
              CHECK(sizeof(ChunkStateT) == 4, "chunk states are fp32");
            }
  if (fails) return 1;
  std::printf("ok\n");
  return 0;
}
