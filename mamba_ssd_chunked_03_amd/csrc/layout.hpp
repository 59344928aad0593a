// Workspace layout of ssd_fwd / ssd_bwd: one region per intermediate, each 256-byte
// aligned, in a fixed order.  Plain C++ (no HIP), so that a host-only test can check
// it.  Every region's element type is named here once, and the kernels that write
// and read the region use the same name, so a change of one's storage type changes
// the region's size with it:
//   chunk states T and their adjoints U (the scan's inputs; also the chained
//   forward's carry)                                             ChunkStateT (fp32)
//   passed states H and their adjoints dE         bf16 where the bf16 kernels run, else fp32
//   delta, within-chunk cumsum, per-token backward pieces, tile partials   fp32
//   C.B^T                                                         io-sized (bf16 or fp32)
//   the head-summed dCB                           bf16 where the bf16 kernels run, else fp32
//   C.B^T transposed, R and K tile partials       only where the bf16 kernels run
#pragma once

#include <cstddef>
#include <cstdint>

namespace ssd {

using ChunkStateT = float;  // T_c and U_c: fp32 always (rounding them would compound along the chunks)
using TokenT = float;       // per-(chunk, head, token) values
using FlagT = int32_t;      // the chained forward's ticket counters, error word and flags
constexpr int kChainSyncWords = 16;  // counters [0, 8), wait error [8], unused up to 16

struct LayoutDims {
  int64_t nck;            // chunk slots
  int64_t H, P, N, G, Q;  // heads, headdim, dstate, groups, chunk size
  int64_t nseq;           // sequences (packed) or batch rows
  bool packed;
  bool bf16;              // io dtype bf16 (else fp32)
  bool wide;              // bf16 io run by the fp32 matrix-core kernels (headdim or dstate 16)
};

constexpr size_t kLayoutAlign = 256;
inline size_t lay_up(size_t x) { return (x + kLayoutAlign - 1) / kLayoutAlign * kLayoutAlign; }
inline size_t io_size(const LayoutDims& d) { return d.bf16 ? 2 : 4; }
// whether the bf16 MFMA kernels run (their intermediates are partly bf16)
inline bool bf16_kernels(const LayoutDims& d) { return d.bf16 && !d.wide; }
// passed states and their adjoints: every consumer on the bf16 kernels' path feeds
// them to bf16 matrix products, so they are stored in bf16 there (fp32 otherwise)
inline size_t passed_size(const LayoutDims& d) { return bf16_kernels(d) ? 2 : 4; }

struct FwdLayout {
  size_t tab, seq_off, delta, acs, decay, T, Hp, CB, sync, end;
};
inline FwdLayout fwd_layout(const LayoutDims& d) {
  FwdLayout l;
  size_t o = 0;
  const size_t nck = (size_t)d.nck, H = (size_t)d.H, st = (size_t)(d.P * d.N);
  l.tab = o;     o += d.packed ? lay_up(nck * 16) : 0;                   // int4 per slot
  l.seq_off = o; o += d.packed ? lay_up(((size_t)d.nseq + 1) * 4) : 0;   // int32 per sequence + 1
  l.delta = o;   o += lay_up(nck * H * d.Q * sizeof(TokenT));
  l.acs = o;     o += lay_up(nck * H * d.Q * sizeof(TokenT));
  l.decay = o;   o += lay_up(nck * H * sizeof(TokenT));
  l.T = o;       o += lay_up(nck * H * st * sizeof(ChunkStateT));
  l.Hp = o;      o += lay_up(nck * H * st * passed_size(d));
  l.CB = o;      o += lay_up(nck * (size_t)d.G * d.Q * d.Q * io_size(d));
  l.sync = o;    o += nck ? lay_up((kChainSyncWords + nck * H) * sizeof(FlagT)) : 0;
  l.end = o;
  return l;
}

struct BwdLayout {
  FwdLayout f;
  size_t CBt, dCBg, Rp, Kp, U, dE, ddd, Ks, rR, last, dDp, dAp, dbp, end;
};
inline BwdLayout bwd_layout(const LayoutDims& d) {
  BwdLayout l;
  l.f = fwd_layout(d);
  size_t o = l.f.end;
  const size_t nck = (size_t)d.nck, H = (size_t)d.H, st = (size_t)(d.P * d.N);
  const bool bk = bf16_kernels(d);
  const size_t cb = bk ? nck * (size_t)d.G * d.Q * d.Q * 2 : 0;
  const size_t tiles = bk ? nck * H * (size_t)(d.Q / 64) * d.Q * sizeof(TokenT) : 0;
  l.CBt = o;  o += lay_up(cb);
  l.dCBg = o; o += lay_up(nck * (size_t)d.G * d.Q * d.Q * (bk ? 2 : 4));
  l.Rp = o;   o += lay_up(tiles);
  l.Kp = o;   o += lay_up(tiles);
  l.U = o;    o += lay_up(nck * H * st * sizeof(ChunkStateT));
  l.dE = o;   o += lay_up(nck * H * st * passed_size(d));
  l.ddd = o;  o += lay_up(nck * H * d.Q * sizeof(TokenT));
  l.Ks = o;   o += lay_up(nck * H * d.Q * sizeof(TokenT));
  l.rR = o;   o += lay_up(nck * H * d.Q * sizeof(TokenT));
  l.last = o; o += lay_up(nck * H * sizeof(TokenT));
  l.dDp = o;  o += lay_up(nck * H * sizeof(TokenT));
  l.dAp = o;  o += lay_up(nck * H * sizeof(TokenT));
  l.dbp = o;  o += lay_up(nck * H * sizeof(TokenT));
  l.end = o;
  return l;
}

}  // namespace ssd
