// The output stage's per-row-block work, shared by the chunk-scan kernel and the
// fused chained forward (both hold a chunk's x tile, its passed state H_c in bf16,
// and the chunk's acs and delta in LDS).  Per 16-row block of the output:
//   1. acc = 2^(acs_e) C_rows . H_c^T on MFMA (K = dstate);
//   2. acc += (CB_ij * column factor) . X over the 32-token blocks before the
//      diagonal block (the A fragment formed in registers from the CB fragments);
//   3. acc *= 2^(acs_i - acs_e) per row, which also turns 1.'s factor into 2^acs_i;
//   4. acc += M . X over the diagonal block, M_ij = CB_ij 2^(acs_i - acs_j) delta_j
//      masked to j <= i;
//   5. + D x_i and the bf16 store.
// The decay 2^(acs_i - acs_j) is factored through the anchor token e = b0 - 1 of
// the row block's first 32-token block b0 (column factors 2^(acs_e - acs_j)
// delta_j tabulated in LDS, row factor on the accumulator), so both factors are
// <= 1 and only the diagonal block has one exp per element.  Products are issued
// with the operands swapped, so each lane owns one output row; the x tile's
// column groups are permuted (common.hpp, pcol), so a lane's outputs are 8
// adjacent columns per tile pair, stored as whole 128-byte row spans.
#pragma once

#include "common.hpp"

namespace ssd {

constexpr int kScanWaves = 8;
constexpr int kScanQmax = 256;

template <int P, int N>
struct ScanRows {
  static constexpr int QMAX = kScanQmax, LDX = P + 8, HLD = N + 8, NW = kScanWaves;
  // LDS operands
  const uint16_t* xs;   // x tile, [token][permuted column], row stride LDX
  const uint16_t* hs;   // H_c in bf16, [p][n], row stride HLD
  const float* sa;      // acs (log2 units) per token
  const float* sd;      // delta per token
  const float* vt;      // column factors, [QMAX / 32][QMAX]
  // global rows of this chunk (range-checked: rows past the chunk's end read zero
  // and are never written)
  brsrc rcm, rcb, ry;
  int Q, len, w, q, r, NB, nii;
  int64_t xrow;  // bytes between tokens of x and y are 2 * xrow
  float Dh;
  u32x4 cf[N / 32], cbf[QMAX / 32], cbd;

  // cb: the chunk's C rows of its group; cbm: its C.B^T (Q x Q, fragment order:
  // common.hpp, cbf_off); yb: its y rows
  __device__ __forceinline__ void init(const uint16_t* cb, int64_t crow, const uint16_t* cbm,
                                       uint16_t* yb, int64_t xrow_, int Q_, int len_, int tid,
                                       float Dh_) {
    Q = Q_;
    len = len_;
    w = tid >> 6;
    const int lane = tid & 63;
    q = lane >> 4;
    r = lane & 15;
    xrow = xrow_;
    Dh = Dh_;
    NB = Q / 16;
    nii = (NB + NW - 1) / NW;
    rcm = make_rsrc(cb, (uint32_t)(len * crow * 2));
    rcb = make_rsrc(cbm, (uint32_t)(((len + 15) & ~15) * Q * 2));  // whole 16-row blocks
    ry = make_rsrc(yb, (uint32_t)(len * xrow * 2));
    crow_ = crow;
  }
  int64_t crow_;

  // row blocks of this wave, in snake order (w and NW-1-w) so the causal work is balanced
  __device__ __forceinline__ int rb_of(int ii) const {
    return NW * ii + ((ii & 1) ? (NW - 1 - w) : w);
  }
  __device__ __forceinline__ bool live(int ii) const {
    return ii < nii && rb_of(ii) < NB && rb_of(ii) * 16 < len;
  }
  // all C and C.B^T fragments of a row block, in flight together (one memory latency)
  __device__ __forceinline__ void load_rb(int rb) {
    const uint32_t irow = rb * 16 + r, nb = rb / 2;
    const uint32_t co = irow * (uint32_t)(crow_ * 2) + q * 16;
    const uint32_t bo = cbf_piece(rb, 0, q * 16 + r, Q);  // block (rb, sx) at bo + 1024 sx
#pragma unroll
    for (int kb = 0; kb < N / 32; ++kb) cf[kb] = buf_load16(rcm, co + 64 * kb);
#pragma unroll
    for (int sx = 0; sx < QMAX / 32; ++sx)
      cbf[sx] = (sx < (int)nb) ? buf_load16(rcb, bo + 1024 * sx) : u32x4{0u, 0u, 0u, 0u};
    cbd = buf_load16(rcb, bo + 1024 * nb);
  }
  __device__ __forceinline__ void prefetch_first() {
    if (live(0)) load_rb(rb_of(0));
  }

  // column factors for anchor e = 32b - 1: 2^(acs_e - acs_j) delta_j for j <= e
  // (every thread of the workgroup; needs sa, sd in LDS; a barrier must follow)
  static __device__ __forceinline__ void column_factors(float* vt_, const float* sa_, const float* sd_,
                                                        int Q_, int tid) {
    for (int idx = tid; idx < (Q_ / 32) * Q_; idx += NW * 64) {
      const int b = idx / Q_, j = idx % Q_;
      vt_[b * QMAX + j] = (b > 0 && j < 32 * b) ? exp2_fast(sa_[32 * b - 1] - sa_[j]) * sd_[j] : 0.f;
    }
  }

  // every row block of this wave (the first one's fragments already in flight)
  __device__ __forceinline__ void run() {
    for (int ii = 0; ii < nii; ++ii) {
      if (!live(ii)) continue;  // chunk sizes with fewer row blocks than wavefronts, short chunks
      const int rb = rb_of(ii);
      const int i0 = rb * 16;
      const int irow = i0 + r;  // the output row of this lane
      const bool rowok = irow < len;
      const int nb = i0 / 32;   // 32-token blocks strictly before the diagonal block
      const float ae = nb > 0 ? sa[32 * nb - 1] : 0.f;
      // acc[tp][rr] = y[i0 + r][pcol(tp, 4 q + rr)]; acc[2s], acc[2s + 1] are the
      // lane's 8 adjacent outputs 32 s + 8 q .. +7
      f32x4 acc[P / 16];
#pragma unroll
      for (int tp = 0; tp < P / 16; ++tp) acc[tp] = f32x4{0.f, 0.f, 0.f, 0.f};
      // 1. state carried in, pre-scaled by 2^acs_e
#pragma unroll
      for (int kb = 0; kb < N / 32; ++kb)
#pragma unroll
        for (int tp = 0; tp < P / 16; ++tp)
          acc[tp] = mfma_bf16(as_bf16x8(*(const u32x4*)(hs + pcol(tp, r) * HLD + kb * 32 + q * 8)),
                              as_bf16x8(cf[kb]), acc[tp]);
      {
        const float s0 = exp2_fast(ae);
#pragma unroll
        for (int tp = 0; tp < P / 16; ++tp) acc[tp] *= s0;
      }
      // 2. blocks before the diagonal block, through the anchor's column factors
      const float* vrow = vt + nb * QMAX;
#pragma unroll
      for (int sx = 0; sx < QMAX / 32; ++sx) {
        if (sx < nb) {
          const float4 f0 = *(const float4*)(vrow + sx * 32 + q * 8);
          const float4 f1 = *(const float4*)(vrow + sx * 32 + q * 8 + 4);
          u32x4 av;
          av[0] = pack_bf2(bf_lo(cbf[sx][0]) * f0.x, bf_hi(cbf[sx][0]) * f0.y);
          av[1] = pack_bf2(bf_lo(cbf[sx][1]) * f0.z, bf_hi(cbf[sx][1]) * f0.w);
          av[2] = pack_bf2(bf_lo(cbf[sx][2]) * f1.x, bf_hi(cbf[sx][2]) * f1.y);
          av[3] = pack_bf2(bf_lo(cbf[sx][3]) * f1.z, bf_hi(cbf[sx][3]) * f1.w);
          const bf16x8 a = as_bf16x8(av);
          const int lane = q * 16 + r;
#pragma unroll
          for (int tp = 0; tp < P / 16; ++tp)
            acc[tp] = mfma_bf16(frag_kmajor(xs + sx * 32 * LDX + tp * 16, LDX, lane), a, acc[tp]);
        }
      }
      // 3. this lane's row factor 2^(acs_i - acs_e), which also turns 1.'s factor into 2^acs_i
      {
        const float u = rowok ? exp2_fast(sa[irow] - ae) : 0.f;
#pragma unroll
        for (int tp = 0; tp < P / 16; ++tp) acc[tp] *= u;
      }
      // 4. the diagonal block, one exp per element
      {
        const float ai = sa[min(irow, Q - 1)];
        u32x4 av;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int j0 = nb * 32 + q * 8 + 2 * d;
          float v0 = bf_lo(cbd[d]) * exp2_fast(ai - sa[j0]) * sd[j0];
          float v1 = bf_hi(cbd[d]) * exp2_fast(ai - sa[j0 + 1]) * sd[j0 + 1];
          v0 = (j0 <= irow) ? v0 : 0.f;
          v1 = (j0 + 1 <= irow) ? v1 : 0.f;
          av[d] = pack_bf2(v0, v1);
        }
        const bf16x8 a = as_bf16x8(av);
        const int lane = q * 16 + r;
#pragma unroll
        for (int tp = 0; tp < P / 16; ++tp)
          acc[tp] = mfma_bf16(frag_kmajor(xs + nb * 32 * LDX + tp * 16, LDX, lane), a, acc[tp]);
      }
      if (live(ii + 1)) load_rb(rb_of(ii + 1));  // the fragments above are dead now
      // 5. skip term; the lane's 8 adjacent outputs per tile pair are stored as whole
      //    128-byte row spans (span_swap) where a row has two pieces per lane
      {
        const uint32_t yo = (uint32_t)irow * (uint32_t)(xrow * 2) + q * 16;
        u32x4 ys_[P / 32];
#pragma unroll
        for (int s = 0; s < P / 32; ++s) {
          const u32x4 xv = lds_cols8_perm(xs + irow * LDX, s, q);
          f32x4 y0 = acc[2 * s], y1 = acc[2 * s + 1];
          y0[0] += Dh * bf_lo(xv[0]);
          y0[1] += Dh * bf_hi(xv[0]);
          y0[2] += Dh * bf_lo(xv[1]);
          y0[3] += Dh * bf_hi(xv[1]);
          y1[0] += Dh * bf_lo(xv[2]);
          y1[1] += Dh * bf_hi(xv[2]);
          y1[2] += Dh * bf_lo(xv[3]);
          y1[3] += Dh * bf_hi(xv[3]);
          ys_[s] = pack_bf8(y0, y1);
        }
        if constexpr (P >= 64) {
          const uint32_t ra = (uint32_t)(rb_of(ii) * 16 + (r & 7)), so = span_off(r, q);
#pragma unroll
          for (int m2 = 0; m2 < P / 64; ++m2) {
            u32x4 a, b;
            span_swap(r, ys_[2 * m2], ys_[2 * m2 + 1], a, b);
            buf_store16(ry, ra * (uint32_t)(xrow * 2) + so + 128 * m2, a);
            buf_store16(ry, (ra + 8) * (uint32_t)(xrow * 2) + so + 128 * m2, b);
          }
        } else {
          buf_store16(ry, yo, ys_[0]);
        }
      }
    }
  }
};

}  // namespace ssd
