// Backward of the chunked scan (the adjoint of the forward stages).
//
// Per chunk c, head h (group g), tokens i, j of the chunk, with
//   L_ij = 2^(acs_i - acs_j) (i >= j), w_j = 2^(acs_last - acs_j),
//   CB_ij = C_i . B_j, dT = dE_c (from the reverse state-passing scan), H = H_c
//   (both stored in bf16 on the bf16 path, fp32 on the fp32 path):
//   dx_j  = delta_j [ sum_{i>=j} CB_ij L_ij dy_i + w_j dT B_j ] + D dy_j
//   dC_i  = sum_h [ 2^acs_i H^T dy_i + sum_{j<=i} dCB_ij B_j ]
//   dB_j  = sum_h [ sum_{i>=j} dCB_ij C_i + w_j delta_j dT^T x_j ]
//   with dCB_ij = (dy_i . x_j) L_ij delta_j.
// Decay gradients: the gradient w.r.t. the within-chunk cumsum at token i is
//   dAcs_i = r_i + R_i - K_i - s_i  (+ at the last token: sum_j s_j + alpha <dE, H>)
// where r_i = 2^acs_i dy_i . (H C_i), R_i = sum_{j<i} M_ij, K_j = sum_{i>j} M_ij,
// s_j = w_j delta_j x_j . (dT B_j), M_ij = (dy_i . x_j) CB_ij L_ij delta_j, and the
// gradient w.r.t. each token's delta*A is the suffix sum ddA_t = sum_{i>=t} dAcs_i.
// The identity sum_{i>=j} (dy_i . x_j) CB_ij L_ij = x_j . U_j, with U_j dx_j's
// intra-chunk bracket, gives the per-token "direct" delta gradient straight from
// the dx accumulator.  R_i and K_j are built together from one set of M values
// (they cancel exactly where the decay gradient subtracts them).
//
// Kernels (bf16 MFMA; the fp32 path's counterparts are in k_f32.hip):
//   bwd_dx   (chunk, head)            dx, direct d(delta), s_j, dD and
//                                     alpha<dE,H> + sum s per chunk
//   bwd_dcb  (chunk, group, 128x128 causal super-tile; 64x64 tiles where the
//            chunk size is 64 or headdim 128)  head-summed dCB_g; per-head
//                                     tile partials of R, K
//   bwd_dc   (chunk, group, 128 rows; 64 at chunk 64)  dC = dCB_g B + sum_h (state term); r_i
//   bwd_db   (chunk, group, 128 rows; 64 at chunk 64)  dB = dCB_g^T C + sum_h (state term)
//   finalize (chunk, 8 heads)     suffix sum of dAcs (DPP scan), d(delta)->ddt,
//                                 per-chunk partials of dA and d_dt_bias
//   reduce   (head)               fixed-order sums over chunks: dA, dD, d_dt_bias
// Every reduction has a fixed order, so results are bitwise reproducible.
#include "internal.hpp"

namespace ssd {

constexpr int QMAX = 256;

// ------------------------------------------------------------ bwd_dx bf16 ----
constexpr int kDxWaves = 8;

template <int P, int N>
__global__ __launch_bounds__(kDxWaves * 64, 4) void bwd_dx_bf16_kernel(
    ChunkMap m, int H, int G, const uint16_t* __restrict__ X, const uint16_t* __restrict__ Bm,
    const uint16_t* __restrict__ DY, const uint16_t* __restrict__ CBt,
    const float* __restrict__ delta, const float* __restrict__ acs,
    const float* __restrict__ decay, const uint16_t* __restrict__ dE,
    const uint16_t* __restrict__ Hs, const float* __restrict__ D, uint16_t* __restrict__ DX,
    float* __restrict__ ddd, float* __restrict__ Ks, float* __restrict__ last_term,
    float* __restrict__ dDp) {
  constexpr int LDY = P + 16;  // dy tile row stride (bf16): odd multiple of 32 bytes
  constexpr int LDT = N + 8;   // dT tile row stride
  __shared__ __attribute__((aligned(16))) uint16_t dyt[QMAX * LDY];
  __shared__ __attribute__((aligned(16))) uint16_t dts[P * LDT];
  __shared__ float sa[QMAX], sd[QMAX];
  __shared__ float red[3][kDxWaves];
  __shared__ __attribute__((aligned(16))) float wt[QMAX / 32][QMAX];  // column factors per anchor

  int k, h;
  chunk_head(H, k, h);
  const ChunkInfo ci = chunk_info(m, k);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t kh = (int64_t)k * H + h;
  if (ci.len <= 0) {
    if (tid == 0) {
      last_term[kh] = 0.f;
      dDp[kh] = 0.f;
    }
    return;
  }
  const int Q = m.Q, len = ci.len;
  const int g = h / (H / G);
  const int q = lane >> 4, r = lane & 15;
  const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N;
  const uint16_t* xb = X + (int64_t)ci.start * xrow + (int64_t)h * P;
  const uint16_t* dyb = DY + (int64_t)ci.start * xrow + (int64_t)h * P;
  const uint16_t* bb = Bm + (int64_t)ci.start * brow + (int64_t)g * N;
  const uint16_t* cbt = CBt + ((int64_t)k * G + g) * Q * Q;

  // Row blocks of this wave (snake order), and their x values, B rows and first
  // and diagonal CBt fragments: the next row block's are loaded before the
  // current one's stores, so the wait for them does not also wait for those
  // stores (one in-order memory counter); the first row block's are in flight
  // during the prologue.
  const int NB = Q / 16, nii = (NB + kDxWaves - 1) / kDxWaves;
  auto rb_of = [&](int ii) { return kDxWaves * ii + ((ii & 1) ? (kDxWaves - 1 - w) : w); };
  auto live = [&](int ii) { return ii < nii && rb_of(ii) < NB && rb_of(ii) * 16 < len; };
  // Buffer resources over the chunk's valid rows: rows past its end read as
  // zero and are not written.
  const brsrc rx = make_rsrc(xb, (uint32_t)(len * xrow * 2)), rbm = make_rsrc(bb, (uint32_t)(len * brow * 2));
  const brsrc rc = make_rsrc(cbt, (uint32_t)(((len + 15) & ~15) * Q * 2));  // fragment order: whole 16-row blocks
  const brsrc rdx = make_rsrc(DX + (int64_t)ci.start * xrow + (int64_t)h * P, (uint32_t)(len * xrow * 2));
  u32x4 px[P / 32];  // x_j, the lane's 8 adjacent columns per tile pair (pcol)
  u32x4 bq[N / 32], pc1, pcd;
  auto load_rb = [&](int rb) {
    const uint32_t jr = rb * 16 + r, c0 = rb / 2;
    const uint32_t xo = jr * (uint32_t)(xrow * 2) + q * 16, bo = jr * (uint32_t)(brow * 2) + q * 16;
    const uint32_t co = cbf_piece(rb, 0, q * 16 + r, Q);  // CBt block (rb, sx) at co + 1024 sx
#pragma unroll
    for (int s = 0; s < P / 32; ++s) px[s] = buf_load16(rx, xo + 64 * s);
#pragma unroll
    for (int kk = 0; kk < N / 32; ++kk) bq[kk] = buf_load16(rbm, bo + 64 * kk);
    pc1 = buf_load16(rc, co + (c0 + 1) * 1024);  // (unused when no later block exists)
    pcd = buf_load16(rc, co + c0 * 1024);
  };
  if (live(0)) load_rb(rb_of(0));
  // every prologue load in flight before the first LDS store waits on one:
  // acs/delta, the dy tile (token-major, rows past the chunk's end zero, column
  // groups permuted so that a lane's outputs are adjacent columns; read once,
  // so loaded nontemporally), and
  // dT = dE_c (bf16, into LDS [p][n]) with H_c for alpha <dE, H> in fp32
  static_assert(QMAX <= kDxWaves * 64, "one acs/delta value per thread");
  const float av = tid < Q ? acs[kh * Q + tid] : 0.f, dv = tid < Q ? delta[kh * Q + tid] : 0.f;
  RowTile<QMAX, P, kDxWaves * 64, true, true> ytile;
  ytile.load(dyb, xrow, len, tid);
  float dot = 0.f;
  {
    constexpr int NT = kDxWaves * 64, NC = (P * N / 8 + NT - 1) / NT;
    const brsrc rde = make_rsrc(dE + kh * (int64_t)(P * N), (uint32_t)(P * N * 2));
    const brsrc rhh = make_rsrc(Hs + kh * (int64_t)(P * N), (uint32_t)(P * N * 2));
    u32x4 ta[NC], tb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = (tid + c * NT) * 8;
      const uint32_t off = e < P * N ? (uint32_t)e * 2u : 0x80000000u;
      ta[c] = buf_load16(rde, off);
      tb[c] = buf_load16(rhh, off);
    }
    ytile.store(dyt, LDY, tid);
    if (tid < Q) {
      sa[tid] = av;
      sd[tid] = dv;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = (tid + c * NT) * 8;
      if (e < P * N) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          dot += bf_lo(ta[c][d]) * bf_lo(tb[c][d]) + bf_hi(ta[c][d]) * bf_hi(tb[c][d]);
        *(u32x4*)(dts + (e / N) * LDT + (e % N)) = ta[c];
      }
    }
  }
  dot = wave_sum(dot);
  __syncthreads();
  // anchor e = 32b + 31: column factors 2^(acs_i - acs_e) for e < i < len
  for (int idx = tid; idx < (Q / 32) * Q; idx += kDxWaves * 64) {
    const int bb2 = idx / Q, i = idx % Q, e = 32 * bb2 + 31;
    wt[bb2][i] = (i > e && i < len) ? exp2_fast(sa[i] - sa[e]) : 0.f;
  }
  __syncthreads();

  const float Dh = D ? D[h] : 0.f;
  const float a_last = sa[len - 1];
  float s_sum = 0.f, dxx_sum = 0.f;  // lanes q == 0 accumulate their rows
  for (int ii = 0; ii < nii; ++ii) {
    if (!live(ii)) continue;  // chunk sizes with fewer row blocks than wavefronts, short chunks
    const int rb = rb_of(ii);
    const int j0 = rb * 16;
    // Products are issued with the operands swapped, so each lane holds the
    // transposed tile acc[tp][rr] = (dx bracket)[j0 + r][pcol(tp, 4 q + rr)]:
    // the lane owns row jrow, row factors are one value per lane, row dots
    // reduce over the four lanes r, r+16, r+32, r+48, and acc[2s], acc[2s + 1]
    // are 8 adjacent columns (16-byte loads of x and stores of dx).
    f32x4 acc[P / 16];
#pragma unroll
    for (int tp = 0; tp < P / 16; ++tp) acc[tp] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int jrow = j0 + r;
    const bool rowok = jrow < len;
    const int cb0 = j0 / 32;                       // 32-token block holding this row block
    const int e = 32 * cb0 + 31;                   // anchor: j <= e < i for later blocks
    const int s_end = (len + 31) / 32;
    const bool has_off = cb0 + 1 < s_end;
    const float ae = has_off ? sa[e] : 0.f;
    const float aj = sa[jrow];                     // jrow < Q always
    u32x4 xq[P / 32];                              // this lane's x values
#pragma unroll
    for (int s = 0; s < P / 32; ++s) xq[s] = px[s];
    // state part: sum_n B_j[n] dT[p][n]
#pragma unroll
    for (int kk = 0; kk < N / 32; ++kk) {
      const bf16x8 b = as_bf16x8(bq[kk]);
#pragma unroll
      for (int tp = 0; tp < P / 16; ++tp)
        acc[tp] = mfma_bf16(as_bf16x8(*(const u32x4*)(dts + pcol(tp, r) * LDT + kk * 32 + q * 8)), b, acc[tp]);
    }
    const float wj = rowok ? exp2_fast(a_last - aj) : 0.f;
    float xs = 0.f;
#pragma unroll
    for (int s = 0; s < P / 32; ++s) xs += dot_bf8(xq[s], acc[2 * s], acc[2 * s + 1]);
    xs *= wj;                                      // this lane's part of x_j . (w_j dT B_j)
    if (has_off) {
      // later blocks through the anchor: acc = 2^(acs_last - acs_e) state
      //   + sum_i CBt[j][i] 2^(acs_i - acs_e) dy_i, then * 2^(acs_e - acs_j)
      const float s0 = exp2_fast(a_last - ae);
#pragma unroll
      for (int tp = 0; tp < P / 16; ++tp) acc[tp] *= s0;
      const float* wrow = &wt[cb0][0];
      u32x4 cvn = pc1;
      const uint32_t co = cbf_piece(rb, 0, q * 16 + r, Q);
      for (int sx = cb0 + 1; sx < s_end; ++sx) {
        const u32x4 cv = cvn;
        if (sx + 1 < s_end) cvn = buf_load16(rc, co + (sx + 1) * 1024);  // one step of lookahead
        const float4 f0 = *(const float4*)(wrow + sx * 32 + q * 8);
        const float4 f1 = *(const float4*)(wrow + sx * 32 + q * 8 + 4);
        u32x4 av;
        av[0] = pack_bf2(bf_lo(cv[0]) * f0.x, bf_hi(cv[0]) * f0.y);
        av[1] = pack_bf2(bf_lo(cv[1]) * f0.z, bf_hi(cv[1]) * f0.w);
        av[2] = pack_bf2(bf_lo(cv[2]) * f1.x, bf_hi(cv[2]) * f1.y);
        av[3] = pack_bf2(bf_lo(cv[3]) * f1.z, bf_hi(cv[3]) * f1.w);
        const bf16x8 a = as_bf16x8(av);
#pragma unroll
        for (int tp = 0; tp < P / 16; ++tp)
          acc[tp] = mfma_bf16(frag_kmajor(dyt + sx * 32 * LDY + tp * 16, LDY, lane), a, acc[tp]);
      }
      const float u = rowok ? exp2_fast(ae - aj) : 0.f;
#pragma unroll
      for (int tp = 0; tp < P / 16; ++tp) acc[tp] *= u;
    } else {
#pragma unroll
      for (int tp = 0; tp < P / 16; ++tp) acc[tp] *= wj;
    }
    // the diagonal block, one exp per element: CBt[j][i] 2^(acs_i - acs_j), j <= i < len
    {
      const u32x4 cv = pcd;
      u32x4 av;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int i0 = cb0 * 32 + q * 8 + 2 * d;
        float v0 = bf_lo(cv[d]) * exp2_fast(sa[i0] - aj);
        float v1 = bf_hi(cv[d]) * exp2_fast(sa[i0 + 1] - aj);
        v0 = (i0 >= jrow && i0 < len) ? v0 : 0.f;
        v1 = (i0 + 1 >= jrow && i0 + 1 < len) ? v1 : 0.f;
        av[d] = pack_bf2(v0, v1);
      }
      const bf16x8 a = as_bf16x8(av);
#pragma unroll
      for (int tp = 0; tp < P / 16; ++tp)
        acc[tp] = mfma_bf16(frag_kmajor(dyt + cb0 * 32 * LDY + tp * 16, LDY, lane), a, acc[tp]);
    }
    if (live(ii + 1)) load_rb(rb_of(ii + 1));  // the fragments above are dead now
    // per-row dots and the store: the lane's 8 adjacent columns per tile pair, written as
    // whole 128-byte row spans (span_swap) where a row has two pieces per lane
    const float dj = rowok ? sd[jrow] : 0.f;
    float xt = 0.f, dxx = 0.f;
    const uint32_t dxo = (uint32_t)jrow * (uint32_t)(xrow * 2) + q * 16;
    u32x4 os[P / 32];
#pragma unroll
    for (int s = 0; s < P / 32; ++s) {
      const u32x4 dq = lds_cols8_perm(dyt + jrow * LDY, s, q);  // rows past the end are zero
      xt += dot_bf8(xq[s], acc[2 * s], acc[2 * s + 1]);
      u32x4 o;
#pragma unroll
      for (int u = 0; u < 2; ++u) {  // tile 2s + u: the lane's columns 32s + 8q + 4u .. +3
        const f32x4 a = acc[2 * s + u];
        const float y0 = bf_lo(dq[2 * u]), y1 = bf_hi(dq[2 * u]);
        const float y2 = bf_lo(dq[2 * u + 1]), y3 = bf_hi(dq[2 * u + 1]);
        dxx += bf_lo(xq[s][2 * u]) * y0 + bf_hi(xq[s][2 * u]) * y1 + bf_lo(xq[s][2 * u + 1]) * y2 +
               bf_hi(xq[s][2 * u + 1]) * y3;
        o[2 * u] = pack_bf2(dj * a[0] + Dh * y0, dj * a[1] + Dh * y1);
        o[2 * u + 1] = pack_bf2(dj * a[2] + Dh * y2, dj * a[3] + Dh * y3);
      }
      os[s] = o;
    }
    if constexpr (P >= 64) {
      const uint32_t ra = (uint32_t)(j0 + (r & 7)), so = span_off(r, q);
#pragma unroll
      for (int m2 = 0; m2 < P / 64; ++m2) {
        u32x4 a, b;
        span_swap(r, os[2 * m2], os[2 * m2 + 1], a, b);
        buf_store16(rdx, ra * (uint32_t)(xrow * 2) + so + 128 * m2, a);
        buf_store16(rdx, (ra + 8) * (uint32_t)(xrow * 2) + so + 128 * m2, b);
      }
    } else {
      buf_store16(rdx, dxo, os[0]);
    }
    xs += __shfl_xor(xs, 16);
    xs += __shfl_xor(xs, 32);
    xt += __shfl_xor(xt, 16);
    xt += __shfl_xor(xt, 32);
    dxx += __shfl_xor(dxx, 16);
    dxx += __shfl_xor(dxx, 32);
    if (q == 0 && rowok) {
      ddd[kh * Q + jrow] = xt;
      Ks[kh * Q + jrow] = dj * xs;  // s_j (K_j comes from bwd_dcb)
      s_sum += dj * xs;
      dxx_sum += dxx;
    }
  }
  // fixed-order workgroup reductions: lanes (w, q) -> wave -> waves 0..3
  s_sum = wave_sum(s_sum);
  dxx_sum = wave_sum(dxx_sum);
  if (lane == 0) {
    red[0][w] = s_sum;
    red[1][w] = dxx_sum;
    red[2][w] = dot;
  }
  __syncthreads();
  if (tid == 0) {
    float S = 0.f, DD = 0.f, HD = 0.f;
    for (int i = 0; i < kDxWaves; ++i) {
      S += red[0][i];
      DD += red[1][i];
      HD += red[2][i];
    }
    last_term[kh] = S + exp2_fast(decay[kh]) * HD;
    dDp[kh] = DD;
  }
}

// ------------------------------------------------------------ bwd_dcb bf16 ----
// One workgroup per (chunk, group, 64x64 causal tile (ti, tj), tj <= ti).  B and
// C are shared by the group's heads, so the intra-chunk parts of dC and dB only
// need the head-summed dCB_g = sum_h dCB^h: it is formed here once per tile, so
// dC and dB each become one GEMM per group (dB reads it down the columns).
// For every head the tile's contributions to R_i (row sums over j < i) and K_j
// (column sums over i > j) of M_ij = dCB_ij CB_ij come from the same values,
// so they cancel exactly where the decay gradient subtracts them.
//
// Wave w owns rows ti*64 + 16w .. +15.  Per head: the tile's 64 x rows are
// staged in LDS by all four waves together (double-buffered, one barrier per
// head), each wave's 16 dy rows stay in registers, and both are loaded one head
// ahead.  D = dy_rows . x_tile^T on MFMA (K = headdim), then times L_ij delta_j:
// an off-diagonal tile factors the decay through its last column e
// (2^(acs_i - acs_e) per row times 2^(acs_e - acs_j) delta_j per column, both
// <= 1), the diagonal tile takes one exp per element and the causal mask.
template <int P>
__global__ __launch_bounds__(256, 4) void bwd_dcb_bf16_kernel(
    ChunkMap m, int H, int G, const uint16_t* __restrict__ X, const uint16_t* __restrict__ DY,
    const uint16_t* __restrict__ CB, const float* __restrict__ delta,
    const float* __restrict__ acs, uint16_t* __restrict__ dCBg,
    float* __restrict__ Rp, float* __restrict__ Kp) {
  constexpr int LX = P + 8;          // x tile row stride (bf16)
  constexpr int LT = 64 + 8;         // output staging row stride
  constexpr int PER = P / 8;         // 16-byte pieces per row
  constexpr int NPX = 64 * PER / 256;  // x pieces per thread per head
  static_assert(NPX >= 1, "headdim");
  __shared__ __attribute__((aligned(16))) uint16_t xt[2][64 * LX];
  __shared__ float kred[8][4][64];
  __shared__ __attribute__((aligned(16))) float sv[8][320];  // per head of a block of 8 (below)
  const int Q = m.Q, T = Q / 64, NT = T * (T + 1) / 2;
  const int lid = xcd_order(blockIdx.x, gridDim.x);  // (chunk, group, tile), tile fastest
  const int tile = lid % NT, k = lid / NT / G, g = (lid / NT) % G;
  const ChunkInfo ci = chunk_info(m, k);
  int ti = 0;
  while ((ti + 1) * (ti + 2) / 2 <= tile) ++ti;
  const int tj = tile - ti * (ti + 1) / 2;
  if (ci.len <= 0 || ti * 64 >= ci.len) return;
  const int len = ci.len;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, r = lane & 15;
  const int hpg = H / G;
  const int64_t xrow = (int64_t)H * P;
  const int i0 = ti * 64 + w * 16, jt0 = tj * 64;
  const int irow = i0 + r;
  const bool diag = ti == tj;
  const int64_t kg = (int64_t)k * G + g;
  const uint16_t* cbm = CB + kg * Q * Q;
  // CB at this lane's 16 outputs: every load unconditional (the chunk's CB
  // tile is whole in memory), then the causal mask j < i < len
  float cbv[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int i = i0 + q * 4 + rr, j = jt0 + b * 16 + r;
      const float c = bf2f(cbm[cbf_off(i, j, Q)]);  // (fragment order)
      cbv[b][rr] = (i < len && j < i) ? c : 0.f;
    }
  f32x4 sum[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) sum[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the next head's rows: this wave's dy fragments and this thread's x pieces
  u32x4 ay[P / 32], px[NPX];
  // (buffer resources over the chunk's valid rows: rows past the end read as zero)
  const uint32_t yo = (uint32_t)irow * (uint32_t)(xrow * 2) + q * 16;
  auto load_head = [&](int h) {
    const brsrc rdy = make_rsrc(DY + (int64_t)ci.start * xrow + (int64_t)h * P, (uint32_t)(len * xrow * 2));
    const brsrc rxt = make_rsrc(X + (int64_t)(ci.start + jt0) * xrow + (int64_t)h * P,
                                (uint32_t)(max(len - jt0, 0) * xrow * 2));
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb) ay[kb] = buf_load16(rdy, yo + 64 * kb);
#pragma unroll
    for (int c = 0; c < NPX; ++c) {
      const uint32_t e = tid + c * 256, row = e / PER, c8 = e % PER;
      px[c] = buf_load16(rxt, row * (uint32_t)(xrow * 2) + c8 * 16);
    }
  };
  // Per head of a block of 8, sv holds acs of the tile's rows [0, 64), acs of
  // its columns [64, 128) and delta of its columns [128, 192); an off-diagonal
  // tile (anchor e = its last column, e < i for every row i) also holds
  //   [192, 256) rho_i = 2^(acs_i - acs_e) (0 past the chunk's end),
  //   [256, 320) gam_j = 2^(acs_e - acs_j) delta_j,
  // so that its per-element factor is rho_i gam_j (a diagonal tile takes one
  // exp per element).  Called at the start of each block of 8 heads: the
  // previous block's readers are done (the column reduction ends in a barrier).
  // Every value of the block is loaded before the first is stored (range-checked
  // buffer loads, no branches: a load-then-store loop would wait for each load
  // in turn), and every slot of sv is written (slots of heads past the group's
  // end get zeros and are never read).
  auto fill_sv = [&](int h0, int nh) {
    const int64_t kh0 = (int64_t)k * H + h0;
    const brsrc ra = make_rsrc(acs + kh0 * Q, (uint32_t)(nh * Q * 4));
    const brsrc rd = make_rsrc(delta + kh0 * Q, (uint32_t)(nh * Q * 4));
    float va[4], vd[2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // acs of the tile's rows [0, 64) and columns [64, 128): 8 x 128
      const int e = tid + u * 256, sl = e >> 7, c = e & 127;
      const int t = (c < 64) ? ti * 64 + c : jt0 + (c - 64);  // < Q: inside the workspace
      va[u] = buf_load_f32(ra, (uint32_t)(sl * Q + t) * 4u);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // delta of its columns [128, 192): 8 x 64
      const int e = tid + u * 256, sl = e >> 6, c = e & 63;
      vd[u] = buf_load_f32(rd, (uint32_t)(sl * Q + jt0 + c) * 4u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + u * 256;
      sv[e >> 7][e & 127] = va[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + u * 256;
      sv[e >> 6][128 + (e & 63)] = vd[u];
    }
    if (!diag) {
      __syncthreads();
      for (int e = tid; e < nh * 128; e += 256) {
        const int sl = e >> 7, c = e & 127;
        const float ae = sv[sl][127];
        sv[sl][192 + c] = (c < 64) ? ((ti * 64 + c < len) ? exp2_fast(sv[sl][c] - ae) : 0.f)
                                   : exp2_fast(ae - sv[sl][c]) * sv[sl][c + 64];
      }
    }
  };
  load_head(g * hpg);
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const int64_t kh = (int64_t)k * H + h;
    uint16_t* xbuf = xt[hh & 1];
    // (the block's decay values are loaded while this head's rows are in flight)
    if ((hh & 7) == 0) fill_sv(h, min(8, hpg - hh));
#pragma unroll
    for (int c = 0; c < NPX; ++c) {
      const int e = tid + c * 256, row = e / PER, c8 = e % PER;
      *(u32x4*)(xbuf + row * LX + c8 * 8) = px[c];
    }
    __syncthreads();
    bf16x8 af[P / 32];
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb) af[kb] = as_bf16x8(ay[kb]);
    if (hh + 1 < hpg) load_head(h + 1);  // in flight during this head's work
    f32x4 dxb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      dxb[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < P / 32; ++kb)
        dxb[b] = mfma_bf16(af[kb], as_bf16x8(*(const u32x4*)(xbuf + (b * 16 + r) * LX + kb * 32 + q * 8)),
                           dxb[b]);
    }
    // v = dCB^h_ij, M_ij = v CB_ij; R_i and K_j both add the exact products
    const float* svh = sv[hh & 7];
    float Rl[4] = {0.f, 0.f, 0.f, 0.f}, Kl[4] = {0.f, 0.f, 0.f, 0.f};
    if (!diag) {
      const float4 rho = *(const float4*)(svh + 192 + w * 16 + q * 4);
      const float rr4[4] = {rho.x, rho.y, rho.z, rho.w};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float gam = svh[256 + b * 16 + r];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float v = dxb[b][rr] * rr4[rr] * gam;
          sum[b][rr] += v;
          Rl[rr] = fmaf(v, cbv[b][rr], Rl[rr]);
          Kl[b] = fmaf(v, cbv[b][rr], Kl[b]);
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float aj = svh[64 + b * 16 + r], dj = svh[128 + b * 16 + r];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int i = i0 + q * 4 + rr, j = jt0 + b * 16 + r;
          float v = dxb[b][rr] * exp2_fast(svh[w * 16 + q * 4 + rr] - aj) * dj;
          v = (j <= i && i < len) ? v : 0.f;
          sum[b][rr] += v;
          Rl[rr] = fmaf(v, cbv[b][rr], Rl[rr]);  // cbv is zero unless j < i < len
          Kl[b] = fmaf(v, cbv[b][rr], Kl[b]);
        }
      }
    }
    {
      // row sums: lane r ends with row i0 + 4q + r/4; lanes r % 4 == 0 store
      const float v = row_reduce_scatter4(Rl[0], Rl[1], Rl[2], Rl[3], r);
      const int i = i0 + q * 4 + (r >> 2);
      if ((r & 3) == 0 && i < len) Rp[(kh * T + tj) * Q + i] = v;
    }
    const int slot = hh & 7;
    // column sums over the wave's rows: lane (r, q) ends with column 16 q + r
    kred[slot][w][q * 16 + r] = col_reduce_scatter4(Kl[0], Kl[1], Kl[2], Kl[3]);
    if (slot == 7 || hh == hpg - 1) {  // cross-wave column sums, fixed order, every 8 heads
      __syncthreads();
      for (int e = tid; e < (slot + 1) * 64; e += 256) {
        const int sl = e >> 6, jj = e & 63, j = jt0 + jj;
        const int64_t khs = (int64_t)k * H + h - slot + sl;
        const float v = kred[sl][0][jj] + kred[sl][1][jj] + kred[sl][2][jj] + kred[sl][3][jj];
        if (j < len) Kp[(khs * T + ti) * Q + j] = v;
      }
      __syncthreads();
    }
  }
  // head-summed tile -> bf16, through LDS to 16-byte row stores
  uint16_t* stg = xt[0];  // every wave is past its last read of the x tiles (barrier above)
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) stg[(w * 16 + q * 4 + rr) * LT + b * 16 + r] = f2bf(sum[b][rr]);
  __syncthreads();
  for (int e = tid; e < 64 * 8; e += 256) {
    const int row = e >> 3, c8 = e & 7;
    *(u32x4*)(dCBg + (kg * Q + ti * 64 + row) * Q + jt0 + c8 * 8) = *(const u32x4*)(stg + row * LT + c8 * 8);
  }
}

// ----------------------------------------------------- bwd_dcb bf16, 128 ----
// The head-summed dCB_g of bwd_dcb_bf16_kernel, on 128x128 super-tiles (si, sj),
// sj <= si, for chunk sizes that are multiples of 128.  A (chunk, group) has
// T2 (T2 + 1) / 2 of them (3 at chunk 256) against T (T + 1) / 2 64x64 tiles
// (10): each head's dy and x rows of 128 tokens serve two 64x64 tiles each way,
// so a chunk's rows are read 12 times per head instead of 20.  Every element is
// formed exactly as in the 64x64 kernel (the 64x64 tiles' decay anchors, the
// same operand order and the same head order of the sum), so dCB_g is the same
// bit for bit; the tile partials of R and K cover 128 columns / rows.
//
// Eight waves; wave w owns rows 128 si + 16 w .. +15 and the super-tile's 8
// column blocks of 16 (on a diagonal super-tile only blocks b <= w: the others
// lie above the diagonal).  Per head, x's 128 rows are staged in LDS by all
// waves (double-buffered), each wave's dy rows stay in registers, and the
// head's decay factors go to LDS (double-buffered), all loaded one head ahead;
// the previous head's column sums are reduced across the waves after the
// barrier that starts the next head.  A wave whose rows all lie past the
// chunk's end does no work (so no value read past the end, where a decay anchor
// of a short chunk can lie, enters a product).
constexpr int kT128Waves = 8;

template <int P>
__global__ __launch_bounds__(kT128Waves * 64, 4) void bwd_dcb_t128_bf16_kernel(
    ChunkMap m, int H, int G, const uint16_t* __restrict__ X, const uint16_t* __restrict__ DY,
    const uint16_t* __restrict__ CB, const float* __restrict__ delta,
    const float* __restrict__ acs, uint16_t* __restrict__ dCBg,
    float* __restrict__ Rp, float* __restrict__ Kp) {
  constexpr int NT = kT128Waves * 64;
  constexpr int LX = P + 8;             // x tile row stride (bf16)
  constexpr int LT = 128 + 8;           // output staging row stride
  constexpr int PER = P / 8;            // 16-byte pieces per row
  constexpr int NPX = 128 * PER / NT;   // x pieces per thread per head
  constexpr int XS = 128 * LX;          // one x buffer
  constexpr int XL = 2 * XS > 128 * LT ? 2 * XS : 128 * LT;
  static_assert(NPX >= 1 && 128 * PER % NT == 0, "headdim");
  __shared__ __attribute__((aligned(16))) uint16_t xt[XL];
  __shared__ __attribute__((aligned(16))) float kred[2][kT128Waves][128];
  __shared__ __attribute__((aligned(16))) float sv[2][384];  // one head's decay factors (below)
  const int Q = m.Q, T2 = Q / 128, NS = T2 * (T2 + 1) / 2;
  const int lid = xcd_order(blockIdx.x, gridDim.x);  // (chunk, group, super-tile), super-tile fastest
  const int tile = lid % NS, k = lid / NS / G, g = (lid / NS) % G;
  const ChunkInfo ci = chunk_info(m, k);
  int si = 0;
  while ((si + 1) * (si + 2) / 2 <= tile) ++si;
  const int sj = tile - si * (si + 1) / 2;
  if (ci.len <= 0 || si * 128 >= ci.len) return;
  const int len = ci.len;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r = lane & 15;
  const int hpg = H / G;
  const int64_t xrow = (int64_t)H * P;
  const int i0 = si * 128 + w * 16, jt0 = sj * 128;
  const bool diag = si == sj;
  const bool live = i0 < len;          // (uniform per wave)
  const int nblk = diag ? w + 1 : 8;   // column blocks this wave works on
  const int64_t kg = (int64_t)k * G + g;
  const uint16_t* cbm = CB + kg * Q * Q;
  // C.B^T at this lane's 32 outputs (rows i0 + 4 q + rr, columns jt0 + 16 b + r),
  // two bf16 values per register, zero unless j < i < len
  // (range-checked 2-byte loads, the mask folded into an offset past the range:
  // no load sits under a branch, so all 32 are in flight together)
  const brsrc rcb = make_rsrc(cbm, (uint32_t)(Q * Q * 2));
  uint32_t cbp[8][2];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    uint32_t v[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int i = i0 + q * 4 + rr, j = jt0 + b * 16 + r;
      const bool ok = live && b < nblk && i < len && j < i;
      v[rr] = __builtin_amdgcn_raw_buffer_load_b16(rcb, ok ? cbf_off(i, j, Q) * 2u : 0x80000000u, 0, 0);
    }
    cbp[b][0] = v[0] | (v[1] << 16);
    cbp[b][1] = v[2] | (v[3] << 16);
  }
  // This thread's decay inputs per head (tokens are chunk positions < Q, inside
  // the workspace; 0x80000000: none).  Off the diagonal, the super-tile's four
  // 64x64 tiles are all off the diagonal, tile (ti, tj) anchored at its last
  // column e = 64 tj + 63:
  //   [0, 256)   rho[a][i] = 2^(acs_i - acs_e(a)) (0 past the chunk's end), a = tj - 2 sj
  //   [256, 384) gam[j] = 2^(acs_e(j) - acs_j) delta_j
  // On the diagonal, tile (2 si + 1, 2 si) is anchored at e = 128 si + 63 and the
  // two diagonal tiles take one exp per element:
  //   [0, 64) rho of rows 64..127, [64, 128) gam of columns 0..63,
  //   [128, 256) acs of the 128 tokens, [256, 384) their delta.
  // Thread t's entry t of that table: its token, its anchor (or -1) and its kind.
  // Formed from an opaque copy of the thread index where used, so that the
  // compiler does not keep them in registers across the head loop.
  struct Role {
    int tok, anc, kind;  // kind: 0 none, 1 rho, 2 gam, 3 acs, 4 delta
  };
  auto role = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    Role o{0, -1, 0};
    if (!diag) {
      if (t < 256) o = Role{si * 128 + (t & 127), sj * 128 + (t >> 7) * 64 + 63, 1};
      else if (t < 384) o = Role{jt0 + t - 256, jt0 + ((t - 256) >> 6) * 64 + 63, 2};
    } else {
      const int e = si * 128 + 63;
      if (t < 64) o = Role{si * 128 + 64 + t, e, 1};
      else if (t < 128) o = Role{si * 128 + t - 64, e, 2};
      else if (t < 256) o = Role{si * 128 + t - 128, -1, 3};
      else if (t < 384) o = Role{si * 128 + t - 256, -1, 4};
    }
    return o;
  };
  f32x4 sum[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) sum[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the next head's rows and decay inputs
  u32x4 ay[P / 32], px[NPX];
  float pa = 0.f, pd = 0.f, pe = 0.f;
  const uint32_t yo = (uint32_t)(i0 + r) * (uint32_t)(xrow * 2) + q * 16;
  auto load_head = [&](int h) {
    const brsrc rdy = make_rsrc(DY + (int64_t)ci.start * xrow + (int64_t)h * P, (uint32_t)(len * xrow * 2));
    const brsrc rxt = make_rsrc(X + (int64_t)(ci.start + jt0) * xrow + (int64_t)h * P,
                                (uint32_t)(max(len - jt0, 0) * xrow * 2));
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb) ay[kb] = buf_load16(rdy, yo + 64 * kb);
#pragma unroll
    for (int c = 0; c < NPX; ++c) {
      const uint32_t e = tid + c * NT, row = e / PER, c8 = e % PER;
      px[c] = buf_load16(rxt, row * (uint32_t)(xrow * 2) + c8 * 16);
    }
    const int64_t kh = (int64_t)k * H + h;
    const brsrc ra = make_rsrc(acs + kh * Q, (uint32_t)(Q * 4));
    const brsrc rd = make_rsrc(delta + kh * Q, (uint32_t)(Q * 4));
    const Role o = role();
    constexpr uint32_t kNone = 0x80000000u;  // past every range: reads zero
    const uint32_t ot = (uint32_t)o.tok * 4u;
    pa = buf_load_f32(ra, (o.kind == 1 || o.kind == 2 || o.kind == 3) ? ot : kNone);
    pd = buf_load_f32(rd, (o.kind == 2 || o.kind == 4) ? ot : kNone);
    pe = buf_load_f32(ra, o.anc >= 0 ? (uint32_t)o.anc * 4u : kNone);
  };
  load_head(g * hpg);
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const int64_t kh = (int64_t)k * H + h;
    const int buf = hh & 1;
    uint16_t* xbuf = xt + buf * XS;
#pragma unroll
    for (int c = 0; c < NPX; ++c) {
      const int e = tid + c * NT, row = e / PER, c8 = e % PER;
      *(u32x4*)(xbuf + row * LX + c8 * 8) = px[c];
    }
    {
      const Role o = role();
      float f = o.kind == 3 ? pa : pd;
      if (o.kind == 1) f = (o.tok < len) ? exp2_fast(pa - pe) : 0.f;
      if (o.kind == 2) f = exp2_fast(pe - pa) * pd;
      if (o.kind) sv[buf][tid] = f;
    }
    __syncthreads();
    if (hh > 0 && tid < 128) {  // the previous head's column sums, fixed order over the waves
      const int j = jt0 + tid;
      float v = 0.f;
#pragma unroll
      for (int u = 0; u < kT128Waves; ++u) v += kred[buf ^ 1][u][tid];
      if (j < len) Kp[((kh - 1) * T2 + si) * Q + j] = v;
    }
    bf16x8 af[P / 32];
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb) af[kb] = as_bf16x8(ay[kb]);
    if (hh + 1 < hpg) load_head(h + 1);  // in flight during this head's work
    const float* svh = sv[buf];
    // this lane's x fragment base (an opaque copy of the lane index: the block and
    // k-step offsets become immediates instead of 16 hoisted addresses)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint16_t* xl = xbuf + (ln & 15) * LX + (ln >> 4) * 8;
    float Rl[4] = {0.f, 0.f, 0.f, 0.f}, Kl[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float kA = 0.f, kB = 0.f;  // column sums over the wave's rows (below)
    if (live) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        if (b == 4) kA = col_reduce_scatter4(Kl[0], Kl[1], Kl[2], Kl[3]);
        if (b >= nblk) continue;
        f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < P / 32; ++kb)
          d = mfma_bf16(af[kb], as_bf16x8(*(const u32x4*)(xl + b * 16 * LX + kb * 32)), d);
        // (unpacked here from opaque copies: hoisted out of the head loop, the 32
        // values would not fit the registers)
        uint32_t c01 = cbp[b][0], c23 = cbp[b][1];
        asm volatile("" : "+v"(c01), "+v"(c23));
        float cb[4];
        cb[0] = __uint_as_float(c01 << 16);
        cb[1] = __uint_as_float(c01 & 0xffff0000u);
        cb[2] = __uint_as_float(c23 << 16);
        cb[3] = __uint_as_float(c23 & 0xffff0000u);
        // v = dCB^h_ij, M_ij = v CB_ij; R_i and K_j both add the exact products
        if (!diag || (w >= 4 && b < 4)) {  // a 64x64 tile off the diagonal
          const int ro = diag ? (w - 4) * 16 + q * 4 : (b >> 2) * 128 + w * 16 + q * 4;
          const float4 rho = *(const float4*)(svh + ro);
          const float rr4[4] = {rho.x, rho.y, rho.z, rho.w};
          const float gam = svh[(diag ? 64 : 256) + b * 16 + r];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float v = d[rr] * rr4[rr] * gam;
            sum[b][rr] += v;
            Rl[rr] = fmaf(v, cb[rr], Rl[rr]);
            Kl[b] = fmaf(v, cb[rr], Kl[b]);
          }
        } else {  // a diagonal 64x64 tile: one exp per element and the causal mask
          const float aj = svh[128 + b * 16 + r], dj = svh[256 + b * 16 + r];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int i = i0 + (ln >> 4) * 4 + rr, j = jt0 + b * 16 + (ln & 15);  // (masks formed per head)
            float v = d[rr] * exp2_fast(svh[128 + w * 16 + q * 4 + rr] - aj) * dj;
            v = (j <= i && i < len) ? v : 0.f;
            sum[b][rr] += v;
            Rl[rr] = fmaf(v, cb[rr], Rl[rr]);  // cb is zero unless j < i < len
            Kl[b] = fmaf(v, cb[rr], Kl[b]);
          }
        }
      }
      kB = col_reduce_scatter4(Kl[4], Kl[5], Kl[6], Kl[7]);
      // row sums: lane r ends with row i0 + 4q + r/4; lanes r % 4 == 0 store
      const float v = row_reduce_scatter4(Rl[0], Rl[1], Rl[2], Rl[3], r);
      const int i = i0 + q * 4 + (r >> 2);
      if ((r & 3) == 0 && i < len) Rp[(kh * T2 + sj) * Q + i] = v;
    }
    // column sums over the wave's rows: lane (r, q) holds columns 16 q + r and 64 + 16 q + r
    kred[buf][w][q * 16 + r] = kA;
    kred[buf][w][64 + q * 16 + r] = kB;
  }
  __syncthreads();
  if (tid < 128) {  // the last head's column sums
    const int64_t khl = (int64_t)k * H + g * hpg + hpg - 1;
    const int j = jt0 + tid;
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < kT128Waves; ++u) v += kred[(hpg - 1) & 1][u][tid];
    if (j < len) Kp[(khl * T2 + si) * Q + j] = v;
  }
  // head-summed tile -> bf16, through LDS to 16-byte row stores of the 64x64
  // tiles that the 64x64 kernel writes (tj <= ti, rows of the tile before the
  // chunk's end)
  uint16_t* stg = xt;  // every wave is past its last read of the x tiles (barrier above)
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) stg[(w * 16 + q * 4 + rr) * LT + b * 16 + r] = f2bf(sum[b][rr]);
  __syncthreads();
  for (int e = tid; e < 128 * 16; e += NT) {
    const int row = e >> 4, c8 = e & 15;
    const bool upper = diag && row < 64 && c8 >= 8;
    if (!upper && si * 128 + (row & ~63) < len)
      *(u32x4*)(dCBg + (kg * Q + si * 128 + row) * Q + jt0 + c8 * 8) = *(const u32x4*)(stg + row * LT + c8 * 8);
  }
}

// ------------------------------------------------------------ bwd_dc bf16 ----
// One workgroup of W waves per (chunk, group, 16 W rows i): W = 8 (128 rows) where
// the chunk size is a multiple of 128, so that each head's H tile is staged once
// for 128 rows (half the requests for it of 64-row workgroups), else W = 4.
// dC_i = sum_{j<=i} dCB_g[i][j] B_j
// (dCB_g fragments straight from its rows, B through LDS one 64-row piece at a
// time and read with transpose reads) + sum_h 2^acs_i H^T dy_i (one K=headdim
// GEMM per head); r_i = C_i . (that head's state term).  Per head, H (bf16) is
// staged in a double-buffered LDS tile (one barrier per head) and the next
// head's H, dy fragments and acs are loaded into registers while this head is
// worked on.  Products are issued with the operands swapped, so each lane owns
// one row i: its r_i reduces over four lanes.  B and H are staged with their
// column groups permuted (common.hpp, pcol), so a lane's outputs are 8 adjacent
// columns per tile pair and C is loaded and dC stored 16 bytes at a time.
template <int P, int N, int W>
__global__ __launch_bounds__(W * 64, 4) void bwd_dc_bf16_kernel(
    ChunkMap m, int H, int G, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ DY, const uint16_t* __restrict__ dCBg,
    const float* __restrict__ acs, const uint16_t* __restrict__ Hs, uint16_t* __restrict__ dC,
    float* __restrict__ rout) {
  constexpr int LDB = N + 16;  // odd multiple of 32 bytes for the transpose reads
  constexpr int ROWS = P > 64 ? P : 64;
  constexpr int NT = W * 64, RW = 16 * W;      // threads; rows per workgroup
  constexpr int NPH = (P * N / 8 + NT - 1) / NT;  // 16-byte pieces of H per thread
  __shared__ __attribute__((aligned(16))) uint16_t ub[2][ROWS * LDB];
  const int T = m.Q / RW;
  const int lid = xcd_order(blockIdx.x, gridDim.x);  // (chunk, group, tile), tile fastest
  const int tile = lid % T, k = lid / T / G, g = (lid / T) % G;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0 || tile * RW >= ci.len) return;
  const int Q = m.Q, len = ci.len;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, r = lane & 15;
  const int hpg = H / G;
  const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N;
  const uint16_t* bb = Bm + (int64_t)ci.start * brow + (int64_t)g * N;
  const uint16_t* cb = Cm + (int64_t)ci.start * brow + (int64_t)g * N;
  const uint16_t* dcb = dCBg + ((int64_t)k * G + g) * Q * Q;
  const int i0 = tile * RW + w * 16;
  const bool active = i0 < len;
  const int irow = i0 + r;
  // buffer resources over the chunk's valid rows (rows past the end: zero, not written)
  const brsrc rdcb = make_rsrc(dcb, (uint32_t)(len * Q * 2)), rcm = make_rsrc(cb, (uint32_t)(len * brow * 2));
  const uint32_t ro = (uint32_t)irow * (uint32_t)(brow * 2) + q * 16;  // this lane's offset in a B/C row
  const uint32_t yo = (uint32_t)irow * (uint32_t)(xrow * 2) + q * 16;  // and in an x/dy row
  // acc[nb][rr] = dC[irow][pcol(nb, 4 q + rr)]
  f32x4 acc[N / 16];
#pragma unroll
  for (int nb = 0; nb < N / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* bt = ub[0];
  for (int jt = 0; jt * 64 < tile * RW + RW && jt * 64 < len; ++jt) {
    // this piece's B rows and this lane's two dCB_g fragments, all in flight
    // together (one memory latency per piece); fragments past the row block's
    // causal end are not needed
    RowTile<64, N, NT, true> btile;
    btile.load(bb + (int64_t)jt * 64 * brow, brow, len - jt * 64, tid);
    const int jend = min(jt * 64 + 64, i0 + 16);
    u32x4 af[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int jb = jt * 64 + 32 * u;
      af[u] = (active && jb < jend) ? buf_load16(rdcb, (uint32_t)irow * (uint32_t)(Q * 2) + jb * 2 + q * 16)
                                    : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();  // every wave is done with the previous piece
    btile.store(bt, LDB, tid);
    __syncthreads();
    if (!active) continue;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (jt * 64 + 32 * u >= jend) break;
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb)
        acc[nb] = mfma_bf16(frag_kmajor(bt + 32 * u * LDB + nb * 16, LDB, lane), as_bf16x8(af[u]), acc[nb]);
    }
  }
  // C_i values of this lane's outputs, 8 adjacent per tile pair
  u32x4 cq[N / 32];
#pragma unroll
  for (int s = 0; s < N / 32; ++s) cq[s] = buf_load16(rcm, ro + 64 * s);
  // the next head's H pieces, dy fragments and acs_i
  u32x4 ph[NPH], py[P / 32];
  float pa = 0.f;
  auto load_head = [&](int h) {
    const int64_t kh = (int64_t)k * H + h;
    // range-checked loads, no branches (rows past the chunk's end read zero)
    const brsrc rh = make_rsrc(Hs + kh * (int64_t)(P * N), (uint32_t)(P * N * 2));
#pragma unroll
    for (int c = 0; c < NPH; ++c) {
      const int e = (tid + c * NT) * 8;
      ph[c] = buf_load16(rh, e < P * N ? (uint32_t)e * 2u : 0x80000000u);
    }
    const brsrc rdy = make_rsrc(DY + (int64_t)ci.start * xrow + (int64_t)h * P, (uint32_t)(len * xrow * 2));
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb) py[kb] = buf_load16(rdy, yo + 64 * kb);
    pa = buf_load_f32(make_rsrc(acs + kh * Q, (uint32_t)(len * 4)), (uint32_t)irow * 4u);
  };
  __syncthreads();  // every wave is done with the B pieces in ub[0]
  load_head(g * hpg);
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const int64_t kh = (int64_t)k * H + h;
    uint16_t* ht = ub[hh & 1];
    // Values that do not change from head to head are made opaque here, so that
    // the compiler forms them inside the loop: hoisted, the unpacked C values and
    // the LDS addresses of H's pieces held ~35 more registers, and the kernel
    // fitted three workgroups per CU instead of four.
    int tz = tid;
    asm volatile("" : "+v"(tz));
#pragma unroll
    for (int s = 0; s < N / 32; ++s) asm volatile("" : "+v"(cq[s]));
#pragma unroll
    for (int c = 0; c < NPH; ++c) {
      const int e = (tz + c * NT) * 8;
      if (e < P * N) lds_piece<true>(ht + (e / N) * LDB, (e % N) / 8, ph[c]);
    }
    __syncthreads();
    // this head's dy fragment scaled by 2^acs_i (one row per lane)
    const float ei = irow < len ? exp2_fast(pa) : 0.f;
    bf16x8 ays[P / 32];
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb) {
      u32x4 sv;
#pragma unroll
      for (int d = 0; d < 4; ++d) sv[d] = pack_bf2(bf_lo(py[kb][d]) * ei, bf_hi(py[kb][d]) * ei);
      ays[kb] = as_bf16x8(sv);
    }
    if (hh + 1 < hpg) load_head(h + 1);  // in flight during this head's work
    if (!active) continue;
    float rsum = 0.f;
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) {
      f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < P / 32; ++kb)
        t = mfma_bf16(frag_kmajor(ht + kb * 32 * LDB + nb * 16, LDB, lane), ays[kb], t);
      const uint32_t c0 = cq[nb >> 1][2 * (nb & 1)], c1 = cq[nb >> 1][2 * (nb & 1) + 1];
      rsum += bf_lo(c0) * t[0] + bf_hi(c0) * t[1] + bf_lo(c1) * t[2] + bf_hi(c1) * t[3];
      acc[nb] += t;
    }
    rsum += __shfl_xor(rsum, 16);
    rsum += __shfl_xor(rsum, 32);
    if (q == 0 && irow < len) rout[kh * Q + irow] = rsum;
  }
  const brsrc rdc = make_rsrc(dC + (int64_t)ci.start * brow + (int64_t)g * N, (uint32_t)(len * brow * 2));
#pragma unroll
  for (int s = 0; s < N / 32; ++s) buf_store16(rdc, ro + 64 * s, pack_bf8(acc[2 * s], acc[2 * s + 1]));
}

// ------------------------------------------------------------ bwd_db bf16 ----
// One workgroup of W waves per (chunk, group, 16 W rows j), W = 8 or 4 as for dC
// (each head's dT tile staged once per 128 rows).  dB_j = sum_{i>=j} dCB_g[i][j] C_i
// (per 64-row piece of i: the piece's C rows and its 64 x 16 W tile of dCB_g
// staged in LDS, the tile read with the transpose read, which hands each lane
// dCB_g down a column j)
// + sum_h w_j delta_j dT^T x_j (one K=headdim GEMM per head).  Per head, dT = dE_c
// (bf16) is staged in a double-buffered LDS tile and the next head's dT, x
// fragments and decay scalars are loaded into registers while this head is
// worked on.  Operands swapped and C, dT staged in the permuted column order as
// in bwd_dc: each lane owns one row j and stores dB 16 bytes at a time.
template <int P, int N, int W>
__global__ __launch_bounds__(W * 64, 4) void bwd_db_bf16_kernel(
    ChunkMap m, int H, int G, const uint16_t* __restrict__ X, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ dCBg, const float* __restrict__ delta,
    const float* __restrict__ acs, const uint16_t* __restrict__ dE, uint16_t* __restrict__ dB) {
  constexpr int LDB = N + 16;
  constexpr int ROWS = P > 64 ? P : 64;
  constexpr int NT = W * 64, RW = 16 * W;  // threads; rows per workgroup
  constexpr int NPH = (P * N / 8 + NT - 1) / NT;
  constexpr int LDT = RW + 8;  // dCB_g tile row stride (bf16)
  constexpr int UB = ROWS * LDB > 64 * LDT ? ROWS * LDB : 64 * LDT;
  __shared__ __attribute__((aligned(16))) uint16_t ub[2][UB];
  const int T = m.Q / RW;
  const int lid = xcd_order(blockIdx.x, gridDim.x);  // (chunk, group, tile), tile fastest
  const int tile = lid % T, k = lid / T / G, g = (lid / T) % G;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0 || tile * RW >= ci.len) return;
  const int Q = m.Q, len = ci.len;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, r = lane & 15;
  const int hpg = H / G;
  const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N;
  const uint16_t* cb = Cm + (int64_t)ci.start * brow + (int64_t)g * N;
  const uint16_t* dcbg = dCBg + ((int64_t)k * G + g) * Q * Q;
  const int j0 = tile * RW + w * 16;
  const bool active = j0 < len;
  const int jrow = j0 + r;
  const bool rowok = jrow < len;
  const uint32_t xo = (uint32_t)jrow * (uint32_t)(xrow * 2) + q * 16;

  f32x4 acc[N / 16];  // acc[nb][rr] = dB[jrow][pcol(nb, 4 q + rr)]
#pragma unroll
  for (int nb = 0; nb < N / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t *ct = ub[0], *dt_ = ub[1];
  for (int it = tile * RW / 64; it * 64 < len; ++it) {
    // C rows of this piece and dCB_g[it-piece rows i][this tile's columns j]
    // (rows past the chunk's end zero; the diagonal tile is zero above i = j),
    // both in flight together: one memory latency per piece
    RowTile<64, N, NT, true> ctile;
    RowTile<64, RW, NT> dtile;
    ctile.load(cb + (int64_t)it * 64 * brow, brow, len - it * 64, tid);
    dtile.load(dcbg + (int64_t)it * 64 * Q + tile * RW, Q, len - it * 64, tid);
    __syncthreads();  // every wave is done with the previous piece
    ctile.store(ct, LDB, tid);
    dtile.store(dt_, LDT, tid);
    __syncthreads();
    if (!active) continue;
    const int ib0 = max(it * 64, (j0 / 32) * 32);  // rows i >= this wave's first 32-block
    for (int ib = ib0; ib < min(it * 64 + 64, len); ib += 32) {
      // a[j][i] = dCB_g[i][j]: tile rows are k = i, the lane's column is j0 + r
      const bf16x8 a = frag_kmajor(dt_ + (ib - it * 64) * LDT + w * 16, LDT, lane);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb)
        acc[nb] = mfma_bf16(frag_kmajor(ct + (ib - it * 64) * LDB + nb * 16, LDB, lane), a, acc[nb]);
    }
  }
  u32x4 ph[NPH], px[P / 32];
  float pl = 0.f, pj = 0.f, pd = 0.f;
  auto load_head = [&](int h) {
    const int64_t kh = (int64_t)k * H + h;
    // range-checked loads, no branches (rows past the chunk's end read zero)
    const brsrc rh = make_rsrc(dE + kh * (int64_t)(P * N), (uint32_t)(P * N * 2));
#pragma unroll
    for (int c = 0; c < NPH; ++c) {
      const int e = (tid + c * NT) * 8;
      ph[c] = buf_load16(rh, e < P * N ? (uint32_t)e * 2u : 0x80000000u);
    }
    const brsrc rxh = make_rsrc(X + (int64_t)ci.start * xrow + (int64_t)h * P, (uint32_t)(len * xrow * 2));
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb) px[kb] = buf_load16(rxh, xo + 64 * kb);
    const brsrc ra = make_rsrc(acs + kh * Q, (uint32_t)(len * 4));
    pl = buf_load_f32(ra, (uint32_t)(len - 1) * 4u);
    pj = buf_load_f32(ra, (uint32_t)jrow * 4u);
    pd = buf_load_f32(make_rsrc(delta + kh * Q, (uint32_t)(len * 4)), (uint32_t)jrow * 4u);
  };
  __syncthreads();  // every wave is done with the C pieces in ub[0]
  load_head(g * hpg);
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    uint16_t* dtt = ub[hh & 1];
#pragma unroll
    for (int c = 0; c < NPH; ++c) {
      const int e = (tid + c * NT) * 8;
      if (e < P * N) lds_piece<true>(dtt + (e / N) * LDB, (e % N) / 8, ph[c]);
    }
    __syncthreads();
    // this head's x fragment scaled by w_j delta_j (one row per lane)
    const float sj = rowok ? exp2_fast(pl - pj) * pd : 0.f;
    bf16x8 axs[P / 32];
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb) {
      u32x4 sv;
#pragma unroll
      for (int d = 0; d < 4; ++d) sv[d] = pack_bf2(bf_lo(px[kb][d]) * sj, bf_hi(px[kb][d]) * sj);
      axs[kb] = as_bf16x8(sv);
    }
    if (hh + 1 < hpg) load_head(h + 1);  // in flight during this head's work
    if (!active) continue;
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb)
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb)
        acc[nb] = mfma_bf16(frag_kmajor(dtt + kb * 32 * LDB + nb * 16, LDB, lane), axs[kb], acc[nb]);
  }
  const brsrc rdb = make_rsrc(dB + (int64_t)ci.start * brow + (int64_t)g * N, (uint32_t)(len * brow * 2));
  const uint32_t bo = (uint32_t)jrow * (uint32_t)(brow * 2) + q * 16;
#pragma unroll
  for (int s = 0; s < N / 32; ++s) buf_store16(rdb, bo + 64 * s, pack_bf8(acc[2 * s], acc[2 * s + 1]));
}

// ---------------------------------------------------------------- finalize ----
// One workgroup per (chunk, 8 heads), one wavefront per head: dAcs_i = rR_i - Ks_i
// + (R, K tile partials, or whole R, K per token: Rf, Kf) (+ last_term at the last
// token); ddA_t = sum_{i>=t} dAcs_i, d(delta)_t = ddd_t + A ddA_t,
// ddt = d(delta) sigmoid(z) when softplus is on; per-chunk partial sums of
// delta*ddA and ddt.  Lane l holds four consecutive tokens, lane 0 the chunk's
// last four, so that the suffix sum is the lane's own tokens summed from its last
// plus a DPP prefix sum of the lane totals.  The per-head arrays are read four
// tokens (16 bytes) at a time.  dt is read and ddt written through LDS, eight
// adjacent heads of a token at a time: a head's values lie H floats apart, and
// read one head per workgroup, every wave instruction touched 64 cache lines.
// Every load is issued before the first wait.
constexpr int kFinHeads = 8;  // heads per workgroup, one per wavefront
__global__ __launch_bounds__(kFinHeads * 64) void bwd_finalize_kernel(
    ChunkMap m, int H, int softplus, const float* __restrict__ dt,
    const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ delta, const float* __restrict__ rR, const float* __restrict__ Ks,
    const float* __restrict__ ddd, const float* __restrict__ last_term,
    const float* __restrict__ Rp, const float* __restrict__ Kp, int ntile, int tsh,
    const float* __restrict__ Rf, const float* __restrict__ Kf, float* __restrict__ ddt,
    float* __restrict__ dAp, float* __restrict__ dbp) {
  constexpr int NT = kFinHeads * 64, NE = kFinHeads * QMAX / NT;
  __shared__ __attribute__((aligned(16))) float tk[kFinHeads][QMAX];  // dt in, then ddt out
  const int k = blockIdx.x, h0 = blockIdx.y * kFinHeads;
  const int nh = min(kFinHeads, H - h0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // this wave's head: h0 + w
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) {
    if (tid < nh) {
      dAp[(int64_t)k * H + h0 + tid] = 0.f;
      dbp[(int64_t)k * H + h0 + tid] = 0.f;
    }
    return;
  }
  const int Q = m.Q, len = ci.len;
  // dt of the workgroup's heads: element e is token e / 8, head e % 8 (range-checked
  // over the chunk's tokens; heads past H get an offset past every range)
  const brsrc rdt = make_rsrc(dt + (int64_t)ci.start * H + h0, (uint32_t)len * (uint32_t)H * 4u);
  float dtv[NE];
#pragma unroll
  for (int c = 0; c < NE; ++c) {
    const int e = tid + NT * c, t = e / kFinHeads, hh = e % kFinHeads;
    dtv[c] = buf_load_f32(rdt, (t < len && hh < nh) ? ((uint32_t)t * (uint32_t)H + hh) * 4u : 0x80000000u);
  }
  // this lane's tokens tb .. tb + 3 (lanes past the chunk size hold none), of head
  // h0 + w (waves past H load nothing)
  const bool hin = w < nh;
  const int tb = Q - 4 * (lane + 1);
  const bool lane_in = tb >= 0;
  const uint32_t o = (lane_in && hin) ? (uint32_t)tb * 4u : 0x80000000u, qb = (uint32_t)Q * 4u;
  const int tt = lane_in ? tb >> tsh : 0, tlast = (len - 1) >> tsh;
  const int64_t kh = (int64_t)k * H + h0 + (hin ? w : 0);
  auto ld4 = [&](const float* base, uint32_t bytes, uint32_t off) {
    const u32x4 v = buf_load16(make_rsrc(base, bytes), off);
    return f32x4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
  };
  const f32x4 vr = ld4(rR + kh * Q, qb, o), vk = ld4(Ks + kh * Q, qb, o);
  const f32x4 vd = ld4(delta + kh * Q, qb, o), v0 = ld4(ddd + kh * Q, qb, o);
  const f32x4 vrf = ld4(Rf ? Rf + kh * Q : rR, qb, Rf ? o : 0x80000000u);
  const f32x4 vkf = ld4(Kf ? Kf + kh * Q : Ks, qb, Kf ? o : 0x80000000u);
  // tile partials (tiles of 2^tsh tokens): R over column tiles <= the lane's, K over
  // row tiles >= it
  f32x4 vrp[4], vkp[4];
  const uint32_t tbytes = (uint32_t)(ntile * Q * 4);
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    const bool ur = tl <= tt && tl < ntile, uk = tl >= tt && tl <= tlast && tl < ntile;
    vrp[tl] = ld4(Rp + kh * ntile * Q, tbytes, ur ? o + (uint32_t)(tl * Q * 4) : 0x80000000u);
    vkp[tl] = ld4(Kp + kh * ntile * Q, tbytes, uk ? o + (uint32_t)(tl * Q * 4) : 0x80000000u);
  }
  const float lt = hin ? last_term[kh] : 0.f;
#pragma unroll
  for (int c = 0; c < NE; ++c) {
    const int e = tid + NT * c;
    tk[e % kFinHeads][e / kFinHeads] = dtv[c];
  }
  __syncthreads();
  if (hin) {  // (uniform per wave)
    const int h = h0 + w;
    const float Ah = A[h], bias = dt_bias ? dt_bias[h] : 0.f;
    const float4 zr = lane_in ? *(const float4*)&tk[w][tb] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float z_[4] = {zr.x, zr.y, zr.z, zr.w};
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tb + j;
      float a = vr[j] - vk[j] + (t == len - 1 ? lt : 0.f) + (vrf[j] - vkf[j]);
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) a += vrp[tl][j];
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) a -= vkp[tl][j];
      v[j] = (lane_in && t < len) ? a : 0.f;
    }
    // suffix sums: the lane's own tokens from its last, then the lanes before it
    // (which hold the later tokens)
    float s[4];
    s[3] = v[3];
    s[2] = v[2] + s[3];
    s[1] = v[1] + s[2];
    s[0] = v[0] + s[1];
    const float incl = wave_inclusive_sum(s[0]);
    float carry = __shfl_up(incl, 1);  // the lanes before this one (no subtraction: exact)
    carry = lane == 0 ? 0.f : carry;
    float pa = 0.f, pb = 0.f, g4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tb + j;
      const bool in = lane_in && t < len;
      const float suf = s[j] + carry;
      const float dd = v0[j] + Ah * suf;
      const float g = softplus ? dd * sigmoid_f(z_[j] + bias) : dd;
      g4[j] = in ? g : 0.f;
      pa += in ? vd[j] * suf : 0.f;
      pb += in ? g : 0.f;
    }
    if (lane_in) *(float4*)&tk[w][tb] = make_float4(g4[0], g4[1], g4[2], g4[3]);  // (own dt read above)
    pa = wave_sum(pa);
    pb = wave_sum(pb);
    if (lane == 0) {
      dAp[kh] = pa;
      dbp[kh] = pb;
    }
  }
  __syncthreads();
  // ddt, eight adjacent heads of a token at a time
  float* dtt = ddt + (int64_t)ci.start * H + h0;
#pragma unroll
  for (int c = 0; c < NE; ++c) {
    const int e = tid + NT * c, t = e / kFinHeads, hh = e % kFinHeads;
    if (t < len && hh < nh) dtt[(int64_t)t * H + hh] = tk[hh][t];
  }
}

// Fixed-order sums over chunk slots: one wavefront per head, lane l takes slots
// l, l + 64, ... in order, then a fixed DPP tree across lanes.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(int nck, int H, const float* __restrict__ dAp,
                                                         const float* __restrict__ dbp,
                                                         const float* __restrict__ dDp,
                                                         float* __restrict__ dA,
                                                         float* __restrict__ d_dt_bias,
                                                         float* __restrict__ dD) {
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (h >= H) return;
  float a = 0.f, b = 0.f, d = 0.f;
  for (int k = lane; k < nck; k += 64) {
    a += dAp[(int64_t)k * H + h];
    b += dbp[(int64_t)k * H + h];
    d += dDp[(int64_t)k * H + h];
  }
  a = wave_sum(a);
  b = wave_sum(b);
  d = wave_sum(d);
  if (lane == 0) {
    dA[h] = a;
    if (d_dt_bias) d_dt_bias[h] = b;
    if (dD) dD[h] = d;
  }
}

// ---------------------------------------------------------------- launchers ----
// The head-summed dCB on 128x128 super-tiles where the chunk size allows and the
// kernel fits its registers and LDS (headdim <= 64); 64x64 tiles otherwise.
static bool dcb_t128(const Prob& p) { return p.Q % 128 == 0 && p.P <= 64; }

template <int P, int N>
static void launch_bwd_bf16(const Prob& p, const BwdArgs& a, int which, hipStream_t st) {
  const int T = p.Q / 64;
  if (!which || which == 1)
  hipLaunchKernelGGL((bwd_dx_bf16_kernel<P, N>), dim3((unsigned)(p.nck * p.H)), dim3(kDxWaves * 64), 0, st, p.map,
                     p.H, p.G, (const uint16_t*)a.x, (const uint16_t*)a.B, (const uint16_t*)a.dout,
                     (const uint16_t*)a.CBt, a.delta, a.acs, a.decay, (const uint16_t*)a.dE, (const uint16_t*)a.Hp, a.D,
                     (uint16_t*)a.dx, a.ddd, a.Ks, a.last_term, a.dDp);
  bool t128 = false;
  if constexpr (P <= 64) {
    if ((!which || which == 2) && dcb_t128(p)) {
      const int T2 = p.Q / 128;
      hipLaunchKernelGGL((bwd_dcb_t128_bf16_kernel<P>), dim3((unsigned)(p.nck * p.G * (T2 * (T2 + 1) / 2))),
                         dim3(kT128Waves * 64), 0, st, p.map, p.H, p.G, (const uint16_t*)a.x,
                         (const uint16_t*)a.dout, (const uint16_t*)a.CB, a.delta, a.acs,
                         (uint16_t*)a.dCBg, a.Rp, a.Kp);
      t128 = true;
    }
  }
  if ((!which || which == 2) && !t128) {
    hipLaunchKernelGGL((bwd_dcb_bf16_kernel<P>), dim3((unsigned)(p.nck * p.G * (T * (T + 1) / 2))),
                       dim3(256), 0, st, p.map, p.H, p.G, (const uint16_t*)a.x,
                       (const uint16_t*)a.dout, (const uint16_t*)a.CB, a.delta, a.acs,
                       (uint16_t*)a.dCBg, a.Rp, a.Kp);
  }
  // dC and dB: 128 rows per workgroup (eight waves) where the chunk size allows
  const bool r128 = p.Q % 128 == 0;
  if ((!which || which == 3) && r128)
  hipLaunchKernelGGL((bwd_dc_bf16_kernel<P, N, 8>), dim3((unsigned)(p.nck * p.G * (p.Q / 128))), dim3(512), 0, st,
                     p.map, p.H, p.G, (const uint16_t*)a.B, (const uint16_t*)a.C,
                     (const uint16_t*)a.dout, (const uint16_t*)a.dCBg, a.acs, (const uint16_t*)a.Hp,
                     (uint16_t*)a.dC, a.rR);
  if ((!which || which == 3) && !r128)
  hipLaunchKernelGGL((bwd_dc_bf16_kernel<P, N, 4>), dim3((unsigned)(p.nck * p.G * T)), dim3(256), 0, st,
                     p.map, p.H, p.G, (const uint16_t*)a.B, (const uint16_t*)a.C,
                     (const uint16_t*)a.dout, (const uint16_t*)a.dCBg, a.acs, (const uint16_t*)a.Hp,
                     (uint16_t*)a.dC, a.rR);
  if ((!which || which == 4) && r128)
  hipLaunchKernelGGL((bwd_db_bf16_kernel<P, N, 8>), dim3((unsigned)(p.nck * p.G * (p.Q / 128))), dim3(512), 0, st,
                     p.map, p.H, p.G, (const uint16_t*)a.x, (const uint16_t*)a.C,
                     (const uint16_t*)a.dCBg, a.delta, a.acs, (const uint16_t*)a.dE, (uint16_t*)a.dB);
  if ((!which || which == 4) && !r128)
  hipLaunchKernelGGL((bwd_db_bf16_kernel<P, N, 4>), dim3((unsigned)(p.nck * p.G * T)), dim3(256), 0, st,
                     p.map, p.H, p.G, (const uint16_t*)a.x, (const uint16_t*)a.C,
                     (const uint16_t*)a.dCBg, a.delta, a.acs, (const uint16_t*)a.dE, (uint16_t*)a.dB);
}

hipError_t launch_bwd_chunk(const Prob& p, const BwdArgs& a, int which, hipStream_t st) {
  if (p.nck == 0) return hipSuccess;
  if (!bf16_kernels(p)) return launch_bwd_f32(p, a, which, st);
#define SSD_BWD_CASE(PP, NN) \
  if (p.P == PP && p.N == NN) { launch_bwd_bf16<PP, NN>(p, a, which, st); return hipGetLastError(); }
  SSD_BWD_CASE(32, 32) SSD_BWD_CASE(32, 64) SSD_BWD_CASE(32, 128)
  SSD_BWD_CASE(64, 32) SSD_BWD_CASE(64, 64) SSD_BWD_CASE(64, 128)
  SSD_BWD_CASE(128, 32) SSD_BWD_CASE(128, 64) SSD_BWD_CASE(128, 128)
#undef SSD_BWD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_finalize(const Prob& p, const BwdArgs& a, hipStream_t st, bool fused) {
  if (p.nck > 0)
    hipLaunchKernelGGL(bwd_finalize_kernel, dim3((unsigned)p.nck, (p.H + kFinHeads - 1) / kFinHeads),
                       dim3(kFinHeads * 64), 0, st,
                       p.map, p.H, p.softplus, a.dt, a.dt_bias, a.A, a.delta, a.rR, a.Ks, a.ddd,
                       a.last_term, a.Rp, a.Kp,
                       (!bf16_kernels(p) || fused) ? 0 : (dcb_t128(p) ? p.Q / 128 : p.Q / 64),
                       dcb_t128(p) ? 7 : 6,
                       fused ? a.Rp : nullptr, fused ? a.Kp : nullptr, a.ddt, a.dAp, a.dbp);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((p.H + 3) / 4), dim3(256), 0, st, (int)p.nck, p.H,
                     a.dAp, a.dbp, a.dDp, a.dA, a.d_dt_bias, a.dD);
  return hipGetLastError();
}

}  // namespace ssd
