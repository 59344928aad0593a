// Stage 5 (ssd_chunk_scan): the per-chunk output
//   y_i = sum_{j<=i} CB_ij 2^(acs_i - acs_j) delta_j x_j   (intra-chunk, causal)
//       + 2^(acs_i) H_c C_i                                 (state carried in)
//       + D_h x_i,
// stored in the io dtype.  Decays only ever appear as differences of the
// within-chunk cumsum (acs_i - acs_j <= 0), so nothing overflows however long
// the chunk's total decay gets.
//
// bf16 path: one workgroup per (chunk, head), eight wavefronts.  LDS holds the
// chunk's x in its natural token-major layout (16-byte copies; the MFMA
// operand, 8 consecutive tokens per lane, comes from the gfx950 transpose read
// ds_read_b64_tr_b16), H_c rounded to bf16 as [p][n], and the chunk's acs and
// delta.  Each wavefront owns 16-row blocks of the output in a snake order (w and
// 15-w for eight waves) so the causal work is balanced.  Per row
// block, all its C and CB fragments are loaded first (one memory latency).
// Products are issued with A and B swapped, so every lane ends up owning one
// output row (one row factor per lane).  The x tile is staged with its column
// groups permuted (common.hpp, pcol), so each lane's outputs are 8 adjacent
// columns per tile pair: the skip term's x and the output go 16 bytes a lane.
// The decay 2^(acs_i - acs_j) is factored through an anchor token e with
// j <= e < i, 2^(acs_i - acs_e) * 2^(acs_e - acs_j), both factors <= 1 (acs never
// increases), so nothing can overflow.  For a row block starting in the 32-token
// block [b0, b0 + 32), every column j < b0 uses e = b0 - 1: the column factors
// 2^(acs_e - acs_j) delta_j are tabulated once per workgroup in LDS, and the row
// factor is applied to the accumulator.  Only the diagonal 32-block needs one
// exp per element.  Per row block:
//   1. acc = 2^(acs_e) C_rows . H_c^T on MFMA (K = dstate);
//   2. acc += (CB_ij * column factor) . X over the blocks before b0 (the A
//      fragment formed in registers from the CB fragments, packed to bf16);
//   3. acc *= 2^(acs_i - acs_e) per row, which also turns 1.'s factor into 2^acs_i;
//   4. acc += M . X over the diagonal block, M_ij = CB_ij 2^(acs_i - acs_j) delta_j
//      masked to j <= i;
//   5. + D x_i and the bf16 store.
// The x and H tiles are read once per workgroup and loaded nontemporally.
//
// fp32 path: one thread per (token, p), plain loops.
#include "internal.hpp"

namespace ssd {

constexpr int kScanWaves = 8;

// HT: element type of the passed states (fp32, or bf16 from the fused forward)
template <int P, int N, typename HT>
__global__ __launch_bounds__(kScanWaves * 64) void chunk_scan_bf16_kernel(
    ChunkMap m, int H, int G, const uint16_t* __restrict__ X, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ CB, const float* __restrict__ delta,
    const float* __restrict__ acs, const HT* __restrict__ Hs, const float* __restrict__ D,
    uint16_t* __restrict__ Y) {
  constexpr int QMAX = 256, LDX = P + 8, HLD = N + 8;
  __shared__ __attribute__((aligned(16))) uint16_t xs[QMAX * LDX];
  __shared__ __attribute__((aligned(16))) uint16_t hs[P * HLD];
  __shared__ float sa[QMAX], sd[QMAX];
  __shared__ __attribute__((aligned(16))) float vt[QMAX / 32][QMAX];  // column factors per anchor

  int k, h;
  chunk_head(H, k, h);
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int Q = m.Q, len = ci.len;
  const int g = h / (H / G);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, r = lane & 15;
  const int64_t kh = (int64_t)k * H + h;
  const int64_t xrow = (int64_t)H * P, crow = (int64_t)G * N;
  const uint16_t* xb = X + (int64_t)ci.start * xrow + (int64_t)h * P;
  const uint16_t* cb = Cm + (int64_t)ci.start * crow + (int64_t)g * N;
  const uint16_t* cbm = CB + ((int64_t)k * G + g) * Q * Q;

  // Row blocks of this wave (snake order), and their C / CB fragments: the next
  // row block's are loaded before the current one's stores, so the wait for
  // them does not also wait for those stores (one in-order memory counter);
  // the first row block's are in flight during the prologue.
  const int NB = Q / 16, nii = (NB + kScanWaves - 1) / kScanWaves;
  auto rb_of = [&](int ii) { return kScanWaves * ii + ((ii & 1) ? (kScanWaves - 1 - w) : w); };
  auto live = [&](int ii) { return ii < nii && rb_of(ii) < NB && rb_of(ii) * 16 < len; };
  // (the diagonal fragment has its own register: indexing the array with the
  // run-time block index would become a select over every element)
  // Buffer resources over the chunk's valid rows: rows past its end read as
  // zero and are not written.
  const brsrc rcm = make_rsrc(cb, (uint32_t)(len * crow * 2)), rcb = make_rsrc(cbm, (uint32_t)(len * Q * 2));
  const brsrc ry = make_rsrc(Y + (int64_t)ci.start * xrow + (int64_t)h * P, (uint32_t)(len * xrow * 2));
  u32x4 cf[N / 32], cbf[QMAX / 32], cbd;
  auto load_rb = [&](int rb) {
    const uint32_t irow = rb * 16 + r, nb = rb / 2;
    const uint32_t co = irow * (uint32_t)(crow * 2) + q * 16, bo = irow * (uint32_t)(Q * 2) + q * 16;
#pragma unroll
    for (int kb = 0; kb < N / 32; ++kb) cf[kb] = buf_load16(rcm, co + 64 * kb);
#pragma unroll
    for (int sx = 0; sx < QMAX / 32; ++sx)
      cbf[sx] = (sx < (int)nb) ? buf_load16(rcb, bo + 64 * sx) : u32x4{0u, 0u, 0u, 0u};
    cbd = buf_load16(rcb, bo + 64 * nb);
  };
  if (live(0)) load_rb(rb_of(0));
  {
    // every prologue load in flight before the first LDS store waits on one
    static_assert(QMAX <= kScanWaves * 64, "one acs/delta value per thread");
    const float av = tid < Q ? acs[kh * Q + tid] : 0.f, dv = tid < Q ? delta[kh * Q + tid] : 0.f;
    RowTile<QMAX, P, kScanWaves * 64, true, true> xt;
    xt.load(xb, xrow, len, tid);
    if constexpr (sizeof(HT) == 2) {
      RowTile<P, N, kScanWaves * 64, false, true> ht;
      ht.load((const uint16_t*)(Hs + kh * (int64_t)(P * N)), N, P, tid);
      xt.store(xs, LDX, tid);
      ht.store(hs, HLD, tid);
    } else {
      xt.store(xs, LDX, tid);
      stage_state_bf16<P, N, kScanWaves * 64>(hs, HLD, Hs + kh * (int64_t)(P * N), tid);
    }
    if (tid < Q) {
      sa[tid] = av;
      sd[tid] = dv;
    }
  }
  __syncthreads();
  // column factors for anchor e = 32b - 1: 2^(acs_e - acs_j) delta_j for j <= e
  for (int idx = tid; idx < (Q / 32) * Q; idx += kScanWaves * 64) {
    const int b = idx / Q, j = idx % Q;
    vt[b][j] = (b > 0 && j < 32 * b) ? exp2_fast(sa[32 * b - 1] - sa[j]) * sd[j] : 0.f;
  }
  __syncthreads();

  const float Dh = D ? D[h] : 0.f;
  for (int ii = 0; ii < nii; ++ii) {
    if (!live(ii)) continue;  // chunk sizes with fewer row blocks than wavefronts, short chunks
    const int rb = rb_of(ii);
    const int i0 = rb * 16;
    const int irow = i0 + r;  // the output row of this lane
    const bool rowok = irow < len;
    const int nb = i0 / 32;   // 32-token blocks strictly before the diagonal block
    const float ae = nb > 0 ? sa[32 * nb - 1] : 0.f;
    // The products are issued with the operands swapped, so each lane holds the
    // transposed tile: acc[tp][rr] = y[i0 + r][pcol(tp, 4 q + rr)].  A row
    // factor is then one value per lane, and acc[2s], acc[2s + 1] are the
    // lane's 8 adjacent outputs 32 s + 8 q .. +7.
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
    const float* vrow = &vt[nb][0];
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

__global__ __launch_bounds__(256) void chunk_scan_f32_kernel(
    ChunkMap m, int H, int G, int P, int N, const float* __restrict__ X,
    const float* __restrict__ Cm, const float* __restrict__ CB, const float* __restrict__ delta,
    const float* __restrict__ acs, const float* __restrict__ Hs, const float* __restrict__ D,
    float* __restrict__ Y) {
  const int k = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int Q = m.Q;
  const int o = blockIdx.z * 256 + threadIdx.x;
  const int i = o / P, p = o % P;
  if (i >= ci.len) return;
  const int g = h / (H / G);
  const int64_t kh = (int64_t)k * H + h;
  const float* ac = acs + kh * Q;
  const float* dl = delta + kh * Q;
  const float* cbr = CB + (((int64_t)k * G + g) * Q + i) * Q;
  const float ai = ac[i];
  float acc = 0.f;
  for (int j = 0; j <= i; ++j)
    acc += cbr[j] * exp2_fast(ai - ac[j]) * dl[j] * X[((int64_t)(ci.start + j) * H + h) * P + p];
  const float* crow = Cm + ((int64_t)(ci.start + i) * G + g) * N;
  const float* hrow = Hs + kh * (int64_t)(P * N) + (int64_t)p * N;
  float inter = 0.f;
  for (int n = 0; n < N; ++n) inter += crow[n] * hrow[n];
  const float xi = X[((int64_t)(ci.start + i) * H + h) * P + p];
  Y[((int64_t)(ci.start + i) * H + h) * P + p] = acc + exp2_fast(ai) * inter + (D ? D[h] : 0.f) * xi;
}

template <int P, int N>
static void launch_scan_bf16(const Prob& p, const void* x, const void* C, const void* CB,
                             const float* delta, const float* acs, const void* passed,
                             int passed_bf16, const float* D, void* out, hipStream_t st) {
  const dim3 grid((unsigned)(p.nck * p.H)), block(kScanWaves * 64);  // XCD-aware (chunk, head)
  if (passed_bf16)
    hipLaunchKernelGGL((chunk_scan_bf16_kernel<P, N, uint16_t>), grid, block, 0, st, p.map, p.H,
                       p.G, (const uint16_t*)x, (const uint16_t*)C, (const uint16_t*)CB, delta, acs,
                       (const uint16_t*)passed, D, (uint16_t*)out);
  else
    hipLaunchKernelGGL((chunk_scan_bf16_kernel<P, N, float>), grid, block, 0, st, p.map, p.H, p.G,
                       (const uint16_t*)x, (const uint16_t*)C, (const uint16_t*)CB, delta, acs,
                       (const float*)passed, D, (uint16_t*)out);
}

hipError_t launch_chunk_scan(const Prob& p, const void* x, const void* C, const void* CB,
                             const float* delta, const float* acs, const void* passed,
                             int passed_bf16, const float* D, void* out, hipStream_t st) {
  if (p.nck == 0) return hipSuccess;
  if (p.io == 0) {
    if (passed_bf16) return hipErrorInvalidValue;
    dim3 grid((unsigned)p.nck, p.H, (p.Q * p.P + 255) / 256);
    hipLaunchKernelGGL(chunk_scan_f32_kernel, grid, dim3(256), 0, st, p.map, p.H, p.G, p.P, p.N,
                       (const float*)x, (const float*)C, (const float*)CB, delta, acs, (const float*)passed, D,
                       (float*)out);
    return hipGetLastError();
  }
#define SSD_SCAN_CASE(PP, NN) \
  if (p.P == PP && p.N == NN) { launch_scan_bf16<PP, NN>(p, x, C, CB, delta, acs, passed, passed_bf16, D, out, st); return hipGetLastError(); }
  SSD_SCAN_CASE(32, 32) SSD_SCAN_CASE(32, 64) SSD_SCAN_CASE(32, 128)
  SSD_SCAN_CASE(64, 32) SSD_SCAN_CASE(64, 64) SSD_SCAN_CASE(64, 128)
  SSD_SCAN_CASE(128, 32) SSD_SCAN_CASE(128, 64) SSD_SCAN_CASE(128, 128)
#undef SSD_SCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
