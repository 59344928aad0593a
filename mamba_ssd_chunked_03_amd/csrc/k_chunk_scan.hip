// Stage 5 (ssd_chunk_scan): the per-chunk output
//   y_i = sum_{j<=i} CB_ij 2^(acs_i - acs_j) delta_j x_j   (intra-chunk, causal)
//       + 2^(acs_i) H_c C_i                                 (state carried in)
//       + D_h x_i,
// stored in the io dtype.  Decays only ever appear as differences of the
// within-chunk cumsum (acs_i - acs_j <= 0), so nothing overflows however long
// the chunk's total decay gets.
//
// bf16 path: one workgroup per (chunk, head), four wavefronts.  LDS holds the
// chunk's x in its natural token-major layout (16-byte copies; the MFMA
// operand, 8 consecutive tokens per lane, comes from the gfx950 transpose read
// ds_read_b64_tr_b16), H_c rounded to bf16 as [p][n], and the chunk's acs and
// delta.  Each wavefront owns 16-row blocks of the output in a snake order (w,
// 7-w, 8+w, 15-w for four waves) so the causal work is balanced.  Per row
// block, all its C and CB fragments are loaded first (one memory latency), then:
//   1. acc = C_rows . H_c^T on MFMA (K = dstate), each row scaled by 2^(acs_i);
//   2. acc += M . X where M_ij = CB_ij 2^(acs_i - acs_j) delta_j (j <= i) is
//      formed in registers from the CB fragments and packed to bf16 as the A
//      fragment; K runs only up to the row block's last token;
//   3. + D x_i and the bf16 store.
//
// fp32 path: one thread per (token, p), plain loops.
#include "internal.hpp"

namespace ssd {

template <int P, int N>
__global__ __launch_bounds__(256) void chunk_scan_bf16_kernel(
    ChunkMap m, int H, int G, const uint16_t* __restrict__ X, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ CB, const float* __restrict__ delta,
    const float* __restrict__ acs, const float* __restrict__ Hs, const float* __restrict__ D,
    uint16_t* __restrict__ Y) {
  constexpr int QMAX = 256, LDX = P + 8, HLD = N + 8;
  __shared__ __attribute__((aligned(16))) uint16_t xs[QMAX * LDX];
  __shared__ __attribute__((aligned(16))) uint16_t hs[P * HLD];
  __shared__ float sa[QMAX], sd[QMAX];

  const int k = blockIdx.x, h = blockIdx.y;
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

  for (int t = tid; t < Q; t += 256) {
    sa[t] = acs[kh * Q + t];
    sd[t] = delta[kh * Q + t];
  }
  stage_rows<QMAX, P>(xs, LDX, xb, xrow, len, tid);
  stage_state_bf16<P, N>(hs, HLD, Hs + kh * (int64_t)(P * N), tid);
  __syncthreads();

  const float Dh = D ? D[h] : 0.f;
  const int NB = Q / 16;
  for (int ii = 0; ii < NB / 4; ++ii) {
    const int rb = 4 * ii + ((ii & 1) ? (3 - w) : w);
    const int i0 = rb * 16;
    if (i0 >= len) continue;
    const int irow = i0 + r;  // the A-fragment row of this lane
    const bool rowok = irow < len;
    const int nks = (i0 + 16 + 31) / 32;  // 32-token steps covering j <= i0 + 15
    u32x4 cf[N / 32], cbf[QMAX / 32];
#pragma unroll
    for (int kb = 0; kb < N / 32; ++kb)
      cf[kb] = rowok ? *(const u32x4*)(cb + (int64_t)irow * crow + kb * 32 + q * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < QMAX / 32; ++s)
      cbf[s] = (rowok && s < nks) ? *(const u32x4*)(cbm + (int64_t)irow * Q + s * 32 + q * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
    f32x4 acc[P / 16];
#pragma unroll
    for (int tp = 0; tp < P / 16; ++tp) acc[tp] = f32x4{0.f, 0.f, 0.f, 0.f};
    // 1. state carried in: C_i . H_c^T, then scale rows by 2^acs_i
#pragma unroll
    for (int kb = 0; kb < N / 32; ++kb)
#pragma unroll
      for (int tp = 0; tp < P / 16; ++tp)
        acc[tp] = mfma_bf16(as_bf16x8(cf[kb]),
                            as_bf16x8(*(const u32x4*)(hs + (tp * 16 + r) * HLD + kb * 32 + q * 8)), acc[tp]);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int i = i0 + q * 4 + rr;
      const float e = (i < len) ? exp2_fast(sa[i]) : 0.f;
#pragma unroll
      for (int tp = 0; tp < P / 16; ++tp) acc[tp][rr] *= e;
    }
    // 2. intra-chunk causal part
    const float ai = sa[min(irow, Q - 1)];
#pragma unroll
    for (int s = 0; s < QMAX / 32; ++s) {
      if (s < nks) {
        u32x4 av;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int j0 = s * 32 + q * 8 + 2 * d;
          float v0 = bf_lo(cbf[s][d]) * exp2_fast(ai - sa[j0]) * sd[j0];
          float v1 = bf_hi(cbf[s][d]) * exp2_fast(ai - sa[j0 + 1]) * sd[j0 + 1];
          v0 = (j0 <= irow) ? v0 : 0.f;
          v1 = (j0 + 1 <= irow) ? v1 : 0.f;
          av[d] = pack_bf2(v0, v1);
        }
        const bf16x8 a = as_bf16x8(av);
#pragma unroll
        for (int tp = 0; tp < P / 16; ++tp)
          acc[tp] = mfma_bf16(a, frag_kmajor(xs + s * 32 * LDX + tp * 16, LDX, lane), acc[tp]);
      }
    }
    // 3. skip term and store
#pragma unroll
    for (int tp = 0; tp < P / 16; ++tp)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = i0 + q * 4 + rr, p = tp * 16 + r;
        if (i < len) {
          const float v = acc[tp][rr] + Dh * bf2f(xs[i * LDX + p]);
          Y[(int64_t)(ci.start + i) * xrow + (int64_t)h * P + p] = f2bf(v);
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
                             const float* delta, const float* acs, const float* passed,
                             const float* D, void* out, hipStream_t st) {
  hipLaunchKernelGGL((chunk_scan_bf16_kernel<P, N>), dim3((unsigned)p.nck, p.H), dim3(256), 0, st,
                     p.map, p.H, p.G, (const uint16_t*)x, (const uint16_t*)C, (const uint16_t*)CB,
                     delta, acs, passed, D, (uint16_t*)out);
}

hipError_t launch_chunk_scan(const Prob& p, const void* x, const void* C, const void* CB,
                             const float* delta, const float* acs, const float* passed,
                             const float* D, void* out, hipStream_t st) {
  if (p.nck == 0) return hipSuccess;
  if (p.io == 0) {
    dim3 grid((unsigned)p.nck, p.H, (p.Q * p.P + 255) / 256);
    hipLaunchKernelGGL(chunk_scan_f32_kernel, grid, dim3(256), 0, st, p.map, p.H, p.G, p.P, p.N,
                       (const float*)x, (const float*)C, (const float*)CB, delta, acs, passed, D,
                       (float*)out);
    return hipGetLastError();
  }
#define SSD_SCAN_CASE(PP, NN) \
  if (p.P == PP && p.N == NN) { launch_scan_bf16<PP, NN>(p, x, C, CB, delta, acs, passed, D, out, st); return hipGetLastError(); }
  SSD_SCAN_CASE(32, 32) SSD_SCAN_CASE(32, 64) SSD_SCAN_CASE(32, 128)
  SSD_SCAN_CASE(64, 32) SSD_SCAN_CASE(64, 64) SSD_SCAN_CASE(64, 128)
  SSD_SCAN_CASE(128, 32) SSD_SCAN_CASE(128, 64) SSD_SCAN_CASE(128, 128)
#undef SSD_SCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
