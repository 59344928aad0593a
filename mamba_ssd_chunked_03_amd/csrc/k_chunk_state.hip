// Stage 2 (ssd_chunk_state) and the backward's dstates contraction.
//
//   kStateFwd:     T_c[p][n] = sum_j delta_j 2^(acs_last - acs_j) x_j[p] B_j[n]
//   kStateDstates: U_c[p][n] = sum_i 2^(acs_i) dy_i[p] C_i[n]
//
// Both are one GEMM per (chunk, head): M = headdim, N = dstate, K = chunk
// tokens, with a per-token scale on the first operand.  The scan carries a
// chunk's end state into the next chunk (scan page, section 3), and this stage
// produces that chunk-local end state.
//
// bf16 path (v_mfma_f32_16x16x32_bf16).  The contraction index is the token
// index, which is the slow index of both operands in memory, while the MFMA
// wants 8 consecutive k values per lane.  Tiles of 64 tokens are therefore
// transposed on their way into LDS: each thread loads an 8x8 block (8 token
// rows x 16 bytes, coalesced across the wavefront), transposes it in registers
// and writes 8 rows of 16 bytes.  The scaled operand is split into bf16 hi +
// lo parts (two MFMAs) so the chunk state keeps ~16 bits of precision; the
// states feed the fp32 final states.  Four wavefronts, each a
// (P/2) x (N/2) tile of 16x16 blocks.
//
// fp32 path: one thread per output element, plain FMA loop (correctness path
// for fp32 inputs; no rounding of any operand).
#include "internal.hpp"

namespace ssd {

// 8x8 transpose of bf16 values: in[r] holds row r (element c in dword c/2,
// half c&1); out[c] holds column c (element r at position r).
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = in[2 * k][c >> 1], b = in[2 * k + 1][c >> 1];
      out[c][k] = (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
  }
}

__device__ __forceinline__ float token_scale(int mode, const float* dl, const float* ac, int j,
                                             float a_last) {
  return mode == kStateFwd ? dl[j] * exp2_fast(a_last - ac[j]) : exp2_fast(ac[j]);
}

template <int P, int N>
__global__ __launch_bounds__(256) void chunk_state_bf16_kernel(ChunkMap m, int H, int G, int mode,
                                                               const uint16_t* __restrict__ X,
                                                               const uint16_t* __restrict__ Y,
                                                               const float* __restrict__ delta,
                                                               const float* __restrict__ acs,
                                                               float* __restrict__ out) {
  constexpr int KS = 64;       // tokens per LDS slice
  constexpr int LD = KS + 8;   // padded row (bf16): b128 reads of 8 rows hit distinct banks
  constexpr int WM = 2, WN = 2;
  constexpr int TM = P / 16 / WM, TN = N / 16 / WN;
  static_assert(TM >= 1 && TN >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t xh[P * LD];
  __shared__ __attribute__((aligned(16))) uint16_t xl[P * LD];
  __shared__ __attribute__((aligned(16))) uint16_t ys[N * LD];
  __shared__ float sc[256];

  const int k = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int Q = m.Q;
  const int g = h / (H / G);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t kh = (int64_t)k * H + h;
  {
    const float* dl = delta + kh * Q;
    const float* ac = acs + kh * Q;
    const float a_last = ac[ci.len - 1];
    for (int t = tid; t < Q; t += 256) sc[t] = (t < ci.len) ? token_scale(mode, dl, ac, t, a_last) : 0.f;
  }
  const int64_t xrow = (int64_t)H * P, yrow = (int64_t)G * N;
  const uint16_t* xb = X + (int64_t)ci.start * xrow + (int64_t)h * P;
  const uint16_t* yb = Y + (int64_t)ci.start * yrow + (int64_t)g * N;

  const int wm = w / WN, wn = w % WN;
  const int p0 = wm * (P / WM), n0 = wn * (N / WN);
  const int q = lane >> 4, r = lane & 15;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NBX = (KS / 8) * (P / 8), NBY = (KS / 8) * (N / 8);
  __syncthreads();
  for (int s0 = 0; s0 < ci.len; s0 += KS) {
    for (int bidx = tid; bidx < NBX + NBY; bidx += 256) {
      const bool isx = bidx < NBX;
      const int bb = isx ? bidx : bidx - NBX;
      const int jb = bb % (KS / 8), cb = bb / (KS / 8);
      u32x4 rows[8], cols[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int j = s0 + jb * 8 + rr;
        if (j < ci.len)
          rows[rr] = isx ? *(const u32x4*)(xb + (int64_t)j * xrow + cb * 8)
                         : *(const u32x4*)(yb + (int64_t)j * yrow + cb * 8);
        else
          rows[rr] = u32x4{0u, 0u, 0u, 0u};
      }
      if (isx) {
        u32x4 lo[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const float s = sc[s0 + jb * 8 + rr];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const float v0 = bf_lo(rows[rr][d]) * s, v1 = bf_hi(rows[rr][d]) * s;
            const uint32_t hi = pack_bf2(v0, v1);
            rows[rr][d] = hi;
            lo[rr][d] = pack_bf2(v0 - bf_lo(hi), v1 - bf_hi(hi));
          }
        }
        transpose8x8(rows, cols);
#pragma unroll
        for (int c = 0; c < 8; ++c) *(u32x4*)(xh + (cb * 8 + c) * LD + jb * 8) = cols[c];
        transpose8x8(lo, cols);
#pragma unroll
        for (int c = 0; c < 8; ++c) *(u32x4*)(xl + (cb * 8 + c) * LD + jb * 8) = cols[c];
      } else {
        transpose8x8(rows, cols);
#pragma unroll
        for (int c = 0; c < 8; ++c) *(u32x4*)(ys + (cb * 8 + c) * LD + jb * 8) = cols[c];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS; kk += 32) {
      bf16x8 ah[TM], al[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        ah[i] = as_bf16x8(*(const u32x4*)(xh + (p0 + i * 16 + r) * LD + kk + q * 8));
        al[i] = as_bf16x8(*(const u32x4*)(xl + (p0 + i * 16 + r) * LD + kk + q * 8));
      }
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
        bv[jj] = as_bf16x8(*(const u32x4*)(ys + (n0 + jj * 16 + r) * LD + kk + q * 8));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) {
          acc[i][jj] = mfma_bf16(ah[i], bv[jj], acc[i][jj]);
          acc[i][jj] = mfma_bf16(al[i], bv[jj], acc[i][jj]);
        }
    }
    __syncthreads();
  }
  float* ob = out + kh * (int64_t)(P * N);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jj = 0; jj < TN; ++jj)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        ob[(p0 + i * 16 + q * 4 + rr) * N + n0 + jj * 16 + r] = acc[i][jj][rr];
}

// fp32: grid (chunk, head, output blocks of 256 elements)
__global__ __launch_bounds__(256) void chunk_state_f32_kernel(ChunkMap m, int H, int G, int P,
                                                              int N, int mode,
                                                              const float* __restrict__ X,
                                                              const float* __restrict__ Y,
                                                              const float* __restrict__ delta,
                                                              const float* __restrict__ acs,
                                                              float* __restrict__ out) {
  const int k = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int o = blockIdx.z * 256 + threadIdx.x;
  if (o >= P * N) return;
  const int p = o / N, n = o % N;
  const int g = h / (H / G);
  const int Q = m.Q;
  const int64_t kh = (int64_t)k * H + h;
  const float* dl = delta + kh * Q;
  const float* ac = acs + kh * Q;
  const float a_last = ac[ci.len - 1];
  float acc = 0.f;
  for (int j = 0; j < ci.len; ++j) {
    const int64_t t = ci.start + j;
    acc += token_scale(mode, dl, ac, j, a_last) * X[(t * H + h) * P + p] * Y[(t * G + g) * N + n];
  }
  out[kh * (int64_t)(P * N) + o] = acc;
}

template <int P, int N>
static void launch_cs_bf16(const Prob& p, const void* X, const void* Y, const float* delta,
                           const float* acs, float* out, int mode, hipStream_t st) {
  hipLaunchKernelGGL((chunk_state_bf16_kernel<P, N>), dim3((unsigned)p.nck, p.H), dim3(256), 0, st,
                     p.map, p.H, p.G, mode, (const uint16_t*)X, (const uint16_t*)Y, delta, acs, out);
}

hipError_t launch_chunk_state(const Prob& p, const void* X, const void* Y, const float* delta,
                              const float* acs, float* out, int mode, hipStream_t st) {
  if (p.nck == 0) return hipSuccess;
  if (p.io == 0) {
    dim3 grid((unsigned)p.nck, p.H, (p.P * p.N + 255) / 256);
    hipLaunchKernelGGL(chunk_state_f32_kernel, grid, dim3(256), 0, st, p.map, p.H, p.G, p.P, p.N,
                       mode, (const float*)X, (const float*)Y, delta, acs, out);
    return hipGetLastError();
  }
#define SSD_CS_CASE(PP, NN) \
  if (p.P == PP && p.N == NN) { launch_cs_bf16<PP, NN>(p, X, Y, delta, acs, out, mode, st); return hipGetLastError(); }
  SSD_CS_CASE(32, 32) SSD_CS_CASE(32, 64) SSD_CS_CASE(32, 128)
  SSD_CS_CASE(64, 32) SSD_CS_CASE(64, 64) SSD_CS_CASE(64, 128)
  SSD_CS_CASE(128, 32) SSD_CS_CASE(128, 64) SSD_CS_CASE(128, 128)
#undef SSD_CS_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
