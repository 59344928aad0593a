// Stage 1 (ssd_chunk_cumsum) plus the packed-sequence chunk table and a plain
// copy kernel.
//
// chunk_cumsum: delta_t = softplus(dt_t + bias_h) (or dt_t + bias_h), and the
// inclusive cumulative sum of delta_t * A_h inside each chunk, stored in log2
// units so that every later decay is a single v_exp_f32.  One workgroup per
// (chunk slot, block of 16 heads): the (tokens x 16 heads) tile of dt is loaded
// once with coalesced row reads into LDS, then each wavefront scans one head at
// a time over the chunk with the DPP wavefront prefix sum (64 tokens per pass,
// the running total carried in a register between passes).
#include "internal.hpp"

namespace ssd {

constexpr int kCumsumHeads = 16;

__global__ __launch_bounds__(256) void chunk_cumsum_kernel(ChunkMap m, int H, int softplus,
                                                           const float* __restrict__ dt,
                                                           const float* __restrict__ dt_bias,
                                                           const float* __restrict__ A,
                                                           float* __restrict__ delta,
                                                           float* __restrict__ acs,
                                                           float* __restrict__ decay) {
  __shared__ float tile[256 * (kCumsumHeads + 1)];
  const int k = blockIdx.x;
  const int h0 = blockIdx.y * kCumsumHeads;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int Q = m.Q;
  const int tid = threadIdx.x;
  {
    constexpr int NC = 256 * kCumsumHeads / 256;  // loads issued together, then stored
    float v[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int idx = tid + c * 256, t = idx / kCumsumHeads, h = h0 + idx % kCumsumHeads;
      v[c] = (t < ci.len && h < H) ? dt[(int64_t)(ci.start + t) * H + h] : 0.f;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int idx = tid + c * 256, t = idx / kCumsumHeads, hh = idx % kCumsumHeads;
      if (t < Q) tile[t * (kCumsumHeads + 1) + hh] = v[c];
    }
  }
  __syncthreads();
  const int w = tid >> 6, lane = tid & 63;
  for (int hh = w; hh < kCumsumHeads; hh += 4) {
    const int h = h0 + hh;
    if (h >= H) break;
    const float bias = dt_bias ? dt_bias[h] : 0.f;
    const float a2 = A[h] * kLog2e;
    const int64_t base = ((int64_t)k * H + h) * Q;
    float carry = 0.f;
    for (int t0 = 0; t0 < Q; t0 += 64) {
      const int t = t0 + lane;
      const bool in = t < ci.len;
      const float d = token_delta(tile[t * (kCumsumHeads + 1) + hh], bias, softplus, in);
      float incl = wave_inclusive_sum(scan_input(d, a2)) + carry;
      carry = wave_last(incl);
      delta[base + t] = d;
      acs[base + t] = in ? incl : 0.f;
      if (t == ci.len - 1) decay[(int64_t)k * H + h] = incl;
    }
  }
}

// Packed sequences: chunk table and per-sequence chunk offsets, built by one
// workgroup on the device so the host never waits for cu_seqlens.  Values are
// clamped into [0, seqlen] so a malformed cu_seqlens cannot send later kernels
// out of bounds.
__global__ __launch_bounds__(256) void build_table_kernel(const int32_t* __restrict__ cu, int nseq,
                                                          int seqlen, int Q, int nck,
                                                          int4* __restrict__ tab,
                                                          int32_t* __restrict__ seq_off) {
  __shared__ int wsum[4];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < nseq; base += 256) {
    const int s = base + tid;
    int cnt = 0;
    if (s < nseq) {
      int a = min(max(cu[s], 0), seqlen);
      int b = min(max(cu[s + 1], a), seqlen);
      cnt = (b - a + Q - 1) / Q;
    }
    float incl = wave_inclusive_sum((float)cnt);  // exact: counts stay far below 2^24
    if (lane == 63) wsum[w] = (int)incl;
    __syncthreads();
    int off = carry_s;
    for (int i = 0; i < w; ++i) off += wsum[i];
    off += (int)incl - cnt;
    if (s < nseq) seq_off[s] = min(off, nck);
    __syncthreads();
    if (tid == 0) carry_s += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  const int total = min(carry_s, nck);
  if (tid == 0) seq_off[nseq] = total;
  __syncthreads();
  for (int s = tid; s < nseq; s += 256) {
    int a = min(max(cu[s], 0), seqlen);
    int b = min(max(cu[s + 1], a), seqlen);
    int n = (b - a + Q - 1) / Q;
    int off = seq_off[s];
    for (int c = 0; c < n && off + c < nck; ++c) {
      int flags = (c == 0 ? 1 : 0) | (c == n - 1 ? 2 : 0);
      tab[off + c] = make_int4(a + c * Q, min(Q, b - a - c * Q), s, flags);
    }
  }
  for (int k = total + tid; k < nck; k += 256) tab[k] = make_int4(0, 0, 0, 0);
}

// One 16-byte piece per thread over a grid that covers the buffer: the resident
// workgroups then sweep one contiguous window of memory.  (A grid-stride loop
// over 8192 workgroups, whose threads each touch addresses far apart, reached
// 4.6 TB/s at 1 GiB; this form 6.2 TB/s.)
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

hipError_t launch_chunk_cumsum(const Prob& p, const float* dt, const float* dt_bias, const float* A,
                               float* delta, float* acs, float* decay, hipStream_t st) {
  if (p.nck == 0) return hipSuccess;
  dim3 grid((unsigned)p.nck, (p.H + kCumsumHeads - 1) / kCumsumHeads);
  hipLaunchKernelGGL(chunk_cumsum_kernel, grid, dim3(256), 0, st, p.map, p.H, p.softplus, dt,
                     dt_bias, A, delta, acs, decay);
  return hipGetLastError();
}

hipError_t launch_build_table(const Prob& p, const int32_t* cu_seqlens, int4* tab, int32_t* seq_off,
                              hipStream_t st) {
  hipLaunchKernelGGL(build_table_kernel, dim3(1), dim3(256), 0, st, cu_seqlens, p.nseq, p.L, p.Q,
                     (int)p.nck, tab, seq_off);
  return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4*)src,
                     (u32x4*)dst, n);
  return hipGetLastError();
}

}  // namespace ssd
