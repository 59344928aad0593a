// Gated RMSNorm of the Mamba-2 layer, the normalisation applied to the SSD
// output y with the gate z (aitrends.kr/articles/109906, "B200에 맞춘 Helion
// Mamba-2 커널 최적화": its backward, _layer_norm_bwd, is the layer's largest
// single kernel gain; the page prints no formula, the Mamba-2 gated RMSNorm,
// normalised after gating, is used).  Per row of D columns, groups of `group`
// columns:
//   s = z sigmoid(z) (1 without a gate), v = y s, r = (mean_group v^2 + eps)^-1/2,
//   out = v r w;
//   backward: c = sum_group w dout v, dv = r w dout - (r^3 / group) c v,
//   dy = dv s, dz = dv y sigmoid(z) (1 + z (1 - sigmoid(z))), dw = sum_rows dout v r.
//
// Layout: y, z, out, dout, dy, dz bf16 (rows, D), D fastest; w, dw fp32 (D);
// r fp32 (rows, D / group).  A row is D/8 16-byte pieces and a workgroup has
// D/8 threads, one piece each, so each load or store instruction of a wave
// covers 1 KB of the row contiguously.  A group of `group` columns is group/8
// consecutive threads: 32 lanes (group 256), one wave (512), or several waves
// (1024, 2048, or the whole row); its sums take DPP row sums, the gfx950 row
// swaps, and across waves a fixed-order sum through LDS.  Every reduction has a
// fixed order: results are bitwise reproducible.
#include "internal.hpp"

namespace ssd {

constexpr int kNormMaxWaves = 16;  // D <= 8192

// sum over the 32 lanes of each half wavefront / over the whole wavefront
__device__ __forceinline__ float half_sum32(float v) {
  v = row_sum16(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float wave_sum64(float v) {
  v = half_sum32(v);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Total over the group holding this thread's piece of per-thread partials q.
// ws: LDS scratch of kNormMaxWaves floats.
__device__ __forceinline__ float group_total(float q, int group, float* ws, int w, int lane, int nw) {
  if (group == 256) return half_sum32(q);
  const float s = wave_sum64(q);
  if (group == 512) return s;
  __syncthreads();  // earlier readers of ws are done
  if (lane == 0) ws[w] = s;
  __syncthreads();
  const int gw = group / 512 < nw ? group / 512 : nw, w0 = w / gw * gw;  // the group's waves, in order
  float t = 0.f;
  for (int u = 0; u < gw; ++u) t += ws[w0 + u];
  return t;
}

// The gate's sigmoid, 1 / (1 + exp(-z)), from the hardware base-2 exponential and
// reciprocal (exp(-|z|) = 2^(-|z| log2 e) <= 1, so nothing overflows).  Their
// error, about 1e-6 of the value here, is far below the bf16 rounding of every
// output that uses it; the library-accurate exp and an IEEE division took ~25
// VALU instructions per element and made these kernels wait on the VALU rather
// than on memory.
__device__ __forceinline__ float gate_sigmoid(float z) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(z) * 1.4426950408889634f);
  const float r = __builtin_amdgcn_rcpf(1.f + e);
  return z >= 0.f ? r : e * r;
}

__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f[2 * d] = bf_lo(v[d]);
    f[2 * d + 1] = bf_hi(v[d]);
  }
}

// kNormFwdRows rows per workgroup of D/8 threads: every row's loads are issued
// before the first is used, and w (fp32, twice a bf16 row's bytes) is read once
// for all of them instead of once per row.  Each row's arithmetic is the same
// whatever the count.  (Independent workgroups schedule better here than a
// persistent loop over rows, which was measured 10 % slower.)
constexpr int kNormFwdRows = 2;

template <bool GATE>
__global__ __launch_bounds__(1024) void gated_rmsnorm_fwd_kernel(
    int rows, int D, int group, float eps, const uint16_t* __restrict__ Y, const uint16_t* __restrict__ Z,
    const float* __restrict__ W, uint16_t* __restrict__ OUT, float* __restrict__ R) {
  constexpr int RR = kNormFwdRows;
  __shared__ float ws[kNormMaxWaves];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, nw = blockDim.x >> 6;
  const int row0 = blockIdx.x * RR, nr = min(RR, rows - row0);  // (uniform; a missing row loads the last)
  u32x4 yv[RR], zv[RR];
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    const int64_t base = (int64_t)(row0 + min(i, nr - 1)) * D;
    yv[i] = __builtin_nontemporal_load((const u32x4*)(Y + base) + tid);
    zv[i] = u32x4{0u, 0u, 0u, 0u};
    if constexpr (GATE) zv[i] = __builtin_nontemporal_load((const u32x4*)(Z + base) + tid);
  }
  const float4 w0 = ((const float4*)W)[2 * tid], w1 = ((const float4*)W)[2 * tid + 1];
  const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    float yf[8], zf[8], v[8];
    unpack8(yv[i], yf);
    unpack8(zv[i], zf);
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = GATE ? yf[e] * (zf[e] * gate_sigmoid(zf[e])) : yf[e];
      q += v[e] * v[e];
    }
    const float r = 1.f / sqrtf(group_total(q, group, ws, w, lane, nw) / (float)group + eps);
    if (i < nr) {
      const int row = row0 + i;
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[d] = pack_bf2(v[2 * d] * r * wv[2 * d], v[2 * d + 1] * r * wv[2 * d + 1]);
      ((u32x4*)(OUT + (int64_t)row * D))[tid] = o;
      if (R && (tid * 8) % group == 0) R[(int64_t)row * (D / group) + tid * 8 / group] = r;
    }
  }
}

// Workgroup b takes rows b, b + gridDim.x, ...; its per-column dw sums go to
// dwp[b] (fixed row order), reduced over workgroups by the next kernel.  The
// next row's inputs are loaded while the current row is worked on.
template <bool GATE>
__global__ __launch_bounds__(1024) void gated_rmsnorm_bwd_kernel(
    int rows, int D, int group, float eps, const uint16_t* __restrict__ DO, const uint16_t* __restrict__ Y,
    const uint16_t* __restrict__ Z, const float* __restrict__ W, uint16_t* __restrict__ DY,
    uint16_t* __restrict__ DZ, float* __restrict__ dwp) {
  __shared__ float ws[2][kNormMaxWaves];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, nw = blockDim.x >> 6;
  const float4 w0 = ((const float4*)W)[2 * tid], w1 = ((const float4*)W)[2 * tid + 1];
  const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  float dw[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) dw[e] = 0.f;
  u32x4 dov, yv, zv = u32x4{0u, 0u, 0u, 0u};
  auto load = [&](int row) {
    const int64_t base = (int64_t)row * D;
    dov = __builtin_nontemporal_load((const u32x4*)(DO + base) + tid);
    yv = __builtin_nontemporal_load((const u32x4*)(Y + base) + tid);
    if constexpr (GATE) zv = __builtin_nontemporal_load((const u32x4*)(Z + base) + tid);
  };
  if ((int)blockIdx.x < rows) load(blockIdx.x);
  for (int row = blockIdx.x; row < rows; row += gridDim.x) {
    float df[8], yf[8], zf[8];
    unpack8(dov, df);
    unpack8(yv, yf);
    unpack8(zv, zf);
    if (row + (int)gridDim.x < rows) load(row + gridDim.x);  // the inputs above are unpacked
    float v[8], sg[8], qv = 0.f, qc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sg[e] = GATE ? gate_sigmoid(zf[e]) : 1.f;
      v[e] = GATE ? yf[e] * (zf[e] * sg[e]) : yf[e];
      qv += v[e] * v[e];
      qc += (wv[e] * df[e]) * v[e];
    }
    const float tv = group_total(qv, group, ws[0], w, lane, nw);
    const float tc = group_total(qc, group, ws[1], w, lane, nw);
    const float r = 1.f / sqrtf(tv / (float)group + eps);
    const float k3 = r * r * r / (float)group * tc;
    u32x4 oy, oz;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float gy[2], gz[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * d + u;
        const float dv = r * (wv[e] * df[e]) - k3 * v[e];
        if constexpr (GATE) {
          gy[u] = dv * (zf[e] * sg[e]);
          gz[u] = dv * yf[e] * sg[e] * (1.f + zf[e] * (1.f - sg[e]));
        } else {
          gy[u] = dv;
          gz[u] = 0.f;
        }
        dw[e] += df[e] * v[e] * r;
      }
      oy[d] = pack_bf2(gy[0], gy[1]);
      oz[d] = pack_bf2(gz[0], gz[1]);
    }
    const int64_t base = (int64_t)row * D;
    ((u32x4*)(DY + base))[tid] = oy;
    if constexpr (GATE) ((u32x4*)(DZ + base))[tid] = oz;
  }
  float4* dst = (float4*)(dwp + (int64_t)blockIdx.x * D) + 2 * tid;
  dst[0] = make_float4(dw[0], dw[1], dw[2], dw[3]);
  dst[1] = make_float4(dw[4], dw[5], dw[6], dw[7]);
}

// dw[i] = sum over the nb workgroup partials dwp[b][i], in a fixed order: the
// 16 waves of a workgroup each sum one segment of consecutive b (one column per
// lane, eight loads in flight), then wave 0 adds the segments in order.
__global__ __launch_bounds__(1024) void norm_dw_reduce_kernel(int nb, int D, const float* __restrict__ dwp,
                                                              float* __restrict__ dw) {
  __shared__ float part[16][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = blockIdx.x * 64 + lane;  // D is a multiple of 64
  const int per = (nb + 15) / 16, b0 = min(nb, w * per), b1 = min(nb, b0 + per);
  float s = 0.f;
  int b = b0;
  for (; b + 8 <= b1; b += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = dwp[(int64_t)(b + u) * D + col];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += t[u];
  }
  for (; b < b1; ++b) s += dwp[(int64_t)b * D + col];
  part[w][lane] = s;
  __syncthreads();
  if (w == 0) {
    float t = 0.f;
    for (int u = 0; u < 16; ++u) t += part[u][lane];
    dw[col] = t;
  }
}

// workgroups of a backward launch: rows are spread over at most 1024 of them
int norm_bwd_blocks(int rows) { return rows < 1024 ? rows : 1024; }

hipError_t launch_gated_rmsnorm(int rows, int D, int group, float eps, const void* y, const void* z,
                                const float* w, void* out, float* r, const void* dout, void* dy, void* dz,
                                float* dwp, float* dw, bool bwd, hipStream_t st) {
  const dim3 block((unsigned)(D / 8));
  const uint16_t *Y = (const uint16_t*)y, *Z = (const uint16_t*)z;
  if (!bwd) {
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + kNormFwdRows - 1) / kNormFwdRows));
    if (z)
      hipLaunchKernelGGL((gated_rmsnorm_fwd_kernel<true>), grid, block, 0, st, rows, D, group, eps, Y, Z, w,
                         (uint16_t*)out, r);
    else
      hipLaunchKernelGGL((gated_rmsnorm_fwd_kernel<false>), grid, block, 0, st, rows, D, group, eps, Y, Z, w,
                         (uint16_t*)out, r);
    return hipGetLastError();
  }
  const int nb = norm_bwd_blocks(rows);
  if (nb > 0) {
    if (z)
      hipLaunchKernelGGL((gated_rmsnorm_bwd_kernel<true>), dim3((unsigned)nb), block, 0, st, rows, D, group, eps,
                         (const uint16_t*)dout, Y, Z, w, (uint16_t*)dy, (uint16_t*)dz, dwp);
    else
      hipLaunchKernelGGL((gated_rmsnorm_bwd_kernel<false>), dim3((unsigned)nb), block, 0, st, rows, D, group, eps,
                         (const uint16_t*)dout, Y, Z, w, (uint16_t*)dy, (uint16_t*)dz, dwp);
  }
  hipLaunchKernelGGL(norm_dw_reduce_kernel, dim3((unsigned)(D / 64)), dim3(1024), 0, st, nb, D, dwp, dw);
  return hipGetLastError();
}

}  // namespace ssd
