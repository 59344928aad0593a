// The fp32 path of every matrix stage, forward and backward: true fp32 products
// on the fp32 matrix cores (v_mfma_f32_16x16x4f32: D(16x16) += A(16x4) B(4x16))
// with fp32 accumulation.  No operand is rounded to bf16 or a reduced fp32 format,
// so the path keeps fp32 accuracy (the stages and equations are those of the
// bf16 path, see k_chunk_state.hip, k_chunk_scan.hip and k_bwd.hip).
//
// Operand fragments come straight from global memory through the caches, with
// no LDS staging.  For an MFMA operand X[m][k] (lane (r, q) = lane % 16, lane /
// 16 supplies m = r, k = q):
//   - if X's rows run along k (k contiguous), lane (r, q) loads 16 bytes,
//     X[m0 + r][k0 + 4q .. 4q + 3], and element s of them serves k-step s;
//   - if they run along m, lane (r, q) loads X[k0 + 4q + s][m0 + r] for k-step s
//     (64 contiguous bytes per 16 lanes).
// Both orders give k-step s the K indices k0 + 4q + s, q = 0..3, so the two
// operands of every product agree on K whichever way each is stored.  Rows past
// a chunk's end read as zero through range-checked buffer resources, and stores
// there are dropped; every per-element decay factor is selected away (not
// multiplied by zero) where its indices fall outside the causal, in-chunk range,
// so an overflowing exp never reaches a sum.
//
// Kernels (workgroups of four wavefronts):
//   chunk_state   (chunk, head)       T or U: output tiles split over the waves
//   bmm_chunk     (chunk, group, 64 rows)   C.B^T, lower triangle
//   scan_rows     (chunk, head)       y (chunk scan) or r_i + R_i (backward);
//                                     16-row blocks, the waves in snake order
//   bwd_dx        (chunk, head)       dx, direct d(delta), K_j + s_j, dD and
//                                     alpha <dE, H> + sum s per chunk
//   bwd_dcb       (chunk, group, causal 64x64 tile)   head-summed dCB_g, zero above
//                                     the diagonal
//   bwd_dc/db     (chunk, group, 16 rows)   dC, dB; the waves split dstate
// Every sum over heads, lanes and waves has a fixed order: results are bitwise
// reproducible.
#include "internal.hpp"

namespace ssd {

namespace {

__device__ __forceinline__ f32x4 ld4(brsrc rs, uint32_t off) { return __builtin_bit_cast(f32x4, buf_load16(rs, off)); }
__device__ __forceinline__ void st1(brsrc rs, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, 0);
}

// V consecutive floats (V = 1, 2 or 4) in one load or store
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
template <int V>
__device__ __forceinline__ void ldv(brsrc rs, uint32_t off, float (&o)[V]) {
  if constexpr (V == 4) {
    const f32x4 t = ld4(rs, off);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = t[i];
  } else if constexpr (V == 2) {
    const u32x2v t = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    o[0] = __uint_as_float(t[0]);
    o[1] = __uint_as_float(t[1]);
  } else {
    o[0] = buf_load_f32(rs, off);
  }
}
template <int V>
__device__ __forceinline__ void stv(brsrc rs, uint32_t off, const float (&o)[V]) {
  if constexpr (V == 4) {
    buf_store16(rs, off, u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])});
  } else if constexpr (V == 2) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2v{__float_as_uint(o[0]), __float_as_uint(o[1])}, rs, off, 0, 0);
  } else {
    st1(rs, off, o[0]);
  }
}

// Permuted output columns.  A row of W = 16 T values (T tiles of 16 columns) is
// split into groups of V tiles (V = min(4, T)); tile c V + t of group c holds the
// columns 16 V c + V r + t, r = 0..15.  Lane r of a row then owns V consecutive
// columns, 16 V c + V r .. + V - 1, one per tile of the group: the operand that
// runs along those columns is loaded, and the output stored, V values a lane.
template <int T>
struct ColGroups {
  static constexpr int V = T < 4 ? T : 4, NG = T / V;
  // first column of lane r in group c
  static __device__ __forceinline__ int col0(int c, int r) { return 16 * V * c + V * r; }
};

}  // namespace

// ------------------------------------------------------------ chunk states ----
// out[p][n] = sum_j s_j X_j[p] Y_j[n] per (chunk, head):
//   kStateFwd:     X = x, Y = B, s_j = delta_j 2^(acs_last - acs_j)  (T_c)
//   kStateDstates: X = dy, Y = C, s_j = 2^(acs_j)                    (U_c)
// Products D[n][p] (A = s_j Y_j[n], B = X_j[p]).  The waves split the output
// tiles along p first (WP waves), then along n (WN), each taking a contiguous run
// of tiles; inside a run the columns are permuted in groups (ColGroups), so each
// token's Y and X values come 4 (or 2) to a load and a lane's outputs of one p
// are consecutive n: vector stores.
template <int P, int N>
__global__ __launch_bounds__(256) void chunk_state_f32_kernel(ChunkMap m, int H, int G, int mode,
                                                              const float* __restrict__ X,
                                                              const float* __restrict__ Y,
                                                              const float* __restrict__ delta,
                                                              const float* __restrict__ acs,
                                                              float* __restrict__ out) {
  constexpr int PT = P / 16, NT = N / 16;
  constexpr int WP = PT < 4 ? PT : 4;
  constexpr int WN = NT < 4 / WP ? NT : 4 / WP;
  constexpr int PTW = PT / WP, NTW = NT / WN;
  using CP = ColGroups<PTW>;
  using CN = ColGroups<NTW>;
  __shared__ float ss[256];
  int k, h;
  chunk_head(H, k, h);
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int Q = m.Q, len = ci.len, g = h / (H / G);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int64_t kh = (int64_t)k * H + h;
  const float a_last = acs[kh * Q + len - 1];
  for (int j = tid; j < Q; j += 256) {
    float s = 0.f;
    if (j < len)
      s = mode == kStateFwd ? delta[kh * Q + j] * exp2_fast(a_last - acs[kh * Q + j]) : exp2_fast(acs[kh * Q + j]);
    ss[j] = s;
  }
  __syncthreads();
  if (w >= WP * WN) return;
  const int wp = w % WP, wn = w / WP;
  const int pb = wp * PTW * 16, nb = wn * NTW * 16;  // this wave's first p and n
  const uint32_t xrow = (uint32_t)(H * P) * 4u, yrow = (uint32_t)(G * N) * 4u;
  const brsrc rx = make_rsrc(X + (int64_t)ci.start * H * P + (int64_t)h * P, (uint32_t)len * xrow);
  const brsrc ry = make_rsrc(Y + (int64_t)ci.start * G * N + (int64_t)g * N, (uint32_t)len * yrow);
  f32x4 acc[NTW][PTW];
#pragma unroll
  for (int u = 0; u < NTW; ++u)
#pragma unroll
    for (int v = 0; v < PTW; ++v) acc[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < len; j0 += 4) {
    const int j = j0 + q;  // <= Q - 1: j0 < len <= Q, both multiples of 4
    const float s = ss[j];
    float a[CN::NG][CN::V], b[CP::NG][CP::V];
#pragma unroll
    for (int c = 0; c < CN::NG; ++c) ldv<CN::V>(ry, (uint32_t)j * yrow + (uint32_t)(nb + CN::col0(c, r)) * 4u, a[c]);
#pragma unroll
    for (int c = 0; c < CP::NG; ++c) ldv<CP::V>(rx, (uint32_t)j * xrow + (uint32_t)(pb + CP::col0(c, r)) * 4u, b[c]);
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
      for (int v = 0; v < PTW; ++v)
        acc[u][v] = mfma_f32(a[u / CN::V][u % CN::V] * s, b[v / CP::V][v % CP::V], acc[u][v]);
  }
  // tile (u, v), element e: n = nb + 16 V c + V (4q + e) + t (u = c V + t), p = pb + col of lane r in v
  float* ob = out + kh * (int64_t)(P * N);
  const brsrc ro = make_rsrc(ob, (uint32_t)(P * N) * 4u);
#pragma unroll
  for (int v = 0; v < PTW; ++v) {
    const int p = pb + CP::col0(v / CP::V, r) + v % CP::V;
#pragma unroll
    for (int c = 0; c < CN::NG; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float o[CN::V];
#pragma unroll
        for (int t = 0; t < CN::V; ++t) o[t] = acc[c * CN::V + t][v][e];
        stv<CN::V>(ro, (uint32_t)(p * N + nb + 16 * CN::V * c + CN::V * (4 * q + e)) * 4u, o);
      }
  }
}

// ------------------------------------------------------------------ C.B^T ----
// CB[i][j] = C_i . B_j for j <= i < len; nothing else is written.  Wave w owns
// rows 16w .. 16w + 15 of the 64-row block and takes its column tiles up to the
// diagonal four at a time; both operands run along dstate (16-byte loads).
__global__ __launch_bounds__(256) void bmm_chunk_f32_kernel(ChunkMap m, int G, int N,
                                                            const float* __restrict__ Bm,
                                                            const float* __restrict__ Cm,
                                                            float* __restrict__ CB) {
  const int Q = m.Q, T = Q / 64;
  const int lid = xcd_order(blockIdx.x, gridDim.x);  // (chunk, group, row block), row block fastest
  const int ti = lid % T, g = (lid / T) % G, k = lid / T / G;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int len = ci.len;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int i0 = ti * 64 + 16 * w;
  if (i0 >= len) return;
  const uint32_t row = (uint32_t)(G * N) * 4u;
  const int64_t base = (int64_t)ci.start * G * N + (int64_t)g * N;
  const brsrc rc = make_rsrc(Cm + base, (uint32_t)len * row), rb = make_rsrc(Bm + base, (uint32_t)len * row);
  const brsrc ro = make_rsrc(CB + ((int64_t)k * G + g) * Q * Q, (uint32_t)(Q * Q) * 4u);
  const int njt = i0 / 16 + 1;  // column tiles up to the diagonal one
  for (int jt0 = 0; jt0 < njt; jt0 += 4) {
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int n0 = 0; n0 < N; n0 += 16) {
      const f32x4 cv = ld4(rc, (uint32_t)(i0 + r) * row + (uint32_t)(n0 + 4 * q) * 4u);
      f32x4 bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) bv[u] = ld4(rb, (uint32_t)((jt0 + u) * 16 + r) * row + (uint32_t)(n0 + 4 * q) * 4u);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = mfma_f32(cv[s], bv[u][s], acc[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 4 * q + e, j = (jt0 + u) * 16 + r;
        if (jt0 + u < njt && j <= i && i < len) st1(ro, (uint32_t)(i * Q + j) * 4u, acc[u][e]);
      }
  }
}

// ---------------------------------------------------- output rows (scan, r+R) ----
// Per (chunk, head) and 16-row block of tokens i, the chunk scan's bracket
//   acc_i[p] = 2^(acs_i) (H_c C_i)[p] + sum_{j<=i} CB_ij 2^(acs_i - acs_j) delta_j x_j[p]
// then either (RR false) y_i = acc_i + D x_i, or (RR true) the backward's
//   r_i + R_i = dy_i . (acc_i - CB_ii delta_i x_i),
// the state term's r_i and R_i = sum_{j<i} (dy_i . x_j) CB_ij L_ij delta_j together.
// Products D[i][p]: A = 2^(acs_i) C_i (16-byte loads along dstate) or the decayed
// C.B^T row (16-byte loads along j), B = H_c[p] (16-byte loads along dstate) or
// x_j[p], whose headdim columns are permuted in groups (ColGroups): a lane loads
// its x, dy and y values 16 bytes at a time.  Row blocks in snake order over the
// four waves.
template <int P, bool RR>
__global__ __launch_bounds__(256) void scan_rows_f32_kernel(
    ChunkMap m, int H, int G, int N, const float* __restrict__ X, const float* __restrict__ Cm,
    const float* __restrict__ CB, const float* __restrict__ delta, const float* __restrict__ acs,
    const float* __restrict__ Hs, const float* __restrict__ D, float* __restrict__ Y,
    const float* __restrict__ DY, float* __restrict__ rR) {
  constexpr int PT = P / 16;
  using CG = ColGroups<PT>;
  constexpr int V = CG::V, NG = CG::NG;
  __shared__ float sa[256], sd[256];
  int k, h;
  chunk_head(H, k, h);
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int Q = m.Q, len = ci.len, g = h / (H / G);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int64_t kh = (int64_t)k * H + h;
  for (int t = tid; t < Q; t += 256) {
    sa[t] = acs[kh * Q + t];
    sd[t] = delta[kh * Q + t];
  }
  __syncthreads();
  const uint32_t xrow = (uint32_t)(H * P) * 4u, crow = (uint32_t)(G * N) * 4u, qrow = (uint32_t)Q * 4u;
  const int64_t xb = (int64_t)ci.start * H * P + (int64_t)h * P;
  const brsrc rx = make_rsrc(X + xb, (uint32_t)len * xrow);
  const brsrc rdy = make_rsrc(RR ? DY + xb : X + xb, (uint32_t)len * xrow);
  const brsrc ry = make_rsrc(RR ? nullptr : Y + xb, RR ? 0u : (uint32_t)len * xrow);
  const brsrc rc = make_rsrc(Cm + (int64_t)ci.start * G * N + (int64_t)g * N, (uint32_t)len * crow);
  const brsrc rcb = make_rsrc(CB + ((int64_t)k * G + g) * Q * Q, (uint32_t)Q * qrow);
  const brsrc rh = make_rsrc(Hs + kh * (int64_t)(P * N), (uint32_t)(P * N) * 4u);
  const float Dh = (!RR && D) ? D[h] : 0.f;
  const int NB = Q / 16;
  for (int ii = 0; ii * 4 < NB; ++ii) {
    const int rb = 4 * ii + ((ii & 1) ? 3 - w : w);
    const int i0 = rb * 16;
    if (i0 >= len) continue;
    const int ir = i0 + r;  // this lane's row of the A operands (< Q)
    f32x4 acc[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the state carried in
    const float sc = ir < len ? exp2_fast(sa[ir]) : 0.f;
    for (int n0 = 0; n0 < N; n0 += 16) {
      const f32x4 cv = ld4(rc, (uint32_t)ir * crow + (uint32_t)(n0 + 4 * q) * 4u) * sc;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const int p = CG::col0(pt / V, r) + pt % V;
        const f32x4 hv = ld4(rh, (uint32_t)(p * N + n0 + 4 * q) * 4u);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[pt] = mfma_f32(cv[s], hv[s], acc[pt]);
      }
    }
    // the chunk's earlier tokens and the diagonal block
    const float ai = sa[ir];
    for (int j0 = 0; j0 <= i0; j0 += 16) {
      const f32x4 cb = ld4(rcb, (uint32_t)ir * qrow + (uint32_t)(j0 + 4 * q) * 4u);
      float mv[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int j = j0 + 4 * q + s;
        const float v = cb[s] * exp2_fast(ai - sa[j]) * sd[j];
        mv[s] = (j <= ir && ir < len) ? v : 0.f;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int c = 0; c < NG; ++c) {
          float xv[V];
          ldv<V>(rx, (uint32_t)(j0 + 4 * q + s) * xrow + (uint32_t)CG::col0(c, r) * 4u, xv);
#pragma unroll
          for (int t = 0; t < V; ++t) acc[c * V + t] = mfma_f32(mv[s], xv[t], acc[c * V + t]);
        }
    }
    // lane (r, q) holds rows i0 + 4q + e, columns col0(c, r) + t of tile c V + t
    if constexpr (!RR) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t io = (uint32_t)(i0 + 4 * q + e) * xrow;
#pragma unroll
        for (int c = 0; c < NG; ++c) {
          const uint32_t o = io + (uint32_t)CG::col0(c, r) * 4u;
          float xv[V], yv[V];
          ldv<V>(rx, o, xv);
#pragma unroll
          for (int t = 0; t < V; ++t) yv[t] = acc[c * V + t][e] + Dh * xv[t];
          stv<V>(ry, o, yv);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 4 * q + e;
        const uint32_t io = (uint32_t)i * xrow;
        float ya = 0.f, yx = 0.f;
#pragma unroll
        for (int c = 0; c < NG; ++c) {
          const uint32_t o = io + (uint32_t)CG::col0(c, r) * 4u;
          float dyv[V], xv[V];
          ldv<V>(rdy, o, dyv);
          ldv<V>(rx, o, xv);
#pragma unroll
          for (int t = 0; t < V; ++t) {
            ya += dyv[t] * acc[c * V + t][e];
            yx += dyv[t] * xv[t];
          }
        }
        const float mii = i < len ? buf_load_f32(rcb, (uint32_t)i * qrow + (uint32_t)i * 4u) * sd[i] : 0.f;
        const float v = row_sum16(ya) - mii * row_sum16(yx);
        if (r == 0 && i < len) rR[kh * Q + i] = v;
      }
    }
  }
}

// ------------------------------------------------------------------ bwd dx ----
// Per (chunk, head) and 16-row block of tokens j, the bracket
//   U_j[p] = w_j (dT B_j)[p] + sum_{i>=j} CB_ij 2^(acs_i - acs_j) dy_i[p],  w_j = 2^(acs_last - acs_j)
// (A = w_j B_j, 16-byte loads along dstate, with B = dE_c[p], 16-byte loads; then
// A = the decayed C.B^T column j, 4-byte loads along j, with B = dy_i[p], headdim
// columns permuted in groups as in the rows kernel above), and
//   dx_j = delta_j U_j + D dy_j,  d(delta)_j direct = x_j . U_j,
//   K_j + s_j = delta_j (x_j . U_j - (x_j . dy_j) CB_jj)   (s_j = delta_j x_j . w_j dT B_j),
// dD's per-chunk part sum_j x_j . dy_j and alpha <dE, H> + sum_j s_j per chunk.
template <int P>
__global__ __launch_bounds__(256) void bwd_dx_f32_kernel(
    ChunkMap m, int H, int G, int N, const float* __restrict__ X, const float* __restrict__ Bm,
    const float* __restrict__ DY, const float* __restrict__ CB, const float* __restrict__ delta,
    const float* __restrict__ acs, const float* __restrict__ decay, const float* __restrict__ dE,
    const float* __restrict__ Hs, const float* __restrict__ D, float* __restrict__ DX,
    float* __restrict__ ddd, float* __restrict__ Ks, float* __restrict__ last_term,
    float* __restrict__ dDp) {
  constexpr int PT = P / 16;
  using CG = ColGroups<PT>;
  constexpr int V = CG::V, NG = CG::NG;
  __shared__ float sa[256], sd[256];
  __shared__ float red[3][4];
  int k, h;
  chunk_head(H, k, h);
  const ChunkInfo ci = chunk_info(m, k);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int64_t kh = (int64_t)k * H + h;
  if (ci.len <= 0) {
    if (tid == 0) {
      last_term[kh] = 0.f;
      dDp[kh] = 0.f;
    }
    return;
  }
  const int Q = m.Q, len = ci.len, g = h / (H / G);
  for (int t = tid; t < Q; t += 256) {
    sa[t] = acs[kh * Q + t];
    sd[t] = delta[kh * Q + t];
  }
  // <dE, H>: this thread's 16-byte pieces in order
  const brsrc rde = make_rsrc(dE + kh * (int64_t)(P * N), (uint32_t)(P * N) * 4u);
  const brsrc rhh = make_rsrc(Hs + kh * (int64_t)(P * N), (uint32_t)(P * N) * 4u);
  float dot = 0.f;
  for (int e = tid * 4; e < P * N; e += 1024) {
    const f32x4 a = ld4(rde, (uint32_t)e * 4u), b = ld4(rhh, (uint32_t)e * 4u);
    dot += a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
  }
  __syncthreads();
  const uint32_t xrow = (uint32_t)(H * P) * 4u, brow = (uint32_t)(G * N) * 4u, qrow = (uint32_t)Q * 4u;
  const int64_t xb = (int64_t)ci.start * H * P + (int64_t)h * P;
  const brsrc rx = make_rsrc(X + xb, (uint32_t)len * xrow), rdy = make_rsrc(DY + xb, (uint32_t)len * xrow);
  const brsrc rdx = make_rsrc(DX + xb, (uint32_t)len * xrow);
  const brsrc rb = make_rsrc(Bm + (int64_t)ci.start * G * N + (int64_t)g * N, (uint32_t)len * brow);
  const brsrc rcb = make_rsrc(CB + ((int64_t)k * G + g) * Q * Q, (uint32_t)Q * qrow);
  const float Dh = D ? D[h] : 0.f;
  const float a_last = sa[len - 1];
  float s_sum = 0.f, dxx_sum = 0.f;
  const int NB = Q / 16;
  for (int ii = 0; ii * 4 < NB; ++ii) {
    const int rb_ = 4 * ii + ((ii & 1) ? 3 - w : w);
    const int j0 = rb_ * 16;
    if (j0 >= len) continue;
    const int jr = j0 + r;  // this lane's row of the A operands (< Q)
    f32x4 acc[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // state part w_j dT B_j
    const float wj = jr < len ? exp2_fast(a_last - sa[jr]) : 0.f;
    for (int n0 = 0; n0 < N; n0 += 16) {
      const f32x4 bv = ld4(rb, (uint32_t)jr * brow + (uint32_t)(n0 + 4 * q) * 4u) * wj;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const int p = CG::col0(pt / V, r) + pt % V;
        const f32x4 ev = ld4(rde, (uint32_t)(p * N + n0 + 4 * q) * 4u);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[pt] = mfma_f32(bv[s], ev[s], acc[pt]);
      }
    }
    // x_j . (state part), rows j0 + 4q + e
    float xs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t jo = (uint32_t)(j0 + 4 * q + e) * xrow;
      float v = 0.f;
#pragma unroll
      for (int c = 0; c < NG; ++c) {
        float xv[V];
        ldv<V>(rx, jo + (uint32_t)CG::col0(c, r) * 4u, xv);
#pragma unroll
        for (int t = 0; t < V; ++t) v += xv[t] * acc[c * V + t][e];
      }
      xs[e] = v;
    }
    // later tokens of the chunk: i >= j
    const float aj = sa[jr];
    for (int i0 = j0; i0 < len; i0 += 16) {
      float mv[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int i = i0 + 4 * q + s;  // < Q: i0 < len <= Q, both multiples of 16
        const float v = buf_load_f32(rcb, (uint32_t)i * qrow + (uint32_t)jr * 4u) * exp2_fast(sa[i] - aj);
        mv[s] = (i >= jr && i < len) ? v : 0.f;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int c = 0; c < NG; ++c) {
          float yv[V];
          ldv<V>(rdy, (uint32_t)(i0 + 4 * q + s) * xrow + (uint32_t)CG::col0(c, r) * 4u, yv);
#pragma unroll
          for (int t = 0; t < V; ++t) acc[c * V + t] = mfma_f32(mv[s], yv[t], acc[c * V + t]);
        }
    }
    // dx, and the per-row dots
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + 4 * q + e;
      const float dj = sd[j];
      const uint32_t jo = (uint32_t)j * xrow;
      float xt = 0.f, dxx = 0.f;
#pragma unroll
      for (int c = 0; c < NG; ++c) {
        const uint32_t o = jo + (uint32_t)CG::col0(c, r) * 4u;
        float xv[V], yv[V], ov[V];
        ldv<V>(rx, o, xv);
        ldv<V>(rdy, o, yv);
#pragma unroll
        for (int t = 0; t < V; ++t) {
          const float a = acc[c * V + t][e];
          xt += xv[t] * a;
          dxx += xv[t] * yv[t];
          ov[t] = dj * a + Dh * yv[t];
        }
        stv<V>(rdx, o, ov);
      }
      xt = row_sum16(xt);
      dxx = row_sum16(dxx);
      const float x_s = row_sum16(xs[e]);
      if (r == 0 && j < len) {
        const float cbjj = buf_load_f32(rcb, (uint32_t)j * qrow + (uint32_t)j * 4u);
        ddd[kh * Q + j] = xt;
        Ks[kh * Q + j] = dj * (xt - dxx * cbjj);
        s_sum += dj * x_s;
        dxx_sum += dxx;
      }
    }
  }
  // fixed-order workgroup sums: lanes -> wave -> waves 0..3
  s_sum = wave_sum(s_sum);
  dxx_sum = wave_sum(dxx_sum);
  dot = wave_sum(dot);
  if (lane == 0) {
    red[0][w] = s_sum;
    red[1][w] = dxx_sum;
    red[2][w] = dot;
  }
  __syncthreads();
  if (tid == 0) {
    float S = 0.f, DD = 0.f, HD = 0.f;
    for (int i = 0; i < 4; ++i) {
      S += red[0][i];
      DD += red[1][i];
      HD += red[2][i];
    }
    last_term[kh] = S + exp2_fast(decay[kh]) * HD;
    dDp[kh] = DD;
  }
}

// -------------------------------------------------------------- bwd dCB_g ----
// dCB_g[i][j] = sum_h (dy_i . x_j) 2^(acs_i - acs_j) delta_j for j <= i < len, zero
// elsewhere in the tiles it writes.  One workgroup per (chunk, group, causal 64 x 64
// tile (ti, tj <= ti)), wave w its rows 16w .. 16w + 15: every tile that dC and dB
// read is written whole, so they read no unwritten value.  A = dy_i (16-byte loads
// along headdim), B = x_j (16-byte loads along headdim); heads summed in order.
__global__ __launch_bounds__(256) void bwd_dcb_f32_kernel(ChunkMap m, int H, int G, int P,
                                                          const float* __restrict__ X,
                                                          const float* __restrict__ DY,
                                                          const float* __restrict__ delta,
                                                          const float* __restrict__ acs,
                                                          float* __restrict__ dCBg) {
  const int Q = m.Q, T = Q / 64, NT = T * (T + 1) / 2;
  const int lid = xcd_order(blockIdx.x, gridDim.x);  // (chunk, group, tile), tile fastest
  const int tile = lid % NT, g = (lid / NT) % G, k = lid / NT / G;
  int ti = 0;
  while ((ti + 1) * (ti + 2) / 2 <= tile) ++ti;
  const int tj = tile - ti * (ti + 1) / 2;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int len = ci.len, hpg = H / G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int i0 = ti * 64 + 16 * w, ir = i0 + r, jb = tj * 64;
  const uint32_t xrow = (uint32_t)(H * P) * 4u;
  f32x4 sum[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sum[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int hh = 0; hh < hpg && i0 < len; ++hh) {
    const int h = g * hpg + hh;
    const int64_t kh = (int64_t)k * H + h, xb = (int64_t)ci.start * H * P + (int64_t)h * P;
    const brsrc rdy = make_rsrc(DY + xb, (uint32_t)len * xrow), rx = make_rsrc(X + xb, (uint32_t)len * xrow);
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < P; p0 += 16) {
      const f32x4 dv = ld4(rdy, (uint32_t)ir * xrow + (uint32_t)(p0 + 4 * q) * 4u);
      f32x4 xv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) xv[u] = ld4(rx, (uint32_t)(jb + u * 16 + r) * xrow + (uint32_t)(p0 + 4 * q) * 4u);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = mfma_f32(dv[s], xv[u][s], acc[u]);
    }
    float ai[4], aj[4], dj[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ai[e] = acs[kh * Q + i0 + 4 * q + e];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      aj[u] = acs[kh * Q + jb + u * 16 + r];
      dj[u] = delta[kh * Q + jb + u * 16 + r];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 4 * q + e, j = jb + u * 16 + r;
        const float v = acc[u][e] * exp2_fast(ai[e] - aj[u]) * dj[u];
        sum[u][e] += (j <= i && i < len) ? v : 0.f;
      }
  }
  float* ob = dCBg + ((int64_t)k * G + g) * Q * Q;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) ob[(int64_t)(i0 + 4 * q + e) * Q + jb + u * 16 + r] = sum[u][e];
}

// ------------------------------------------------------------ bwd dC, dB ----
// One workgroup per (chunk, group, 16 rows); its waves split the dstate tiles
// (wave w takes tiles w, w + WN, ...), so every wave shares the rows' A operand
// (L1 hits) and the grid has a workgroup per 16 rows.
template <int N>
struct DstateSplit {
  static constexpr int NT = N / 16, WN = NT < 4 ? NT : 4, NTW = NT / WN;
};

// dC_i = sum_{j<=i} dCB_g[i][j] B_j + sum_h 2^(acs_i) H_h^T dy_i
//   (A = dCB_g row i, 16-byte loads along j, with B = B_j[n], 4-byte loads; then
//   A = 2^(acs_i) dy_i, 16-byte loads along headdim, with B = H_h[p][n], 4-byte loads)
template <int N>
__global__ __launch_bounds__(256) void bwd_dc_f32_kernel(ChunkMap m, int H, int G, int P,
                                                         const float* __restrict__ Bm,
                                                         const float* __restrict__ DY,
                                                         const float* __restrict__ dCBg,
                                                         const float* __restrict__ acs,
                                                         const float* __restrict__ Hs,
                                                         float* __restrict__ dC) {
  using S = DstateSplit<N>;
  const int Q = m.Q, NB = Q / 16;
  const int lid = xcd_order(blockIdx.x, gridDim.x);  // (chunk, group, 16-row block), block fastest
  const int rb = lid % NB, g = (lid / NB) % G, k = lid / NB / G;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int len = ci.len, hpg = H / G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int i0 = rb * 16, ir = i0 + r;
  if (i0 >= len || w >= S::WN) return;
  const uint32_t xrow = (uint32_t)(H * P) * 4u, brow = (uint32_t)(G * N) * 4u, qrow = (uint32_t)Q * 4u;
  const int64_t bbase = (int64_t)ci.start * G * N + (int64_t)g * N;
  const brsrc rb_ = make_rsrc(Bm + bbase, (uint32_t)len * brow), ro = make_rsrc(dC + bbase, (uint32_t)len * brow);
  const brsrc rcb = make_rsrc(dCBg + ((int64_t)k * G + g) * Q * Q, (uint32_t)Q * qrow);
  f32x4 acc[S::NTW];
#pragma unroll
  for (int u = 0; u < S::NTW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 <= i0; j0 += 16) {
    const f32x4 cv = ld4(rcb, (uint32_t)ir * qrow + (uint32_t)(j0 + 4 * q) * 4u);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < S::NTW; ++u)
        acc[u] = mfma_f32(
            cv[s], buf_load_f32(rb_, (uint32_t)(j0 + 4 * q + s) * brow + (uint32_t)((w + S::WN * u) * 16 + r) * 4u),
            acc[u]);
  }
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const int64_t kh = (int64_t)k * H + h;
    const float sc = ir < len ? exp2_fast(acs[kh * Q + ir]) : 0.f;
    const brsrc rdy = make_rsrc(DY + (int64_t)ci.start * H * P + (int64_t)h * P, (uint32_t)len * xrow);
    const brsrc rh = make_rsrc(Hs + kh * (int64_t)(P * N), (uint32_t)(P * N) * 4u);
    for (int p0 = 0; p0 < P; p0 += 16) {
      const f32x4 dv = ld4(rdy, (uint32_t)ir * xrow + (uint32_t)(p0 + 4 * q) * 4u) * sc;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < S::NTW; ++u)
          acc[u] = mfma_f32(dv[s], buf_load_f32(rh, (uint32_t)((p0 + 4 * q + s) * N + (w + S::WN * u) * 16 + r) * 4u),
                            acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < S::NTW; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      st1(ro, (uint32_t)(i0 + 4 * q + e) * brow + (uint32_t)((w + S::WN * u) * 16 + r) * 4u, acc[u][e]);
}

// dB_j = sum_{i>=j} dCB_g[i][j] C_i + sum_h w_j delta_j dE_h^T x_j
//   (A = dCB_g column j, 4-byte loads along j, with B = C_i[n], 4-byte loads; then
//   A = w_j delta_j x_j, 16-byte loads along headdim, with B = dE_h[p][n], 4-byte loads)
template <int N>
__global__ __launch_bounds__(256) void bwd_db_f32_kernel(ChunkMap m, int H, int G, int P,
                                                         const float* __restrict__ X,
                                                         const float* __restrict__ Cm,
                                                         const float* __restrict__ dCBg,
                                                         const float* __restrict__ delta,
                                                         const float* __restrict__ acs,
                                                         const float* __restrict__ dE,
                                                         float* __restrict__ dB) {
  using S = DstateSplit<N>;
  const int Q = m.Q, NB = Q / 16;
  const int lid = xcd_order(blockIdx.x, gridDim.x);
  const int rb = lid % NB, g = (lid / NB) % G, k = lid / NB / G;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int len = ci.len, hpg = H / G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int j0 = rb * 16, jr = j0 + r;
  if (j0 >= len || w >= S::WN) return;
  const uint32_t xrow = (uint32_t)(H * P) * 4u, crow = (uint32_t)(G * N) * 4u, qrow = (uint32_t)Q * 4u;
  const int64_t cbase = (int64_t)ci.start * G * N + (int64_t)g * N;
  const brsrc rc = make_rsrc(Cm + cbase, (uint32_t)len * crow), ro = make_rsrc(dB + cbase, (uint32_t)len * crow);
  const brsrc rcb = make_rsrc(dCBg + ((int64_t)k * G + g) * Q * Q, (uint32_t)Q * qrow);
  f32x4 acc[S::NTW];
#pragma unroll
  for (int u = 0; u < S::NTW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i0 = j0; i0 < len; i0 += 16) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = i0 + 4 * q + s;  // < Q
      const float v = buf_load_f32(rcb, (uint32_t)i * qrow + (uint32_t)jr * 4u);
      const float a = i < len ? v : 0.f;
#pragma unroll
      for (int u = 0; u < S::NTW; ++u)
        acc[u] = mfma_f32(a, buf_load_f32(rc, (uint32_t)i * crow + (uint32_t)((w + S::WN * u) * 16 + r) * 4u), acc[u]);
    }
  }
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const int64_t kh = (int64_t)k * H + h;
    const float sc = jr < len ? exp2_fast(acs[kh * Q + len - 1] - acs[kh * Q + jr]) * delta[kh * Q + jr] : 0.f;
    const brsrc rx = make_rsrc(X + (int64_t)ci.start * H * P + (int64_t)h * P, (uint32_t)len * xrow);
    const brsrc rde = make_rsrc(dE + kh * (int64_t)(P * N), (uint32_t)(P * N) * 4u);
    for (int p0 = 0; p0 < P; p0 += 16) {
      const f32x4 xv = ld4(rx, (uint32_t)jr * xrow + (uint32_t)(p0 + 4 * q) * 4u) * sc;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < S::NTW; ++u)
          acc[u] = mfma_f32(xv[s], buf_load_f32(rde, (uint32_t)((p0 + 4 * q + s) * N + (w + S::WN * u) * 16 + r) * 4u),
                            acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < S::NTW; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      st1(ro, (uint32_t)(j0 + 4 * q + e) * crow + (uint32_t)((w + S::WN * u) * 16 + r) * 4u, acc[u][e]);
}

// -------------------------------------------------------------- launchers ----
#define SSD_F32_P(MACRO) \
  MACRO(16) MACRO(32) MACRO(64) MACRO(128)

hipError_t launch_chunk_state_f32(const Prob& p, const float* X, const float* Y, const float* delta,
                                  const float* acs, float* out, int mode, hipStream_t st) {
  const dim3 grid((unsigned)(p.nck * p.H)), block(256);
#define SSD_CS32(PP, NN)                                                                              \
  if (p.P == PP && p.N == NN) {                                                                       \
    hipLaunchKernelGGL((chunk_state_f32_kernel<PP, NN>), grid, block, 0, st, p.map, p.H, p.G, mode, X, \
                       Y, delta, acs, out);                                                           \
    return hipGetLastError();                                                                         \
  }
#define SSD_CS32_N(PP) SSD_CS32(PP, 16) SSD_CS32(PP, 32) SSD_CS32(PP, 64) SSD_CS32(PP, 128)
  SSD_F32_P(SSD_CS32_N)
#undef SSD_CS32_N
#undef SSD_CS32
  return hipErrorInvalidValue;
}

hipError_t launch_bmm_chunk_f32(const Prob& p, const float* B, const float* C, float* CB, hipStream_t st) {
  hipLaunchKernelGGL(bmm_chunk_f32_kernel, dim3((unsigned)(p.nck * p.G * (p.Q / 64))), dim3(256), 0, st,
                     p.map, p.G, p.N, B, C, CB);
  return hipGetLastError();
}

hipError_t launch_chunk_scan_f32(const Prob& p, const float* x, const float* C, const float* CB,
                                 const float* delta, const float* acs, const float* passed,
                                 const float* D, float* out, hipStream_t st) {
  const dim3 grid((unsigned)(p.nck * p.H)), block(256);
#define SSD_SCAN32(PP)                                                                                  \
  if (p.P == PP) {                                                                                      \
    hipLaunchKernelGGL((scan_rows_f32_kernel<PP, false>), grid, block, 0, st, p.map, p.H, p.G, p.N, x, C, \
                       CB, delta, acs, passed, D, out, nullptr, nullptr);                               \
    return hipGetLastError();                                                                           \
  }
  SSD_F32_P(SSD_SCAN32)
#undef SSD_SCAN32
  return hipErrorInvalidValue;
}

template <int P, int N>
static void launch_bwd_f32_pn(const Prob& p, const BwdArgs& a, int which, hipStream_t st) {
  const int T = p.Q / 64;
  const dim3 heads((unsigned)(p.nck * p.H)), tiles((unsigned)(p.nck * p.G * (T * (T + 1) / 2)));
  const dim3 rows((unsigned)(p.nck * p.G * (p.Q / 16))), block(256);
  const float *x = (const float*)a.x, *B = (const float*)a.B, *C = (const float*)a.C, *dy = (const float*)a.dout;
  const float *CB = (const float*)a.CB, *Hp = (const float*)a.Hp, *dE = (const float*)a.dE;
  float* dCBg = (float*)a.dCBg;
  if (!which || which == 1)
    hipLaunchKernelGGL((bwd_dx_f32_kernel<P>), heads, block, 0, st, p.map, p.H, p.G, N, x, B, dy, CB, a.delta,
                       a.acs, a.decay, dE, Hp, a.D, (float*)a.dx, a.ddd, a.Ks, a.last_term, a.dDp);
  if (!which || which == 2) {
    hipLaunchKernelGGL(bwd_dcb_f32_kernel, tiles, block, 0, st, p.map, p.H, p.G, P, x, dy, a.delta, a.acs, dCBg);
    hipLaunchKernelGGL((scan_rows_f32_kernel<P, true>), heads, block, 0, st, p.map, p.H, p.G, N, x, C, CB, a.delta,
                       a.acs, Hp, nullptr, nullptr, dy, a.rR);
  }
  if (!which || which == 3)
    hipLaunchKernelGGL((bwd_dc_f32_kernel<N>), rows, block, 0, st, p.map, p.H, p.G, P, B, dy, dCBg, a.acs, Hp,
                       (float*)a.dC);
  if (!which || which == 4)
    hipLaunchKernelGGL((bwd_db_f32_kernel<N>), rows, block, 0, st, p.map, p.H, p.G, P, x, C, dCBg, a.delta, a.acs,
                       dE, (float*)a.dB);
}

// which: 0 every kernel; 1 dx; 2 the head-summed dCB and the r + R rows; 3 dC; 4 dB
hipError_t launch_bwd_f32(const Prob& p, const BwdArgs& a, int which, hipStream_t st) {
#define SSD_BWD32(PP, NN) \
  if (p.P == PP && p.N == NN) { launch_bwd_f32_pn<PP, NN>(p, a, which, st); return hipGetLastError(); }
#define SSD_BWD32_N(PP) SSD_BWD32(PP, 16) SSD_BWD32(PP, 32) SSD_BWD32(PP, 64) SSD_BWD32(PP, 128)
  SSD_F32_P(SSD_BWD32_N)
#undef SSD_BWD32_N
#undef SSD_BWD32
  return hipErrorInvalidValue;
}

#undef SSD_F32_P

}  // namespace ssd
