// The fp32 matrix-core path of every matrix stage, forward and backward: true
// fp32 products (v_mfma_f32_16x16x4f32: D(16x16) += A(16x4) B(4x16)) with fp32
// accumulation.  It runs every fp32 problem, and the bf16 problems whose headdim
// or dstate is 16 (below the bf16 kernels' 32-wide operand tiles): the
// input/output tensors (x, B, C, dy, y, dx, dB, dC and C.B^T) are then read and
// written in bf16 (element type IT) and widened to fp32 in registers, every
// product and sum in fp32.  The stages and equations are those of the bf16 path
// (k_chunk_state.hip, k_chunk_scan.hip and k_bwd.hip).
//
// Operand fragments come straight from global memory through the caches, with
// no LDS staging.  For an MFMA operand X[m][k] (lane (r, q) = lane % 16, lane /
// 16 supplies m = r, k = q):
//   - if X's rows run along k (k contiguous), lane (r, q) loads 4 elements,
//     X[m0 + r][k0 + 4q .. 4q + 3], and element s of them serves k-step s;
//   - if they run along m, lane (r, q) loads X[k0 + 4q + s][m0 + r] for k-step s
//     (16 contiguous elements per 16 lanes).
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

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// A tensor of element type IT (float, or uint16_t holding bf16) seen through a
// range-checked buffer resource over its first n elements.  Offsets are element
// indices; values are fp32 in registers (bf16 widened on load, rounded to nearest
// even on store).  V consecutive elements (V = 1, 2, 4) move in one access; the
// callers keep such runs aligned to V elements.
template <typename IT>
struct Tn {
  static constexpr bool kF32 = sizeof(IT) == 4;
  brsrc r;
  __device__ __forceinline__ Tn(const IT* p, uint32_t n) : r(make_rsrc(p, n * (uint32_t)sizeof(IT))) {}
  __device__ __forceinline__ float ld1(uint32_t e) const {
    if constexpr (kF32)
      return buf_load_f32(r, e * 4u);
    else
      return bf2f(__builtin_amdgcn_raw_buffer_load_b16(r, e * 2u, 0, 0));
  }
  template <int V>
  __device__ __forceinline__ void ldv(uint32_t e, float (&o)[V]) const {
    if constexpr (kF32) {
      if constexpr (V == 4) {
        const u32x4 t = buf_load16(r, e * 4u);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(t[i]);
      } else if constexpr (V == 2) {
        const u32x2v t = __builtin_amdgcn_raw_buffer_load_b64(r, e * 4u, 0, 0);
        o[0] = __uint_as_float(t[0]);
        o[1] = __uint_as_float(t[1]);
      } else {
        o[0] = ld1(e);
      }
    } else {
      if constexpr (V == 4) {
        const u32x2v t = __builtin_amdgcn_raw_buffer_load_b64(r, e * 2u, 0, 0);
        o[0] = bf_lo(t[0]);
        o[1] = bf_hi(t[0]);
        o[2] = bf_lo(t[1]);
        o[3] = bf_hi(t[1]);
      } else if constexpr (V == 2) {
        const uint32_t t = __builtin_amdgcn_raw_buffer_load_b32(r, e * 2u, 0, 0);
        o[0] = bf_lo(t);
        o[1] = bf_hi(t);
      } else {
        o[0] = ld1(e);
      }
    }
  }
  __device__ __forceinline__ f32x4 ld4(uint32_t e) const {
    float o[4];
    ldv<4>(e, o);
    return f32x4{o[0], o[1], o[2], o[3]};
  }
  __device__ __forceinline__ void st1(uint32_t e, float v) const {
    if constexpr (kF32)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, e * 4u, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b16(f2bf(v), r, e * 2u, 0, 0);
  }
  template <int V>
  __device__ __forceinline__ void stv(uint32_t e, const float (&o)[V]) const {
    if constexpr (kF32) {
      if constexpr (V == 4)
        buf_store16(r, e * 4u, u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                                     __float_as_uint(o[3])});
      else if constexpr (V == 2)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2v{__float_as_uint(o[0]), __float_as_uint(o[1])}, r, e * 4u, 0, 0);
      else
        st1(e, o[0]);
    } else {
      if constexpr (V == 4)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2v{pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3])}, r, e * 2u, 0, 0);
      else if constexpr (V == 2)
        __builtin_amdgcn_raw_buffer_store_b32(pack_bf2(o[0], o[1]), r, e * 2u, 0, 0);
      else
        st1(e, o[0]);
    }
  }
};

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
template <int P, int N, typename IT>
__global__ __launch_bounds__(256) void chunk_state_f32_kernel(ChunkMap m, int H, int G, int mode,
                                                              const IT* __restrict__ X,
                                                              const IT* __restrict__ Y,
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
  const uint32_t xs = (uint32_t)(H * P), ys = (uint32_t)(G * N);  // elements between tokens
  const Tn<IT> tx(X + (int64_t)ci.start * H * P + (int64_t)h * P, (uint32_t)len * xs);
  const Tn<IT> ty(Y + (int64_t)ci.start * G * N + (int64_t)g * N, (uint32_t)len * ys);
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
    for (int c = 0; c < CN::NG; ++c) ty.template ldv<CN::V>((uint32_t)j * ys + (uint32_t)(nb + CN::col0(c, r)), a[c]);
#pragma unroll
    for (int c = 0; c < CP::NG; ++c) tx.template ldv<CP::V>((uint32_t)j * xs + (uint32_t)(pb + CP::col0(c, r)), b[c]);
#pragma unroll
    for (int u = 0; u < NTW; ++u)
#pragma unroll
      for (int v = 0; v < PTW; ++v)
        acc[u][v] = mfma_f32(a[u / CN::V][u % CN::V] * s, b[v / CP::V][v % CP::V], acc[u][v]);
  }
  // tile (u, v), element e: n = nb + 16 V c + V (4q + e) + t (u = c V + t), p = pb + col of lane r in v
  const Tn<float> to(out + kh * (int64_t)(P * N), (uint32_t)(P * N));
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
        to.template stv<CN::V>((uint32_t)(p * N + nb + 16 * CN::V * c + CN::V * (4 * q + e)), o);
      }
  }
}

// ------------------------------------------------------------------ C.B^T ----
// CB[i][j] = C_i . B_j for j <= i < len; nothing else is written.  Wave w owns
// rows 16w .. 16w + 15 of the 64-row block and takes its column tiles up to the
// diagonal four at a time; both operands run along dstate (4-element loads).
template <typename IT>
__global__ __launch_bounds__(256) void bmm_chunk_f32_kernel(ChunkMap m, int G, int N,
                                                            const IT* __restrict__ Bm,
                                                            const IT* __restrict__ Cm,
                                                            IT* __restrict__ CB) {
  const int Q = m.Q, T = Q / 64;
  const int lid = xcd_order(blockIdx.x, gridDim.x);  // (chunk, group, row block), row block fastest
  const int ti = lid % T, g = (lid / T) % G, k = lid / T / G;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int len = ci.len;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int i0 = ti * 64 + 16 * w;
  if (i0 >= len) return;
  const uint32_t rs = (uint32_t)(G * N);
  const int64_t base = (int64_t)ci.start * G * N + (int64_t)g * N;
  const Tn<IT> tc(Cm + base, (uint32_t)len * rs), tb(Bm + base, (uint32_t)len * rs);
  const Tn<IT> to(CB + ((int64_t)k * G + g) * Q * Q, (uint32_t)(Q * Q));
  const int njt = i0 / 16 + 1;  // column tiles up to the diagonal one
  for (int jt0 = 0; jt0 < njt; jt0 += 4) {
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int n0 = 0; n0 < N; n0 += 16) {
      const f32x4 cv = tc.ld4((uint32_t)(i0 + r) * rs + (uint32_t)(n0 + 4 * q));
      f32x4 bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) bv[u] = tb.ld4((uint32_t)((jt0 + u) * 16 + r) * rs + (uint32_t)(n0 + 4 * q));
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
        if (jt0 + u < njt && j <= i && i < len) to.st1((uint32_t)(i * Q + j), acc[u][e]);
      }
  }
}

// ---------------------------------------------------- output rows (scan, r+R) ----
// Per (chunk, head) and 16-row block of tokens i, the chunk scan's bracket
//   acc_i[p] = 2^(acs_i) (H_c C_i)[p] + sum_{j<=i} CB_ij 2^(acs_i - acs_j) delta_j x_j[p]
// then either (RR false) y_i = acc_i + D x_i, or (RR true) the backward's
//   r_i + R_i = dy_i . (acc_i - CB_ii delta_i x_i),
// the state term's r_i and R_i = sum_{j<i} (dy_i . x_j) CB_ij L_ij delta_j together.
// Products D[i][p]: A = 2^(acs_i) C_i (4-element loads along dstate) or the
// decayed C.B^T row (4-element loads along j), B = H_c[p] (4-element loads along
// dstate) or x_j[p], whose headdim columns are permuted in groups (ColGroups): a
// lane loads its x, dy and y values 4 at a time.  Row blocks in snake order over
// the four waves.
template <int P, bool RR, typename IT>
__global__ __launch_bounds__(256) void scan_rows_f32_kernel(
    ChunkMap m, int H, int G, int N, const IT* __restrict__ X, const IT* __restrict__ Cm,
    const IT* __restrict__ CB, const float* __restrict__ delta, const float* __restrict__ acs,
    const float* __restrict__ Hs, const float* __restrict__ D, IT* __restrict__ Y,
    const IT* __restrict__ DY, float* __restrict__ rR) {
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
  const uint32_t xs = (uint32_t)(H * P), cs = (uint32_t)(G * N);  // elements between tokens
  const int64_t xb = (int64_t)ci.start * H * P + (int64_t)h * P;
  const Tn<IT> tx(X + xb, (uint32_t)len * xs);
  const Tn<IT> tdy(RR ? DY + xb : X + xb, (uint32_t)len * xs);
  const Tn<IT> ty(RR ? nullptr : Y + xb, RR ? 0u : (uint32_t)len * xs);
  const Tn<IT> tc(Cm + (int64_t)ci.start * G * N + (int64_t)g * N, (uint32_t)len * cs);
  const Tn<IT> tcb(CB + ((int64_t)k * G + g) * Q * Q, (uint32_t)(Q * Q));
  const Tn<float> th(Hs + kh * (int64_t)(P * N), (uint32_t)(P * N));
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
      const f32x4 cv = tc.ld4((uint32_t)ir * cs + (uint32_t)(n0 + 4 * q)) * sc;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const int p = CG::col0(pt / V, r) + pt % V;
        const f32x4 hv = th.ld4((uint32_t)(p * N + n0 + 4 * q));
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[pt] = mfma_f32(cv[s], hv[s], acc[pt]);
      }
    }
    // the chunk's earlier tokens and the diagonal block
    const float ai = sa[ir];
    for (int j0 = 0; j0 <= i0; j0 += 16) {
      const f32x4 cb = tcb.ld4((uint32_t)(ir * Q + j0 + 4 * q));
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
          tx.template ldv<V>((uint32_t)(j0 + 4 * q + s) * xs + (uint32_t)CG::col0(c, r), xv);
#pragma unroll
          for (int t = 0; t < V; ++t) acc[c * V + t] = mfma_f32(mv[s], xv[t], acc[c * V + t]);
        }
    }
    // lane (r, q) holds rows i0 + 4q + e, columns col0(c, r) + t of tile c V + t
    if constexpr (!RR) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t io = (uint32_t)(i0 + 4 * q + e) * xs;
#pragma unroll
        for (int c = 0; c < NG; ++c) {
          const uint32_t o = io + (uint32_t)CG::col0(c, r);
          float xv[V], yv[V];
          tx.template ldv<V>(o, xv);
#pragma unroll
          for (int t = 0; t < V; ++t) yv[t] = acc[c * V + t][e] + Dh * xv[t];
          ty.template stv<V>(o, yv);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 4 * q + e;
        const uint32_t io = (uint32_t)i * xs;
        float ya = 0.f, yx = 0.f;
#pragma unroll
        for (int c = 0; c < NG; ++c) {
          const uint32_t o = io + (uint32_t)CG::col0(c, r);
          float dyv[V], xv[V];
          tdy.template ldv<V>(o, dyv);
          tx.template ldv<V>(o, xv);
#pragma unroll
          for (int t = 0; t < V; ++t) {
            ya += dyv[t] * acc[c * V + t][e];
            yx += dyv[t] * xv[t];
          }
        }
        const float mii = i < len ? tcb.ld1((uint32_t)(i * Q + i)) * sd[i] : 0.f;
        const float v = row_sum16(ya) - mii * row_sum16(yx);
        if (r == 0 && i < len) rR[kh * Q + i] = v;
      }
    }
  }
}

// ------------------------------------------------------------------ bwd dx ----
// Per (chunk, head) and 16-row block of tokens j, the bracket
//   U_j[p] = w_j (dT B_j)[p] + sum_{i>=j} CB_ij 2^(acs_i - acs_j) dy_i[p],  w_j = 2^(acs_last - acs_j)
// (A = w_j B_j, 4-element loads along dstate, with B = dE_c[p], 4-element loads;
// then A = the decayed C.B^T column j, 1-element loads along j, with B = dy_i[p],
// headdim columns permuted in groups as in the rows kernel above), and
//   dx_j = delta_j U_j + D dy_j,  d(delta)_j direct = x_j . U_j,
//   K_j + s_j = delta_j (x_j . U_j - (x_j . dy_j) CB_jj)   (s_j = delta_j x_j . w_j dT B_j),
// dD's per-chunk part sum_j x_j . dy_j and alpha <dE, H> + sum_j s_j per chunk.
template <int P, typename IT>
__global__ __launch_bounds__(256) void bwd_dx_f32_kernel(
    ChunkMap m, int H, int G, int N, const IT* __restrict__ X, const IT* __restrict__ Bm,
    const IT* __restrict__ DY, const IT* __restrict__ CB, const float* __restrict__ delta,
    const float* __restrict__ acs, const float* __restrict__ decay, const float* __restrict__ dE,
    const float* __restrict__ Hs, const float* __restrict__ D, IT* __restrict__ DX,
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
  // <dE, H>: this thread's 4-element pieces in order
  const Tn<float> tde(dE + kh * (int64_t)(P * N), (uint32_t)(P * N));
  const Tn<float> thh(Hs + kh * (int64_t)(P * N), (uint32_t)(P * N));
  float dot = 0.f;
  for (int e = tid * 4; e < P * N; e += 1024) {
    const f32x4 a = tde.ld4((uint32_t)e), b = thh.ld4((uint32_t)e);
    dot += a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
  }
  __syncthreads();
  const uint32_t xs = (uint32_t)(H * P), bs = (uint32_t)(G * N);  // elements between tokens
  const int64_t xb = (int64_t)ci.start * H * P + (int64_t)h * P;
  const Tn<IT> tx(X + xb, (uint32_t)len * xs), tdy(DY + xb, (uint32_t)len * xs);
  const Tn<IT> tdx(DX + xb, (uint32_t)len * xs);
  const Tn<IT> tb(Bm + (int64_t)ci.start * G * N + (int64_t)g * N, (uint32_t)len * bs);
  const Tn<IT> tcb(CB + ((int64_t)k * G + g) * Q * Q, (uint32_t)(Q * Q));
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
      const f32x4 bv = tb.ld4((uint32_t)jr * bs + (uint32_t)(n0 + 4 * q)) * wj;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const int p = CG::col0(pt / V, r) + pt % V;
        const f32x4 ev = tde.ld4((uint32_t)(p * N + n0 + 4 * q));
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[pt] = mfma_f32(bv[s], ev[s], acc[pt]);
      }
    }
    // x_j . (state part), rows j0 + 4q + e
    float xsum[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t jo = (uint32_t)(j0 + 4 * q + e) * xs;
      float v = 0.f;
#pragma unroll
      for (int c = 0; c < NG; ++c) {
        float xv[V];
        tx.template ldv<V>(jo + (uint32_t)CG::col0(c, r), xv);
#pragma unroll
        for (int t = 0; t < V; ++t) v += xv[t] * acc[c * V + t][e];
      }
      xsum[e] = v;
    }
    // later tokens of the chunk: i >= j
    const float aj = sa[jr];
    for (int i0 = j0; i0 < len; i0 += 16) {
      float mv[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int i = i0 + 4 * q + s;  // < Q: i0 < len <= Q, both multiples of 16
        const float v = tcb.ld1((uint32_t)(i * Q + jr)) * exp2_fast(sa[i] - aj);
        mv[s] = (i >= jr && i < len) ? v : 0.f;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int c = 0; c < NG; ++c) {
          float yv[V];
          tdy.template ldv<V>((uint32_t)(i0 + 4 * q + s) * xs + (uint32_t)CG::col0(c, r), yv);
#pragma unroll
          for (int t = 0; t < V; ++t) acc[c * V + t] = mfma_f32(mv[s], yv[t], acc[c * V + t]);
        }
    }
    // dx, and the per-row dots
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + 4 * q + e;
      const float dj = sd[j];
      const uint32_t jo = (uint32_t)j * xs;
      float xt = 0.f, dxx = 0.f;
#pragma unroll
      for (int c = 0; c < NG; ++c) {
        const uint32_t o = jo + (uint32_t)CG::col0(c, r);
        float xv[V], yv[V], ov[V];
        tx.template ldv<V>(o, xv);
        tdy.template ldv<V>(o, yv);
#pragma unroll
        for (int t = 0; t < V; ++t) {
          const float a = acc[c * V + t][e];
          xt += xv[t] * a;
          dxx += xv[t] * yv[t];
          ov[t] = dj * a + Dh * yv[t];
        }
        tdx.template stv<V>(o, ov);
      }
      xt = row_sum16(xt);
      dxx = row_sum16(dxx);
      const float x_s = row_sum16(xsum[e]);
      if (r == 0 && j < len) {
        const float cbjj = tcb.ld1((uint32_t)(j * Q + j));
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
// elsewhere in the tiles it writes (fp32).  One workgroup per (chunk, group,
// causal 64 x 64 tile (ti, tj <= ti)), wave w its rows 16w .. 16w + 15: every tile
// that dC and dB read is written whole, so they read no unwritten value.  A = dy_i
// (4-element loads along headdim), B = x_j (4-element loads along headdim); heads
// summed in order.
template <typename IT>
__global__ __launch_bounds__(256) void bwd_dcb_f32_kernel(ChunkMap m, int H, int G, int P,
                                                          const IT* __restrict__ X,
                                                          const IT* __restrict__ DY,
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
  const uint32_t xs = (uint32_t)(H * P);
  f32x4 sum[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sum[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int hh = 0; hh < hpg && i0 < len; ++hh) {
    const int h = g * hpg + hh;
    const int64_t kh = (int64_t)k * H + h, xb = (int64_t)ci.start * H * P + (int64_t)h * P;
    const Tn<IT> tdy(DY + xb, (uint32_t)len * xs), tx(X + xb, (uint32_t)len * xs);
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < P; p0 += 16) {
      const f32x4 dv = tdy.ld4((uint32_t)ir * xs + (uint32_t)(p0 + 4 * q));
      f32x4 xv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) xv[u] = tx.ld4((uint32_t)(jb + u * 16 + r) * xs + (uint32_t)(p0 + 4 * q));
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
// and the grid has a workgroup per 16 rows.
template <int N>
struct DstateSplit {
  static constexpr int NT = N / 16, WN = NT < 4 ? NT : 4, NTW = NT / WN;
};

// dC_i = sum_{j<=i} dCB_g[i][j] B_j + sum_h 2^(acs_i) H_h^T dy_i
//   (A = dCB_g row i, 4-element loads along j, with B = B_j[n], 1-element loads;
//   then A = 2^(acs_i) dy_i, 4-element loads along headdim, with B = H_h[p][n],
//   1-element loads)
template <int N, typename IT>
__global__ __launch_bounds__(256) void bwd_dc_f32_kernel(ChunkMap m, int H, int G, int P,
                                                         const IT* __restrict__ Bm,
                                                         const IT* __restrict__ DY,
                                                         const float* __restrict__ dCBg,
                                                         const float* __restrict__ acs,
                                                         const float* __restrict__ Hs,
                                                         IT* __restrict__ dC) {
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
  const uint32_t xs = (uint32_t)(H * P), bs = (uint32_t)(G * N);
  const int64_t bbase = (int64_t)ci.start * G * N + (int64_t)g * N;
  const Tn<IT> tb(Bm + bbase, (uint32_t)len * bs), to(dC + bbase, (uint32_t)len * bs);
  const Tn<float> tcb(dCBg + ((int64_t)k * G + g) * Q * Q, (uint32_t)(Q * Q));
  f32x4 acc[S::NTW];
#pragma unroll
  for (int u = 0; u < S::NTW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 <= i0; j0 += 16) {
    const f32x4 cv = tcb.ld4((uint32_t)(ir * Q + j0 + 4 * q));
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < S::NTW; ++u)
        acc[u] = mfma_f32(cv[s], tb.ld1((uint32_t)(j0 + 4 * q + s) * bs + (uint32_t)((w + S::WN * u) * 16 + r)),
                          acc[u]);
  }
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const int64_t kh = (int64_t)k * H + h;
    const float sc = ir < len ? exp2_fast(acs[kh * Q + ir]) : 0.f;
    const Tn<IT> tdy(DY + (int64_t)ci.start * H * P + (int64_t)h * P, (uint32_t)len * xs);
    const Tn<float> th(Hs + kh * (int64_t)(P * N), (uint32_t)(P * N));
    for (int p0 = 0; p0 < P; p0 += 16) {
      const f32x4 dv = tdy.ld4((uint32_t)ir * xs + (uint32_t)(p0 + 4 * q)) * sc;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < S::NTW; ++u)
          acc[u] = mfma_f32(dv[s], th.ld1((uint32_t)((p0 + 4 * q + s) * N + (w + S::WN * u) * 16 + r)), acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < S::NTW; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      to.st1((uint32_t)(i0 + 4 * q + e) * bs + (uint32_t)((w + S::WN * u) * 16 + r), acc[u][e]);
}

// dB_j = sum_{i>=j} dCB_g[i][j] C_i + sum_h w_j delta_j dE_h^T x_j
//   (A = dCB_g column j, 1-element loads along j, with B = C_i[n], 1-element loads;
//   then A = w_j delta_j x_j, 4-element loads along headdim, with B = dE_h[p][n],
//   1-element loads)
template <int N, typename IT>
__global__ __launch_bounds__(256) void bwd_db_f32_kernel(ChunkMap m, int H, int G, int P,
                                                         const IT* __restrict__ X,
                                                         const IT* __restrict__ Cm,
                                                         const float* __restrict__ dCBg,
                                                         const float* __restrict__ delta,
                                                         const float* __restrict__ acs,
                                                         const float* __restrict__ dE,
                                                         IT* __restrict__ dB) {
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
  const uint32_t xs = (uint32_t)(H * P), cs = (uint32_t)(G * N);
  const int64_t cbase = (int64_t)ci.start * G * N + (int64_t)g * N;
  const Tn<IT> tc(Cm + cbase, (uint32_t)len * cs), to(dB + cbase, (uint32_t)len * cs);
  const Tn<float> tcb(dCBg + ((int64_t)k * G + g) * Q * Q, (uint32_t)(Q * Q));
  f32x4 acc[S::NTW];
#pragma unroll
  for (int u = 0; u < S::NTW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i0 = j0; i0 < len; i0 += 16) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = i0 + 4 * q + s;  // < Q
      const float v = tcb.ld1((uint32_t)(i * Q + jr));
      const float a = i < len ? v : 0.f;
#pragma unroll
      for (int u = 0; u < S::NTW; ++u)
        acc[u] = mfma_f32(a, tc.ld1((uint32_t)i * cs + (uint32_t)((w + S::WN * u) * 16 + r)), acc[u]);
    }
  }
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const int64_t kh = (int64_t)k * H + h;
    const float sc = jr < len ? exp2_fast(acs[kh * Q + len - 1] - acs[kh * Q + jr]) * delta[kh * Q + jr] : 0.f;
    const Tn<IT> tx(X + (int64_t)ci.start * H * P + (int64_t)h * P, (uint32_t)len * xs);
    const Tn<float> tde(dE + kh * (int64_t)(P * N), (uint32_t)(P * N));
    for (int p0 = 0; p0 < P; p0 += 16) {
      const f32x4 xv = tx.ld4((uint32_t)jr * xs + (uint32_t)(p0 + 4 * q)) * sc;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < S::NTW; ++u)
          acc[u] = mfma_f32(xv[s], tde.ld1((uint32_t)((p0 + 4 * q + s) * N + (w + S::WN * u) * 16 + r)), acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < S::NTW; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      to.st1((uint32_t)(j0 + 4 * q + e) * cs + (uint32_t)((w + S::WN * u) * 16 + r), acc[u][e]);
}

// -------------------------------------------------------------- launchers ----
// The io tensors' element type: fp32, or bf16 (a bf16 problem with headdim or
// dstate 16).  Intermediates (chunk states, passed states and their adjoints,
// the head-summed dCB, per-token values) are fp32 on this path in either case.
#define SSD_F32_P(MACRO) \
  MACRO(16) MACRO(32) MACRO(64) MACRO(128)

template <typename IT>
static hipError_t chunk_state_f32_it(const Prob& p, const void* X, const void* Y, const float* delta,
                                     const float* acs, float* out, int mode, hipStream_t st) {
  const dim3 grid((unsigned)(p.nck * p.H)), block(256);
#define SSD_CS32(PP, NN)                                                                                   \
  if (p.P == PP && p.N == NN) {                                                                            \
    hipLaunchKernelGGL((chunk_state_f32_kernel<PP, NN, IT>), grid, block, 0, st, p.map, p.H, p.G, mode,    \
                       (const IT*)X, (const IT*)Y, delta, acs, out);                                       \
    return hipGetLastError();                                                                              \
  }
#define SSD_CS32_N(PP) SSD_CS32(PP, 16) SSD_CS32(PP, 32) SSD_CS32(PP, 64) SSD_CS32(PP, 128)
  SSD_F32_P(SSD_CS32_N)
#undef SSD_CS32_N
#undef SSD_CS32
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_state_f32(const Prob& p, const void* X, const void* Y, const float* delta,
                                  const float* acs, float* out, int mode, hipStream_t st) {
  return p.io == 1 ? chunk_state_f32_it<uint16_t>(p, X, Y, delta, acs, out, mode, st)
                   : chunk_state_f32_it<float>(p, X, Y, delta, acs, out, mode, st);
}

hipError_t launch_bmm_chunk_f32(const Prob& p, const void* B, const void* C, void* CB, hipStream_t st) {
  const dim3 grid((unsigned)(p.nck * p.G * (p.Q / 64))), block(256);
  if (p.io == 1)
    hipLaunchKernelGGL(bmm_chunk_f32_kernel<uint16_t>, grid, block, 0, st, p.map, p.G, p.N, (const uint16_t*)B,
                       (const uint16_t*)C, (uint16_t*)CB);
  else
    hipLaunchKernelGGL(bmm_chunk_f32_kernel<float>, grid, block, 0, st, p.map, p.G, p.N, (const float*)B,
                       (const float*)C, (float*)CB);
  return hipGetLastError();
}

template <typename IT>
static hipError_t chunk_scan_f32_it(const Prob& p, const void* x, const void* C, const void* CB,
                                    const float* delta, const float* acs, const float* passed,
                                    const float* D, void* out, hipStream_t st) {
  const dim3 grid((unsigned)(p.nck * p.H)), block(256);
#define SSD_SCAN32(PP)                                                                                       \
  if (p.P == PP) {                                                                                           \
    hipLaunchKernelGGL((scan_rows_f32_kernel<PP, false, IT>), grid, block, 0, st, p.map, p.H, p.G, p.N,      \
                       (const IT*)x, (const IT*)C, (const IT*)CB, delta, acs, passed, D, (IT*)out, nullptr,  \
                       nullptr);                                                                             \
    return hipGetLastError();                                                                                \
  }
  SSD_F32_P(SSD_SCAN32)
#undef SSD_SCAN32
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_scan_f32(const Prob& p, const void* x, const void* C, const void* CB,
                                 const float* delta, const float* acs, const float* passed,
                                 const float* D, void* out, hipStream_t st) {
  return p.io == 1 ? chunk_scan_f32_it<uint16_t>(p, x, C, CB, delta, acs, passed, D, out, st)
                   : chunk_scan_f32_it<float>(p, x, C, CB, delta, acs, passed, D, out, st);
}

template <int P, int N, typename IT>
static void launch_bwd_f32_pn(const Prob& p, const BwdArgs& a, int which, hipStream_t st) {
  const int T = p.Q / 64;
  const dim3 heads((unsigned)(p.nck * p.H)), tiles((unsigned)(p.nck * p.G * (T * (T + 1) / 2)));
  const dim3 rows((unsigned)(p.nck * p.G * (p.Q / 16))), block(256);
  const IT *x = (const IT*)a.x, *B = (const IT*)a.B, *C = (const IT*)a.C, *dy = (const IT*)a.dout;
  const IT* CB = (const IT*)a.CB;
  const float *Hp = (const float*)a.Hp, *dE = (const float*)a.dE;
  float* dCBg = (float*)a.dCBg;
  if (!which || which == 1)
    hipLaunchKernelGGL((bwd_dx_f32_kernel<P, IT>), heads, block, 0, st, p.map, p.H, p.G, N, x, B, dy, CB,
                       a.delta, a.acs, a.decay, dE, Hp, a.D, (IT*)a.dx, a.ddd, a.Ks, a.last_term, a.dDp);
  if (!which || which == 2) {
    hipLaunchKernelGGL(bwd_dcb_f32_kernel<IT>, tiles, block, 0, st, p.map, p.H, p.G, P, x, dy, a.delta, a.acs,
                       dCBg);
    hipLaunchKernelGGL((scan_rows_f32_kernel<P, true, IT>), heads, block, 0, st, p.map, p.H, p.G, N, x, C, CB,
                       a.delta, a.acs, Hp, nullptr, nullptr, dy, a.rR);
  }
  if (!which || which == 3)
    hipLaunchKernelGGL((bwd_dc_f32_kernel<N, IT>), rows, block, 0, st, p.map, p.H, p.G, P, B, dy, dCBg, a.acs,
                       Hp, (IT*)a.dC);
  if (!which || which == 4)
    hipLaunchKernelGGL((bwd_db_f32_kernel<N, IT>), rows, block, 0, st, p.map, p.H, p.G, P, x, C, dCBg, a.delta,
                       a.acs, dE, (IT*)a.dB);
}

// which: 0 every kernel; 1 dx; 2 the head-summed dCB and the r + R rows; 3 dC; 4 dB
hipError_t launch_bwd_f32(const Prob& p, const BwdArgs& a, int which, hipStream_t st) {
#define SSD_BWD32(PP, NN)                                                           \
  if (p.P == PP && p.N == NN) {                                                     \
    if (p.io == 1)                                                                  \
      launch_bwd_f32_pn<PP, NN, uint16_t>(p, a, which, st);                         \
    else                                                                            \
      launch_bwd_f32_pn<PP, NN, float>(p, a, which, st);                            \
    return hipGetLastError();                                                       \
  }
#define SSD_BWD32_N(PP) SSD_BWD32(PP, 16) SSD_BWD32(PP, 32) SSD_BWD32(PP, 64) SSD_BWD32(PP, 128)
  SSD_F32_P(SSD_BWD32_N)
#undef SSD_BWD32_N
#undef SSD_BWD32
  return hipErrorInvalidValue;
}

#undef SSD_F32_P

}  // namespace ssd
