// Backward, intra-chunk part of dB and dC with their decay-gradient sums, in one
// pass over a group's x and dy rows (the adjoint of the output stage; the
// notation is that of k_bwd.hip).  The opt-in form (SSD_FLAG_BWD_FUSED) of what
// bwd_dcb, bwd_dc and bwd_db compute: it moves ~40 % fewer bytes, but its phase A
// holds ~165 registers per lane (the T tiles' sums, the next head's blocks, the
// C.B^T values), so one 8-wave workgroup runs per compute unit, and each head's
// load, barrier, product sequence is then bound by memory latency; on MI355X the
// three kernels, at three or four workgroups per compute unit, are faster.
//
// One workgroup per (chunk, group, 64-row block b), 8 wavefronts.  With T = Q/64
// blocks per chunk, dC on the rows of block b needs the head-summed tiles
// dCB_g[b][0..b] and dB on the rows of b needs dCB_g[b..T-1][b]: T tiles for
// every b (the diagonal tile serves both), so every workgroup does the same work.
// Three phases:
//   A  per head h: dy_i . x_j on MFMA over those tiles (the column tiles computed
//      transposed, x_j . dy_i), times L_ij delta_j (off-diagonal tiles through the
//      anchor token at their last column, as bwd_dcb), summed over the heads in
//      fp32 registers.  The decay-gradient sums of M_ij = dCB^h_ij CB_ij,
//      R_i = sum_{j<i} M_ij for the rows i of block b and K_j = sum_{i>j} M_ij for
//      its columns j, are whole inside the workgroup and are written once per
//      token (no tile partials).
//   B  dCB_g through LDS in bf16; waves 0-3 start dC_b = sum_{jb<=b} dCB_g[b][jb] B_jb,
//      waves 4-7 dB_b = sum_{ib>=b} dCB_g[ib][b]^T C_ib.
//   C  per head: the state terms 2^acs_i H^T dy_i (waves 0-3, with
//      r_i = C_i . that term) and w_j delta_j dT^T x_j (waves 4-7).
// The values, the order of every sum that forms dB and dC, and the rounding are
// those of bwd_dcb, bwd_dc and bwd_db, so dB and dC come out bit for bit the
// same; only R and K are summed in another order.  Across the T workgroups of a
// (chunk, group), which run one after the other on one XCD, each x and dy block
// comes from memory once (the three kernels read x and dy twice each); phase C's
// second look at block b's own rows is a cache hit.  (Launched with at most two
// waves per SIMD: capped at 128 registers it spilled to scratch inside the head
// loop and ran 1.6 times slower still.)
#include "internal.hpp"

namespace ssd {

namespace {

constexpr int QMAXF = 256;
constexpr int TMF = QMAXF / 64;  // blocks per chunk, at most

template <int P, int N>
struct DbcShape {
  static constexpr int PER = P / 8;                        // 16-byte pieces of an x / dy row
  static constexpr int LX = P + 8;                         // x / dy block row stride (bf16)
  static constexpr int LT = 64 + 8;                        // dCB tile row stride
  static constexpr int LDB = N + 16;                       // B, C, H, dE rows: odd multiple of 32 bytes
  static constexpr int NPA = ((TMF + 1) * 64 * PER + 511) / 512;  // phase A block pieces per thread
  static constexpr int NPB = 64 * (N / 8) / 512 > 0 ? 64 * (N / 8) / 512 : 1;  // B or C block pieces
  static constexpr int NPC = (P * N / 8 + 511) / 512;      // H or dE pieces per thread
  static constexpr int SZA = (TMF + 1) * 64 * LX;
  static constexpr int SZT = TMF * 64 * LT;                // dCB tiles
  static constexpr int SZB = SZT + 2 * 64 * LDB;           // tiles + one B and one C block
  static constexpr int SZC1 = 2 * P * LDB;                 // H and dE of one head
  static constexpr int NBUF = SZC1 * 2 * 2 <= 76 * 1024 ? 2 : 1;  // phase C buffers
  static constexpr int SZC = NBUF * SZC1;
  static constexpr int SZ = SZA > SZB ? (SZA > SZC ? SZA : SZC) : (SZB > SZC ? SZB : SZC);
};

}  // namespace

template <int P, int N>
__global__ __launch_bounds__(512, 2) void bwd_dbc_bf16_kernel(
    ChunkMap m, int H, int G, const uint16_t* __restrict__ X, const uint16_t* __restrict__ DY,
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ CB, const float* __restrict__ delta,
    const float* __restrict__ acs, const uint16_t* __restrict__ Hs,
    const uint16_t* __restrict__ dE, uint16_t* __restrict__ dB, uint16_t* __restrict__ dC,
    float* __restrict__ rout, float* __restrict__ Rf, float* __restrict__ Kf) {
  using S = DbcShape<P, N>;
  constexpr int PER = S::PER, LX = S::LX, LT = S::LT, LDB = S::LDB;
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::SZ];
  __shared__ float sa[QMAXF], sd[QMAXF];                 // this head's acs and delta
  __shared__ float redr[2][64], redkc[2][64], redkd[4][64];

  const int T = m.Q / 64;
  const int lid = xcd_order(blockIdx.x, gridDim.x);  // (chunk, group, block), block fastest
  const int rb = lid % T, k = lid / T / G, g = (lid / T) % G;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0 || rb * 64 >= ci.len) return;
  const int Q = m.Q, len = ci.len;
  const int nT = (len + 63) / 64;  // blocks holding tokens
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w & 3, wc = w >> 2;
  const int q = lane >> 4, r = lane & 15;
  const int hpg = H / G;
  const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N;
  const int64_t kg = (int64_t)k * G + g;
  const int t0 = rb * 64;              // first token of block b
  const int rowA = 16 * wr + 4 * q;    // phase A: this lane's rows rowA + rr of block b
  const int row1 = t0 + 16 * wr + r;   // phases B, C: this lane's one row (and phase A's A operand row)
  const uint32_t xo1 = (uint32_t)row1 * (uint32_t)(xrow * 2) + q * 16;
  auto ccol = [&](int c) { return (2 * wc + c) * 16 + r; };  // phase A: this lane's columns of a tile

  // ------------------------------------------------------------------ A ----
  // Tile s of the workgroup: s <= b the row tile (b, s), rows i of b, columns j of
  // s; s > b the column tile (s, b), computed transposed: rows j of b, columns i
  // of s.  LDS slot s < T holds x block s (s <= b) or dy block s (s > b), the B
  // operand of tile s, and slot T holds dy block b; the A operands are this wave's
  // 16 rows of block b, of dy (slot T) for row tiles and of x (slot b) for column
  // tiles.  CB at this lane's outputs, strictly lower (j < i < len), is loaded
  // once (the chunk's C.B^T tile is whole in memory) and kept as bf16 pairs.
  const uint16_t* cbm = CB + kg * Q * Q;
  uint32_t cbp[TMF][2][2];
#pragma unroll
  for (int s = 0; s < TMF; ++s)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        uint32_t v = 0u;
        if (s < T) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int a = t0 + rowA + 2 * h2 + u, o = s * 64 + ccol(c);
            const int i = s <= rb ? a : o, j = s <= rb ? o : a;
            const uint32_t cv = cbm[cbf_off(i, j, Q)];  // (fragment order)
            v |= ((i < len && j < i) ? cv : 0u) << (16 * u);
          }
        }
        cbp[s][c][h2] = v;
      }
  auto cbv = [&](int s, int c, int rr) {
    return (rr & 1) ? bf_hi(cbp[s][c][rr >> 1]) : bf_lo(cbp[s][c][rr >> 1]);
  };
  f32x4 sum[TMF][2];
#pragma unroll
  for (int s = 0; s < TMF; ++s) sum[s][0] = sum[s][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 px[S::NPA];
  float pa = 0.f, pd = 0.f;
  // the next head's LDS blocks and the head's acs and delta: every load
  // unconditional, range-checked (rows past the chunk read zero)
  auto load_a = [&](int h) {
    const int64_t hoff = (int64_t)ci.start * xrow + (int64_t)h * P;
    const brsrc rx = make_rsrc(X + hoff, (uint32_t)(len * xrow * 2));
    const brsrc ry = make_rsrc(DY + hoff, (uint32_t)(len * xrow * 2));
#pragma unroll
    for (int c = 0; c < S::NPA; ++c) {
      const int e = tid + c * 512;
      const int s = __builtin_amdgcn_readfirstlane(e / (64 * PER));  // whole wavefronts per slot
      const int rem = e % (64 * PER), row = rem / PER, c8 = rem % PER;
      const int sb = s < T ? s : rb;  // source block of slot s (slot T: dy block b)
      const uint32_t off = s <= T ? (uint32_t)(sb * 64 + row) * (uint32_t)(xrow * 2) + c8 * 16 : 0x80000000u;
      px[c] = buf_load16(s <= rb ? rx : ry, off);
    }
    const int64_t kh = (int64_t)k * H + h;
    const uint32_t to = tid < Q ? (uint32_t)tid * 4u : 0x80000000u;
    pa = buf_load_f32(make_rsrc(acs + kh * Q, (uint32_t)(Q * 4)), to);
    pd = buf_load_f32(make_rsrc(delta + kh * Q, (uint32_t)(Q * 4)), to);
  };
  // R and K of head h from the reduction arrays (after a barrier)
  auto write_rk = [&](int h) {
    const int64_t kh = (int64_t)k * H + h;
    if (tid < 64) {
      if (t0 + tid < len) Rf[kh * Q + t0 + tid] = redr[0][tid] + redr[1][tid];
    } else if (tid < 128) {
      const int j = tid - 64;
      if (t0 + j < len)
        Kf[kh * Q + t0 + j] =
            ((redkd[0][j] + redkd[1][j]) + (redkd[2][j] + redkd[3][j])) + (redkc[0][j] + redkc[1][j]);
    }
  };

  uint16_t* blk = lds;
  load_a(g * hpg);
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    __syncthreads();  // every wave is done with the previous head's blocks and sums
    if (hh > 0) write_rk(h - 1);
#pragma unroll
    for (int c = 0; c < S::NPA; ++c) {
      const int e = tid + c * 512;
      const int s = e / (64 * PER), rem = e % (64 * PER), row = rem / PER, c8 = rem % PER;
      if (s <= T) *(u32x4*)(blk + (s * 64 + row) * LX + c8 * 8) = px[c];
    }
    if (tid < Q) {
      sa[tid] = pa;
      sd[tid] = pd;
    }
    __syncthreads();
    if (hh + 1 < hpg) load_a(h + 1);  // in flight during this head's products

    // Per-lane indices (and a zero LDS base) made opaque once per head: the masks,
    // factors and LDS addresses below are then formed where they are used, not
    // hoisted out of the head loop, where they held ~100 registers; the bf16 pairs
    // of CB stay packed.
    int rowv = rowA, colv = 16 * (2 * wc) + r, arv = 16 * wr + r, z = 0;
    asm volatile("" : "+v"(rowv), "+v"(colv), "+v"(arv), "+v"(z));
    const float* sa_ = sa + z;  // (LDS addresses from one opaque base plus immediates)
    const float* sd_ = sd + z;
    const uint16_t* blk_ = blk + z;
#pragma unroll
    for (int s = 0; s < TMF; ++s)
#pragma unroll
      for (int c = 0; c < 2; ++c) asm volatile("" : "+v"(cbp[s][c][0]), "+v"(cbp[s][c][1]));
    float ai[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) ai[rr] = sa_[t0 + rowv + rr];
    float Rl[4] = {0.f, 0.f, 0.f, 0.f}, Kc[4] = {0.f, 0.f, 0.f, 0.f}, Kd[2] = {0.f, 0.f};
#pragma unroll
    for (int s = 0; s < TMF; ++s) {
      if (s < nT) {  // (T <= TMF; tiles past the chunk's last token are zero)
        const uint16_t* bt = blk_ + s * 64 * LX;
        const uint16_t* arow = blk_ + (s <= rb ? T : rb) * 64 * LX + arv * LX + q * 8;
        bf16x8 fa[P / 32];
#pragma unroll
        for (int kb = 0; kb < P / 32; ++kb) fa[kb] = as_bf16x8(*(const u32x4*)(arow + kb * 32));
        f32x4 d[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          d[c] = f32x4{0.f, 0.f, 0.f, 0.f};
          const uint16_t* brow_ = bt + (colv + 16 * c) * LX + q * 8;
#pragma unroll
          for (int kb = 0; kb < P / 32; ++kb)
            d[c] = mfma_bf16(fa[kb], as_bf16x8(*(const u32x4*)(brow_ + kb * 32)), d[c]);
        }
        if (s < rb) {
          // off-diagonal row tile (b, s): anchor e = s's last token, e < i for every row
          const float ae = sa_[s * 64 + 63];
          float rho[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) rho[rr] = (t0 + rowv + rr < len) ? exp2_fast(ai[rr] - ae) : 0.f;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int tc = s * 64 + colv + 16 * c;
            const float gam = exp2_fast(ae - sa_[tc]) * sd_[tc];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const float v = d[c][rr] * rho[rr] * gam;
              sum[s][c][rr] += v;
              Rl[rr] = fmaf(v, cbv(s, c, rr), Rl[rr]);
            }
          }
        } else if (s == rb) {
          // diagonal tile: one exp per element, the causal mask j <= i < len
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int tc = s * 64 + colv + 16 * c;
            const float aj = sa_[tc], dj = sd_[tc];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int i = t0 + rowv + rr;
              float v = d[c][rr] * exp2_fast(ai[rr] - aj) * dj;
              v = (tc <= i && i < len) ? v : 0.f;
              sum[s][c][rr] += v;
              Rl[rr] = fmaf(v, cbv(s, c, rr), Rl[rr]);
              Kd[c] = fmaf(v, cbv(s, c, rr), Kd[c]);
            }
          }
        } else {
          // column tile (s, b), transposed: d[c][rr] = dy_i . x_j at j = row rr, i = tc;
          // anchor e = block b's last token (the tile exists only when b is whole)
          const float ae = sa_[t0 + 63];
          float gj[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) gj[rr] = exp2_fast(ae - ai[rr]) * sd_[t0 + rowv + rr];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int tc = s * 64 + colv + 16 * c;
            const float rho = tc < len ? exp2_fast(sa_[tc] - ae) : 0.f;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const float v = d[c][rr] * rho * gj[rr];
              sum[s][c][rr] += v;
              Kc[rr] = fmaf(v, cbv(s, c, rr), Kc[rr]);
            }
          }
        }
      }
    }
    {
      // row sums over the wave's 32 columns: lane r ends with row rowA + r/4
      const float rv = row_reduce_scatter4(Rl[0], Rl[1], Rl[2], Rl[3], r);
      const float kv = row_reduce_scatter4(Kc[0], Kc[1], Kc[2], Kc[3], r);
      if ((r & 3) == 0) {
        redr[wc][z + rowv + (r >> 2)] = rv;
        redkc[wc][z + rowv + (r >> 2)] = kv;
      }
      // the diagonal tile's column sums over the wave's 16 rows
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float kd = Kd[c];
        kd += __shfl_xor(kd, 16);
        kd += __shfl_xor(kd, 32);
        if (q == 0) redkd[wr][z + colv + 16 * c] = kd;
      }
    }
  }
  __syncthreads();  // every wave is done with the blocks; the last head's sums are in
  write_rk(g * hpg + hpg - 1);

  // ------------------------------------------------------------------ B ----
  // dCB_g tiles to LDS in bf16, [i][j] inside each tile (column tiles transposed back)
  uint16_t* dct = lds;
#pragma unroll
  for (int s = 0; s < TMF; ++s) {
    if (s >= T) break;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint16_t v = f2bf(sum[s][c][rr]);
        if (s <= rb)
          dct[s * 64 * LT + (rowA + rr) * LT + ccol(c)] = v;
        else
          dct[s * 64 * LT + ccol(c) * LT + rowA + rr] = v;
      }
  }
  const bool dcw = wc == 0;  // waves 0-3: dC rows; waves 4-7: dB rows
  f32x4 acc[N / 16];         // acc[nb][rr] = (dC or dB)[row1][pcol(nb, 4 q + rr)]
#pragma unroll
  for (int nb = 0; nb < N / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    uint16_t* bt = lds + S::SZT;
    uint16_t* ct = bt + 64 * LDB;
    const uint16_t* bb = Bm + (int64_t)ci.start * brow + (int64_t)g * N;
    const uint16_t* cb = Cm + (int64_t)ci.start * brow + (int64_t)g * N;
    const int nsteps = max(rb + 1, nT - rb);
    const int i0 = t0 + 16 * wr;  // this wave's first row
    for (int st = 0; st < nsteps; ++st) {
      // step st: B block st (dC) and C block b + st (dB), loaded together
      const int jb = st, it = rb + st;
      RowTile<64, N, 512, true> btile, ctile;
      btile.load(bb + (int64_t)jb * 64 * brow, brow, jb <= rb ? len - jb * 64 : 0, tid);
      ctile.load(cb + (int64_t)it * 64 * brow, brow, it < nT ? len - it * 64 : 0, tid);
      __syncthreads();  // every wave is done with the previous blocks (and the tiles are in)
      btile.store(bt, LDB, tid);
      ctile.store(ct, LDB, tid);
      __syncthreads();
      if (dcw) {
        if (jb <= rb) {
          const int jend = min(jb * 64 + 64, i0 + 16);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if (jb * 64 + 32 * u >= jend) break;
            const bf16x8 a = as_bf16x8(*(const u32x4*)(dct + jb * 64 * LT + (16 * wr + r) * LT + 32 * u + q * 8));
#pragma unroll
            for (int nb = 0; nb < N / 16; ++nb)
              acc[nb] = mfma_bf16(frag_kmajor(bt + 32 * u * LDB + nb * 16, LDB, lane), a, acc[nb]);
          }
        }
      } else if (it < nT) {
        const int ib0 = (it == rb) ? (i0 / 32) * 32 : it * 64;
        for (int ib = ib0; ib < min(it * 64 + 64, len); ib += 32) {
          // a[j][i] = dCB_g[i][j]: tile rows are k = i, the lane's column is row1
          const bf16x8 a = frag_kmajor(dct + it * 64 * LT + (ib - it * 64) * LT + 16 * wr, LT, lane);
#pragma unroll
          for (int nb = 0; nb < N / 16; ++nb)
            acc[nb] = mfma_bf16(frag_kmajor(ct + (ib - it * 64) * LDB + nb * 16, LDB, lane), a, acc[nb]);
        }
      }
    }
  }

  // ------------------------------------------------------------------ C ----
  // Per head, H (dC waves) and dT = dE (dB waves) staged in LDS [p][n] with their
  // column groups permuted; this lane's dy or x row scaled by 2^acs_i or
  // w_j delta_j.  The next head's pieces, row and scalars are loaded during this
  // head's products.
  const brsrc rcm = make_rsrc(Cm + (int64_t)ci.start * brow + (int64_t)g * N, (uint32_t)(len * brow * 2));
  const uint32_t ro = (uint32_t)row1 * (uint32_t)(brow * 2) + q * 16;
  u32x4 cq[N / 32];  // C_i at this lane's outputs, 8 adjacent per tile pair (dC waves)
#pragma unroll
  for (int s = 0; s < N / 32; ++s) cq[s] = buf_load16(rcm, dcw ? ro + 64 * s : 0x80000000u);
  u32x4 ph[S::NPC], pe[S::NPC], pr[P / 32];
  float pl = 0.f, pj = 0.f, pdl = 0.f;
  auto load_c = [&](int h) {
    const int64_t kh = (int64_t)k * H + h;
    const brsrc rh = make_rsrc(Hs + kh * (int64_t)(P * N), (uint32_t)(P * N * 2));
    const brsrc re = make_rsrc(dE + kh * (int64_t)(P * N), (uint32_t)(P * N * 2));
#pragma unroll
    for (int c = 0; c < S::NPC; ++c) {
      const int e = (tid + c * 512) * 8;
      const uint32_t off = e < P * N ? (uint32_t)e * 2u : 0x80000000u;
      ph[c] = buf_load16(rh, off);
      pe[c] = buf_load16(re, off);
    }
    const brsrc rrow = make_rsrc((dcw ? DY : X) + (int64_t)ci.start * xrow + (int64_t)h * P,
                                 (uint32_t)(len * xrow * 2));
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb) pr[kb] = buf_load16(rrow, xo1 + 64 * kb);
    const brsrc ra = make_rsrc(acs + kh * Q, (uint32_t)(len * 4));
    pl = buf_load_f32(ra, (uint32_t)(len - 1) * 4u);
    pj = buf_load_f32(ra, (uint32_t)row1 * 4u);
    pdl = buf_load_f32(make_rsrc(delta + kh * Q, (uint32_t)(len * 4)), (uint32_t)row1 * 4u);
  };
  __syncthreads();  // every wave is done with the B and C blocks and the dCB tiles
  load_c(g * hpg);
  const bool rowok = row1 < len;
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const int64_t kh = (int64_t)k * H + h;
    uint16_t* ht = lds + (S::NBUF == 2 ? (hh & 1) * S::SZC1 : 0);
    uint16_t* et = ht + P * LDB;
    if (S::NBUF == 1 && hh > 0) __syncthreads();  // one buffer: the previous head is read
#pragma unroll
    for (int c = 0; c < S::NPC; ++c) {
      const int e = (tid + c * 512) * 8;
      if (e < P * N) {
        lds_piece<true>(ht + (e / N) * LDB, (e % N) / 8, ph[c]);
        lds_piece<true>(et + (e / N) * LDB, (e % N) / 8, pe[c]);
      }
    }
    __syncthreads();
    // dC waves: dy_i 2^acs_i; dB waves: x_j 2^(acs_last - acs_j) delta_j
    const float sc = rowok ? (dcw ? exp2_fast(pj) : exp2_fast(pl - pj) * pdl) : 0.f;
    bf16x8 as_[P / 32];
#pragma unroll
    for (int kb = 0; kb < P / 32; ++kb) {
      u32x4 sv;
#pragma unroll
      for (int d = 0; d < 4; ++d) sv[d] = pack_bf2(bf_lo(pr[kb][d]) * sc, bf_hi(pr[kb][d]) * sc);
      as_[kb] = as_bf16x8(sv);
    }
    if (hh + 1 < hpg) load_c(h + 1);  // in flight during this head's products
    if (dcw) {
      float rsum = 0.f;
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) {
        f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < P / 32; ++kb)
          t = mfma_bf16(frag_kmajor(ht + kb * 32 * LDB + nb * 16, LDB, lane), as_[kb], t);
        const uint32_t c0 = cq[nb >> 1][2 * (nb & 1)], c1 = cq[nb >> 1][2 * (nb & 1) + 1];
        rsum += bf_lo(c0) * t[0] + bf_hi(c0) * t[1] + bf_lo(c1) * t[2] + bf_hi(c1) * t[3];
        acc[nb] += t;
      }
      rsum += __shfl_xor(rsum, 16);
      rsum += __shfl_xor(rsum, 32);
      if (q == 0 && rowok) rout[kh * Q + row1] = rsum;
    } else {
#pragma unroll
      for (int kb = 0; kb < P / 32; ++kb)
#pragma unroll
        for (int nb = 0; nb < N / 16; ++nb)
          acc[nb] = mfma_bf16(frag_kmajor(et + kb * 32 * LDB + nb * 16, LDB, lane), as_[kb], acc[nb]);
    }
  }
  const brsrc rout_ = make_rsrc((dcw ? dC : dB) + (int64_t)ci.start * brow + (int64_t)g * N,
                                (uint32_t)(len * brow * 2));
#pragma unroll
  for (int s = 0; s < N / 32; ++s) buf_store16(rout_, ro + 64 * s, pack_bf8(acc[2 * s], acc[2 * s + 1]));
}

template <int P, int N>
static void launch_dbc(const Prob& p, const BwdArgs& a, hipStream_t st) {
  const int T = p.Q / 64;
  hipLaunchKernelGGL((bwd_dbc_bf16_kernel<P, N>), dim3((unsigned)(p.nck * p.G * T)), dim3(512), 0, st,
                     p.map, p.H, p.G, (const uint16_t*)a.x, (const uint16_t*)a.dout,
                     (const uint16_t*)a.B, (const uint16_t*)a.C, (const uint16_t*)a.CB, a.delta,
                     a.acs, (const uint16_t*)a.Hp, (const uint16_t*)a.dE, (uint16_t*)a.dB,
                     (uint16_t*)a.dC, a.rR, a.Rp, a.Kp);
}

bool bwd_fused_supported(const Prob& p) { return bf16_kernels(p) && p.Q <= QMAXF && p.P >= 32 && p.N >= 32; }

hipError_t launch_bwd_dbc(const Prob& p, const BwdArgs& a, hipStream_t st) {
  if (p.nck == 0) return hipSuccess;
#define SSD_DBC_CASE(PP, NN) \
  if (p.P == PP && p.N == NN) { launch_dbc<PP, NN>(p, a, st); return hipGetLastError(); }
  SSD_DBC_CASE(32, 32) SSD_DBC_CASE(32, 64) SSD_DBC_CASE(32, 128)
  SSD_DBC_CASE(64, 32) SSD_DBC_CASE(64, 64) SSD_DBC_CASE(64, 128)
  SSD_DBC_CASE(128, 32) SSD_DBC_CASE(128, 64) SSD_DBC_CASE(128, 128)
#undef SSD_DBC_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
