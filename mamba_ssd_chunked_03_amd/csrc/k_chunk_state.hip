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
// index, the slow index of both operands in memory, while the MFMA wants 8
// consecutive k values per lane.  Slices of 64 tokens are copied into LDS in
// their natural token-major layout with 16-byte moves and the fragments are
// read with the gfx950 transpose read (ds_read_b64_tr_b16), which hands each
// lane 8 consecutive tokens of one column.  The next slice's global loads are
// issued before the current slice's MFMAs, so memory latency overlaps compute.
// The scaled operand is split into bf16 hi + lo parts (two MFMAs) so the chunk
// state keeps ~16 bits of precision; the states feed the fp32 final states.
// Four wavefronts per head, each a (P/2) x (N/2) tile of 16x16 blocks.  Where a
// group has an even number of heads and the tiles fit, one workgroup holds two
// heads of a group (eight wavefronts): the second operand (B, or C) is the
// group's, so each slice of it is loaded and staged once for both heads, which
// halves the L2 read requests for it.
//
// kStateFwdCumsum also forms stage 1 for its (chunk, head) first: wave w scans
// tokens 64w .. 64w + 63 (delta, then the inclusive sum of delta A in log2
// units) and adds the totals of the waves before it in order, which is the
// cumsum kernel's pass-by-pass carry, so delta, acs and the chunk decay come out
// with the same bits.  They are written for the later stages, and the token
// scales are formed from the values in registers (no second read).
//
// With two heads per workgroup, kStateFwdCumsum can also form the chunk's
// C.B^T (the input of the output stage) from the same staged B slices: where a
// group's head pairs are as many as the chunk's 64-row blocks (8 heads per group,
// chunk 256), pair ib forms row block ib, in both orientations (the backward
// reads the transpose), and no separate C.B^T kernel runs.
//
// fp32 path: k_f32.hip (fp32 matrix cores, no rounding of any operand).
#include "internal.hpp"

namespace ssd {

static_assert(sizeof(ChunkStateT) == 4 && (ChunkStateT)0.5f == 0.5f,
              "the chunk states and their adjoints are written here as fp32 (float4 stores)");

constexpr int QMAX_STATE = 256;  // largest chunk size: one token per thread of a head

// MODE (kStateFwd / kStateDstates) is a template argument so that profiles
// tell the forward chunk states and the backward adjoint states apart.
// Stage-1 inputs of kStateFwdCumsum (unused by the other modes).
struct CumsumIn {
  const float *dt, *dt_bias, *A;
  int softplus;
  float* decay;
  // C.B^T formed here too when C is set (two heads per workgroup, a group's
  // head pairs one per 64-row block of the chunk): CB[i][j], and CBt[j][i] if set
  const uint16_t* C;
  uint16_t *CB, *CBt;
};

template <int P, int N, int MODE, int HP>
__global__ __launch_bounds__(256 * HP, 4) void chunk_state_bf16_kernel(ChunkMap m, int H, int G,
                                                               const uint16_t* __restrict__ X,
                                                               const uint16_t* __restrict__ Y,
                                                               float* __restrict__ delta,
                                                               float* __restrict__ acs,
                                                               float* __restrict__ out, CumsumIn cs) {
  constexpr int KS = 64;       // tokens per LDS slice
  constexpr int LDX = P + 16;  // row strides: odd multiples of 32 bytes for the transpose reads
  constexpr int LDY = N + 16;
  constexpr int WM = 2, WN = 2;
  constexpr int TM = P / 16 / WM, TN = N / 16 / WN;
  constexpr int XC = KS * (P / 8) / 256;  // 16-byte chunks per thread per slice
  constexpr int YC = KS * (N / 8) / (256 * HP);  // shared operand: pieces per thread of the workgroup
  static_assert(TM >= 1 && TN >= 1 && XC >= 1 && YC >= 1 && KS * (N / 8) % (256 * HP) == 0,
                "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t xh_[HP][KS * LDX];
  __shared__ __attribute__((aligned(16))) uint16_t xl_[HP][KS * LDX];
  __shared__ __attribute__((aligned(16))) uint16_t ys[KS * LDY];
  __shared__ float sc_[HP][256];
  // C.B^T tile staging (see below): both orientations, so that every store
  // instruction writes whole 128-byte rows
  constexpr bool kCanFuseCB = MODE == kStateFwdCumsum && HP == 2;
  constexpr int LT = 64 + 8;
  __shared__ __attribute__((aligned(16))) uint16_t tcb[kCanFuseCB ? 64 * LT : 1];
  __shared__ __attribute__((aligned(16))) uint16_t tcbt[kCanFuseCB ? 64 * LT : 1];

  int k, h;
  chunk_head(H / HP, k, h);
  const int half = HP == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / 256);
  h = h * HP + half;
  uint16_t* xh = xh_[half];
  uint16_t* xl = xl_[half];
  float* sc = sc_[half];
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int Q = m.Q, len = ci.len;
  const int g = h / (H / G);
  // tid: thread of this head's four wavefronts; gid: thread of the workgroup
  const int gid = threadIdx.x, tid = HP == 1 ? gid : gid % 256, w = tid >> 6, lane = tid & 63;
  const int64_t kh = (int64_t)k * H + h;
  const int64_t xrow = (int64_t)H * P, yrow = (int64_t)G * N;
  const uint16_t* xb = X + (int64_t)ci.start * xrow + (int64_t)h * P;
  const uint16_t* yb = Y + (int64_t)ci.start * yrow + (int64_t)g * N;

  const int wm = w / WN, wn = w % WN;
  const int p0 = wm * (P / WM), n0 = wn * (N / WN);
  const int r = lane & 15;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Buffer resources over the chunk's valid rows: rows past its end read as
  // zero, with no branch (a load under a branch can leave its register shared
  // with the other path's zero, whose move then waits for the load).
  const brsrc rx = make_rsrc(xb, (uint32_t)(len * xrow * 2)), ry = make_rsrc(yb, (uint32_t)(len * yrow * 2));
  u32x4 xr[XC], yr[YC];
  auto load_slice = [&](int s0) {
#pragma unroll
    for (int c = 0; c < XC; ++c) {
      const int e = tid + c * 256, j = s0 + e / (P / 8), c8 = e % (P / 8);
      xr[c] = buf_load16(rx, (uint32_t)j * (uint32_t)(xrow * 2) + c8 * 16);
    }
#pragma unroll
    for (int c = 0; c < YC; ++c) {
      const int e = gid + c * 256 * HP, j = s0 + e / (N / 8), c8 = e % (N / 8);
      yr[c] = buf_load16(ry, (uint32_t)j * (uint32_t)(yrow * 2) + c8 * 16);
    }
  };
  // kStateFwdCumsum: this thread's token (256 threads, chunks of at most 256
  // tokens; wave w holds the cumsum's pass w).  Its dt is loaded before the
  // first slice, so that waiting for it does not also wait for the slice (the
  // memory counter completes in order).
  // The other modes load this thread's acs (and delta, and the chunk's last acs)
  // the same way.  Range-checked buffer loads: tokens past the chunk's end read
  // as zero, with no branch.
  const int t = tid;
  const bool in = t < len;
  float dtv = 0.f, acv = 0.f, dlv = 0.f, alv = 0.f;
  if constexpr (MODE == kStateFwdCumsum) {
    const brsrc rdt = make_rsrc(cs.dt + (int64_t)ci.start * H + h, (uint32_t)(len * H * 4));
    dtv = buf_load_f32(rdt, (uint32_t)(t * H * 4));
  } else {
    const brsrc ra = make_rsrc(acs + kh * Q, (uint32_t)(len * 4));
    acv = buf_load_f32(ra, (uint32_t)(t * 4));
    if constexpr (MODE == kStateFwd) {
      const brsrc rd = make_rsrc(delta + kh * Q, (uint32_t)(len * 4));
      dlv = buf_load_f32(rd, (uint32_t)(t * 4));
      alv = buf_load_f32(ra, (uint32_t)((len - 1) * 4));
    }
  }
  // (kept ahead of the slice's loads: the scheduler would otherwise sink them
  // below, and waiting for them would then wait for the slice too)
  __builtin_amdgcn_sched_barrier(0);
  load_slice(0);  // independent of the token scales: in flight while they are formed
  // C.B^T (kStateFwdCumsum with two heads): this workgroup's head pair is pair ib
  // of its group, and it forms row block ib (rows 64 ib .. 64 ib + 63) of the
  // chunk's C.B^T from each staged B slice j <= ib: wave w8 owns rows
  // 64 ib + 16 (w8 % 4) + 0..15 and columns 32 (w8 / 4) .. +31 of each 64 x 64
  // tile, and holds its 16 C rows as MFMA fragments for the whole chunk.
  const bool fuse_cb = kCanFuseCB && cs.C != nullptr;
  const int lq = lane >> 4, w8 = gid >> 6, ri = w8 & 3, cj = w8 >> 2;
  const int ib = ((h % (H / G)) / HP);
  u32x4 cfr[N / 32];
  if constexpr (kCanFuseCB) {
    if (fuse_cb) {
      const brsrc rcm = make_rsrc(cs.C + (int64_t)ci.start * yrow + (int64_t)g * N, (uint32_t)(len * yrow * 2));
      const uint32_t co = (uint32_t)(ib * 64 + ri * 16 + r) * (uint32_t)(yrow * 2) + lq * 16;
#pragma unroll
      for (int kk = 0; kk < N / 32; ++kk) cfr[kk] = buf_load16(rcm, co + 64 * kk);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // (and all issued before the first wait)
  if constexpr (MODE == kStateFwdCumsum) {
    __shared__ float wtot_[HP][4], alast_[HP];
    float* wtot = wtot_[half];
    float& alast = alast_[half];
    const float bias = cs.dt_bias ? cs.dt_bias[h] : 0.f;
    const float a2 = cs.A[h] * kLog2e;
    const float d = token_delta(dtv, bias, cs.softplus, in);
    const float sw = wave_inclusive_sum(scan_input(d, a2));
    if (lane == 63) wtot[w] = sw;
    __syncthreads();
    float carry = 0.f;
    for (int v = 0; v < w; ++v) carry = wtot[v] + carry;
    const float incl = sw + carry;
    if (t < Q) {
      delta[kh * Q + t] = d;
      acs[kh * Q + t] = in ? incl : 0.f;
    }
    if (t == len - 1) {
      cs.decay[kh] = incl;
      alast = incl;
    }
    __syncthreads();
    if (t < Q) sc[t] = in ? d * exp2_fast(alast - incl) : 0.f;
  } else {
    // (every thread writes its entry, so the loads above are not sunk into a branch)
    const float v = MODE == kStateFwd ? dlv * exp2_fast(alv - acv) : exp2_fast(acv);
    sc[t] = in ? v : 0.f;
  }
  __syncthreads();
  for (int s0 = 0; s0 < len; s0 += KS) {
#pragma unroll
    for (int c = 0; c < XC; ++c) {
      const int e = tid + c * 256, jj = e / (P / 8), c8 = e % (P / 8);
      const float sv = sc[s0 + jj];
      u32x4 hi, lo;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float v0 = bf_lo(xr[c][d]) * sv, v1 = bf_hi(xr[c][d]) * sv;
        hi[d] = pack_bf2(v0, v1);
        lo[d] = pack_bf2(v0 - bf_lo(hi[d]), v1 - bf_hi(hi[d]));
      }
      *(u32x4*)(xh + jj * LDX + c8 * 8) = hi;
      *(u32x4*)(xl + jj * LDX + c8 * 8) = lo;
    }
#pragma unroll
    for (int c = 0; c < YC; ++c) {
      const int e = gid + c * 256 * HP, jj = e / (N / 8), c8 = e % (N / 8);
      *(u32x4*)(ys + jj * LDY + c8 * 8) = yr[c];
    }
    __syncthreads();
    if (s0 + KS < len) load_slice(s0 + KS);  // in flight during the MFMAs below
#pragma unroll
    for (int kk = 0; kk < KS; kk += 32) {
      bf16x8 ah[TM], al[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        ah[i] = frag_kmajor(xh + kk * LDX + p0 + i * 16, LDX, lane);
        al[i] = frag_kmajor(xl + kk * LDX + p0 + i * 16, LDX, lane);
      }
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) bv[jj] = frag_kmajor(ys + kk * LDY + n0 + jj * 16, LDY, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) {
          acc[i][jj] = mfma_bf16(bv[jj], ah[i], acc[i][jj]);
          acc[i][jj] = mfma_bf16(bv[jj], al[i], acc[i][jj]);
        }
    }
    if constexpr (kCanFuseCB) {
      // tile (ib, s0 / 64) of C.B^T from this slice of B (rows of ys, dstate
      // contiguous, so the fragments are plain 16-byte LDS reads).  Both
      // orientations come from the MFMA: with B as the first operand, lane
      // (lq, r) holds CB[i = r][j = 4 lq .. +3] of its 16 x 16 block, with C
      // first CB[i = 4 lq .. +3][j = r], i.e. CBt[j][i .. i + 3].  The two
      // 64 x 64 tiles go through LDS, then each thread stores one 16-byte piece
      // of each in fragment order (common.hpp, cbf_off): wave f writes block
      // (f / 2, f % 2) of each tile, 1 KB contiguous per store instruction.
      if (fuse_cb && s0 / KS <= ib) {
        const int il = ri * 16;
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
          const int jl = cj * 32 + bj * 16;
          f32x4 d1 = f32x4{0.f, 0.f, 0.f, 0.f}, d2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < N / 32; ++kk) {
            const bf16x8 bfr = as_bf16x8(*(const u32x4*)(ys + (jl + r) * LDY + kk * 32 + lq * 8));
            d1 = mfma_bf16(bfr, as_bf16x8(cfr[kk]), d1);
            d2 = mfma_bf16(as_bf16x8(cfr[kk]), bfr, d2);
          }
          *(uint2*)(tcb + (il + r) * LT + jl + 4 * lq) = make_uint2(pack_bf2(d1[0], d1[1]), pack_bf2(d1[2], d1[3]));
          *(uint2*)(tcbt + (jl + r) * LT + il + 4 * lq) = make_uint2(pack_bf2(d2[0], d2[1]), pack_bf2(d2[2], d2[3]));
        }
        __syncthreads();
        const int64_t kg = (int64_t)k * G + g;
        // 512 threads: 8 blocks of 16 rows x 32 columns, lane (q, r) = row r, columns 8q .. +7
        const int f = gid >> 6, fl = gid & 63, rr = f >> 1, cc = f & 1, fq = fl >> 4, fr = fl & 15;
        const int lo = (rr * 16 + fr) * LT + cc * 32 + fq * 8;
        *(u32x4*)((char*)(cs.CB + kg * Q * Q) + cbf_piece(ib * 4 + rr, s0 / 32 + cc, fl, Q)) = *(const u32x4*)(tcb + lo);
        if (cs.CBt)
          *(u32x4*)((char*)(cs.CBt + kg * Q * Q) + cbf_piece(s0 / 16 + rr, ib * 2 + cc, fl, Q)) = *(const u32x4*)(tcbt + lo);
      }
    }
    __syncthreads();
  }
  // operands were swapped: acc[i][jj][rr] = T[p0 + 16 i + r][n0 + 16 jj + 4 q + rr], so each
  // lane stores 16 contiguous bytes
  const int q = lane >> 4;
  float* ob = out + kh * (int64_t)(P * N);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jj = 0; jj < TN; ++jj)
      *(float4*)(ob + (p0 + i * 16 + r) * N + n0 + jj * 16 + q * 4) =
          make_float4(acc[i][jj][0], acc[i][jj][1], acc[i][jj][2], acc[i][jj][3]);
}

template <int P, int N, int HP>
static void launch_cs_hp(const Prob& p, const void* X, const void* Y, float* delta, float* acs,
                         float* out, int mode, const CumsumIn& cs, hipStream_t st) {
  const dim3 grid((unsigned)(p.nck * (p.H / HP)));  // (chunk, head group of HP) in the XCD-aware order
  const dim3 block(256 * HP);
  const uint16_t *x = (const uint16_t*)X, *y = (const uint16_t*)Y;
  if (mode == kStateFwd)
    hipLaunchKernelGGL((chunk_state_bf16_kernel<P, N, kStateFwd, HP>), grid, block, 0, st, p.map, p.H,
                       p.G, x, y, delta, acs, out, cs);
  else if (mode == kStateDstates)
    hipLaunchKernelGGL((chunk_state_bf16_kernel<P, N, kStateDstates, HP>), grid, block, 0, st, p.map,
                       p.H, p.G, x, y, delta, acs, out, cs);
  else
    hipLaunchKernelGGL((chunk_state_bf16_kernel<P, N, kStateFwdCumsum, HP>), grid, block, 0, st, p.map,
                       p.H, p.G, x, y, delta, acs, out, cs);
}

// LDS bytes of a chunk-state workgroup holding hp heads (the arrays above)
constexpr int cs_lds_bytes(int P, int N, int hp) {
  return hp * (2 * 64 * (P + 16) * 2 + 256 * 4 + 5 * 4) + 64 * (N + 16) * 2;
}

// two heads per workgroup need the shared operand to split evenly over 512
// threads and two such workgroups to fit a CU's LDS
constexpr bool cs_two_ok(int P, int N) { return 64 * (N / 8) % 512 == 0 && cs_lds_bytes(P, N, 2) <= 80 * 1024; }

template <int P, int N>
static void launch_cs_bf16(const Prob& p, const void* X, const void* Y, float* delta, float* acs,
                           float* out, int mode, const CumsumIn& cs, hipStream_t st) {
  if constexpr (cs_two_ok(P, N)) {
    if (cs_variant_for(p) >= kCsTwoHeads) return launch_cs_hp<P, N, 2>(p, X, Y, delta, acs, out, mode, cs, st);
  }
  if (cs.C) return;  // C.B^T is formed only by the two-head kernel (cb_in_chunk_state)
  launch_cs_hp<P, N, 1>(p, X, Y, delta, acs, out, mode, cs, st);
}

static hipError_t launch_cs(const Prob& p, const void* X, const void* Y, float* delta, float* acs,
                            float* out, int mode, const CumsumIn& cs, hipStream_t st) {
#define SSD_CS_CASE(PP, NN) \
  if (p.P == PP && p.N == NN) { launch_cs_bf16<PP, NN>(p, X, Y, delta, acs, out, mode, cs, st); return hipGetLastError(); }
  SSD_CS_CASE(32, 32) SSD_CS_CASE(32, 64) SSD_CS_CASE(32, 128)
  SSD_CS_CASE(64, 32) SSD_CS_CASE(64, 64) SSD_CS_CASE(64, 128)
  SSD_CS_CASE(128, 32) SSD_CS_CASE(128, 64) SSD_CS_CASE(128, 128)
#undef SSD_CS_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_state(const Prob& p, const void* X, const void* Y, const float* delta,
                              const float* acs, float* out, int mode, hipStream_t st) {
  if (p.nck == 0) return hipSuccess;
  if (!bf16_kernels(p)) return launch_chunk_state_f32(p, X, Y, delta, acs, out, mode, st);
  if (p.Q > QMAX_STATE) return hipErrorInvalidValue;  // one token per thread
  // (the kStateFwd and kStateDstates modes only read delta and acs)
  return launch_cs(p, X, Y, const_cast<float*>(delta), const_cast<float*>(acs), out, mode, CumsumIn{}, st);
}

bool cs_variant_valid(const Prob& p, int v) {
  if (v == kCsOneHead) return true;
  if (!bf16_kernels(p) || p.G <= 0 || (v != kCsTwoHeads && v != kCsTwoHeadsCB)) return false;
  const int hpg = p.H / p.G;
  if (hpg % 2 || !cs_two_ok(p.P, p.N)) return false;
  // C.B^T inside: chunks of four 64-row blocks and four head pairs per group
  return v == kCsTwoHeads || (p.Q == 256 && hpg == 8);
}

// The tuned table's chunk-state rows, measured by tuning/sweep.py and turned into
// tuned_cs.inc by build.py (an empty table leaves the widest valid form).
struct CsEntry {
  int32_t P, N, hpg, Q;  // headdim, dstate, heads per group, chunk size of the measured shape
  int32_t variant;       // the fastest forward there (kCsOneHead .. kCsTwoHeadsCB)
};
#if __has_include("tuned_cs.inc")
#include "tuned_cs.inc"
#else
static const CsEntry kTunedCs[] = {{0, 0, 0, 0, 0}};
static const int kTunedCsCount = 0;
#endif

int cs_variant_for(const Prob& p) {
  const int f = (p.flags >> kCsVariantShift) & 3;
  if (f != kCsTable) return f;  // (make_prob refuses a variant the problem cannot run)
  if (!bf16_kernels(p) || p.G <= 0) return kCsOneHead;
  const int hpg = p.H / p.G;
  for (int i = 0; i < kTunedCsCount; ++i) {
    const CsEntry& e = kTunedCs[i];
    if (e.P == p.P && e.N == p.N && e.hpg == hpg && e.Q == p.Q && cs_variant_valid(p, e.variant))
      return e.variant;
  }
  for (int v = kCsTwoHeadsCB; v > kCsOneHead; --v)
    if (cs_variant_valid(p, v)) return v;
  return kCsOneHead;
}

bool cb_in_chunk_state(const Prob& p) { return bf16_kernels(p) && cs_variant_for(p) == kCsTwoHeadsCB; }

hipError_t launch_cumsum_chunk_state(const Prob& p, const void* X, const void* Bm, const float* dt,
                                     const float* dt_bias, const float* A, float* delta, float* acs,
                                     float* decay, float* T, hipStream_t st, const void* C, void* CB,
                                     void* CBt) {
  if (p.nck == 0) return hipSuccess;
  if (C && !cb_in_chunk_state(p)) return hipErrorInvalidValue;
  if (!bf16_kernels(p) || p.Q > 256) {
    const hipError_t e = launch_chunk_cumsum(p, dt, dt_bias, A, delta, acs, decay, st);
    if (e != hipSuccess) return e;
    return launch_chunk_state(p, X, Bm, delta, acs, T, kStateFwd, st);
  }
  const CumsumIn cs{dt, dt_bias, A, p.softplus, decay, (const uint16_t*)C, C ? (uint16_t*)CB : nullptr,
                    C ? (uint16_t*)CBt : nullptr};
  return launch_cs(p, X, Bm, delta, acs, T, kStateFwdCumsum, cs, st);
}

}  // namespace ssd
