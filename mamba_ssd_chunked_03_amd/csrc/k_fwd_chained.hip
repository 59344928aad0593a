// Fused single-pass forward with a chained scan across chunks.
//
// The scan page (gigipick.blogspot.com "LLM Mamba ...") fuses the scan's stages
// to cut global-memory traffic (section 3, "kernel fusion") and keeps the chunk
// carry on chip, one chunk's carry-out seeding the next chunk's carry-in ("memory
// hierarchy").  Here one workgroup per (chunk, head) unit forms the chunk's state
// T_c = sum_j delta_j 2^(acs_last - acs_j) x_j B_j^T, takes the state entering the
// chunk, H_c = E_{c-1}, from the unit of the previous chunk (the chain), publishes
// E_c = 2^(acs_last) H_c + T_c for the next one, and writes the chunk's output
// y = (CB o L o delta) X + 2^acs C H_c^T + D x in the same launch.  Neither the
// chunk states nor the passed states make a round trip through memory; x is read
// once.  C.B^T comes from the C.B^T kernel launched before this one.
//
// Units are handed out by tickets, so that a unit only ever waits for units that
// took their tickets earlier (resident, or done) and every wait ends.  Units go
// to 8 queues by head (a queue's heads together, so a group's C and C.B^T are
// shared in one L2); a workgroup serves the queue of the XCD it runs on first,
// then any other queue that still has units.  Within a queue, tickets run chunk by
// chunk, each sequence's chunks in order.  The carry's hand-off uses the device's
// agent-scope memory model: E_c stored, every wave's stores complete, a
// workgroup barrier, then a release store of the unit's flag; the waiting unit
// spins on relaxed loads of its predecessor's flag (with a bound that records an
// error and goes on, so the kernel always finishes), then an acquire fence before
// reading E_{c-1}.  The flags and ticket counters are cleared by a small kernel
// queued just before.
//
// x is staged once, token-major with permuted column groups (as the output
// stage reads it), and serves as the contraction's second operand for T; the
// per-token scale is applied to B's slices instead of x, split into bf16 hi + lo
// (16-bit-accurate states).  LDS: the x tile, and one region holding first the B
// slices, then H_c in bf16 and the output stage's column factors.
#include "internal.hpp"
#include "scan_rows.hpp"

namespace ssd {

static_assert(sizeof(ChunkStateT) == 4 && (ChunkStateT)0.5f == 0.5f,
              "the carry is read and written as fp32 float4");

struct ChainArgs {
  const uint16_t *x, *B, *C, *CB;
  const float *dt, *dt_bias, *A, *D, *init;
  int softplus;
  uint16_t* y;
  float* final_states;
  float* E;         // (nck, H, P, N) fp32: the carry out of every unit
  int32_t* flags;   // (nck, H): nonzero once that unit's E is published
  int32_t* sync;    // [0, 8) ticket counters of the queues; [8] set when a wait hit its bound
  float *delta, *acs, *decay;  // the saved context (null when not kept)
  uint16_t* Hp;                // passed states in bf16 (null when not kept)
  int32_t nq[8];    // units in each queue
  int32_t nhq[8];   // heads in each queue
  int32_t hpq;      // a queue's heads come in blocks of hpq consecutive heads
  int32_t rows;     // batch rows (batched layout)
};

// Longest wait for a predecessor, in polls (each at least one memory round trip,
// so ~0.1 s; a legitimate wait is at most the chain's latency over the units in
// flight, tens of microseconds).  A unit whose wait runs out records the error,
// goes on and still publishes, so its successors do not wait for it too.
constexpr int kMaxPolls = 1 << 16;

__device__ __forceinline__ int xcc_id() {
  // HW_REG_XCC_ID (register 20), bits 0..3: which XCD this wave runs on
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 7;
}

template <int P, int N>
__global__ __launch_bounds__(kScanWaves * 64, 4) void fwd_chained_kernel(ChunkMap m, int H, int G,
                                                                      ChainArgs a) {
  using Rows = ScanRows<P, N>;
  constexpr int QMAX = Rows::QMAX, LDX = Rows::LDX, HLD = Rows::HLD, NT = kScanWaves * 64;
  constexpr int KS = 64, LDB = N + 16;                 // B slice: 64 tokens, row stride N + 16
  constexpr int TM = P / 32, TN = N / 64;              // 2 x 4 waves over (p, n)
  constexpr int YC = KS * (N / 8) / NT;                // 16-byte B pieces per thread per slice
  static_assert(TM >= 1 && TN >= 1 && YC >= 1 && KS * (N / 8) % NT == 0, "shape");
  constexpr int SLICE_BYTES = 2 * KS * LDB * 2;
  constexpr int SCAN_BYTES = P * HLD * 2 + (QMAX / 32) * QMAX * 4;
  constexpr int UNI = SLICE_BYTES > SCAN_BYTES ? SLICE_BYTES : SCAN_BYTES;
  __shared__ __attribute__((aligned(16))) uint16_t xs[QMAX * LDX];
  __shared__ __attribute__((aligned(16))) char uni[UNI];
  __shared__ float sa[QMAX], sd[QMAX], sc[QMAX];
  __shared__ float wtot[4], alast_s;
  __shared__ int s_unit, s_queue;
  uint16_t* bh = (uint16_t*)uni;                       // phase 1: scaled B slice, hi and lo
  uint16_t* bl = bh + KS * LDB;
  uint16_t* hs = (uint16_t*)uni;                       // phase 2: H_c in bf16, then column factors
  float* vt = (float*)(uni + P * HLD * 2);

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int q4 = lane >> 4, r = lane & 15;
  const int home = __builtin_amdgcn_readfirstlane(xcc_id());
  {
    // ---------------------------------------------------------------- ticket ----
    // As many workgroups as units, one ticket each: a queue's counter passes its
    // unit count only once all its tickets are taken, so a workgroup that found
    // every queue taken would leave a unit to nobody, which one ticket per
    // workgroup and as many workgroups as units rule out.
    if (tid == 0) {
      int got = -1, gq = -1;
      for (int i = 0; i < 8 && got < 0; ++i) {
        const int qq = (home + i) & 7;
        if (a.nq[qq] == 0) continue;
        if (__hip_atomic_load(a.sync + qq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= a.nq[qq])
          continue;
        const int t = __hip_atomic_fetch_add(a.sync + qq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (t < a.nq[qq]) {
          got = t;
          gq = qq;
        }
      }
      s_unit = got;
      s_queue = gq;
    }
    __syncthreads();
    // (uniform: read into scalar registers, so that everything derived from the
    // unit -- chunk, head, pointers, buffer descriptors -- stays scalar)
    const int u = __builtin_amdgcn_readfirstlane(s_unit), qq = __builtin_amdgcn_readfirstlane(s_queue);
    if (u < 0) return;
    // unit -> (chunk slot k, head h): chunk by chunk; batch rows interleaved
    const int nh = a.nhq[qq];
    int k, hi;
    if (!m.packed) {
      const int c = u / (a.rows * nh), rem = u % (a.rows * nh);
      k = (rem / nh) * m.ncs + c;
      hi = rem % nh;
    } else {
      k = u / nh;
      hi = u % nh;
    }
    const int h = (qq + 8 * (hi / a.hpq)) * a.hpq + hi % a.hpq;
    const ChunkInfo ci = chunk_info(m, k);
    if (ci.len <= 0) return;  // an unused packed slot: no successor waits on it
    const int Q = m.Q, len = ci.len;
    const int g = h / (H / G);
    const int64_t kh = (int64_t)k * H + h;
    const int64_t xrow = (int64_t)H * P, yrow = (int64_t)G * N;
    const uint16_t* xb = a.x + (int64_t)ci.start * xrow + (int64_t)h * P;
    const uint16_t* bb = a.B + (int64_t)ci.start * yrow + (int64_t)g * N;

    // ---------------------------------------------- loads, within-chunk cumsum ----
    const bool in = tid < len;
    const brsrc rdt = make_rsrc(a.dt + (int64_t)ci.start * H + h, (uint32_t)(len * H * 4));
    const float dtv = buf_load_f32(rdt, (uint32_t)(tid * H * 4));
    RowTile<QMAX, P, NT, true, true> xt;
    xt.load(xb, xrow, len, tid);
    const brsrc rb = make_rsrc(bb, (uint32_t)(len * yrow * 2));
    u32x4 yr[YC];
    auto load_slice = [&](int s0) {
#pragma unroll
      for (int c = 0; c < YC; ++c) {
        const int e = tid + c * NT, j = s0 + e / (N / 8), c8 = e % (N / 8);
        yr[c] = buf_load16(rb, (uint32_t)j * (uint32_t)(yrow * 2) + c8 * 16);
      }
    };
    load_slice(0);
    {
      // the chunk-state kernel's cumsum, step for step (same bits): wave w < 4 scans
      // tokens 64w .. 64w + 63 and adds the earlier waves' totals in order
      const float bias = a.dt_bias ? a.dt_bias[h] : 0.f;
      const float a2 = a.A[h] * kLog2e;
      const float d = token_delta(dtv, bias, a.softplus, in);
      const float sw = wave_inclusive_sum(scan_input(d, a2));
      if (lane == 63 && w < 4) wtot[w] = sw;
      __syncthreads();
      float carry = 0.f;
      for (int v = 0; v < w && v < 4; ++v) carry = wtot[v] + carry;
      const float incl = sw + carry;
      if (tid < Q) {
        sa[tid] = in ? incl : 0.f;
        sd[tid] = d;
        if (a.delta) {
          a.delta[kh * Q + tid] = d;
          a.acs[kh * Q + tid] = in ? incl : 0.f;
        }
      }
      if (tid == len - 1) {
        alast_s = incl;
        if (a.decay) a.decay[kh] = incl;
      }
      __syncthreads();
      if (tid < Q) sc[tid] = in ? d * exp2_fast(alast_s - incl) : 0.f;
    }
    xt.store(xs, LDX, tid);
    __syncthreads();

    // ------------------------------------------- chunk state T (MFMA, in registers) ----
    // wave w owns p tiles (w & 1) * TM .. +TM-1 (LDS column tiles of the permuted x) and
    // n tiles (w >> 1) * TN .. +TN-1; lane (q4, r) ends up with T[pcol(tp, r)][16 tn + 4 q4 + 0..3]
    const int tp0 = (w & 1) * TM, tn0 = (w >> 1) * TN;
    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < len; s0 += KS) {
#pragma unroll
      for (int c = 0; c < YC; ++c) {
        const int e = tid + c * NT, jj = e / (N / 8), c8 = e % (N / 8);
        const float sv = sc[s0 + jj];
        u32x4 hv, lv;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float v0 = bf_lo(yr[c][d]) * sv, v1 = bf_hi(yr[c][d]) * sv;
          hv[d] = pack_bf2(v0, v1);
          lv[d] = pack_bf2(v0 - bf_lo(hv[d]), v1 - bf_hi(hv[d]));
        }
        *(u32x4*)(bh + jj * LDB + c8 * 8) = hv;
        *(u32x4*)(bl + jj * LDB + c8 * 8) = lv;
      }
      __syncthreads();
      if (s0 + KS < len) load_slice(s0 + KS);  // in flight during the MFMAs below
#pragma unroll
      for (int kk = 0; kk < KS; kk += 32) {
        bf16x8 xf[TM], fh[TN], fl[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) xf[i] = frag_kmajor(xs + (s0 + kk) * LDX + (tp0 + i) * 16, LDX, lane);
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) {
          fh[jj] = frag_kmajor(bh + kk * LDB + (tn0 + jj) * 16, LDB, lane);
          fl[jj] = frag_kmajor(bl + kk * LDB + (tn0 + jj) * 16, LDB, lane);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int jj = 0; jj < TN; ++jj) {
            acc[i][jj] = mfma_bf16(fh[jj], xf[i], acc[i][jj]);
            acc[i][jj] = mfma_bf16(fl[jj], xf[i], acc[i][jj]);
          }
      }
      __syncthreads();
    }

    // ------------------------------------------------------------- the carry ----
    Rows rows;
    rows.xs = xs;
    rows.hs = hs;
    rows.sa = sa;
    rows.sd = sd;
    rows.vt = vt;
    rows.init(a.C + (int64_t)ci.start * yrow + (int64_t)g * N, yrow, a.CB + ((int64_t)k * G + g) * Q * Q,
              a.y + (int64_t)ci.start * xrow + (int64_t)h * P, xrow, Q, len, tid, a.D ? a.D[h] : 0.f);
    const int64_t st_off = kh * (int64_t)(P * N);
    if (!ci.first) {
      if (tid == 0) {
        const int32_t* f = a.flags + kh - H;  // unit (k - 1, h)
        int polls = 0;
        while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
          if (++polls > kMaxPolls) {
            __hip_atomic_store(a.sync + 8, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
    }
    const float* hsrc = ci.first ? (a.init ? a.init + ((int64_t)ci.seq * H + h) * (P * N) : nullptr)
                                 : a.E + st_off - (int64_t)H * (P * N);
    const float alpha = exp2_fast(alast_s);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int p = pcol(tp0 + i, r);
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) {
        const int n = (tn0 + jj) * 16 + 4 * q4;
        const float4 hv = hsrc ? *(const float4*)(hsrc + p * N + n) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 ev = make_float4(alpha * hv.x + acc[i][jj][0], alpha * hv.y + acc[i][jj][1],
                                      alpha * hv.z + acc[i][jj][2], alpha * hv.w + acc[i][jj][3]);
        if (ci.last) {
          if (a.final_states) *(float4*)(a.final_states + ((int64_t)ci.seq * H + h) * (P * N) + p * N + n) = ev;
        } else {
          *(float4*)(a.E + st_off + p * N + n) = ev;
        }
        const uint2 hb = make_uint2(pack_bf2(hv.x, hv.y), pack_bf2(hv.z, hv.w));
        *(uint2*)(hs + p * HLD + n) = hb;
        if (a.Hp) *(uint2*)(a.Hp + st_off + p * N + n) = hb;
      }
    }
    if (!ci.last) {
      // every wave's E stores complete, then one release store of the flag
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_store(a.flags + kh, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }

    // --------------------------------------------------------------- output ----
    rows.prefetch_first();  // the first row block's C and C.B^T fragments
    __syncthreads();  // hs complete
    Rows::column_factors(vt, sa, sd, Q, tid);
    __syncthreads();
    rows.run();
  }
}

// A sequence without tokens has no unit: its final state is its initial state
// (zero without one).  Grid (sequence, head), one 16-byte piece per thread.
__global__ __launch_bounds__(256) void chain_empty_final_kernel(ChunkMap m, int H, int PN,
                                                                const float* __restrict__ init,
                                                                float* __restrict__ final_states) {
  const int s = blockIdx.x, h = blockIdx.y;
  int c0, c1;
  seq_chunks(m, s, c0, c1);
  if (c1 > c0) return;
  const int64_t base = ((int64_t)s * H + h) * PN;
  for (int e = threadIdx.x * 4; e < PN; e += 256 * 4)
    *(float4*)(final_states + base + e) = init ? *(const float4*)(init + base + e) : make_float4(0.f, 0.f, 0.f, 0.f);
}

// flags and ticket counters back to zero before each chained launch (a kernel, so
// that the call can be captured into a graph)
__global__ void chain_clear_kernel(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

bool chained_supported(const Prob& p) {
  return bf16_kernels(p) && p.Q <= kScanQmax && (p.P == 32 || p.P == 64 || p.P == 128) &&
         (p.N == 64 || p.N == 128);
}

hipError_t launch_fwd_chained(const Prob& p, const ChainIO& io, hipStream_t st) {
  if (!chained_supported(p)) return hipErrorInvalidValue;
  if (io.final_states && p.nseq > 0)
    hipLaunchKernelGGL(chain_empty_final_kernel, dim3(p.nseq, p.H), dim3(256), 0, st, p.map, p.H,
                       p.P * p.N, io.init, io.final_states);
  if (p.nck == 0) return hipGetLastError();
  ChainArgs a;
  a.x = (const uint16_t*)io.x;
  a.B = (const uint16_t*)io.B;
  a.C = (const uint16_t*)io.C;
  a.CB = (const uint16_t*)io.CB;
  a.dt = io.dt;
  a.dt_bias = io.dt_bias;
  a.A = io.A;
  a.D = io.D;
  a.init = io.init;
  a.softplus = p.softplus;
  a.y = (uint16_t*)io.y;
  a.final_states = io.final_states;
  a.E = io.E;
  a.flags = io.sync + kChainSyncWords;
  a.sync = io.sync;
  a.delta = io.delta;
  a.acs = io.acs;
  a.decay = io.decay;
  a.Hp = (uint16_t*)io.Hp;
  a.rows = p.packed ? 1 : p.B;
  a.hpq = p.H >= 8 ? p.H / 8 : 1;
  int64_t total = 0;
  for (int x = 0; x < 8; ++x) {
    int cnt = 0;
    for (int h = 0; h < p.H; ++h)
      if ((h / a.hpq) % 8 == x) ++cnt;
    a.nhq[x] = cnt;
    a.nq[x] = (int32_t)(p.nck * cnt);
    total += a.nq[x];
  }
  const int64_t words = kChainSyncWords + p.nck * (int64_t)p.H;
  hipLaunchKernelGGL(chain_clear_kernel, dim3((unsigned)std::min<int64_t>(1024, (words + 255) / 256)),
                     dim3(256), 0, st, io.sync, words);
  const int64_t grid = total;  // one unit per workgroup
#define SSD_CHAIN_CASE(PP, NN)                                                                       \
  if (p.P == PP && p.N == NN) {                                                                      \
    hipLaunchKernelGGL((fwd_chained_kernel<PP, NN>), dim3((unsigned)grid), dim3(kScanWaves * 64), 0, \
                       st, p.map, p.H, p.G, a);                                                      \
    return hipGetLastError();                                                                        \
  }
  SSD_CHAIN_CASE(32, 64) SSD_CHAIN_CASE(32, 128) SSD_CHAIN_CASE(64, 64) SSD_CHAIN_CASE(64, 128)
  SSD_CHAIN_CASE(128, 64) SSD_CHAIN_CASE(128, 128)
#undef SSD_CHAIN_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
