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
// fp32 path: k_f32.hip.
#include "internal.hpp"
#include "scan_rows.hpp"

namespace ssd {

// HT: element type of the passed states (fp32, or bf16 from the fused forward)
template <int P, int N, typename HT>
__global__ __launch_bounds__(kScanWaves * 64) void chunk_scan_bf16_kernel(
    ChunkMap m, int H, int G, const uint16_t* __restrict__ X, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ CB, const float* __restrict__ delta,
    const float* __restrict__ acs, const HT* __restrict__ Hs, const float* __restrict__ D,
    uint16_t* __restrict__ Y) {
  using Rows = ScanRows<P, N>;
  constexpr int QMAX = Rows::QMAX, LDX = Rows::LDX, HLD = Rows::HLD;
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
  const int tid = threadIdx.x;
  const int64_t kh = (int64_t)k * H + h;
  const int64_t xrow = (int64_t)H * P, crow = (int64_t)G * N;
  const uint16_t* xb = X + (int64_t)ci.start * xrow + (int64_t)h * P;

  Rows rows;
  rows.xs = xs;
  rows.hs = hs;
  rows.sa = sa;
  rows.sd = sd;
  rows.vt = &vt[0][0];
  rows.init(Cm + (int64_t)ci.start * crow + (int64_t)g * N, crow, CB + ((int64_t)k * G + g) * Q * Q,
            Y + (int64_t)ci.start * xrow + (int64_t)h * P, xrow, Q, len, tid, D ? D[h] : 0.f);
  // the first row block's C and C.B^T fragments are in flight during the prologue;
  // the next one's are loaded before the current one's stores, so the wait for them
  // does not also wait for those stores (one in-order memory counter)
  rows.prefetch_first();
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
  Rows::column_factors(&vt[0][0], sa, sd, Q, tid);
  __syncthreads();
  rows.run();
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
  if (!bf16_kernels(p)) {
    if (passed_bf16) return hipErrorInvalidValue;
    return launch_chunk_scan_f32(p, x, C, CB, delta, acs, (const float*)passed, D, out, st);
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
