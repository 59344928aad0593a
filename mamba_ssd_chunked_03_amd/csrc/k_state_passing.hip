// Stage 3 (ssd_state_passing): the cross-chunk recurrence as an associative scan.
//
// Per sequence, head and state element, chunk c contributes the pair
// (l_c, T_c) with l_c = log2 of the chunk's total decay.  Pairs combine as the
// composition of affine maps (scan page, section 2; its formula was lost, the
// reading is):
//     (l1, b1) (+) (l2, b2) = (l1 + l2, 2^l2 * b1 + b2)
// The forward output is H_c, the state entering chunk c (the exclusive prefix
// seeded with the sequence's init state), and the final state E_last.  The
// per-chunk outputs are stored in fp32 or, where every consumer feeds them to
// bf16 matrix cores anyway, in bf16 (half the bytes); the carry itself and the
// final state stay fp32.  The
// backward runs the same scan over the chunks in reverse order (dE_c out,
// d_final in, d_init out), replacing the sequential state-passing loop in both
// directions (aitrends.kr/articles/109906, "Helion-based B200 kernel redesign").
//
// Mapping (reduce, scan, re-walk):
//  * a workgroup owns one (sequence, head, slab of 256 state elements); each
//    lane owns 4 consecutive elements, so every global access of a wavefront is
//    one contiguous 1 KB row (state arrays are (chunk, head, P*N));
//  * the W wavefronts split the chunk axis into W segments of S chunks; each
//    lane folds its segment in registers (loads for all S chunks issued first);
//  * the W segment summaries are scanned with a log-depth Hillis-Steele over
//    the 16 lanes of a DPP row (row_shr 1, 2, 4, 8; each step reads the
//    previous step's value from the neighbour lane, so there is no
//    read-after-write race), four state elements per wavefront instruction;
//  * the carry into each segment goes back through LDS and each wavefront
//    re-walks its segment from its carry, writing the states;
//  * sequences longer than W*S chunks are processed block by block with the
//    block's end state carried in LDS.
#include <cmath>

#include "internal.hpp"

namespace ssd {

static_assert(sizeof(ChunkStateT) == 4 && (ChunkStateT)0.5f == 0.5f,
              "the scan reads its inputs (chunk states, their adjoints) as fp32 float4");

// REV (0 forward, 1 reverse) is a template argument so that profiles tell the
// two directions apart.
template <int W, int S, typename OutT, int REV>
__global__ __launch_bounds__(W * 64) void state_passing_kernel(ChunkMap m, int H, int PN,
                                                               const float* __restrict__ T,
                                                               const float* __restrict__ decay,
                                                               const float* __restrict__ init,
                                                               OutT* __restrict__ Hout,
                                                               float* __restrict__ final_states) {
  constexpr bool reverse = REV != 0;
  __shared__ float4 sumB[W][64];  // segment summaries, b part
  __shared__ float sumL[W];       // segment summaries, log2 decay part
  __shared__ float cin[W][256];   // carry into each segment (scalar per element)
  __shared__ float4 nxt[64];      // carry into the next block of chunks

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int slab = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int pn = slab * 256 + lane * 4;
  const int64_t hstride = PN;               // between heads
  const int64_t cstride = (int64_t)H * PN;  // between chunks
  int c0, c1;
  seq_chunks(m, s, c0, c1);
  const int n = c1 - c0;

  float4 carry = make_float4(0.f, 0.f, 0.f, 0.f);
  if (init) carry = *(const float4*)(init + ((int64_t)s * H + h) * hstride + pn);

  for (int base = 0; base < n; base += W * S) {
    const int seg0 = base + w * S;
    const int cnt = max(0, min(S, n - seg0));
    float4 tv[S];
    float lg[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      if (i < cnt) {
        const int c = reverse ? (c1 - 1 - (seg0 + i)) : (c0 + seg0 + i);
        tv[i] = *(const float4*)(T + (int64_t)c * cstride + (int64_t)h * hstride + pn);
        lg[i] = decay[(int64_t)c * H + h];
      } else {
        tv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        lg[i] = 0.f;
      }
    }
    // local fold of the segment from the identity (0, 0)
    float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const float a = exp2_fast(lg[i]);
      b.x = a * b.x + tv[i].x;
      b.y = a * b.y + tv[i].y;
      b.z = a * b.z + tv[i].z;
      b.w = a * b.w + tv[i].w;
      L += lg[i];
    }
    sumB[w][lane] = b;
    if (lane == 0) sumL[w] = L;
    if (w == 0) nxt[lane] = carry;
    __syncthreads();

    // Log-depth scan over segments: DPP row r of wavefront w handles state
    // element e = (w * 4 + r) + 4 * W * it of the slab; lane j of the row holds
    // segment j (identity for j >= W).
    const int j = lane & 15, r = lane >> 4;
    for (int e = w * 4 + r; e < 256; e += 4 * W) {
      float lj = (j < W) ? sumL[j] : 0.f;
      const float* sb = (const float*)&sumB[0][0];
      float bj = (j < W) ? sb[j * 256 + e] : 0.f;
      // inclusive Hillis-Steele: (l, b) <- (l_prev + l, 2^l * b_prev + b)
      {
        float lp = dpp_f<kRowShr1>(0.f, lj), bp = dpp_f<kRowShr1>(0.f, bj);
        bj = exp2_fast(lj) * bp + bj; lj += lp;
      }
      {
        float lp = dpp_f<kRowShr2>(0.f, lj), bp = dpp_f<kRowShr2>(0.f, bj);
        bj = exp2_fast(lj) * bp + bj; lj += lp;
      }
      {
        float lp = dpp_f<kRowShr4>(0.f, lj), bp = dpp_f<kRowShr4>(0.f, bj);
        bj = exp2_fast(lj) * bp + bj; lj += lp;
      }
      {
        float lp = dpp_f<kRowShr8>(0.f, lj), bp = dpp_f<kRowShr8>(0.f, bj);
        bj = exp2_fast(lj) * bp + bj; lj += lp;
      }
      // exclusive prefix = inclusive of the previous lane (identity for lane 0)
      const float le = dpp_f<kRowShr1>(0.f, lj), be = dpp_f<kRowShr1>(0.f, bj);
      const float cv = ((const float*)nxt)[e];
      if (j < W) cin[j][e] = exp2_fast(le) * cv + be;
      // element e belongs to this DPP row alone: the row reads nxt[e] before lane W-1 rewrites it
      if (j == W - 1) ((float*)nxt)[e] = exp2_fast(lj) * cv + bj;
    }
    __syncthreads();

    // re-walk the segment from its carry, writing the state entering each chunk
    float4 E;
    E.x = cin[w][lane * 4 + 0];
    E.y = cin[w][lane * 4 + 1];
    E.z = cin[w][lane * 4 + 2];
    E.w = cin[w][lane * 4 + 3];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      if (i < cnt) {
        const int c = reverse ? (c1 - 1 - (seg0 + i)) : (c0 + seg0 + i);
        store4(Hout + (int64_t)c * cstride + (int64_t)h * hstride + pn, E);
        const float a = exp2_fast(lg[i]);
        E.x = a * E.x + tv[i].x;
        E.y = a * E.y + tv[i].y;
        E.z = a * E.z + tv[i].z;
        E.w = a * E.w + tv[i].w;
      }
    }
    carry = nxt[lane];
    __syncthreads();  // nxt / cin / sums are rewritten by the next block
  }
  if (final_states && w == 0)
    *(float4*)(final_states + ((int64_t)s * H + h) * hstride + pn) = carry;
}

// The sequential-carry form: each lane owns 4 consecutive state elements of one
// (sequence, head) and walks that sequence's chunks in order,
// E = 2^l_c * E + T_c, writing the state entering each chunk as it goes.  Same
// traffic as the scan above (one read of T and the decays, one write of the
// states); what differs is the dependency depth, as long as the sequence's chunk
// count, walked by B * H * P * N / 4 independent lanes.  The loads do not depend
// on the carry, so D chunks of them are kept in flight (a ring of D registers,
// refilled as each is consumed; past the sequence's end the refill re-reads its
// last chunk, which is never used) and the chain waits on memory only once per D
// chunks.  D = 1 is the plain loop that the associative scan replaces
// (SSD_FLAG_SEQUENTIAL_SCAN, the comparison point); deeper rings stream.
template <typename OutT, int REV, int D>
__global__ __launch_bounds__(256) void state_passing_seq_kernel(ChunkMap m, int H, int PN,
                                                                const float* __restrict__ T,
                                                                const float* __restrict__ decay,
                                                                const float* __restrict__ init,
                                                                OutT* __restrict__ Hout,
                                                                float* __restrict__ final_states) {
  constexpr bool reverse = REV != 0;
  const int pn = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int h = blockIdx.y, s = blockIdx.z;
  if (pn >= PN) return;  // (PN is a multiple of 4: every lane's 4 elements are in range)
  const int64_t hoff = (int64_t)h * PN + pn;
  const int64_t cstride = (int64_t)H * PN;
  int c0, c1;
  seq_chunks(m, s, c0, c1);
  const int n = c1 - c0;
  float4 E = make_float4(0.f, 0.f, 0.f, 0.f);
  if (init) E = *(const float4*)(init + (int64_t)s * H * PN + hoff);
  auto chunk = [&](int i) { return reverse ? c1 - 1 - i : c0 + i; };
  if (n > 0) {
    float4 buf[D];
    float lb[D];
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int c = chunk(min(u, n - 1));
      buf[u] = *(const float4*)(T + (int64_t)c * cstride + hoff);
      lb[u] = decay[(int64_t)c * H + h];
    }
    for (int i0 = 0; i0 < n; i0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int i = i0 + u;
        if (i < n) {  // (the same for every lane of the workgroup)
          const float4 tv = buf[u];
          const float lv = lb[u];
          const int cn = chunk(min(i + D, n - 1));
          buf[u] = *(const float4*)(T + (int64_t)cn * cstride + hoff);
          lb[u] = decay[(int64_t)cn * H + h];
          store4(Hout + (int64_t)chunk(i) * cstride + hoff, E);
          const float a = exp2_fast(lv);
          E.x = a * E.x + tv.x;
          E.y = a * E.y + tv.y;
          E.z = a * E.z + tv.z;
          E.w = a * E.w + tv.w;
        }
      }
    }
  }
  if (final_states) *(float4*)(final_states + (int64_t)s * H * PN + hoff) = E;
}

template <int D>
static void launch_seq(const Prob& p, const float* states, const float* decay, const float* init,
                       void* passed, int passed_bf16, float* final_states, int reverse, hipStream_t st) {
  const int PN = p.P * p.N;
  const dim3 g((PN / 4 + 255) / 256, p.H, p.nseq);
  if (passed_bf16 && reverse)
    hipLaunchKernelGGL((state_passing_seq_kernel<uint16_t, 1, D>), g, dim3(256), 0, st, p.map, p.H, PN,
                       states, decay, init, (uint16_t*)passed, final_states);
  else if (passed_bf16)
    hipLaunchKernelGGL((state_passing_seq_kernel<uint16_t, 0, D>), g, dim3(256), 0, st, p.map, p.H, PN,
                       states, decay, init, (uint16_t*)passed, final_states);
  else if (reverse)
    hipLaunchKernelGGL((state_passing_seq_kernel<float, 1, D>), g, dim3(256), 0, st, p.map, p.H, PN,
                       states, decay, init, (float*)passed, final_states);
  else
    hipLaunchKernelGGL((state_passing_seq_kernel<float, 0, D>), g, dim3(256), 0, st, p.map, p.H, PN,
                       states, decay, init, (float*)passed, final_states);
}

template <int W, int S>
static void launch_sp(const Prob& p, dim3 grid, const float* states, const float* decay,
                      const float* init, void* passed, int passed_bf16, float* final_states,
                      int reverse, hipStream_t st) {
  const int PN = p.P * p.N;
  if (passed_bf16 && reverse)
    hipLaunchKernelGGL((state_passing_kernel<W, S, uint16_t, 1>), grid, dim3(W * 64), 0, st, p.map,
                       p.H, PN, states, decay, init, (uint16_t*)passed, final_states);
  else if (passed_bf16)
    hipLaunchKernelGGL((state_passing_kernel<W, S, uint16_t, 0>), grid, dim3(W * 64), 0, st, p.map,
                       p.H, PN, states, decay, init, (uint16_t*)passed, final_states);
  else if (reverse)
    hipLaunchKernelGGL((state_passing_kernel<W, S, float, 1>), grid, dim3(W * 64), 0, st, p.map,
                       p.H, PN, states, decay, init, (float*)passed, final_states);
  else
    hipLaunchKernelGGL((state_passing_kernel<W, S, float, 0>), grid, dim3(W * 64), 0, st, p.map,
                       p.H, PN, states, decay, init, (float*)passed, final_states);
}

// The tuned per-shape table: (chunks per sequence, independent lanes) -> variant,
// measured by tuning/sweep.py and turned into tuned_scan.inc by build.py.  An
// empty table leaves the rule below.
struct ScanEntry {
  int32_t chunks;  // chunks per sequence of the measured shape
  int64_t lanes;   // sequences x heads x headdim x dstate / 4 of the measured shape
  int32_t variant;
};
#if __has_include("tuned_scan.inc")
#include "tuned_scan.inc"
#else
static const ScanEntry kTunedScan[] = {{0, 0, 0}};
static const int kTunedScanCount = 0;
#endif

int scan_variant_for(const Prob& p) {
  const int v = (p.flags >> kScanVariantShift) & 15;
  if (v != kScanTable) return v;
  if (p.flags & kFlagSequentialScan) return kScanSeq1;
  // chunks per sequence: exact for batched rows, the packed slots' average otherwise
  const int64_t chain = p.packed ? (p.nck + p.nseq - 1) / (p.nseq > 0 ? p.nseq : 1)
                                 : p.nck / (p.B > 0 ? p.B : 1);
  const int64_t lanes = (int64_t)p.nseq * p.H * p.P * p.N / 4;
  if (kTunedScanCount > 0 && chain > 0 && lanes > 0) {
    // the nearest measured shape, distance in log2 of both coordinates
    const double lc = std::log2((double)chain), ll = std::log2((double)lanes);
    double best = 1e300;
    int bv = kScanTable;
    for (int i = 0; i < kTunedScanCount; ++i) {
      const double dc = lc - std::log2((double)kTunedScan[i].chunks);
      const double dl = ll - std::log2((double)kTunedScan[i].lanes);
      const double d = dc * dc + dl * dl;
      if (d < best) {
        best = d;
        bv = kTunedScan[i].variant;
      }
    }
    if (bv >= kScanAssoc4x2 && bv <= kScanSeq8) return bv;
  }
  // no table: segments sized to the chain
  if (chain <= 8) return kScanAssoc4x2;
  if (chain <= 32) return kScanAssoc8x4;
  if (chain <= 64) return kScanAssoc16x4;
  return kScanAssoc16x8;
}

hipError_t launch_state_passing(const Prob& p, const float* states, const float* decay,
                                const float* init, void* passed, int passed_bf16,
                                float* final_states, int reverse, hipStream_t st) {
  const int PN = p.P * p.N;  // a multiple of 256 for every supported (P, N)
  if (p.nseq == 0) return hipSuccess;
  const dim3 grid(PN / 256, p.H, p.nseq);
  switch (scan_variant_for(p)) {
    case kScanAssoc4x2:
      launch_sp<4, 2>(p, grid, states, decay, init, passed, passed_bf16, final_states, reverse, st);
      break;
    case kScanAssoc8x4:
      launch_sp<8, 4>(p, grid, states, decay, init, passed, passed_bf16, final_states, reverse, st);
      break;
    case kScanAssoc16x4:
      launch_sp<16, 4>(p, grid, states, decay, init, passed, passed_bf16, final_states, reverse, st);
      break;
    case kScanAssoc16x8:
      launch_sp<16, 8>(p, grid, states, decay, init, passed, passed_bf16, final_states, reverse, st);
      break;
    case kScanSeq1:
      launch_seq<1>(p, states, decay, init, passed, passed_bf16, final_states, reverse, st);
      break;
    case kScanSeq4:
      launch_seq<4>(p, states, decay, init, passed, passed_bf16, final_states, reverse, st);
      break;
    case kScanSeq8:
      launch_seq<8>(p, states, decay, init, passed, passed_bf16, final_states, reverse, st);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ssd
