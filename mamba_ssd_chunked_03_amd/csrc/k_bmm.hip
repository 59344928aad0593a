// Stage 4 (ssd_bmm_chunk): CB_ij = C_i . B_j for every chunk and group, the
// intra-chunk Gram matrix that the output stage weights by the decay mask.
//
// bf16 path: one workgroup per (chunk, group); the lower triangle of the QxQ
// product is cut into 64x64 tiles (j-tile <= i-tile), handed to the four
// wavefronts round-robin.  Both operands keep dstate (the contraction index)
// contiguous in memory, so MFMA fragments are read straight from global memory
// (16 bytes per lane) without LDS staging.  Tiles above the diagonal are never
// computed; inside diagonal tiles the upper part is written but unspecified.
// The backward also reads the transpose, CBt[j][i] = CB[i][j]: when asked, each
// lower tile is stored a second time, transposed, from the same LDS copy.  Both
// are stored in fragment order (common.hpp, cbf_off): each store instruction of
// a wave writes one 1 KB block.
//
// fp32 path: k_f32.hip (fp32 matrix cores).
#include "internal.hpp"

namespace ssd {

// out[a][b] = R_a . S_b on the lower tile triangle.
// Each wavefront's 64x64 tile goes through LDS so that every store instruction
// writes one 16 x 32 block in fragment order; with DUAL the transposed tile is
// stored too (outT[b][a]), which the backward reads when the forward keeps its
// intermediates.
template <int N, bool DUAL>
__global__ __launch_bounds__(256) void bmm_chunk_bf16_kernel(ChunkMap m, int G,
                                                             const uint16_t* __restrict__ Sm,
                                                             const uint16_t* __restrict__ Rm,
                                                             uint16_t* __restrict__ CB,
                                                             uint16_t* __restrict__ CBt) {
  constexpr int LT = 64 + 8;
  __shared__ __attribute__((aligned(16))) uint16_t tls[4][64 * LT];
  const int k = blockIdx.x, g = blockIdx.y;
  const ChunkInfo ci = chunk_info(m, k);
  if (ci.len <= 0) return;
  const int Q = m.Q;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, r = lane & 15;
  const int T = Q / 64;
  const int ntiles = T * (T + 1) / 2;
  const int64_t row = (int64_t)G * N;
  const uint16_t* cb0 = Rm + (int64_t)ci.start * row + (int64_t)g * N;
  const uint16_t* bb0 = Sm + (int64_t)ci.start * row + (int64_t)g * N;
  uint16_t* out = CB + ((int64_t)k * G + g) * Q * Q;
  uint16_t* tl = tls[w];
  // range-checked buffer loads over the chunk's valid rows (rows past its end read
  // as zero, with no branch: a load under a branch can leave its register shared
  // with the other path's zero, whose move then waits for the load)
  const brsrc rcr = make_rsrc(cb0, (uint32_t)(ci.len * row * 2)), rbr = make_rsrc(bb0, (uint32_t)(ci.len * row * 2));
  for (int tile = w; tile < ntiles; tile += 4) {
    int lo = 0;
    while ((lo + 1) * (lo + 2) / 2 <= tile) ++lo;
    const int hi = tile - lo * (lo + 1) / 2;  // hi <= lo
    const int ti = lo, tj = hi;
    if (ti * 64 >= ci.len) continue;  // rows past the chunk's end are never read
    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < N; kk += 32) {
      bf16x8 af[4], bf[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint32_t i = ti * 64 + a * 16 + r;
        const uint32_t j = tj * 64 + a * 16 + r;
        af[a] = as_bf16x8(buf_load16(rcr, i * (uint32_t)(row * 2) + (kk + q * 8) * 2));
        bf[a] = as_bf16x8(buf_load16(rbr, j * (uint32_t)(row * 2) + (kk + q * 8) * 2));
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma_bf16(af[a], bf[b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) tl[(a * 16 + q * 4 + rr) * LT + b * 16 + r] = f2bf(acc[a][b][rr]);
    __builtin_amdgcn_wave_barrier();
    // block (rr, cc) of the tile: lane (q, r) holds row 16 rr + r, columns
    // 32 cc + 8 q .. +7 (and of the transposed tile, row and column swapped)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int rr = c >> 1, cc = c & 1;
      *(u32x4*)((char*)out + cbf_piece(ti * 4 + rr, tj * 2 + cc, lane, Q)) =
          *(const u32x4*)(tl + (rr * 16 + r) * LT + cc * 32 + q * 8);
      if (DUAL) {
        u32x4 t;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          t[d] = (uint32_t)tl[(cc * 32 + q * 8 + 2 * d) * LT + rr * 16 + r] |
                 ((uint32_t)tl[(cc * 32 + q * 8 + 2 * d + 1) * LT + rr * 16 + r] << 16);
        *(u32x4*)((char*)(CBt + ((int64_t)k * G + g) * Q * Q) + cbf_piece(tj * 4 + rr, ti * 2 + cc, lane, Q)) = t;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_bmm_chunk(const Prob& p, const void* B, const void* C, void* CB, hipStream_t st,
                            void* CBt) {
  if (p.nck == 0) return hipSuccess;
  if (!bf16_kernels(p)) return launch_bmm_chunk_f32(p, B, C, CB, st);
  dim3 grid((unsigned)p.nck, p.G);
#define SSD_BMM_CASE(NN)                                                                   \
  if (p.N == NN) {                                                                         \
    if (CBt)                                                                               \
      hipLaunchKernelGGL((bmm_chunk_bf16_kernel<NN, true>), grid, dim3(256), 0, st,  \
                         p.map, p.G, (const uint16_t*)B, (const uint16_t*)C, (uint16_t*)CB, \
                         (uint16_t*)CBt);                                                  \
    else                                                                                   \
      hipLaunchKernelGGL((bmm_chunk_bf16_kernel<NN, false>), grid, dim3(256), 0, st, \
                         p.map, p.G, (const uint16_t*)B, (const uint16_t*)C, (uint16_t*)CB, \
                         nullptr);                                                         \
    return hipGetLastError();                                                              \
  }
  SSD_BMM_CASE(32) SSD_BMM_CASE(64) SSD_BMM_CASE(128)
#undef SSD_BMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd
