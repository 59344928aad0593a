// Device-side building blocks shared by the libssd kernels (gfx950 / CDNA4).
//
// - bf16 storage and conversion (hardware round-to-nearest-even on gfx950),
// - MFMA wrappers with the lane layouts of v_mfma_f32_16x16x32_bf16 and
//   v_mfma_f32_16x16x4_f32 (64-lane wavefronts),
// - DPP-based wavefront scans (row_shr within 16-lane rows, row_bcast15/31
//   across rows),
// - the chunk map: which tokens a chunk slot covers, for batched rows and for
//   packed sequences.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// log2(e): decays are stored and evaluated in base 2 so each exp is one v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}
// two floats -> packed bf16 pair (lo in bits 0..15): one v_cvt_pk_bf16_f32 with
// both sources (converting the two halves separately costs two converts, a
// shift and an or)
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const f32x2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------------------------------ exp ----
// 2^x with the hardware v_exp_f32 (results below 2^-126 flush to zero, which the
// scan accepts: such decays are below fp32's normal range anyway).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// softplus(z) = max(z, 0) + log1p(exp(-|z|)), from its definition.
__device__ __forceinline__ float softplus_f(float z) {
  return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}
// d softplus / dz = 1 / (1 + exp(-z)), in a form that never overflows.
__device__ __forceinline__ float sigmoid_f(float z) {
  float e = expf(-fabsf(z));
  float r = 1.f / (1.f + e);
  return z >= 0.f ? r : e * r;
}

// delta of one token (zero past the chunk's end): softplus(dt + bias) or dt + bias.
// Shared by the cumsum kernel and the chunk-state kernel that forms it inline,
// so that both produce the same bits.
__device__ __forceinline__ float token_delta(float dtv, float bias, int softplus, bool in) {
  const float z = dtv + bias;
  const float d = softplus ? softplus_f(z) : z;
  return in ? d : 0.f;
}

// The cumsum's per-token increment delta * A in log2 units, never fused into a
// following add, so that every kernel that scans it rounds it the same way.
__device__ __forceinline__ float scan_input(float d, float a2) {
#pragma clang fp contract(off)
  return d * a2;
}

// ----------------------------------------------------------------- MFMA ----
// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l holds A[l%16][8*(l/16) + 0..7], B[8*(l/16) + 0..7][l%16] and
// D[4*(l/16) + r][l%16] for r = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16) += A(16x4) * B(4x16), true fp32.  Lane l holds A[l%16][l/16],
// B[l/16][l%16] and D[4*(l/16) + r][l%16].
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// MFMA operand fragment from an LDS tile stored K-major (tile[k][col], row
// stride `ld` bf16 elements) with the gfx950 transpose read ds_read_b64_tr_b16:
// in each 16-lane group, output lane i, slot s comes from source lane 4s + i/4,
// element i%4.  Pointing lane j of group q at row 8q + j/4, columns 4(j%4)..+3
// makes two reads (rows +0 and +4) deliver tile[8q + 0..7][col0 + lane%16],
// the 16x16x32 operand layout.  `tile` points at tile[k0][col0].
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ int tr_offset(int lane, int ld) {
  return (8 * (lane >> 4) + ((lane & 15) >> 2)) * ld + 4 * (lane & 3);
}
__device__ __forceinline__ bf16x8 frag_kmajor(const uint16_t* tile, int ld, int lane) {
  const uint16_t* p = tile + tr_offset(lane, ld);
  v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * ld));
  v8i16 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// --------------------------------------------------------- buffer access ----
// A buffer resource over the `bytes` bytes that start at p.  Accesses at byte
// offsets >= bytes (vector, instruction and scalar offset together) are range
// checked by the hardware: loads return zero and stores are dropped, without
// touching memory.  With `bytes` ending at a chunk's last valid row, a tile's
// rows past the chunk's end read as zero and are never written, with no branch,
// and every offset is a 32-bit value (callers keep a chunk's span below 2^31
// bytes).  Dword 3 of the descriptor selects the 32-bit data format with no
// swizzling, the untyped layout of this GPU family.
typedef __amdgpu_buffer_rsrc_t brsrc;
__device__ __forceinline__ brsrc make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(brsrc r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(brsrc r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// the same load marked nontemporal (the cache-policy operand's NT bit)
__device__ __forceinline__ u32x4 buf_load16_nt(brsrc r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ void buf_store16(brsrc r, uint32_t off, u32x4 v) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, 0);
}

// ------------------------------------------------- C.B^T fragment order ----
// A chunk's C.B^T (and its transpose) on the bf16 path is a Q x Q bf16 matrix
// stored as 16 x 32 blocks of 1 KB, in the order an MFMA A-operand load reads
// them: block (R, S) = rows 16R..16R+15, columns 32S..32S+31 at element offset
// (R * Q/32 + S) * 512, and inside it the 16 bytes of lane l = 16 q + r holding
// the 8 consecutive columns 32S + 8q .. +7 of row 16R + r.
// A wave's fragment load is then 1 KB contiguous (8 whole 128-byte lines), where
// row-major storage makes it 16 half-lines of 16 rows: with most of these reads
// hitting the L2 (a group's heads share the matrix), the texture address unit
// and the L1 then take about twice as long per load.  Row block R occupies the
// same bytes as rows 16R..16R+15 of the row-major matrix, so a range check that
// ends at a whole row block keeps the "rows past the end" rule.
__host__ __device__ __forceinline__ uint32_t cbf_off(int i, int j, int Q) {  // element offset of (i, j)
  return (uint32_t)(((i >> 4) * (Q >> 5) + (j >> 5)) * 512 + (((j & 31) >> 3) * 16 + (i & 15)) * 8 + (j & 7));
}
// byte offset of the 16-byte piece that lane (q, r) loads of block (R, S)
__host__ __device__ __forceinline__ uint32_t cbf_piece(int R, int S, int lane, int Q) {
  return (uint32_t)((R * (Q >> 5) + S) * 1024 + lane * 16);
}

// ---------------------------------------------- column order of MFMA rows ----
// A row of W outputs (W a multiple of 32) computed as W/16 transposed 16x16
// tiles, the column index coming from a K-major LDS operand read with
// frag_kmajor, leaves lane group q (lanes 16q..16q+15) of tile t holding the
// LDS columns 16t + 4q + 0..3.  The operand is staged with its 4-column groups
// permuted inside every 32-column block (logical group 2g + u stored as group
// 4u + g), so those LDS columns hold the logical columns
// 32(t/2) + 8q + 4(t%2) + 0..3 (pcol below): a lane then owns 8 consecutive
// logical columns in the tile pair 2s, 2s + 1, and its part of a row is read
// and written 16 bytes at a time (64 contiguous bytes per row per instruction,
// where the natural order gives 32).  The transpose reads are untouched, so
// their LDS bank pattern stays that of the natural layout.
__device__ __forceinline__ int pcol(int t, int c) {  // logical column of tile t's column c
  return 32 * (t >> 1) + 8 * (c >> 2) + 4 * (t & 1) + (c & 3);
}
// LDS columns of the low and high 8 bytes of logical 16-byte piece c8 (columns 8 c8 .. +7)
__device__ __forceinline__ int perm_lo(int c8) { return 32 * (c8 >> 2) + 4 * (c8 & 3); }
__device__ __forceinline__ int perm_hi(int c8) { return 32 * (c8 >> 2) + 16 + 4 * (c8 & 3); }
// one 16-byte piece of an LDS row, in the natural or the permuted column order
template <bool PERM>
__device__ __forceinline__ void lds_piece(uint16_t* row, int c8, u32x4 v) {
  if constexpr (PERM) {
    *(uint2*)(row + perm_lo(c8)) = make_uint2(v[0], v[1]);
    *(uint2*)(row + perm_hi(c8)) = make_uint2(v[2], v[3]);
  } else {
    *(u32x4*)(row + c8 * 8) = v;
  }
}
// a lane's 8 logical columns 32s + 8q .. +7 of a permuted LDS row
__device__ __forceinline__ u32x4 lds_cols8_perm(const uint16_t* row, int s, int q) {
  const uint2 lo = *(const uint2*)(row + 32 * s + 4 * q);
  const uint2 hi = *(const uint2*)(row + 32 * s + 16 + 4 * q);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}
// sum of a lane's 8 bf16 values (columns 32s + 8q .. +7) times its outputs of tiles 2s, 2s + 1
__device__ __forceinline__ float dot_bf8(u32x4 v, f32x4 a, f32x4 b) {
  return bf_lo(v[0]) * a[0] + bf_hi(v[0]) * a[1] + bf_lo(v[1]) * a[2] + bf_hi(v[1]) * a[3] +
         bf_lo(v[2]) * b[0] + bf_hi(v[2]) * b[1] + bf_lo(v[3]) * b[2] + bf_hi(v[3]) * b[3];
}
// two adjacent tiles' 4 outputs of one lane (columns 32s + 8q .. +7) as 8 bf16
__device__ __forceinline__ u32x4 pack_bf8(f32x4 a, f32x4 b) {
  return u32x4{pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3])};
}

// --------------------------------------------------------- LDS staging ----
// fp32 P x N state (row-major) -> bf16 LDS [p][n] with row stride ld; loads first
// (range-checked buffer loads, no branches).
template <int P, int N, int NT = 256>
__device__ __forceinline__ void stage_state_bf16(uint16_t* dst, int ld, const float* src, int tid) {
  constexpr int NC = (P * N / 4 + NT - 1) / NT;
  const brsrc rs = make_rsrc(src, (uint32_t)(P * N * 4));
  float4 t[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int e = (tid + c * NT) * 4;
    const u32x4 v = buf_load16(rs, e < P * N ? (uint32_t)e * 4u : 0x80000000u);
    t[c] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int e = (tid + c * NT) * 4;
    if (e < P * N) {
      uint32_t* d = (uint32_t*)(dst + (e / N) * ld + (e % N));
      d[0] = pack_bf2(t[c].x, t[c].y);
      d[1] = pack_bf2(t[c].z, t[c].w);
    }
  }
}

// A tile of ROWS token rows of W bf16 copied into LDS in two steps (load, then
// store), so that several tiles' loads (and other loads) can all be in flight
// before the first LDS store waits for its data.  STREAM
// marks the loads nontemporal: for a tile that this kernel reads exactly once,
// it keeps the tile from displacing the operands that other workgroups re-read
// from the cache.  The loads go through a buffer resource that ends at row
// nvalid, so rows past it read as zero with no branch: a load under a branch,
// with zero on the other path, lets the register allocator give the two paths
// one register, and the zero's move must then wait for the load in flight,
// which serialises the tile's loads.  (nvalid * srow * 2 bytes stay below
// 2^31: one chunk's rows at most.)
template <int ROWS, int W, int NT = 256, bool PERM = false, bool STREAM = false>
struct RowTile {
  static constexpr int PER = W / 8;
  static constexpr int NC = (ROWS * PER + NT - 1) / NT;
  // every thread's every piece lies inside the tile: no test at all
  static constexpr bool EXACT = (ROWS * PER) % NT == 0;
  static_assert(!PERM || W % 32 == 0, "permuted rows are whole 32-column blocks");
  u32x4 t[NC];
  __device__ __forceinline__ void load(const uint16_t* src, int64_t srow, int nvalid, int tid) {
    const brsrc rs = make_rsrc(src, nvalid > 0 ? (uint32_t)nvalid * (uint32_t)(srow * 2) : 0u);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = tid + c * NT, j = e / PER, c8 = e % PER;
      // pieces past the tile (a partial last round) get an offset beyond any range
      const uint32_t off =
          (EXACT || e < ROWS * PER) ? (uint32_t)j * (uint32_t)(srow * 2) + c8 * 16 : 0x80000000u;
      if constexpr (STREAM)
        t[c] = buf_load16_nt(rs, off);
      else
        t[c] = buf_load16(rs, off);
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int ld, int tid) const {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = tid + c * NT, j = e / PER, c8 = e % PER;
      if (EXACT || e < ROWS * PER) lds_piece<PERM>(dst + j * ld, c8, t[c]);
    }
  }
};

// Four consecutive state elements to global memory as fp32 or bf16.
__device__ __forceinline__ void store4(float* dst, float4 v) { *(float4*)dst = v; }
__device__ __forceinline__ void store4(uint16_t* dst, float4 v) {
  *(uint2*)dst = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
}

// ------------------------------------------------------------------ DPP ----
// DPP controls (GFX9 encoding).
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowRor8 = 0x128, kRowHalfMirror = 0x141, kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Stores of 128-byte row spans, whole.  In a 16-row MFMA tile, lane (q, r) owns
// row r and the 16-byte pieces at bytes q*16 (piece 0) and 64 + q*16 (piece 1)
// of a 128-byte span.  Stored directly, each instruction would cover half of
// every row's span; instead the first store covers rows 0..7 whole (lanes r < 8
// piece 0 of row r, lanes r >= 8 piece 1 of row r - 8) and the second rows
// 8..15, after a row rotate by 8 (lane r <-> lane r ^ 8) has moved the pieces:
// half as many partial-line writes reach the L2.
__device__ __forceinline__ uint32_t span_off(int r, int q) { return (r < 8 ? 0u : 64u) + q * 16; }
// the lane's own (piece 0, piece 1) -> (a, b): a goes to row r & 7, b to row 8 + (r & 7),
// both at byte span_off(r, q) of the span
__device__ __forceinline__ void span_swap(int r, const u32x4& o0, const u32x4& o1, u32x4& a, u32x4& b) {
  const bool lo = r < 8;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t recv =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(lo ? o1[d] : o0[d]), kRowRor8, 0xf, 0xf, false);
    a[d] = lo ? o0[d] : recv;
    b[d] = lo ? recv : o1[d];
  }
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                    ROW_MASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wavefront (Hillis-Steele with
// DPP: shifts 1, 2, 4, 8 inside each 16-lane row, then the row carries).
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  v += dpp_f<kRowShr1>(0.f, v);
  v += dpp_f<kRowShr2>(0.f, v);
  v += dpp_f<kRowShr4>(0.f, v);
  v += dpp_f<kRowShr8>(0.f, v);
  v += dpp_f<kRowBcast15, 0xa>(0.f, v);
  v += dpp_f<kRowBcast31, 0xc>(0.f, v);
  return v;
}

// Sum over the 16 lanes of each DPP row (every lane of the row gets the sum):
// rotations by 8, 4, 2, 1 inside the row.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<0x128>(0.f, v);  // row_ror:8
  v += dpp_f<0x124>(0.f, v);  // row_ror:4
  v += dpp_f<0x122>(0.f, v);  // row_ror:2
  v += dpp_f<0x121>(0.f, v);  // row_ror:1
  return v;
}

// Reduce-scatter of four per-lane values over the 16 lanes of each DPP row:
// on return, lane r of a row holds that row's sum of v[r / 4].  Three exchange
// steps (lanes r ^ 8, the mirror inside each half-row, then the quad) move half
// of the remaining values each, 11 instructions instead of 4 x 8.
__device__ __forceinline__ float row_reduce_scatter4(float v0, float v1, float v2, float v3, int r) {
  const bool h8 = r >= 8;  // lanes below 8 keep values 0, 1; the others 2, 3
  const float t0 = (h8 ? v2 : v0) + dpp_f<kRowRor8>(0.f, h8 ? v0 : v2);
  const float t1 = (h8 ? v3 : v1) + dpp_f<kRowRor8>(0.f, h8 ? v1 : v3);
  const bool h4 = (r & 7) >= 4;  // then lanes 0-3 of each half keep t0, lanes 4-7 t1
  float u = (h4 ? t1 : t0) + dpp_f<kRowHalfMirror>(0.f, h4 ? t0 : t1);
  u += dpp_f<kQuadXor1>(0.f, u);
  u += dpp_f<kQuadXor2>(0.f, u);
  return u;
}

// Reduce-scatter of four per-lane values over the four rows of a wavefront
// (lanes r, r + 16, r + 32, r + 48): on return lane r of row q holds the sum of
// v[q] over those lanes.  gfx950's row swaps: permlane16_swap exchanges the odd
// rows of its first operand with the even rows of its second, permlane32_swap
// the upper half of the first with the lower half of the second.
__device__ __forceinline__ float col_reduce_scatter4(float v0, float v1, float v2, float v3) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
  const float s01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // rows 0, 2: v0; rows 1, 3: v1
  const float s23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Sum over all 64 lanes (result valid in every lane).
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Broadcast lane 63's value to the whole wavefront.
__device__ __forceinline__ float wave_last(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ------------------------------------------------------- XCD-aware order ----
// Workgroups are handed to the 8 XCDs round-robin (linear id L goes to XCD
// L % 8) and each XCD has its own L2.  xcd_order(L, W) renumbers a 1-D grid of
// W workgroups so that consecutive logical ids run on the same XCD, one after
// the other: tiles that share operands (the row tiles of one chunk and group)
// then find them in that XCD's L2 instead of fetching them again from HBM.
constexpr int kNumXcd = 8;
__host__ __device__ __forceinline__ int xcd_order(int L, int W) {
  const int x = L % kNumXcd, s = L / kNumXcd;
  const int per = W / kNumXcd, rem = W % kNumXcd;
  return x * per + (x < rem ? x : rem) + s;
}

// xcd_order, and inside each XCD's sequence of slots s = L / 8, every block of
// 32 R slots laid out so that R consecutive logical ids take slots c, c + 32,
// ..., c + 32 (R - 1).  An XCD has 32 compute units and hands its workgroups to
// them in turn, so slots s and s + 32 tend to run on one unit at the same time:
// R neighbouring ids (heads of one group) then request the lines they share at
// about the same moment.  Only the speed depends on this; every order covers
// each id once.
constexpr int kCusPerXcd = 32;
__host__ __device__ __forceinline__ int xcd_order_cu(int L, int W, int R) {
  const int x = L % kNumXcd, s = L / kNumXcd;
  const int per = W / kNumXcd, rem = W % kNumXcd;
  const int blk = kCusPerXcd * R;
  int sp = s;
  if (s < (per / blk) * blk) sp = (s / blk) * blk + (s % kCusPerXcd) * R + (s % blk) / kCusPerXcd;
  return x * per + (x < rem ? x : rem) + sp;
}

// (chunk slot, head) of a workgroup of a 1-D grid over nck x H slots: in the
// XCD-aware order above, head fastest, with pairs of neighbouring heads placed
// to share a compute unit.  Each XCD then works through all heads of one chunk
// together: a token's row of x (every head) is read whole, and a group's B and
// C.B^T tiles stay in that XCD's L2 for the group's heads.
__device__ __forceinline__ void chunk_head(int H, int& k, int& h) {
  const int l = xcd_order_cu(blockIdx.x, gridDim.x, 2);
  k = l / H;
  h = l % H;
}

// ------------------------------------------------------------ chunk map ----
// A chunk slot k covers tokens [start, start + len) of the flattened
// (batch * seqlen) token axis, inside sequence `seq`.  Batched rows: row b is
// sequence b, cut into ceil(seqlen / Q) chunks from its first token.  Packed
// sequences: a table built on the device from cu_seqlens (len 0 = unused slot).
struct ChunkMap {
  int32_t Q;        // chunk size
  int32_t nck;      // number of chunk slots
  int32_t packed;   // 0: batched rows; 1: table
  int32_t seqlen;   // batched: tokens per row
  int32_t ncs;      // batched: chunks per row
  const int4* tab;  // packed: {start, len, seq, flags (1 first, 2 last)}
  const int32_t* seq_off;  // packed: first chunk slot of each sequence (nseq + 1)
};

struct ChunkInfo {
  int32_t start, len, seq;
  bool first, last;
};

__device__ __forceinline__ ChunkInfo chunk_info(const ChunkMap& m, int k) {
  ChunkInfo ci;
  if (!m.packed) {
    int b = k / m.ncs, c = k - b * m.ncs;
    ci.start = b * m.seqlen + c * m.Q;
    ci.len = min(m.Q, m.seqlen - c * m.Q);
    ci.seq = b;
    ci.first = (c == 0);
    ci.last = (c == m.ncs - 1);
  } else {
    int4 e = m.tab[k];
    ci.start = e.x;
    ci.len = e.y;
    ci.seq = e.z;
    ci.first = (e.w & 1) != 0;
    ci.last = (e.w & 2) != 0;
  }
  return ci;
}

// Chunk slots [c0, c1) of sequence s.
__device__ __forceinline__ void seq_chunks(const ChunkMap& m, int s, int& c0, int& c1) {
  if (!m.packed) {
    c0 = s * m.ncs;
    c1 = c0 + m.ncs;
  } else {
    c0 = m.seq_off[s];
    c1 = m.seq_off[s + 1];
  }
}

}  // namespace ssd
