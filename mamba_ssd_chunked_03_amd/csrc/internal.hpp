// Host-side launch interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "layout.hpp"

namespace ssd {

// Validated problem, as the kernels see it.
struct Prob {
  int32_t B, L, H, P, N, G;
  int32_t nseq;      // number of state slots (batch rows, or packed sequences)
  int32_t io;        // io tensors: 0 fp32, 1 bf16
  int32_t wide;      // 1: bf16 io with headdim or dstate 16, run by the fp32 matrix-core
                     // kernels (bf16 tensors widened to fp32 in registers)
  int32_t softplus;  // delta = softplus(dt + bias)
  int32_t Q;         // chunk size
  int32_t packed;
  int32_t flags;     // SSD_FLAG_* bits
  int64_t nck;       // chunk slots
  ChunkMap map;      // device view of the chunk layout (table pointers set when packed)
};

// Whether the bf16 MFMA kernels run (bf16 io, headdim and dstate >= 32); otherwise
// the fp32 matrix-core kernels of k_f32.hip, with fp32 intermediates.
inline bool bf16_kernels(const Prob& p) { return p.io == 1 && !p.wide; }

// Prob::flags bit (SSD_FLAG_SEQUENTIAL_SCAN of ssd.h): state passing, forward and
// reverse, runs the sequential-carry kernel instead of the associative scan.
constexpr int kFlagSequentialScan = 8;
// Prob::flags bits 16..19 (SSD_FLAG_SCAN_VARIANT of ssd.h): the state-passing
// kernel, 0 = the tuned table's choice (scan_variant_for below).
constexpr int kScanVariantShift = 16;
enum { kScanTable = 0, kScanAssoc4x2 = 1, kScanAssoc8x4 = 2, kScanAssoc16x4 = 3, kScanAssoc16x8 = 4,
       kScanSeq1 = 5, kScanSeq4 = 6, kScanSeq8 = 7 };
// The variant a problem's state passing runs: the flag's choice, else the tuned
// table's entry nearest to the problem's chain length and lane count.
int scan_variant_for(const Prob& p);
// Prob::flags bits 20..21 (SSD_FLAG_CS_VARIANT of ssd.h): the shape of the
// chunk-state kernels on the bf16 path, 0 = the tuned table's choice.
constexpr int kCsVariantShift = 20;
enum { kCsTable = 0, kCsOneHead = 1, kCsTwoHeads = 2, kCsTwoHeadsCB = 3 };
// Whether variant v (1..3) can run this problem: two heads per workgroup need an
// even head count per group and a shape whose shared operand and LDS fit; C.B^T
// inside the kernel needs bf16, chunk 256 and eight heads per group (one 64-row
// block of C.B^T per head pair).  The fp32 matrix-core path has one form (1).
bool cs_variant_valid(const Prob& p, int v);
// The variant the chunk-state kernels run: the flag's choice, else the tuned
// table's entry for the problem's (headdim, dstate, heads per group, chunk), else
// the widest valid form.
int cs_variant_for(const Prob& p);

// mode of the chunk-state contraction
enum { kStateFwd = 0,        // T_c = sum_j delta_j 2^(acs_last - acs_j) x_j B_j^T
       kStateDstates = 1,    // U_c = sum_i 2^(acs_i) dy_i C_i^T
       kStateFwdCumsum = 2   // kStateFwd with delta and acs formed in the kernel (stage 1 inline)
};

hipError_t launch_build_table(const Prob& p, const int32_t* cu_seqlens, int4* tab, int32_t* seq_off,
                              hipStream_t st);
hipError_t launch_chunk_cumsum(const Prob& p, const float* dt, const float* dt_bias, const float* A,
                               float* delta, float* acs, float* decay, hipStream_t st);
hipError_t launch_chunk_state(const Prob& p, const void* X, const void* Y, const float* delta,
                              const float* acs, ChunkStateT* out, int mode, hipStream_t st);
// Stages 1 and 2 together: delta, acs and the chunk decays are written as
// launch_chunk_cumsum writes them (bit for bit), and the chunk states T.  One
// kernel on the bf16 path; the two kernels one after the other on the fp32 path.
// With C set (only where cb_in_chunk_state(p)), the same kernel also forms
// C.B^T into CB and, if CBt is set, its transpose, as launch_bmm_chunk does.
hipError_t launch_cumsum_chunk_state(const Prob& p, const void* X, const void* Bm, const float* dt,
                                     const float* dt_bias, const float* A, float* delta, float* acs,
                                     float* decay, ChunkStateT* T, hipStream_t st, const void* C = nullptr,
                                     void* CB = nullptr, void* CBt = nullptr);
// Whether the chunk-state kernel forms C.B^T for this problem (so that no
// separate C.B^T kernel is launched).
bool cb_in_chunk_state(const Prob& p);
// passed: fp32, or bf16 when passed_bf16 (the carry and final_states stay fp32)
hipError_t launch_state_passing(const Prob& p, const ChunkStateT* states, const float* decay,
                                const float* init, void* passed, int passed_bf16,
                                float* final_states, int reverse, hipStream_t st);
// CBt (bf16 only, may be null): also store the transpose of every lower tile.
hipError_t launch_bmm_chunk(const Prob& p, const void* B, const void* C, void* CB, hipStream_t st,
                            void* CBt = nullptr);
// passed: fp32, or bf16 when passed_bf16 (bf16 io only)
hipError_t launch_chunk_scan(const Prob& p, const void* x, const void* C, const void* CB,
                             const float* delta, const float* acs, const void* passed,
                             int passed_bf16, const float* D, void* out, hipStream_t st);
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t st);
// Gated RMSNorm (validated shapes): forward (out, r) or backward (dy, dz, dw via
// the per-workgroup partials dwp of norm_bwd_blocks(rows) x D floats).
int norm_bwd_blocks(int rows);
hipError_t launch_gated_rmsnorm(int rows, int D, int group, float eps, const void* y, const void* z,
                                const float* w, void* out, float* r, const void* dout, void* dy, void* dz,
                                float* dwp, float* dw, bool bwd, hipStream_t st);

// Everything the backward chunk kernels read and write.
struct BwdArgs {
  const void *x, *B, *C, *dout;
  const float *dt, *dt_bias, *A, *D;
  const float *delta, *acs, *decay;
  const void *Hp, *dE;  // per (chunk, head) P x N: bf16 on the bf16 path, fp32 otherwise
  const void *CB, *CBt;
  void* dCBg;          // head-summed dCB per (chunk, group), (Q, Q) row-major
  float *Rp, *Kp;      // per (chunk, head, tile of 64 or 128 tokens, token): R and K partials
  void *dx, *dB, *dC;
  float *ddt, *dA, *dD, *d_dt_bias;
  // per token (nck, H, Q): direct d(delta); s (bf16 path) or K+s (fp32 path);
  // r (bf16 path) or r+R (fp32 path)
  float *ddd, *Ks, *rR;
  // per (chunk, head): alpha<dE,H> + sum s, and partials of dD, dA, d_dt_bias
  float *last_term, *dDp, *dAp, *dbp;
};
// The fused chained forward (k_fwd_chained.hip).  `sync` holds kChainSyncWords
// words (ticket counters, wait error) followed by one flag per (chunk slot, head).
struct ChainIO {
  const void *x, *B, *C, *CB;
  const float *dt, *dt_bias, *A, *D, *init;
  void* y;
  float* final_states;
  ChunkStateT* E;  // (nck, H, P, N) carry buffer (the chunk-state region)
  FlagT* sync;     // kChainSyncWords + nck * H words
  float *delta, *acs, *decay;  // saved context, or null
  void* Hp;                    // bf16 passed states, or null
};
bool chained_supported(const Prob& p);
hipError_t launch_fwd_chained(const Prob& p, const ChainIO& io, hipStream_t st);

// which: 0 every chunk kernel; 1 dx, 2 dCB (fp32: dCB, then the r + R rows), 3 dC, 4 dB
hipError_t launch_bwd_chunk(const Prob& p, const BwdArgs& a, int which, hipStream_t st);
// The fp32 matrix-core path (k_f32.hip), where !bf16_kernels(p): the same stages;
// the io tensors (x, B, C, C.B^T, y and the gradients) in p.io's type.
hipError_t launch_chunk_state_f32(const Prob& p, const void* X, const void* Y, const float* delta,
                                  const float* acs, float* out, int mode, hipStream_t st);
hipError_t launch_bmm_chunk_f32(const Prob& p, const void* B, const void* C, void* CB, hipStream_t st);
hipError_t launch_chunk_scan_f32(const Prob& p, const void* x, const void* C, const void* CB,
                                 const float* delta, const float* acs, const float* passed,
                                 const float* D, void* out, hipStream_t st);
hipError_t launch_bwd_f32(const Prob& p, const BwdArgs& a, int which, hipStream_t st);
// dB and dC, their dCB, r and whole R, K in one kernel (k_bwd_dbc.hip): R into
// a.Rp and K into a.Kp, one value per (chunk, head, token); r into a.rR.
bool bwd_fused_supported(const Prob& p);
hipError_t launch_bwd_dbc(const Prob& p, const BwdArgs& a, hipStream_t st);
// fused: R and K are whole per token (launch_bwd_dbc) rather than tile partials
hipError_t launch_bwd_finalize(const Prob& p, const BwdArgs& a, hipStream_t st, bool fused = false);

}  // namespace ssd
