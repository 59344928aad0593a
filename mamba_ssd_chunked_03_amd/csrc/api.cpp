// C ABI of libssd: argument validation, workspace layout and launch order.
//
// Every check the host can make happens before the first launch.  The library
// allocates no memory.  Its only state across calls is one side stream and four
// events per device, created at the first call that forks to them and kept until
// the process ends (side_lane below).  A launch that fails after a call has forked
// to the side stream still joins it back to the caller's stream before the call
// returns SSD_ERR_HIP, so whatever was queued stays ordered on the caller's stream.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdlib>
#include <cstring>
#include <cmath>
#include <mutex>
#include <vector>

#include "internal.hpp"
#include "layout.hpp"
#include "ssd.h"

using namespace ssd;

static_assert(kFlagSequentialScan == SSD_FLAG_SEQUENTIAL_SCAN, "flag bit seen by the kernels");
static_assert(kScanVariantShift == 16 && SSD_FLAG_SCAN_VARIANT(1) == 1 << kScanVariantShift,
              "variant field seen by the kernels");
static_assert(SSD_FLAG_CS_VARIANT(1) == 1 << kCsVariantShift, "chunk-state variant field seen by the kernels");

namespace {

inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool okdim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Validate sizes and fill the kernel-side problem (device pointers unset).
ssd_status make_prob(const ssd_problem* pr, int32_t Q, int packed, Prob& p) {
  if (!pr) return SSD_ERR_NULL;
  if (pr->batch < 0 || pr->seqlen < 0 || pr->nheads <= 0 || pr->headdim <= 0 ||
      pr->dstate <= 0 || pr->ngroups <= 0)
    return SSD_ERR_SHAPE;
  if (pr->nheads % pr->ngroups) return SSD_ERR_SHAPE;
  if (pr->dt_softplus != 0 && pr->dt_softplus != 1) return SSD_ERR_SHAPE;
  if (pr->flags & ~(SSD_FLAG_SAVE_FOR_BWD | SSD_FLAG_FROM_SAVED | SSD_FLAG_ONE_STREAM |
                    SSD_FLAG_SEQUENTIAL_SCAN | SSD_FLAG_CHAINED_FWD | SSD_FLAG_BWD_FUSED | SSD_FLAG_BWD_KERNEL(7) |
                    SSD_FLAG_FWD_KERNEL(7) | SSD_FLAG_SCAN_VARIANT(15) | SSD_FLAG_CS_VARIANT(3)))
    return SSD_ERR_UNSUPPORTED;
  if ((pr->flags & SSD_FLAG_CHAINED_FWD) && (pr->flags & SSD_FLAG_FWD_KERNEL(7))) return SSD_ERR_UNSUPPORTED;
  if (((pr->flags >> 16) & 15) > 7) return SSD_ERR_UNSUPPORTED;
  if ((pr->flags & SSD_FLAG_SEQUENTIAL_SCAN) && ((pr->flags >> 16) & 15) != 0) return SSD_ERR_UNSUPPORTED;
  if ((pr->flags & SSD_FLAG_BWD_KERNEL(7)) && !(pr->flags & SSD_FLAG_FROM_SAVED))
    return SSD_ERR_UNSUPPORTED;
  if (((pr->flags >> 12) & 7) > 4) return SSD_ERR_UNSUPPORTED;
  if (packed && (pr->batch != 1 || pr->nseq < 0)) return SSD_ERR_SHAPE;
  if (pr->io_dtype != SSD_F32 && pr->io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
  if (Q != 64 && Q != 128 && Q != 256) return SSD_ERR_UNSUPPORTED;
  if (!okdim(pr->headdim) || !okdim(pr->dstate)) return SSD_ERR_UNSUPPORTED;
  const int64_t tokens = (int64_t)pr->batch * pr->seqlen;
  if (tokens > INT32_MAX / 2 || (int64_t)pr->nheads > 65535 || (int64_t)pr->ngroups > 65535)
    return SSD_ERR_UNSUPPORTED;
  // kernels address a chunk's token rows with 32-bit byte offsets
  if ((int64_t)Q * pr->nheads * pr->headdim * 4 > INT32_MAX ||
      (int64_t)Q * pr->ngroups * pr->dstate * 4 > INT32_MAX)
    return SSD_ERR_UNSUPPORTED;
  p.B = pr->batch;
  p.L = pr->seqlen;
  p.H = pr->nheads;
  p.P = pr->headdim;
  p.N = pr->dstate;
  p.G = pr->ngroups;
  p.io = pr->io_dtype;
  // bf16 io below the bf16 kernels' 32-wide operand tiles: the fp32 matrix-core kernels
  p.wide = p.io == SSD_BF16 && (pr->headdim < 32 || pr->dstate < 32);
  p.softplus = pr->dt_softplus;
  p.Q = Q;
  p.packed = packed;
  p.flags = pr->flags;
  p.nseq = packed ? pr->nseq : pr->batch;
  if (packed) {
    if (p.nseq > 65535) return SSD_ERR_UNSUPPORTED;
    p.nck = ((int64_t)p.L + (int64_t)p.nseq * (Q - 1)) / Q;
  } else {
    p.nck = (int64_t)p.B * ((p.L + Q - 1) / Q);
  }
  // 1-D grids over (chunk, head) and (chunk, group, tile) slots stay below 2^31 workgroups
  if (p.nck > INT32_MAX / 4 || p.nck * (int64_t)p.H > INT32_MAX / 16) return SSD_ERR_UNSUPPORTED;
  std::memset(&p.map, 0, sizeof(p.map));
  p.map.Q = Q;
  p.map.nck = (int32_t)p.nck;
  p.map.packed = packed;
  p.map.seqlen = p.L;
  p.map.ncs = (p.L + Q - 1) / Q;
  const int csv = (p.flags >> kCsVariantShift) & 3;
  if (csv != kCsTable && !cs_variant_valid(p, csv)) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

inline size_t esize(const Prob& p) { return p.io == SSD_BF16 ? 2 : 4; }

LayoutDims dims(const Prob& p) {
  LayoutDims d;
  d.nck = p.nck;
  d.H = p.H;
  d.P = p.P;
  d.N = p.N;
  d.G = p.G;
  d.Q = p.Q;
  d.nseq = p.nseq;
  d.packed = p.packed != 0;
  d.bf16 = p.io == SSD_BF16;
  d.wide = p.wide != 0;
  return d;
}
FwdLayout fwd_layout(const Prob& p) { return ssd::fwd_layout(dims(p)); }
BwdLayout bwd_layout(const Prob& p) { return ssd::bwd_layout(dims(p)); }

// Whether ssd_bwd forms dB and dC with the one kernel (launch_bwd_dbc).
bool bwd_fused(const Prob& p) { return (p.flags & SSD_FLAG_BWD_FUSED) && bwd_fused_supported(p); }
size_t stage_ws(const Prob& p) { return fwd_layout(p).delta; }

// Point the chunk map at the table inside a workspace and queue its build.
// build = false: the workspace already holds the table (single-kernel relaunch).
// debug_check = false: no SSD_DEBUG check of cu_seqlens (it copies to the host and
// synchronises the stream).
ssd_status setup_map(Prob& p, const int32_t* cu, char* ws, hipStream_t st, bool build = true,
                     bool debug_check = true) {
  if (!p.packed) return SSD_OK;
  FwdLayout l = fwd_layout(p);
  p.map.tab = (const int4*)(ws + l.tab);
  p.map.seq_off = (const int32_t*)(ws + l.seq_off);
  if (!build) return SSD_OK;
  if (debug_check && std::getenv("SSD_DEBUG") && std::getenv("SSD_DEBUG")[0] == '1') {
    std::vector<int32_t> h((size_t)p.nseq + 1);
    if (hipMemcpyAsync(h.data(), cu, h.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return SSD_ERR_HIP;
    if (h[0] != 0 || h[p.nseq] != p.L) return SSD_ERR_VARLEN;
    for (int s = 0; s < p.nseq; ++s)
      if (h[s + 1] < h[s]) return SSD_ERR_VARLEN;
  }
  if (launch_build_table(p, cu, (int4*)(ws + l.tab), (int32_t*)(ws + l.seq_off), st) != hipSuccess)
    return SSD_ERR_HIP;
  return SSD_OK;
}

// A second stream per device, with four events, created on first use (default
// priority) and kept for the life of the process: kernels of one call that do
// not depend on the ones queued before them run there; the caller's stream forks
// to it and joins it again through the events, so each call stays ordered on the
// caller's stream as a whole.  The lock is held while a call queues its work, so
// calls from several host threads do not interleave their event records.  A
// caller's stream that belongs to another device than the current one gets no
// second stream (every kernel of the call then runs on the caller's stream).
struct SideLane {
  bool tried = false, ok = false;
  hipStream_t stream = nullptr;
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
};
SideLane* side_lane(hipStream_t caller, std::unique_lock<std::mutex>& lock) {
  static std::mutex mu;
  static SideLane lanes[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (caller != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(caller, &sdev) != hipSuccess) {
      (void)hipGetLastError();  // not the caller's error: the call goes on without a second stream
      return nullptr;
    }
    if (sdev != dev) return nullptr;
  }
  lock = std::unique_lock<std::mutex>(mu);
  SideLane& l = lanes[dev];
  if (!l.tried) {
    l.tried = true;
    l.ok = hipStreamCreateWithFlags(&l.stream, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; l.ok && i < 4; ++i)
      l.ok = hipEventCreateWithFlags(&l.ev[i], hipEventDisableTiming) == hipSuccess;
  }
  if (!l.ok) {
    lock.unlock();
    return nullptr;
  }
  return &l;
}

#define SSD_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return SSD_ERR_HIP; \
  } while (0)

// After a fork to the side stream: on a failed launch, join the side stream back
// to the caller's stream (event 2) before returning, so that the work already
// queued there stays ordered on the caller's stream.
ssd_status join_failed(SideLane* side, hipStream_t st) {
  if (side) {
    (void)hipEventRecord(side->ev[2], side->stream);
    (void)hipStreamWaitEvent(st, side->ev[2], 0);
  }
  return SSD_ERR_HIP;
}
#define SSD_TRY_FORKED(expr)                                 \
  do {                                                       \
    if ((expr) != hipSuccess) return join_failed(side, st);  \
  } while (0)

bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* q : ps)
    if (q && !al16(q)) return false;
  return true;
}

}  // namespace

// ---------------------------------------------------- fixed device scratch ----
// The workspace of ssd_fwd_noalloc: a file-scope device array of a fixed size.
// Each device the library runs on holds its own copy, at its own address, until
// the process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is looked up once per device, with that
// device current, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {
// The current device's address of `scratch`.  `stream` must belong to the current
// device (a stream of another device would run its kernels on that device, whose
// copy has another address): SSD_ERR_UNSUPPORTED otherwise.
ssd_status noalloc_scratch(hipStream_t stream, void** out) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SSD_ERR_HIP;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SSD_ERR_HIP;
    if (sdev != dev) return SSD_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) return SSD_ERR_HIP;
    addr[dev] = a;
  }
  *out = addr[dev];
  return SSD_OK;
}
}  // namespace

extern "C" {

int32_t ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_status_string(int32_t s) {
  switch (s) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL: return "a required pointer is NULL";
    case SSD_ERR_SHAPE: return "negative or inconsistent sizes";
    case SSD_ERR_UNSUPPORTED: return "configuration outside the supported set";
    case SSD_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_VARLEN: return "cu_seqlens failed the debug check";
    case SSD_ERR_HIP: return "HIP call or kernel launch failed";
    default: return "unknown status";
  }
}

int64_t ssd_num_chunks(const ssd_problem* pr, int32_t Q, int32_t packed) {
  Prob p;
  if (make_prob(pr, Q, packed, p) != SSD_OK) return -1;
  return p.nck;
}

int64_t ssd_fwd_chained_error_offset(const ssd_problem* pr, int32_t Q, int32_t packed) {
  Prob p;
  if (make_prob(pr, Q, packed, p) != SSD_OK) return -1;
  return (int64_t)(fwd_layout(p).sync + 8 * 4);
}

int32_t ssd_scan_variant(const ssd_problem* pr, int32_t Q, int32_t packed) {
  Prob p;
  if (make_prob(pr, Q, packed, p) != SSD_OK) return 0;
  return scan_variant_for(p);
}

int32_t ssd_cs_variant(const ssd_problem* pr, int32_t Q, int32_t packed) {
  Prob p;
  if (make_prob(pr, Q, packed, p) != SSD_OK) return 0;
  return cs_variant_for(p);
}

int32_t ssd_fwd_kernel_mask(const ssd_problem* pr, int32_t Q, int32_t packed) {
  Prob p;
  if (make_prob(pr, Q, packed, p) != SSD_OK) return 0;
  return cb_in_chunk_state(p) ? 0xB : 0xF;
}

int32_t ssd_bwd_kernel_mask(const ssd_problem* pr, int32_t Q, int32_t packed) {
  Prob p;
  if (make_prob(pr, Q, packed, p) != SSD_OK) return 0;
  return bwd_fused(p) ? 0x4F : 0x7F;
}

size_t ssd_fwd_workspace_bytes(const ssd_problem* pr, int32_t Q, int32_t packed) {
  Prob p;
  if (make_prob(pr, Q, packed, p) != SSD_OK) return 0;
  return fwd_layout(p).end;
}

size_t ssd_bwd_workspace_bytes(const ssd_problem* pr, int32_t Q, int32_t packed) {
  Prob p;
  if (make_prob(pr, Q, packed, p) != SSD_OK) return 0;
  return bwd_layout(p).end;
}

size_t ssd_stage_workspace_bytes(const ssd_problem* pr, int32_t Q, int32_t packed) {
  Prob p;
  if (make_prob(pr, Q, packed, p) != SSD_OK) return 0;
  return stage_ws(p);
}

// The forward of ssd_fwd on a given workspace; debug_check as in setup_map.
static ssd_status fwd_run(const ssd_problem* pr, const void* x, const float* dt,
                          const float* dt_bias, const float* A, const void* B, const void* C,
                          const float* D, const float* init_states, const int32_t* cu_seqlens,
                          int32_t Q, void* out, float* final_states, void* workspace,
                          size_t workspace_bytes, void* stream, bool debug_check) {
  Prob p;
  ssd_status s = make_prob(pr, Q, cu_seqlens != nullptr, p);
  if (s != SSD_OK) return s;
  const bool has_tokens = (int64_t)p.B * p.L > 0;
  if (has_tokens && (!x || !dt || !A || !B || !C || !out)) return SSD_ERR_NULL;
  if (!all_aligned({x, dt, dt_bias, A, B, C, D, init_states, cu_seqlens, out, final_states, workspace}))
    return SSD_ERR_ALIGN;
  const FwdLayout l = fwd_layout(p);
  const bool save = (p.flags & SSD_FLAG_SAVE_FOR_BWD) != 0;
  const size_t need = save ? bwd_layout(p).end : l.end;
  if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int only = (p.flags >> 12) & 7;  // 0: every kernel
  if ((p.flags & SSD_FLAG_CHAINED_FWD) && !chained_supported(p)) return SSD_ERR_UNSUPPORTED;
  s = setup_map(p, cu_seqlens, ws, st, only == 0, debug_check);
  if (s != SSD_OK) return s;
  if (p.flags & SSD_FLAG_CHAINED_FWD) {
    // C.B^T (and its transpose for a saved context), then the fused chained kernel;
    // the carry buffer is the chunk-state slot, the flags the sync slot
    void* CBt = (save && bf16_kernels(p)) ? (void*)(ws + bwd_layout(p).CBt) : nullptr;
    if (p.nck > 0) SSD_TRY(launch_bmm_chunk(p, B, C, ws + l.CB, st, CBt));
    ChainIO io;
    io.x = x; io.B = B; io.C = C; io.CB = ws + l.CB;
    io.dt = dt; io.dt_bias = dt_bias; io.A = A; io.D = D; io.init = init_states;
    io.y = out; io.final_states = final_states;
    io.E = (float*)(ws + l.T);
    io.sync = (int32_t*)(ws + l.sync);
    io.delta = save ? (float*)(ws + l.delta) : nullptr;
    io.acs = save ? (float*)(ws + l.acs) : nullptr;
    io.decay = save ? (float*)(ws + l.decay) : nullptr;
    io.Hp = save ? (void*)(ws + l.Hp) : nullptr;
    SSD_TRY(launch_fwd_chained(p, io, st));
    return SSD_OK;
  }
  float* delta = (float*)(ws + l.delta);
  float* acs = (float*)(ws + l.acs);
  float* decay = (float*)(ws + l.decay);
  float* T = (float*)(ws + l.T);
  void* Hp = ws + l.Hp;
  const int hb = bf16_kernels(p);
  void* CB = ws + l.CB;
  void* CBt = (save && bf16_kernels(p)) ? (void*)(ws + bwd_layout(p).CBt) : nullptr;
  // Where the chunk-state kernel forms C.B^T itself (it stages every B slice of
  // the chunk already), the call is three kernels on `stream`.  Otherwise C.B^T,
  // which needs only B and C, runs on the side stream beside the cumsum and chunk
  // states (one kernel on the bf16 path) and the state passing; the chunk scan
  // waits for it.
  const bool cb_fused = cb_in_chunk_state(p);
  std::unique_lock<std::mutex> lane_lock;
  const bool one_stream = (p.flags & SSD_FLAG_ONE_STREAM) != 0;
  SideLane* side = (!only && p.nck > 0 && !cb_fused && !one_stream) ? side_lane(st, lane_lock) : nullptr;
  if (side) {  // events: 0 fork, 1 C.B^T done
    SSD_TRY_FORKED(hipEventRecord(side->ev[0], st));
    SSD_TRY_FORKED(hipStreamWaitEvent(side->stream, side->ev[0], 0));
    SSD_TRY_FORKED(launch_bmm_chunk(p, B, C, CB, side->stream, CBt));
    SSD_TRY_FORKED(hipEventRecord(side->ev[1], side->stream));
  }
  if (!only || only == 1)
    SSD_TRY_FORKED(launch_cumsum_chunk_state(p, x, B, dt, dt_bias, A, delta, acs, decay, T, st,
                                      cb_fused ? C : nullptr, CB, CBt));
  if (!only || only == 2)
    SSD_TRY_FORKED(launch_state_passing(p, T, decay, init_states, Hp, hb, final_states, 0, st));
  if (side) {
    SSD_TRY_FORKED(hipStreamWaitEvent(st, side->ev[1], 0));
  } else if ((!only || only == 3) && !cb_fused) {
    SSD_TRY_FORKED(launch_bmm_chunk(p, B, C, CB, st, CBt));
  }
  if (!only || only == 4) SSD_TRY_FORKED(launch_chunk_scan(p, x, C, CB, delta, acs, Hp, hb, D, out, st));
  return SSD_OK;
}

ssd_status ssd_fwd(const ssd_problem* pr, const void* x, const float* dt, const float* dt_bias,
                   const float* A, const void* B, const void* C, const float* D,
                   const float* init_states, const int32_t* cu_seqlens, int32_t Q, void* out,
                   float* final_states, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_run(pr, x, dt, dt_bias, A, B, C, D, init_states, cu_seqlens, Q, out, final_states,
                 workspace, workspace_bytes, stream, true);
}

ssd_status ssd_fwd_noalloc(const ssd_problem* pr, const void* x, const float* dt,
                           const float* dt_bias, const float* A, const void* B, const void* C,
                           const float* D, const float* init_states, const int32_t* cu_seqlens,
                           int32_t Q, void* out, float* final_states, void* stream) {
  Prob p;
  ssd_status s = make_prob(pr, Q, cu_seqlens != nullptr, p);
  if (s != SSD_OK) return s;
  if (p.flags & ~SSD_FLAG_ONE_STREAM) return SSD_ERR_UNSUPPORTED;
  // the host-detectable errors first, before any HIP call (as ssd_fwd checks them)
  if ((int64_t)p.B * p.L > 0 && (!x || !dt || !A || !B || !C || !out)) return SSD_ERR_NULL;
  if (!all_aligned({x, dt, dt_bias, A, B, C, D, init_states, cu_seqlens, out, final_states}))
    return SSD_ERR_ALIGN;
  if (fwd_layout(p).end > (size_t)SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_WORKSPACE;
  void* ws = nullptr;
  s = noalloc_scratch((hipStream_t)stream, &ws);
  if (s != SSD_OK) return s;
  ssd_problem one = *pr;
  one.flags = SSD_FLAG_ONE_STREAM;
  return fwd_run(&one, x, dt, dt_bias, A, B, C, D, init_states, cu_seqlens, Q, out, final_states,
                 ws, (size_t)SSD_NOALLOC_SCRATCH_BYTES, stream, false);
}

ssd_status ssd_bwd(const ssd_problem* pr, const void* x, const float* dt, const float* dt_bias,
                   const float* A, const void* B, const void* C, const float* D,
                   const float* init_states, const int32_t* cu_seqlens, int32_t Q,
                   const void* dout, const float* d_final_states, void* dx, float* ddt, float* dA,
                   void* dB, void* dC, float* dD, float* d_dt_bias, float* d_init_states,
                   void* workspace, size_t workspace_bytes, void* stream) {
  Prob p;
  ssd_status s = make_prob(pr, Q, cu_seqlens != nullptr, p);
  if (s != SSD_OK) return s;
  const bool has_tokens = (int64_t)p.B * p.L > 0;
  if (has_tokens && (!x || !dt || !A || !B || !C || !dout || !dx || !ddt || !dB || !dC))
    return SSD_ERR_NULL;
  if (!dA || (D && !dD)) return SSD_ERR_NULL;
  if (!all_aligned({x, dt, dt_bias, A, B, C, D, init_states, cu_seqlens, dout, d_final_states, dx,
                    ddt, dA, dB, dC, dD, d_dt_bias, d_init_states, workspace}))
    return SSD_ERR_ALIGN;
  const BwdLayout l = bwd_layout(p);
  if (!workspace || workspace_bytes < l.end) return SSD_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int only = (p.flags >> 8) & 7;  // 0: every kernel
  s = setup_map(p, cu_seqlens, ws, st, only == 0);
  if (s != SSD_OK) return s;
  float* delta = (float*)(ws + l.f.delta);
  float* acs = (float*)(ws + l.f.acs);
  float* decay = (float*)(ws + l.f.decay);
  float* T = (float*)(ws + l.f.T);
  void* Hp = ws + l.f.Hp;
  const int hb = bf16_kernels(p);
  void* CB = ws + l.f.CB;
  void* CBt = ws + l.CBt;
  float* U = (float*)(ws + l.U);
  void* dE = ws + l.dE;
  if (!(p.flags & SSD_FLAG_FROM_SAVED)) {  // forward intermediates, recomputed
    const bool cb_fused = cb_in_chunk_state(p);
    SSD_TRY(launch_cumsum_chunk_state(p, x, B, dt, dt_bias, A, delta, acs, decay, T, st,
                                      cb_fused ? C : nullptr, CB, CBt));
    SSD_TRY(launch_state_passing(p, T, decay, init_states, Hp, hb, nullptr, 0, st));
    if (!cb_fused) SSD_TRY(launch_bmm_chunk(p, B, C, CB, st, bf16_kernels(p) ? CBt : nullptr));
  }
  BwdArgs a;
  a.x = x; a.B = B; a.C = C; a.dout = dout;
  a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.D = D;
  a.delta = delta; a.acs = acs; a.decay = decay; a.Hp = Hp; a.dE = dE;
  a.CB = CB; a.CBt = CBt;
  a.dCBg = ws + l.dCBg;
  a.Rp = (float*)(ws + l.Rp); a.Kp = (float*)(ws + l.Kp);
  a.dx = dx; a.dB = dB; a.dC = dC;
  a.ddt = ddt; a.dA = dA; a.dD = dD; a.d_dt_bias = d_dt_bias;
  a.ddd = (float*)(ws + l.ddd); a.Ks = (float*)(ws + l.Ks); a.rR = (float*)(ws + l.rR);
  a.last_term = (float*)(ws + l.last); a.dDp = (float*)(ws + l.dDp);
  a.dAp = (float*)(ws + l.dAp); a.dbp = (float*)(ws + l.dbp);
  // dB and dC on the bf16 path: three kernels, the head-summed dCB (with R, K
  // tile partials), then dC, which need only forward quantities, and dB, which
  // needs dCB and the reverse scan's dE; with SSD_FLAG_BWD_FUSED one kernel forms
  // all of them with whole R, K from one pass over x and dy, after the reverse
  // scan.  Those run on a side stream (the first two from the start, dB or the
  // one kernel after an event from the reverse scan) beside the adjoint states,
  // the reverse scan and dx; the finalize waits for dCB and dC (or the one
  // kernel) and runs beside dB, and the call ends once dB is done too.
  const bool fused = bwd_fused(p);
  std::unique_lock<std::mutex> lane_lock;
  const bool one_stream = (p.flags & SSD_FLAG_ONE_STREAM) != 0;
  SideLane* side =
      (!only && bf16_kernels(p) && p.nck > 0 && !one_stream) ? side_lane(st, lane_lock) : nullptr;
  // events: 0 fork, 1 reverse scan done, 2 what the finalize reads from the side
  // stream is done (dCB's partials and dC's r; or the one kernel), 3 dB done
  if (side && !fused) {
    SSD_TRY_FORKED(hipEventRecord(side->ev[0], st));
    SSD_TRY_FORKED(hipStreamWaitEvent(side->stream, side->ev[0], 0));
    SSD_TRY_FORKED(launch_bwd_chunk(p, a, 2, side->stream));
    SSD_TRY_FORKED(launch_bwd_chunk(p, a, 3, side->stream));
    SSD_TRY_FORKED(hipEventRecord(side->ev[2], side->stream));
  }
  // adjoint of the state carried into each chunk, then the reverse scan
  if (!only || only == 1)
    SSD_TRY_FORKED(launch_chunk_state(p, dout, C, delta, acs, U, kStateDstates, st));
  if (!only || only == 2)
    SSD_TRY_FORKED(launch_state_passing(p, U, decay, d_final_states, dE, hb, d_init_states, 1, st));
  if (side) {
    // dB (or the one kernel) after the reverse scan; the finalize, which reads
    // nothing dB writes, runs beside dB once dx and dC are done
    SSD_TRY_FORKED(hipEventRecord(side->ev[1], st));
    SSD_TRY_FORKED(hipStreamWaitEvent(side->stream, side->ev[1], 0));
    SSD_TRY_FORKED(fused ? launch_bwd_dbc(p, a, side->stream) : launch_bwd_chunk(p, a, 4, side->stream));
    SSD_TRY_FORKED(hipEventRecord(side->ev[fused ? 2 : 3], side->stream));
    SSD_TRY_FORKED(launch_bwd_chunk(p, a, 1, st));
    SSD_TRY_FORKED(hipStreamWaitEvent(st, side->ev[2], 0));
    SSD_TRY_FORKED(launch_bwd_finalize(p, a, st, fused));
    if (!fused) SSD_TRY_FORKED(hipStreamWaitEvent(st, side->ev[3], 0));
    return SSD_OK;
  } else if (fused) {
    if (!only || only == 3) SSD_TRY_FORKED(launch_bwd_chunk(p, a, 1, st));
    if (!only || only == 4) SSD_TRY_FORKED(launch_bwd_dbc(p, a, st));
  } else if (!only || (only >= 3 && only <= 6)) {
    SSD_TRY_FORKED(launch_bwd_chunk(p, a, only ? only - 2 : 0, st));
  }
  if (!only || only == 7) SSD_TRY_FORKED(launch_bwd_finalize(p, a, st, fused));
  return SSD_OK;
}

ssd_status ssd_stage_chunk_cumsum(const ssd_problem* pr, const float* dt, const float* dt_bias,
                                  const float* A, const int32_t* cu_seqlens, int32_t Q,
                                  float* delta, float* acs, float* chunk_decay, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Prob p;
  ssd_status s = make_prob(pr, Q, cu_seqlens != nullptr, p);
  if (s != SSD_OK) return s;
  if (p.nck > 0 && (!dt || !A || !delta || !acs || !chunk_decay)) return SSD_ERR_NULL;
  if (!all_aligned({dt, dt_bias, A, cu_seqlens, delta, acs, chunk_decay, workspace})) return SSD_ERR_ALIGN;
  const size_t need = stage_ws(p);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  s = setup_map(p, cu_seqlens, (char*)workspace, st);
  if (s != SSD_OK) return s;
  SSD_TRY(launch_chunk_cumsum(p, dt, dt_bias, A, delta, acs, chunk_decay, st));
  return SSD_OK;
}

ssd_status ssd_stage_chunk_state(const ssd_problem* pr, const void* x, const void* B,
                                 const float* delta, const float* acs, const int32_t* cu_seqlens,
                                 int32_t Q, float* states, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  Prob p;
  ssd_status s = make_prob(pr, Q, cu_seqlens != nullptr, p);
  if (s != SSD_OK) return s;
  if (p.nck > 0 && (!x || !B || !delta || !acs || !states)) return SSD_ERR_NULL;
  if (!all_aligned({x, B, delta, acs, cu_seqlens, states, workspace})) return SSD_ERR_ALIGN;
  const size_t need = stage_ws(p);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  s = setup_map(p, cu_seqlens, (char*)workspace, st);
  if (s != SSD_OK) return s;
  SSD_TRY(launch_chunk_state(p, x, B, delta, acs, states, kStateFwd, st));
  return SSD_OK;
}

ssd_status ssd_stage_state_passing(const ssd_problem* pr, const float* states,
                                   const float* chunk_decay, const float* init_states,
                                   const int32_t* cu_seqlens, int32_t Q, float* passed,
                                   float* final_states, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  Prob p;
  ssd_status s = make_prob(pr, Q, cu_seqlens != nullptr, p);
  if (s != SSD_OK) return s;
  if (p.nck > 0 && (!states || !chunk_decay || !passed)) return SSD_ERR_NULL;
  if (!all_aligned({states, chunk_decay, init_states, cu_seqlens, passed, final_states, workspace}))
    return SSD_ERR_ALIGN;
  const size_t need = stage_ws(p);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  s = setup_map(p, cu_seqlens, (char*)workspace, st);
  if (s != SSD_OK) return s;
  SSD_TRY(launch_state_passing(p, states, chunk_decay, init_states, passed, 0, final_states, 0, st));
  return SSD_OK;
}

ssd_status ssd_stage_bmm_chunk(const ssd_problem* pr, const void* B, const void* C,
                               const int32_t* cu_seqlens, int32_t Q, void* CB, void* workspace,
                               size_t workspace_bytes, void* stream) {
  Prob p;
  ssd_status s = make_prob(pr, Q, cu_seqlens != nullptr, p);
  if (s != SSD_OK) return s;
  if (p.nck > 0 && (!B || !C || !CB)) return SSD_ERR_NULL;
  if (!all_aligned({B, C, cu_seqlens, CB, workspace})) return SSD_ERR_ALIGN;
  const size_t need = stage_ws(p);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  s = setup_map(p, cu_seqlens, (char*)workspace, st);
  if (s != SSD_OK) return s;
  SSD_TRY(launch_bmm_chunk(p, B, C, CB, st));
  return SSD_OK;
}

ssd_status ssd_stage_chunk_scan(const ssd_problem* pr, const void* x, const void* C,
                                const void* CB, const float* delta, const float* acs,
                                const float* passed, const float* D, const int32_t* cu_seqlens,
                                int32_t Q, void* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  Prob p;
  ssd_status s = make_prob(pr, Q, cu_seqlens != nullptr, p);
  if (s != SSD_OK) return s;
  if (p.nck > 0 && (!x || !C || !CB || !delta || !acs || !passed || !out)) return SSD_ERR_NULL;
  if (!all_aligned({x, C, CB, delta, acs, passed, D, cu_seqlens, out, workspace})) return SSD_ERR_ALIGN;
  const size_t need = stage_ws(p);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  s = setup_map(p, cu_seqlens, (char*)workspace, st);
  if (s != SSD_OK) return s;
  SSD_TRY(launch_chunk_scan(p, x, C, CB, delta, acs, passed, 0, D, out, st));
  return SSD_OK;
}

}  // extern "C"

namespace {
ssd_status norm_check(const ssd_norm_problem* pr) {
  if (!pr) return SSD_ERR_NULL;
  if (pr->rows < 0 || pr->dim <= 0 || pr->group <= 0) return SSD_ERR_SHAPE;
  if (pr->io_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
  if (pr->dim % 512 || pr->dim > 8192) return SSD_ERR_UNSUPPORTED;
  const int g = pr->group;
  if (g != pr->dim && !((g == 256 || g == 512 || g == 1024 || g == 2048) && pr->dim % g == 0))
    return SSD_ERR_UNSUPPORTED;
  if (!(pr->eps >= 0.f) || !std::isfinite(pr->eps)) return SSD_ERR_UNSUPPORTED;
  if ((int64_t)pr->rows * pr->dim > INT32_MAX / 2) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}
}  // namespace

extern "C" {

size_t ssd_gated_rmsnorm_bwd_workspace_bytes(const ssd_norm_problem* pr) {
  if (norm_check(pr) != SSD_OK) return 0;
  return (size_t)norm_bwd_blocks(pr->rows) * pr->dim * 4;
}

ssd_status ssd_gated_rmsnorm_fwd(const ssd_norm_problem* pr, const void* y, const void* z,
                                 const float* weight, void* out, float* rstd, void* stream) {
  ssd_status s = norm_check(pr);
  if (s != SSD_OK) return s;
  if (pr->rows > 0 && (!y || !weight || !out)) return SSD_ERR_NULL;
  if (!all_aligned({y, z, weight, out, rstd})) return SSD_ERR_ALIGN;
  if (pr->rows == 0) return SSD_OK;
  SSD_TRY(launch_gated_rmsnorm(pr->rows, pr->dim, pr->group, pr->eps, y, z, weight, out, rstd, nullptr,
                               nullptr, nullptr, nullptr, nullptr, false, (hipStream_t)stream));
  return SSD_OK;
}

ssd_status ssd_gated_rmsnorm_bwd(const ssd_norm_problem* pr, const void* dout, const void* y,
                                 const void* z, const float* weight, void* dy, void* dz,
                                 float* dweight, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  ssd_status s = norm_check(pr);
  if (s != SSD_OK) return s;
  if (!weight || !dweight) return SSD_ERR_NULL;
  if (pr->rows > 0 && (!dout || !y || !dy)) return SSD_ERR_NULL;
  if ((z == nullptr) != (dz == nullptr)) return SSD_ERR_NULL;
  if (!all_aligned({dout, y, z, weight, dy, dz, dweight, workspace})) return SSD_ERR_ALIGN;
  const size_t need = ssd_gated_rmsnorm_bwd_workspace_bytes(pr);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_WORKSPACE;
  SSD_TRY(launch_gated_rmsnorm(pr->rows, pr->dim, pr->group, pr->eps, y, z, weight, nullptr, nullptr,
                               dout, dy, dz, (float*)workspace, dweight, true, (hipStream_t)stream));
  return SSD_OK;
}

ssd_status ssd_util_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes == 0) return SSD_OK;
  if (!dst || !src) return SSD_ERR_NULL;
  if (!al16(dst) || !al16(src) || (bytes & 15)) return SSD_ERR_ALIGN;
  SSD_TRY(launch_copy(dst, src, bytes, (hipStream_t)stream));
  return SSD_OK;
}

}  // extern "C"
