/*
 * libssd — Mamba-2 selective state-space (SSD) chunked scan for AMD MI355X (gfx950).
 *
 * What it computes.  Per sequence and head h (group g = h / (nheads/ngroups)),
 * with the state S = h^T of shape (headdim P, dstate N):
 *
 *     delta_t = softplus(dt_t + dt_bias_h)  (dt_softplus = 1)   or   dt_t + dt_bias_h
 *     S_t     = exp(delta_t * A_h) * S_{t-1} + delta_t * x_t B_t^T
 *     y_t     = S_t C_t + D_h * x_t,        S_{-1} = init,   final = S_last
 *
 * This is the selective SSM recurrence of gigipick.blogspot.com "LLM Mamba ...",
 * section 1 (its printed equation was lost; the Mamba-2 form with one scalar decay
 * per head is used).  It runs as a chunked scan: a per-chunk cumulative sum of
 * delta*A, per-chunk states, cross-chunk state passing as an associative scan
 * (scan page, section 2; aitrends.kr/articles/109906, "Helion-based B200 kernel
 * redesign", which replaces the sequential state-passing loops forward and
 * backward by an associative scan), and a per-chunk output stage.  The chunk
 * carry (one chunk's final state seeds the next) follows the scan page,
 * section 3 ("memory hierarchy").
 *
 * Conventions for every entry point.
 *  - Tensors are dense, row-major (last index fastest):
 *        x, out, dout, dx        (batch, seqlen, nheads, headdim)     io dtype
 *        dt, ddt                 (batch, seqlen, nheads)              fp32
 *        B, C, dB, dC            (batch, seqlen, ngroups, dstate)     io dtype
 *        dt_bias, A, D, dA, dD, d_dt_bias   (nheads)                 fp32
 *        init, final, d_final, d_init       (nstates, nheads, headdim, dstate)  fp32
 *            nstates = batch, or nseq when cu_seqlens is given
 *        cu_seqlens              (nseq + 1) int32, device memory, rising from 0 to seqlen
 *  - With cu_seqlens the problem is one packed row (batch must be 1) holding nseq
 *    sequences; each is chunked from its own first token, starts from its own init
 *    state, and no state crosses a boundary.  Empty sequences are allowed (their
 *    final state is their init).
 *  - Every pointer except `problem` is DEVICE memory owned by the caller.  The
 *    library allocates nothing, keeps no pointer after returning, and modifies no
 *    input.  Outputs must not alias inputs or the workspace.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is queued on
 *    it and the call returns before it runs; keep buffers alive until then.
 *  - State kept across calls: none, except this.  ssd_fwd and ssd_bwd run kernels
 *    that do not depend on each other on a second stream of the library's own
 *    (one per device, with four events, created by the first call that uses it,
 *    default priority, kept until the process ends; ssd_fwd uses none where its
 *    chunk-state kernel forms C.B^T, see ssd_fwd_kernel_mask), forked from and
 *    joined back to `stream` with events: the call as a whole stays ordered on
 *    `stream`, also when a launch fails after the fork, and it can be captured
 *    into a HIP graph.  Calls issued on different streams at the same time share
 *    that second stream (they stay correct; their side kernels queue behind each
 *    other).  The second stream belongs to the current device: when `stream`
 *    belongs to another device, the call queues all of its kernels on `stream`
 *    alone, and so does every call with SSD_FLAG_ONE_STREAM, which then creates
 *    no stream and no event.
 *  - Every error the host can detect (NULL, shape, alignment, workspace size,
 *    unsupported configuration) is returned BEFORE anything is queued.  A failed
 *    launch returns SSD_ERR_HIP.  Nothing is printed; no exception crosses the ABI.
 *  - Pointers must be 16-byte aligned.
 *  - Supported: io dtype f32 or bf16; headdim and dstate in {16, 32, 64, 128}
 *    (a bf16 problem with headdim or dstate 16 runs on the fp32 matrix-core
 *    kernels: its bf16 tensors are widened to fp32 in registers, its
 *    intermediates are fp32, and its outputs are rounded to bf16);
 *    chunk_size in {64, 128, 256}; nheads % ngroups == 0; chunk_size * nheads *
 *    headdim * 4 and chunk_size * ngroups * dstate * 4 at most 2^31 - 1 (one
 *    chunk's token rows are addressed with 32-bit byte offsets); any seqlen >= 0
 *    and any sequence lengths (partial chunks are masked).  Anything else returns
 *    SSD_ERR_UNSUPPORTED.
 *  - cu_seqlens contents are the caller's contract; with the environment variable
 *    SSD_DEBUG=1 they are copied to the host and checked (SSD_ERR_VARLEN).  That
 *    check synchronises the stream.
 *  - Results are bitwise reproducible run to run (every reduction has a fixed
 *    order); they differ from a sequential evaluation only by rounding order.
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 11

typedef enum {
  SSD_OK = 0,
  SSD_ERR_NULL = 1,        /* a required pointer is NULL */
  SSD_ERR_SHAPE = 2,       /* negative or inconsistent sizes */
  SSD_ERR_UNSUPPORTED = 3, /* valid, but outside the supported set above */
  SSD_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  SSD_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  SSD_ERR_VARLEN = 6,      /* cu_seqlens failed the SSD_DEBUG check */
  SSD_ERR_HIP = 7          /* a HIP call or kernel launch failed */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* ssd_problem.flags (bit set).
 * SSD_FLAG_SAVE_FOR_BWD: ssd_fwd keeps its intermediates (delta, the cumsum, the
 *   passed states and C.B^T in both orientations) in the workspace, which must then
 *   hold ssd_bwd_workspace_bytes().
 * SSD_FLAG_FROM_SAVED: ssd_bwd takes those intermediates from its workspace instead
 *   of recomputing them.  The workspace must be the one a SAVE_FOR_BWD ssd_fwd call
 *   on the same problem, inputs and chunk size last wrote, unmodified since; nothing
 *   checks this. */
#define SSD_FLAG_SAVE_FOR_BWD 1
#define SSD_FLAG_FROM_SAVED 2
/* SSD_FLAG_ONE_STREAM: every kernel of the call runs on `stream`; the library
 *   creates and uses no stream or event of its own.  Results are identical. */
#define SSD_FLAG_ONE_STREAM 4
/* SSD_FLAG_SEQUENTIAL_SCAN: the cross-chunk state passing (forward, and the reverse
 *   pass of ssd_bwd) walks each sequence's chunks in order with one carry per state
 *   element, the sequential loop that the associative scan replaces
 *   (aitrends.kr/articles/109906, "Helion-based B200 kernel redesign"), instead of
 *   the log-depth scan.  A comparison point for measurement; results agree with
 *   the default to rounding (the association order differs).  Valid on ssd_fwd,
 *   ssd_bwd and ssd_stage_state_passing. */
#define SSD_FLAG_SEQUENTIAL_SCAN 8
/* SSD_FLAG_SCAN_VARIANT(v), v = 0..7: which kernel runs the cross-chunk state
 *   passing (forward and reverse).  0 (the default) takes the library's tuned
 *   per-shape table (measured on this GPU by mamba_ssd_chunked_03_amd/tuning/sweep.py,
 *   compiled into the library): the analogue of the pages' configuration files
 *   written by an offline sweep and loaded at training time (aitrends.kr/articles/
 *   109906, "putting autotune results into the training pipeline").  1..4: the
 *   log-depth associative scan with W waves x S chunks per wave of
 *   4x2, 8x4, 16x4, 16x8; 5..7: the sequential carry with 1, 4, 8 chunks of loads
 *   in flight (5 is SSD_FLAG_SEQUENTIAL_SCAN).  Results agree to rounding. */
#define SSD_FLAG_SCAN_VARIANT(v) ((v) << 16)
/* SSD_FLAG_CS_VARIANT(v), v = 0..3: the form of the chunk-state kernels (the
 *   forward's chunk states with the inline cumsum, and the backward's adjoint
 *   chunk states) on the bf16 path.  0 (the default) takes the tuned per-shape
 *   table's entry for the problem's (headdim, dstate, heads per group, chunk size),
 *   measured on this GPU by mamba_ssd_chunked_03_amd/tuning/sweep.py and compiled
 *   into the library (aitrends.kr/articles/109906, "putting autotune results into
 *   the training pipeline"), else the widest form the shape allows.  1: one head
 *   per workgroup, C.B^T by its own kernel; 2: two heads of a group per workgroup
 *   (sharing each staged slice of B or C), C.B^T by its own kernel; 3: two heads per
 *   workgroup, C.B^T formed inside the chunk-state kernel.  2 needs an even number
 *   of heads per group (and, with dstate 32 or headdim 128 at dstate 128, is
 *   outside the kernel's shapes); 3 also needs chunk_size 256 and eight heads per
 *   group; a variant the problem cannot run, or 2 or 3 where the fp32 matrix-core
 *   kernels run (fp32 io, or bf16 with headdim or dstate 16), returns
 *   SSD_ERR_UNSUPPORTED.  Results are bitwise the same for every variant. */
#define SSD_FLAG_CS_VARIANT(v) ((v) << 20)
/* SSD_FLAG_CHAINED_FWD: ssd_fwd runs the fused single-pass forward: after the
 *   C.B^T kernel, one kernel forms each chunk's state, takes the state entering the
 *   chunk from the previous chunk's workgroup (a chained scan: work is handed out
 *   in chunk order, each chunk's carry-out published through memory with a release
 *   store of a flag and picked up with an acquire), and writes the output, so the
 *   chunk states and passed states never make a round trip through memory (scan
 *   page, section 3, "kernel fusion" and "memory hierarchy": the chunk carry kept
 *   on chip).  Every wait is bounded: a wait that runs out sets an error word
 *   (ssd_fwd_chained_error) and the kernel still finishes.  Supported for bf16 io
 *   with headdim in {32, 64, 128} and dstate in {64, 128} (SSD_ERR_UNSUPPORTED
 *   otherwise), with or without SSD_FLAG_SAVE_FOR_BWD (the saved context is the one
 *   ssd_bwd expects), not with SSD_FLAG_FWD_KERNEL.  All kernels run on `stream`.
 *   Results agree with the default forward to rounding. */
#define SSD_FLAG_CHAINED_FWD 16
/* SSD_FLAG_BWD_FUSED: ssd_bwd forms dB and dC, their head-summed dCB and the
 *   decay-gradient sums with one kernel, from one pass over x and dy (the scan page,
 *   section 3, "kernel fusion": fewer global-memory passes), instead of three
 *   kernels (the head-summed dCB with per-tile partials of the decay-gradient sums,
 *   then dC, then dB, which read x and dy twice each).  A comparison point for
 *   measurement (it moves fewer bytes but runs one workgroup per compute unit, and
 *   is slower on MI355X): dB and dC are bitwise the same; ddt, dA and d_dt_bias
 *   agree to rounding (their decay-gradient sums are added in another order).  bf16
 *   io with headdim and dstate >= 32 only; no effect where the fp32 matrix-core
 *   kernels run, which always form dB and dC their own way. */
#define SSD_FLAG_BWD_FUSED 32
/* SSD_FLAG_BWD_KERNEL(k), k = 1..7: a profiling aid, valid only together with
 *   SSD_FLAG_FROM_SAVED.  ssd_bwd launches only its k-th kernel: 1 adjoint chunk
 *   states, 2 reverse state passing, 3 dx (with the direct delta gradient),
 *   4 head-summed dCB with the decay-gradient partials, 5 dC, 6 dB, 7 finalize
 *   (ddt and the per-head sums); where ssd_bwd_kernel_mask() leaves bits 4 and 5
 *   clear (SSD_FLAG_BWD_FUSED), 4 is the one kernel forming dB and dC, and 5, 6
 *   launch nothing.  The
 *   workspace and the gradient buffers must hold the results of a complete ssd_bwd
 *   call on the same arguments, so that the kernel finds its inputs; it rewrites
 *   its own outputs with the same values. */
#define SSD_FLAG_BWD_KERNEL(k) ((k) << 8)
/* SSD_FLAG_FWD_KERNEL(k), k = 1..4: the same for ssd_fwd, whose workspace and
 *   outputs must hold a complete call's results on the same arguments: 1 chunk
 *   cumsum and chunk states (one kernel on the bf16 path), 2 state passing,
 *   3 C.B^T, 4 chunk scan.  Where ssd_fwd_kernel_mask() leaves bit 2 clear, C.B^T
 *   is formed by kernel 1 and k = 3 launches nothing. */
#define SSD_FLAG_FWD_KERNEL(k) ((k) << 12)

typedef struct {
  int32_t batch;       /* B (1 when cu_seqlens is given) */
  int32_t seqlen;      /* L: tokens per batch row (total packed tokens with cu_seqlens) */
  int32_t nheads;      /* H */
  int32_t headdim;     /* P */
  int32_t dstate;      /* N */
  int32_t ngroups;     /* G; heads h*G/H share B and C of group h / (H/G) */
  int32_t nseq;        /* number of packed sequences; read only when cu_seqlens != NULL */
  int32_t io_dtype;    /* ssd_dtype of x, B, C, out, dout, dx, dB, dC */
  int32_t dt_softplus; /* 1: delta = softplus(dt + dt_bias); 0: delta = dt + dt_bias */
  int32_t flags;       /* SSD_FLAG_* bits, 0 for none */
} ssd_problem;

/* ABI version (SSD_ABI_VERSION) and a static message for a status code. */
int32_t ssd_abi_version(void);
const char* ssd_status_string(int32_t status);

/* Which of the four forward kernels (bit k-1 for SSD_FLAG_FWD_KERNEL(k)) a complete
 * ssd_fwd call on this problem launches: 0xF, or 0xB where the chunk-state kernel
 * also forms C.B^T (bf16, chunk_size 256, eight heads per group, so that each pair
 * of a group's heads holds one 64-row block of the chunk's C.B^T).  A profiling and
 * accounting aid; the results do not depend on it.  Returns 0 for an invalid problem. */
int32_t ssd_fwd_kernel_mask(const ssd_problem* problem, int32_t chunk_size, int32_t packed);

/* Which chunk-state form (SSD_FLAG_CS_VARIANT numbering, 1..3) ssd_fwd and ssd_bwd
 * run for this problem: the variant forced by problem->flags, else the tuned
 * table's entry, else the widest valid form.  0 for an invalid problem. */
int32_t ssd_cs_variant(const ssd_problem* problem, int32_t chunk_size, int32_t packed);

/* Which of the seven backward kernels (bit k-1 for SSD_FLAG_BWD_KERNEL(k)) a complete
 * ssd_bwd call on this problem launches: 0x7F, or 0x4F where one kernel forms dB and
 * dC (bf16 with SSD_FLAG_BWD_FUSED).  A profiling and accounting aid.  Returns 0
 * for an invalid problem. */
int32_t ssd_bwd_kernel_mask(const ssd_problem* problem, int32_t chunk_size, int32_t packed);

/* Which state-passing kernel (SSD_FLAG_SCAN_VARIANT numbering, 1..7) ssd_fwd and
 * ssd_bwd run for this problem: the variant forced by problem->flags, else the
 * tuned table's entry nearest to the problem's chunks per sequence and lane count
 * (sequences x nheads x headdim x dstate / 4).  0 for an invalid problem. */
int32_t ssd_scan_variant(const ssd_problem* problem, int32_t chunk_size, int32_t packed);

/* Byte offset, inside the workspace of an SSD_FLAG_CHAINED_FWD ssd_fwd call, of the
 * int32 word that the call's fused kernel sets when a wait for the previous chunk's
 * carry ran out (0: every wait ended normally; the results are then valid).  -1 for
 * an invalid problem. */
int64_t ssd_fwd_chained_error_offset(const ssd_problem* problem, int32_t chunk_size, int32_t packed);

/* Number of chunk slots the per-chunk stage arrays below must hold:
 * batch * ceil(seqlen / chunk_size), or floor((seqlen + nseq*(chunk_size-1)) / chunk_size)
 * with cu_seqlens (an upper bound; unused trailing slots are never written).
 * Returns -1 for an invalid problem. */
int64_t ssd_num_chunks(const ssd_problem* problem, int32_t chunk_size, int32_t packed);

/* Workspace sizes in bytes (0 for an invalid problem).  `packed` = 1 when
 * cu_seqlens will be passed.  The forward workspace holds the chunk table,
 * delta, the within-chunk cumsum, the chunk states (fp32), the passed states
 * (bf16 where the bf16 kernels run, which only feed them to bf16 matrix
 * products; fp32 otherwise) and C.B^T per chunk; the backward one adds the
 * adjoint states. */
size_t ssd_fwd_workspace_bytes(const ssd_problem* problem, int32_t chunk_size, int32_t packed);
size_t ssd_bwd_workspace_bytes(const ssd_problem* problem, int32_t chunk_size, int32_t packed);
/* Workspace for the ssd_stage_* entries (the chunk table only). */
size_t ssd_stage_workspace_bytes(const ssd_problem* problem, int32_t chunk_size, int32_t packed);

/* Forward pass: out = y, final_states = S_last (optional, may be NULL).
 * dt_bias, D, init_states and cu_seqlens may be NULL (zero bias, no skip term,
 * zero initial state, unpacked batch).
 * What it computes: the selective-SSM recurrence of the scan page
 * (gigipick.blogspot.com "LLM Mamba ...", section 1), evaluated chunk by chunk:
 * within-chunk cumsum, chunk states, the cross-chunk carry as an associative
 * scan (section 2 and its Hillis-Steele pseudo-code; aitrends.kr/articles/109906,
 * "Helion-based B200 kernel redesign", for _state_passing_fwd), and the per-chunk
 * output with C.h_prev and the D skip term fused (scan page, section 3, "kernel
 * fusion" and "memory hierarchy").  One call replaces the whole forward module
 * (aitrends.kr/articles/109906, "putting autotune results into the training
 * pipeline": a 1:1 drop-in module). */
ssd_status ssd_fwd(const ssd_problem* problem,
                   const void* x, const float* dt, const float* dt_bias, const float* A,
                   const void* B, const void* C, const float* D,
                   const float* init_states, const int32_t* cu_seqlens, int32_t chunk_size,
                   void* out, float* final_states,
                   void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): ssd_fwd with its workspace
 * in a fixed device array of SSD_NOALLOC_SCRATCH_BYTES bytes inside the library,
 * one per device, held from the library's first use on that device until the
 * process ends.  Arguments and results are those of ssd_fwd (the same kernels, all
 * on `stream`), without workspace and workspace_bytes.
 *  - problem->flags must be 0 or SSD_FLAG_ONE_STREAM (no saved context, no
 *    single-kernel launches): SSD_ERR_UNSUPPORTED otherwise.
 *  - A problem whose forward workspace (ssd_fwd_workspace_bytes) exceeds
 *    SSD_NOALLOC_SCRATCH_BYTES returns SSD_ERR_WORKSPACE before anything is queued.
 *  - `stream` must belong to the current device (SSD_ERR_UNSUPPORTED otherwise).
 *  - Nothing is allocated: no hipMalloc, hipFree, stream or event creation.  The
 *    first call on a device looks up that device's array address once.  The
 *    SSD_DEBUG check of cu_seqlens is not run (it would copy to the host).
 *  - Every call on a device uses that device's one array, which keeps the last
 *    call's contents (no value a call reads comes from an earlier call).  Calls
 *    that overlap in time on one device -- on different streams, or from several
 *    host threads before their work has finished -- race on it and give undefined
 *    results: order them on one stream. */
#define SSD_NOALLOC_SCRATCH_BYTES (64u << 20)
ssd_status ssd_fwd_noalloc(const ssd_problem* problem,
                           const void* x, const float* dt, const float* dt_bias, const float* A,
                           const void* B, const void* C, const float* D,
                           const float* init_states, const int32_t* cu_seqlens, int32_t chunk_size,
                           void* out, float* final_states, void* stream);

/* Backward pass for the loss L = <dout, y> + <d_final_states, final>: the adjoint
 * of ssd_fwd's recurrence (scan page, section 1), with the cross-chunk part as the
 * reverse associative scan that replaces _state_passing_bwd's sequential loop
 * (aitrends.kr/articles/109906, "Helion-based B200 kernel redesign"), and every
 * reduction over tokens or heads in a fixed order (the fixed-order tree fold of the
 * FlashInfer Cake RMSNorm page, "key optimisation techniques"), so results are
 * bitwise reproducible.
 * Inputs are those of ssd_fwd plus dout and d_final_states (NULL = 0).
 * Outputs: dx, dB, dC (io dtype; dB and dC summed over each group's heads in
 * fp32 before rounding), ddt (w.r.t. the raw dt input), dA (required), and the
 * optional dD (required iff D != NULL; computed whenever given), d_dt_bias,
 * d_init_states.  The forward intermediates are recomputed inside unless
 * problem->flags has SSD_FLAG_FROM_SAVED (see above). */
ssd_status ssd_bwd(const ssd_problem* problem,
                   const void* x, const float* dt, const float* dt_bias, const float* A,
                   const void* B, const void* C, const float* D,
                   const float* init_states, const int32_t* cu_seqlens, int32_t chunk_size,
                   const void* dout, const float* d_final_states,
                   void* dx, float* ddt, float* dA, void* dB, void* dC,
                   float* dD, float* d_dt_bias, float* d_init_states,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Single-stage entry points (testing and per-stage timing).  Each queues exactly
 * the kernels of one stage of ssd_fwd on explicit buffers.  nck = ssd_num_chunks().
 * Per-chunk layouts (fp32 unless noted):
 *     delta, acs     (nck, nheads, chunk_size); acs = within-chunk inclusive cumsum
 *                    of delta*A in LOG2 units (natural-log value * log2(e));
 *                    entries past a chunk's length are zero
 *     chunk_decay    (nck, nheads) = acs at the chunk's last token (log2 units)
 *     states, passed (nck, nheads, headdim, dstate): chunk-local end state T_c, and
 *                    the state H_c entering each chunk
 *     CB             (nck, ngroups, chunk_size, chunk_size) io dtype: C_i . B_j for
 *                    j <= i (entries above the diagonal are not written).  Where
 *                    the bf16 matrix-core kernels run (bf16 io, headdim and dstate
 *                    >= 32) each chunk's Q x Q matrix is stored in fragment order:
 *                    element (i, j) at offset ((i/16)(Q/32) + j/32) 512
 *                    + ((j%32)/8 16 + i%16) 8 + j%8, i.e. 16 x 32 blocks of 1 KB, each
 *                    laid out as the 64 lanes of an MFMA operand load read it; the
 *                    fp32 matrix-core kernels store it row-major.  ssd_stage_bmm_chunk
 *                    writes and ssd_stage_chunk_scan reads the same order.
 */
/* Stage 1 — per-chunk cumulative sum of delta*A (wavefront prefix sum): the
 * log-decays of the recurrence (scan page, section 1) summed within each chunk of
 * the chunked form (scan page, "memory hierarchy": work in chunks whose carry
 * seeds the next).  dt_bias may be NULL. */
ssd_status ssd_stage_chunk_cumsum(const ssd_problem* problem, const float* dt,
                                  const float* dt_bias, const float* A,
                                  const int32_t* cu_seqlens, int32_t chunk_size,
                                  float* delta, float* acs, float* chunk_decay,
                                  void* workspace, size_t workspace_bytes, void* stream);
/* Stage 2 — chunk states T_c = sum_j delta_j exp(acs_last - acs_j) x_j B_j^T (MFMA):
 * each chunk's end state from a zero start, the carry-out of the scan page's
 * "memory hierarchy" section, i.e. the b part of the chunk's pair in section 2. */
ssd_status ssd_stage_chunk_state(const ssd_problem* problem, const void* x, const void* B,
                                 const float* delta, const float* acs,
                                 const int32_t* cu_seqlens, int32_t chunk_size, float* states,
                                 void* workspace, size_t workspace_bytes, void* stream);
/* Stage 3 — cross-chunk state passing E_c = exp(chunk_decay_c) H_c + T_c as an
 * associative scan (scan page, section 2 and its Hillis-Steele pseudo-code;
 * aitrends.kr/articles/109906, "Helion-based B200 kernel redesign": the sequential
 * _state_passing_fwd loop turned into an associative scan); passed = H_c,
 * final_states = E_last (may be NULL).  init_states may be NULL (zero). */
ssd_status ssd_stage_state_passing(const ssd_problem* problem, const float* states,
                                   const float* chunk_decay, const float* init_states,
                                   const int32_t* cu_seqlens, int32_t chunk_size,
                                   float* passed, float* final_states,
                                   void* workspace, size_t workspace_bytes, void* stream);
/* Stage 4 — CB = C B^T per chunk and group (MFMA), lower triangle: the
 * within-chunk interaction matrix of the chunked form of the recurrence (scan page,
 * section 1, unrolled over one chunk), shared by the group's heads. */
ssd_status ssd_stage_bmm_chunk(const ssd_problem* problem, const void* B, const void* C,
                               const int32_t* cu_seqlens, int32_t chunk_size, void* CB,
                               void* workspace, size_t workspace_bytes, void* stream);
/* Stage 5 — y_i = sum_{j<=i} CB_ij exp(acs_i - acs_j) delta_j x_j
 *               + exp(acs_i) H_c C_i + D x_i   (MFMA, bf16/fp32 store):
 * the recurrence's output (scan page, section 1) inside a chunk, seeded by the
 * carried-in state, with the skip term and the store fused into the same kernel
 * (scan page, section 3, "kernel fusion").  D may be NULL. */
ssd_status ssd_stage_chunk_scan(const ssd_problem* problem, const void* x, const void* C,
                                const void* CB, const float* delta, const float* acs,
                                const float* passed, const float* D,
                                const int32_t* cu_seqlens, int32_t chunk_size, void* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gated RMSNorm of the Mamba-2 layer, the normalisation applied to the SSD
 * output y with the gate z (aitrends.kr/articles/109906, "B200에 맞춘 Helion
 * Mamba-2 커널 최적화": the layer's _layer_norm_bwd kernel; the page prints no
 * formula, the Mamba-2 gated RMSNorm normalised after gating is used).  Per row of
 * `dim` columns, in groups of `group` consecutive columns:
 *     s = z * sigmoid(z) (1 when z is NULL), v = y * s,
 *     r = 1 / sqrt(mean over the group of v^2 + eps),  out = v * r * weight.
 * Layouts: y, z, out, dout, dy, dz (rows, dim) io dtype, dim fastest; weight and
 * dweight (dim) fp32; rstd (rows, dim / group) fp32.  The SSD output (batch,
 * seqlen, nheads, headdim) is such a matrix with rows = batch * seqlen and
 * dim = nheads * headdim.
 * Supported: io_dtype SSD_BF16; dim a multiple of 512, at most 8192; group in
 * {256, 512, 1024, 2048} dividing dim, or group == dim; eps >= 0 and finite;
 * 16-byte aligned pointers.  Anything else returns SSD_ERR_UNSUPPORTED (or
 * SSD_ERR_SHAPE / SSD_ERR_NULL / SSD_ERR_ALIGN) before anything is queued.
 * Every reduction has a fixed order: results are bitwise reproducible.
 */
typedef struct {
  int32_t rows;      /* tokens */
  int32_t dim;       /* columns per row */
  int32_t group;     /* columns per normalisation group */
  int32_t io_dtype;  /* ssd_dtype of y, z, out, dout, dy, dz (SSD_BF16) */
  float eps;
} ssd_norm_problem;

/* Workspace of ssd_gated_rmsnorm_bwd in bytes: per-workgroup partial sums of
 * dweight, min(rows, 1024) x dim fp32 (0 for an invalid problem). */
size_t ssd_gated_rmsnorm_bwd_workspace_bytes(const ssd_norm_problem* problem);
/* Forward: out, and rstd (may be NULL) = r per (row, group).  z may be NULL (no gate). */
ssd_status ssd_gated_rmsnorm_fwd(const ssd_norm_problem* problem, const void* y, const void* z,
                                 const float* weight, void* out, float* rstd, void* stream);
/* Backward for the loss <dout, out>: dy, dz (NULL iff z is NULL) and dweight
 * (summed over rows).  r is recomputed from y and z. */
ssd_status ssd_gated_rmsnorm_bwd(const ssd_norm_problem* problem, const void* dout, const void* y,
                                 const void* z, const float* weight, void* dy, void* dz,
                                 float* dweight, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Plain device-to-device copy kernel of `bytes` bytes (16-byte multiple), used to
 * calibrate hardware traffic counters against a kernel of known traffic. */
ssd_status ssd_util_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBSSD_SSD_H */
