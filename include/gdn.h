/*
 * libgdn -- gated delta-rule linear-attention scan for AMD Instinct MI355X (gfx950).
 *
 * The operator is the gated delta-net linear attention with a matrix-valued
 * recurrent state per head ("[Research] Explore linear attention for the
 * streaming video models", section "We already ship a hybrid linear-attention
 * model"); the state is written one token at a time as standard delta-rule
 * linear attention does ("Video DeltaNet: A Video-Native Hybrid Attention for
 * Livestream Video Generation", section "Methodology in Plain English").
 * Per (batch b, head h), with the state S in R^{dv x dk} (fp32):
 *
 *   q^_t = q_t / max(|q_t|_2, 1e-6),   k^_t = k_t / max(|k_t|_2, 1e-6)
 *   S_t  = a_t S_{t-1} (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T,  a_t = exp(log_alpha_t)
 *   o_t  = S_t q^_t
 *
 * Directions:
 *   GDN_DIR_FORWARD       causal scan t = 0..T-1; the forward-only causal
 *                         form used for streaming rollout (the issue's
 *                         "Open questions and risks": causal streaming scan).
 *   GDN_DIR_REVERSE       the same recurrence run from t = T-1 down to 0.
 *   GDN_DIR_BIDIRECTIONAL out = forward readout + reverse readout, each
 *                         direction with its own (log_alpha, beta) and its own
 *                         initial state ("Video DeltaNet", "Methodology in
 *                         Plain English": forward and backward recurrent
 *                         states whose readouts are added).  Both readouts
 *                         include the current token unless an exclusive
 *                         option bit (below) says otherwise.
 *
 * Streaming: the final state of one call is the initial state of the next
 * (the streaming state lifecycle of the issue's "Suggested phases", phase 1);
 * chaining calls over consecutive token ranges equals one call over their
 * concatenation.
 *
 * Layouts (all row-major and contiguous; base pointers 16-byte aligned):
 *   q, k       [B, T, H, dk]   dtype (fp32 or bf16), finite (any length:
 *                              the scan normalises them itself)
 *   v          [B, T, H, dv]   dtype, finite
 *   log_alpha  [dirs, B, T, H] fp32, finite and <= 0 (caller's contract)
 *   beta       [dirs, B, T, H] fp32, finite (beta in [0,1] keeps the
 *                              transition non-expansive)
 *   state_in   [dirs, B, H, dv, dk] fp32, or NULL for a zero initial state
 *   state_out  [dirs, B, H, dv, dk] fp32, or NULL to skip writing it
 *   out        [B, T, H, dv]   fp32
 * dirs = 2 for GDN_DIR_BIDIRECTIONAL, else 1 (slot 0 then holds the single
 * direction's gates and states).
 *
 * Ownership and execution: every pointer is caller-owned device memory; the
 * library allocates no device memory, does not synchronise and reads no
 * environment variables.  The work is ordered on `stream` (NULL: the default
 * stream) and completes asynchronously.  For long single-direction scans
 * whose state chain leaves compute units free (and fp32 bidirectional ones
 * with few sequences) the chunk
 * preparation runs concurrently with the state chain, on a library stream
 * forked from `stream` and joined back to it with events (one stream and two
 * events per device, created on the first such call and kept until the
 * process ends): the work still starts after earlier work on `stream`, and
 * later work on `stream` still waits for all of it.  While `stream` is being
 * captured into a HIP graph, both kernels are enqueued one after the other on
 * `stream` (no library stream or event is created or used), so a captured
 * call -- the first call of the process included -- replays the serial order.
 * GDN_OPT_SERIAL keeps everything on `stream` always.
 * Calls may come from several host threads at once, each with its own
 * buffers and workspace: the library stream and events are shared under a
 * lock, and the preparation passes of concurrent calls run one after another
 * on that stream (results are those of the same calls made one at a time).
 * state_in == state_out is allowed (in-place streaming carry); any other
 * overlap between `out`, the state buffers, the workspace and the inputs is
 * rejected.  Results are bitwise deterministic for fixed inputs and chunk
 * size, concurrent or not: there are no atomic reductions (the second visit
 * of a chunk in a bidirectional scan adds the stored readout of the first
 * visit in a fixed order; it waits for that readout's flag for about a
 * second at most, after which the outputs it could not combine are NaN).  The value-tile width changes the schedule, never
 * the arithmetic.
 *
 * Errors: argument problems are reported before anything is enqueued and
 * leave every output untouched.  GDN_ERR_HIP reports a failed launch; faults
 * during execution surface at the caller's next synchronisation, as with any
 * stream work.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARGUMENT = 1,   /* NULL/misaligned pointer, bad size, overlap, bad direction */
  GDN_ERR_UNSUPPORTED = 2,        /* dk, dv, chunk, tile or dtype outside the compiled set */
  GDN_ERR_WORKSPACE_TOO_SMALL = 3,
  GDN_ERR_HIP = 4                 /* a kernel launch failed */
} gdn_status_t;

typedef enum {
  GDN_DIR_FORWARD = 0,
  GDN_DIR_REVERSE = 1,
  GDN_DIR_BIDIRECTIONAL = 2
} gdn_direction_t;

typedef enum {
  GDN_DTYPE_F32 = 0,
  GDN_DTYPE_BF16 = 1
} gdn_dtype_t;

/* Bits of gdn_problem_t.options. */
typedef enum {
  GDN_OPT_SERIAL = 1,       /* run both kernels one after the other on `stream` */
  GDN_OPT_NO_ERASE = 2,     /* the erase-free variant: S_t = a_t S_{t-1} + beta_t v_t k^_t^T,
                               i.e. gated linear attention with per-token write strength
                               beta (SANA-Video 2.0 review: the hybrid's linear layers are
                               gated linear attention, and its "Future work" relates them to
                               the delta rule by dropping the delta-rule update) */
  GDN_OPT_EXCLUSIVE_FORWARD = 4,  /* the forward direction reads its memory before the
                               token's own write: o_t = a_t S_{t-1} q^_t */
  GDN_OPT_EXCLUSIVE_REVERSE = 8   /* the same for the reverse direction: o_t = a_t S_{t+1} q^_t.
                               Both bits: the two scans of a bidirectional call cover the
                               disjoint regions s < t and s > t (the current token is left to
                               a local operator); the reverse bit alone: s <= t and s > t,
                               every token once ("Video DeltaNet", "Methodology in Plain
                               English": each direction sees its own non-overlapping part
                               of the sequence, and the prompt's state enters each
                               direction at half weight, S_T / 2 -- here the caller's
                               state_in).
                               Final states are unchanged by either bit. */,
  GDN_OPT_TEST_NO_PREPARATION = 1 << 16  /* testing only: the chunk preparation pass is not
                               launched, so the state chain waits on ready flags that never
                               clear; its bounded waits expire (about a second) and every
                               output and final state is NaN.  This exercises the behaviour
                               under a preparation pass starved of the GPU: results that
                               cannot be trusted are NaN, never silently wrong. */
} gdn_option_t;

/* Problem description.  Supported: dk in {64, 128}; dv in {64, 128};
 * chunk in {0 (= 64), 16, 32, 64, 128} (the chunked form is exact at any chunk
 * length: "Video DeltaNet", Key Contributions item 4, chunk-wise scans; results
 * agree between chunk lengths to rounding, 64 is the fastest on MI355X);
 * dv_tile in {0, 16, 32} (0: 32 when 16-wide
 * state-chain workgroups would outnumber the compute units of the current
 * device, else 16; exclusive readouts on bf16 operands take 16 and reject
 * 32: they carry the state and the decayed q.k tile as bf16 hi + lo parts,
 * whose staging fits 16-column tiles only).  16- and 128-token chunks: bf16
 * operands reject the exclusive readouts and the readout epilogue (their low
 * parts are carried by the 32/64-token chain only); 128-token chunks: fp32
 * operands with dk = 128
 * take dv_tile 16 and reject 32 (the chain's staging would exceed a compute
 * unit's LDS); B, H >= 1, B*H <= 65535;
 * 0 <= T <= 2^30 and
 * (T + 64) * H * max(dk, dv) * 4 < 2^32 (one batch element's rows, fp32,
 * fit 32-bit byte offsets). */
typedef struct {
  int64_t B, T, H, dk, dv;
  int32_t dtype;            /* gdn_dtype_t: type of q, k, v */
  int32_t chunk;            /* tokens per chunk of the chunked evaluation */
  int32_t dv_tile;          /* value columns per workgroup of the state chain */
  int32_t options;          /* OR of gdn_option_t bits (0: delta rule, chosen schedule);
                               other bits are invalid */
  void* workspace;          /* caller-owned device memory, 256-byte aligned */
  size_t workspace_bytes;
  void* stream;             /* hipStream_t; NULL = default stream */
  void* timing_events;      /* NULL, or hipEvent_t[4] (caller-owned): recorded
                               before and after the chunk-preparation kernel on
                               the stream it runs on, then before and after the
                               state-chain kernel on `stream` (per-kernel
                               timing; the epilogue, if any, runs after the
                               last of them) */
  /* Readout epilogue ("Video DeltaNet", "Key Contributions" item 1: the
   * linear branch's readout is RMS-normalised and sigmoid-gated).  With
   * gate != NULL, after the scan, every (token, head) row of `out` becomes
   *   out = norm_weight * o / sqrt(mean_dv(o^2) + norm_eps) * sigmoid(gate),
   * o being the row as the scan computed it (inclusive or exclusive, both
   * directions summed).  A separate pass on `stream`: the channels of one
   * row are split over several state-chain workgroups.  Zero-initialise
   * these fields (as make_problem-style helpers do) for no epilogue. */
  const void* gate;          /* NULL, or [B, T, H, dv] of the type of q, 16-byte aligned */
  const float* norm_weight;  /* [dv] fp32, shared by the heads; required with gate */
  float norm_eps;            /* epilogue only: finite, >= 0 */
} gdn_problem_t;

/* Bytes of workspace gdn_forward needs for this problem and direction
 * (0 if the problem is invalid or unsupported, and for T = 0, which needs
 * none).  It depends on p->options as well: exclusive readouts on bf16
 * operands need about 2 C bytes more per token and head.  Pure host
 * arithmetic. */
size_t gdn_workspace_bytes(const gdn_problem_t* p, int32_t direction);

/* Enqueue the scan described by `p` on p->stream.  See the file comment for
 * layouts; `direction` is a gdn_direction_t. */
gdn_status_t gdn_forward(const gdn_problem_t* p,
                         const void* q, const void* k, const void* v,
                         const float* log_alpha, const float* beta,
                         const float* state_in, float* state_out,
                         float* out, int32_t direction);

/* ---- The same scan without a caller-provided workspace ----------------------
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * workspace is a fixed array the library holds in device memory,
 * GDN_NOALLOC_SCRATCH_BYTES per device that loads the library, kept until the
 * process ends.  Arguments, layouts, results and errors are those of
 * gdn_forward, except:
 *  - p->workspace and p->workspace_bytes are ignored;
 *  - a problem whose workspace (gdn_workspace_bytes) exceeds
 *    GDN_NOALLOC_SCRATCH_BYTES is rejected with GDN_ERR_WORKSPACE_TOO_SMALL
 *    before anything is enqueued (e.g. 480p streaming frames of 1560 tokens at
 *    12 heads need about 6 MB; a whole 480p bidirectional block, about 300 MB,
 *    does not fit);
 *  - both kernels always run one after the other on p->stream (no library
 *    stream or event is created);
 *  - the first call on a device looks up that device's array
 *    (hipGetSymbolAddress); no call allocates device memory.
 * Every call on one device uses that device's single array, which keeps the
 * last call's contents: calls that overlap in time on one device (on
 * different streams, or from several host threads) race on it and must be
 * ordered by the caller.  Nothing in the array has to start at zero. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

gdn_status_t gdn_forward_noalloc(const gdn_problem_t* p,
                                 const void* q, const void* k, const void* v,
                                 const float* log_alpha, const float* beta,
                                 const float* state_in, float* state_out,
                                 float* out, int32_t direction);

/* ---- Frame-wise delta operator (Video Delta Attention) ---------------------
 *
 * The memory is written once per latent frame instead of once per token.
 * The write is a regularised least-squares problem: the new memory balances
 * its squared distance from the decayed previous memory against the squared
 * recall errors of all the frame's keys at once ("Video DeltaNet", "Key
 * Contributions" item 2 and "Methodology in Plain English").  Its solution is
 * the page's closed form
 *
 *   S_t = (a_t S_{t-1} + B_t) (I + A_t)^{-1},
 *   A_t = sum_{i in frame t} beta_i k^_i k^_i^T,  B_t = sum_{i in frame t} beta_i v_i k^_i^T,
 *
 * and every token i of frame t reads o_i = S_t q^_i (q^, k^ normalised as
 * above).  Frames are consecutive runs of `frame` tokens (the last may be
 * shorter).  One decay per frame, a_t = exp(log_alpha_t); one write strength
 * per token (beta >= 0 keeps the transition non-expansive).  Directions as for
 * gdn_forward: the reverse scan visits the frames last to first, the
 * bidirectional output is the sum of both readouts.
 *
 * Options on the same machinery:
 *  - GDN_VDA_OPT_ADDITIVE: the additive frame write the page contrasts the
 *    operator with ("Main Findings", last item: SANA-WM's batched per-token
 *    corrections with 1/sqrt(U) key scaling, U = the frame's token count):
 *    S_t = a_t S_{t-1} (I - A_t / U) + B_t / sqrt(U).
 *  - readout_lag = d > 0: the disjoint-region readout ("Methodology in Plain
 *    English": the forward and reverse memories see non-overlapping parts of
 *    the video, and the text's state starts each direction at half weight,
 *    S_T/2).  A token of
 *    frame t reads the forward state after frame t - d and the reverse state
 *    after frame t + d; where that frame does not exist, the direction's
 *    initial state (zero without state_in).  d = 0 reads its own frame's state.
 *  - gate != NULL: the readout epilogue ("Key Contributions" item 1: the
 *    linear branch's RMS normalisation and sigmoid gate), applied to the
 *    summed readout o of each (token, head) before it is stored:
 *    out = norm_weight * o / sqrt(mean_dv(o^2) + norm_eps) * sigmoid(gate).
 *
 * Layouts: q, k, v, beta, state_in, state_out and out as for gdn_forward;
 *   log_alpha  [dirs, B, NF, H] fp32, NF = ceil(T / frame);
 *   gate       [B, T, H, dv] of the type of q (16-byte aligned);
 *   norm_weight [dv] fp32, shared by the heads.
 * Supported: dk, dv in {64, 128}; frame >= 1; fp32 or bf16 q, k, v; the same
 * size limit as gdn_problem_t.  Same ownership, execution and error contract
 * as gdn_forward (everything on `stream`; no allocation; no synchronisation;
 * `out` must not overlap any input, gate and norm_weight included). */
typedef enum { GDN_VDA_OPT_ADDITIVE = 1 } gdn_vda_option_t;

typedef struct {
  int64_t B, T, H, dk, dv;
  int64_t frame;            /* tokens per frame */
  int32_t dtype;            /* gdn_dtype_t: type of q, k, v and gate */
  int32_t options;          /* 0 or GDN_VDA_OPT_ADDITIVE */
  int32_t readout_lag;      /* >= 0 */
  float norm_eps;           /* epilogue only: finite, >= 0 */
  const void* gate;         /* NULL (no epilogue) or [B, T, H, dv] */
  const float* norm_weight; /* [dv]; required with gate */
  void* workspace;          /* caller-owned device memory, 256-byte aligned */
  size_t workspace_bytes;
  void* stream;             /* hipStream_t; NULL = default stream */
  void* timing_events;      /* NULL, or hipEvent_t[4] (caller-owned), recorded on
                               `stream` before the per-frame kernel, after it,
                               after the frame chain and after the readout */
} gdn_vda_problem_t;

/* Workspace bytes of gdn_vda_forward (0 if invalid or unsupported, or T = 0):
 * three fp32 matrices per frame, head and direction. */
size_t gdn_vda_workspace_bytes(const gdn_vda_problem_t* p, int32_t direction);

/* Enqueue the frame-wise operator described by `p` on p->stream. */
gdn_status_t gdn_vda_forward(const gdn_vda_problem_t* p,
                             const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta,
                             const float* state_in, float* state_out,
                             float* out, int32_t direction);

/* Static description of a status code. */
const char* gdn_status_string(int32_t status);

/* Library version string. */
const char* gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
