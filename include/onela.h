/*
 * onela.h - C ABI of the MI355X (gfx950) large-beam Gated DeltaNet decode step.
 *
 * What it computes.  Generative recommendation decodes hundreds of beams that all start from one
 * prompt-derived recurrent state ("Scientific Impact Assessment: OneLA", §1 Core Contribution; paper
 * index page "OneLA: Scaling Linear-Attention Decoding to Large Beams in Generative Recommendation",
 * Abstract).  Per (request, head) the library keeps:
 *   - the shared post-prefill state S_ctx (d_v x d_k),
 *   - one append-only transition record per beam and step, (alpha_t, k_t, u_t) with
 *     u_t = beta_t (v_t - alpha_t S_{t-1} k_t), so that S_t = alpha_t S_{t-1} + u_t k_t^T: the
 *     gated delta rule of Gated DeltaNet (listed under "Builds on" on the index page) rewritten so a
 *     record costs O(d_v + d_k) (review §1 item (1)),
 *   - an ancestry index: for every live beam, the slots of the records on its history (review §1
 *     item (3)); pruning, reordering and fan-out only rewrite this index, records never move.
 * A decode step computes S_{t-1} k_t and S_t q_t by projection replay (review §1 item (2) and
 * "Additional Observations"): a decayed contraction of S_ctx plus a replay of the beam's records,
 * never forming a per-beam d_v x d_k matrix.  One fused GPU kernel shares each S_ctx tile across all
 * beams of its request (review §1; Abstract).  The output is o_t = S_t q_t (post-update state).
 *
 * Conventions.
 *   - Step t = 1..max_steps.  Before step 1 there is one pseudo-beam (index 0) holding S_ctx.
 *   - The record of beam b at step t lives in slot (t-1)*max_beams + b of its (request, head)
 *     arena; slot numbers are the same for every head.
 *   - chain table after step t: [R][max_beams][max_steps] int32; row b lists the slots of beam b's
 *     history oldest first: its parent's row for steps 1..t-1, then its own slot, then -1.  Rows of
 *     beams >= n_beams are all -1.  Parents are per (request, beam) and shared by all heads.
 *   - Tensor layouts are row-major, innermost index last.  bf16 is IEEE bfloat16 (bit pattern).
 *
 * Memory and ownership.  The library never allocates device memory.  The caller allocates one
 * workspace of onela_workspace_size() bytes (256-byte aligned) and every input/output buffer; the
 * library only borrows those pointers, which must stay valid until the stream has run the work
 * enqueued on them.  The handle itself is a small host object owned by the library.
 *
 * Streams and errors.  Every call that enqueues GPU work takes a hipStream_t passed as void*
 * (NULL = the null stream) and returns without waiting.  Argument and state errors are detected on
 * the host and returned synchronously: nothing is enqueued and no state changes.  A parent index out
 * of range can only be seen on the device: it raises a sticky device flag that onela_get_status()
 * reports as ONELA_ERR_BAD_PARENT (the offending beam is then decoded as a child of beam 0 so every
 * access stays in bounds; that request's outputs are meaningless).  The flag clears on
 * onela_set_context(), onela_prefill() and onela_reset().  HIP launch failures return
 * ONELA_ERR_DEVICE.  onela_last_error() gives a message for the last failing call of this thread.
 *
 * Threading.  A handle is not thread-safe; use one handle per stream.
 */
#ifndef ONELA_H
#define ONELA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct onela_ctx* onela_handle;

typedef enum {
  ONELA_OK = 0,
  ONELA_ERR_INVALID_ARG = 1, /* bad pointer, size, dtype, mode or beam count */
  ONELA_ERR_STATE = 2,       /* call out of order, e.g. a step before any context */
  ONELA_ERR_CAPACITY = 3,    /* max_steps steps already taken, or workspace too small */
  ONELA_ERR_DEVICE = 4,      /* a HIP call failed */
  ONELA_ERR_BAD_PARENT = 5,  /* a parent index was out of range (device-side, sticky) */
  ONELA_ERR_UNSUPPORTED = 6  /* a valid request this build does not implement */
} onela_status;

typedef enum { ONELA_F32 = 0, ONELA_BF16 = 1 } onela_dtype;

typedef enum {
  ONELA_MODE_REPLAY = 0,   /* shared S_ctx + records + ancestry index (the method) */
  ONELA_MODE_FULLSTATE = 1 /* controlled comparison: a dense state per beam, gathered from its parent
                              and updated every step ("Scientific Impact Assessment: OneLA", §2:
                              the Controlled FullState baseline) */
} onela_mode;

/* onela_config.flags */
enum {
  ONELA_FLAG_FORCE_GENERIC = 1, /* replay mode: run the plain fp32-FMA kernel even where the fused
                                   bf16-MFMA kernel applies (for A/B checks) */
  ONELA_FLAG_MATERIALIZE = 2    /* replay mode: comparison path that rebuilds every beam's dense parent
                                   state from S_ctx and its chain each step, then projects it
                                   ("Scientific Impact Assessment: OneLA", §1 and "Additional
                                   Observations": the replay of shared history that the method avoids).
                                   Same records, index and outputs as the projection replay. */
};

typedef struct {
  int32_t num_requests; /* R >= 1 */
  int32_t num_heads;    /* H >= 1 */
  int32_t d_k;          /* 1..256 (the fused MFMA kernel needs d_k of 64, 128 or 256) */
  int32_t d_v;          /* 1..256 (the fused MFMA kernel needs d_v % 32 == 0) */
  int32_t max_beams;    /* B_max >= 1: beams per request and step */
  int32_t max_steps;    /* L_max in 1..64: decode steps per context */
  int32_t qkv_dtype;    /* onela_dtype of q, k, v and of the stored record keys */
  int32_t mode;         /* onela_mode */
  int32_t flags;        /* ONELA_FLAG_* */
  int32_t tile_beams;   /* beams per tile of the fused kernel: 0 = automatic, else 16 or 32 */
} onela_config;

/* Read-only view of the decode state, for inspection and tests.  Device pointers into the workspace. */
typedef struct {
  int32_t t;          /* steps taken since the last context or reset */
  int32_t n_beams;    /* beams alive after step t (1 before the first step: the shared state) */
  int32_t slots;      /* record slots per (request, head) = max_beams * max_steps */
  int32_t fused;      /* 1 if steps run the fused bf16-MFMA kernel, 0 for the fp32-FMA kernel */
  void* rec_k;        /* REPLAY: [R][H][slots][d_k] in qkv_dtype (exact copies of the step's k) */
  float* rec_u;       /* REPLAY: [R][H][slots][d_v] float32 */
  float* rec_alpha;   /* REPLAY: [R][H][slots] float32 (exact copies of the step's alpha) */
  int32_t* chains;    /* [max_steps][R][max_beams][max_steps]: the table after step t at index t-1 */
  float* sctx_t;      /* S_ctx transposed, [R][H][d_k][d_v] float32 */
  float* fullstate;   /* FULLSTATE: [2][R][H][max_beams][d_k][d_v] float32, the states after step t
                         (transposed) are in buffer t % 2; NULL in REPLAY mode */
} onela_view;

/* Workspace bytes a configuration needs.  Fails with ONELA_ERR_INVALID_ARG on a bad configuration. */
onela_status onela_workspace_size(const onela_config* cfg, size_t* bytes);

/* Create a handle on a caller-owned device workspace (>= onela_workspace_size() bytes, 256-byte
 * aligned, on the current HIP device).  No context is set yet. */
onela_status onela_create(const onela_config* cfg, void* d_workspace, size_t workspace_bytes,
                          onela_handle* out);

/* Free the host handle.  The workspace stays the caller's; wait for the stream first. */
onela_status onela_destroy(onela_handle h);

/* Install the shared post-prefill state that every beam of a request starts from ("Scientific Impact
 * Assessment: OneLA", §1 Core Contribution, mechanism (1): one S_ctx per request and head; OneLA index page,
 * Abstract: a single shared prompt-derived state).  d_sctx is [R][H][d_v][d_k] float32 on the device.  It is
 * copied (transposed, and split into bf16 high and low parts for the fused kernel), so the caller may
 * reuse d_sctx once the stream has passed this call.  Starts a new decode (t = 0). */
onela_status onela_set_context(onela_handle h, const float* d_sctx, void* stream);

/* Prefill a prompt of n_tokens GDN steps from the zero state and install the result as the context,
 * as onela_set_context would ("Scientific Impact Assessment: OneLA", §1: the post-prefill state).
 * d_k: [R][n_tokens][H][d_k], d_v: [R][n_tokens][H][d_v], d_alpha/d_beta: [R][n_tokens][H], all
 * float32.  If d_sctx_out is not NULL the state is also written there as [R][H][d_v][d_k] float32.
 * Any head size the handle accepts (d_k, d_v <= 256); n_tokens = 0 installs the zero state.  The work is
 * 4 d_k d_v float32 FLOPs per token and (request, head).  The decode state of the workspace (chain tables
 * and records, or the per-beam states), which a prefill starts afresh, serves as its scratch: with d_k = 128
 * and d_v in {16, 32, 64, 128, 256} the chunked form keeps 4480 bytes per 32-token chunk and (request, head)
 * there, in as many passes over the prompt as that space needs, and falls back to a token-by-token float32
 * recurrence when not even one chunk fits. */
onela_status onela_prefill(onela_handle h, int32_t n_tokens, const float* d_k, const float* d_v,
                           const float* d_alpha, const float* d_beta, float* d_sctx_out, void* stream);

/* One decode step for every request and head ("Scientific Impact Assessment: OneLA", §1 Core Contribution,
 * mechanisms (1)-(3), and the fused kernel that reuses S_ctx across beams; OneLA index page, Abstract).  In
 * REPLAY mode each beam's S_{t-1} k and S_t q come from the decayed S_ctx contraction plus a replay of the
 * records on the beam's chain (mechanism (2): only two vector projections of the state, never the matrix);
 * the new record (alpha, k, u = beta (v - alpha S_{t-1} k)) is appended (mechanism (1)) and the chain table
 * extended through the parents (mechanism (3)).  FULLSTATE mode keeps a dense state per beam instead (the
 * controlled comparison of §2 Methodological Rigor).  n_beams in 1..max_beams new beams per request:
 *   d_q, d_k    [R][n_beams][H][d_k]  qkv_dtype
 *   d_v         [R][n_beams][H][d_v]  qkv_dtype
 *   d_alpha     [R][n_beams][H]       float32 (decay, usually in (0, 1])
 *   d_beta      [R][n_beams][H]       float32 (write strength)
 *   d_parent_idx[R][n_beams]          int32, in [0, B_prev): B_prev = 1 at step 1, else the n_beams of
 *                                     the previous step
 *   d_o         [R][n_beams][H][d_v]  float32 output S_t q_t
 * Appends one record per (request, beam, head) and the new chain table.  ONELA_ERR_STATE without a
 * context, ONELA_ERR_CAPACITY once max_steps steps were taken. */
onela_status onela_step(onela_handle h, int32_t n_beams, const void* d_q, const void* d_k,
                        const void* d_v, const float* d_alpha, const float* d_beta,
                        const int32_t* d_parent_idx, float* d_o, void* stream);

/* Drop every record and chain (logically) and return to t = 0 on the same context: records sit where they
 * were written and are never moved ("Scientific Impact Assessment: OneLA", §1 Core Contribution, mechanism
 * (3): immutable physical record placement), so a new decode only restarts the step counter and the chain
 * tables; no device work is enqueued and the stream argument is accepted for symmetry.  Also clears the
 * parent-error flag for the new decode. */
onela_status onela_reset(onela_handle h, void* stream);

/* Wait for the stream, then report the sticky device flag of the current decode: ONELA_OK, or
 * ONELA_ERR_BAD_PARENT if some step named a parent outside the previous step's beams (a chain the ancestry
 * index of "Scientific Impact Assessment: OneLA", §1 Core Contribution, mechanism (3), cannot follow; that
 * step's outputs for the beam are then computed from parent 0).  Returns ONELA_ERR_DEVICE if the stream
 * fails. */
onela_status onela_get_status(onela_handle h, void* stream);

/* Fill *view with the current decode state (host-side only; no synchronisation). */
onela_status onela_get_view(onela_handle h, onela_view* view);

/* ---- Beam selection (stateless; no handle) ----------------------------------------------------------
 * The step that produces the next decode step's parents: beams are pruned, reordered and fanned out, each
 * survivor naming its parent ("Scientific Impact Assessment: OneLA", §1 Core Contribution).  The pages do
 * not state the rule; this is the plain beam-search step.  For each request r, every current beam b (of
 * n_prev) proposes every candidate token c (of n_cand) with the float32 score
 *     s = d_beam_scores[r][b] + d_logp[r][b][c]      (one addition, round to nearest even);
 * the n_beams candidates with the highest scores survive, best first, equal scores ordered by the smaller
 * flat index b * n_cand + c (-0 and +0 are equal).  Survivor i of request r is written as
 *     d_parent_idx[r][i] = b,  d_token[r][i] = c,  d_scores[r][i] = s,
 * so d_parent_idx can be passed straight to onela_step and d_scores become the next beam scores.
 *   d_beam_scores [R][n_prev] float32, d_logp [R][n_prev][n_cand] float32 (finite or -inf; NaN has no
 *   rank and gives unspecified survivors), outputs [R][n_beams].
 * d_scratch: device memory of at least onela_beam_select_scratch(...) bytes (may be NULL when that is 0),
 * owned by the caller; the call allocates nothing.  All device pointers must stay valid until the stream
 * reaches the work.  Errors (host-side, nothing enqueued): ONELA_ERR_INVALID_ARG for sizes < 1, n_beams >
 * n_prev * n_cand, n_prev * n_cand >= 2^31, a NULL buffer or a scratch smaller than required;
 * ONELA_ERR_UNSUPPORTED for n_beams > 2048; ONELA_ERR_DEVICE for a failed launch. */
onela_status onela_beam_select_scratch(int32_t num_requests, int32_t n_prev, int32_t n_cand, int32_t n_beams,
                                       size_t* bytes);
onela_status onela_beam_select(int32_t num_requests, int32_t n_prev, int32_t n_cand, int32_t n_beams,
                               const float* d_beam_scores, const float* d_logp, int32_t* d_parent_idx,
                               int32_t* d_token, float* d_scores, void* d_scratch, size_t scratch_bytes,
                               void* stream);

/* onela_beam_select without a caller scratch, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments, rule, outputs
 * and errors as onela_beam_select, minus d_scratch / scratch_bytes: the keys that survive a first pass live
 * in an 8 MiB array the library holds on each GPU for the life of the process (looked up on the first call
 * on that device; no call allocates).  Selections whose onela_beam_select_scratch exceeds 8 MiB are
 * rejected with ONELA_ERR_CAPACITY (nothing enqueued): e.g. 32 requests x 512 beams x 256 candidates ->
 * 512 needs 4 MiB.  Every call on one GPU shares that GPU's array: calls on one GPU must not overlap (two
 * streams, or two threads, running it at once race and give wrong survivors); calls that follow each other
 * in stream order are safe.  Nothing in the array needs clearing between calls: every call overwrites what
 * it reads. */
onela_status onela_beam_select_noalloc(int32_t num_requests, int32_t n_prev, int32_t n_cand, int32_t n_beams,
                                       const float* d_beam_scores, const float* d_logp, int32_t* d_parent_idx,
                                       int32_t* d_token, float* d_scores, void* stream);

/* Static text for a status code; message of this thread's last failing call ("" if none). */
const char* onela_status_string(onela_status s);
const char* onela_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ONELA_H */
