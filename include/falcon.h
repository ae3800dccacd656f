/*
 * falcon.h - C interface of libfalcon: the Falcon fast-weight state update and
 * read-after-write readout on AMD Instinct MI355X (gfx950).
 *
 * The method (arXiv 2608.27763, "Fast Weight Attention for Continual
 * Learning", as described by the papers.ananclaw.com explainer, section
 * 核心方法 §1-§3, and the 163.com article, sections 01 and 02):
 *
 *   per (batch b, head h), t = 1..L, value rows i = 1..dv
 *     x_t = k_{t-1}  (x_1 = k_prev, or the zero vector when k_prev == NULL)
 *     y_t = v_t
 *     W_t = { max(1, t-B+1), ..., t }     (B = window; 1 except Falcon-3/3A)
 *     n_t = sum_{j in W_t} ||x_j||^2
 *     eta_t = beta_t / (eps + n_t)        (one per value row for Falcon-2/2A)
 *     regression   (Falcon-1/2/3):  S_t = (1 - eta_t lambda) S_{t-1}
 *                                   + eta_t sum_{j in W_t} (y_j - S_{t-1} x_j) x_j^T
 *     inner product (Falcon-1A/2A/3A): S_t = (1 - eta_t lambda) S_{t-1}
 *                                   + eta_t sum_{j in W_t} y_j x_j^T
 *     o_t = S_t q_t
 *
 * S is dv x dk (it maps key space to value space).  A fresh sequence starts
 * from S_0 = 0 with x_1 = 0, which leaves S_1 = 0 (the step with x_1 = 0 is
 * taken with unit decay and zero write; that equals the literal step because
 * S_0 = 0).
 *
 * Layouts (all row-major and contiguous, element = dtype unless stated):
 *   q, k     [batch, heads, L, dk]          v        [batch, heads, L, dv]
 *   k_prev   [batch, heads, dk]             o        [batch, heads, L, dv]  float32
 *   S0, S_out [batch, heads, dv, dk]  float32
 *   beta_t   NULL (scalar beta), [batch, heads, L] (FALCON_BETA_TOKEN) or
 *            [batch, heads, L, dv] (FALCON_BETA_CHANNEL, Falcon-2/2A only)
 *
 * Ownership: every pointer is device memory owned by the caller.  The library
 * allocates nothing, keeps no mutable global state and is reentrant (except
 * falcon_bwd_chunk_noalloc, which uses a device array of its own).  Work is
 * enqueued on `stream` (a hipStream_t passed as void*, NULL = the default
 * stream) and is asynchronous; buffers must stay alive until it completes.
 *
 * Errors: the return value is the only channel (no printing, no abort).  All
 * validation happens before any HIP call; a call that returns an error
 * enqueues nothing.  FALCON_ERR_HIP reports a failed launch.
 *
 * Determinism: fixed reduction order and no atomics, so repeated calls give
 * bitwise identical results.
 */
#ifndef FALCON_H
#define FALCON_H

#ifdef __cplusplus
extern "C" {
#endif

#define FALCON_ABI_VERSION 4

/* The six update rules (explainer, section 核心方法 §2, variant table;
 * 163.com section 02: objective axis x granularity axis). */
typedef enum {
  FALCON_1 = 0,  /* squared error, one eta shared by all value channels */
  FALCON_2 = 1,  /* squared error, one eta per value channel (row of S) */
  FALCON_3 = 2,  /* squared error, sliding window of the B latest samples */
  FALCON_1A = 3, /* negative inner product, shared eta */
  FALCON_2A = 4, /* negative inner product, per-channel eta */
  FALCON_3A = 5  /* negative inner product, sliding window */
} falcon_variant;

/* Element type of q, k, v, k_prev and beta_t.  S, o are always float32. */
typedef enum { FALCON_BF16 = 0, FALCON_F32 = 1 } falcon_dtype;

/* Shape of beta_t. */
typedef enum {
  FALCON_BETA_SCALAR = 0,  /* beta_t must be NULL; the float `beta` is used */
  FALCON_BETA_TOKEN = 1,   /* one gain per (batch, head, token) */
  FALCON_BETA_CHANNEL = 2  /* one gain per (batch, head, token, value channel) */
} falcon_beta_kind;

typedef enum {
  FALCON_OK = 0,
  FALCON_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad enum, misalignment,
                                 non-finite or negative hyper-parameter, ... */
  FALCON_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels cover */
  FALCON_ERR_HIP = 3          /* the HIP runtime reported a launch failure */
} falcon_status;

/* Returns FALCON_ABI_VERSION. */
int falcon_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* falcon_status_string(int status);

/*
 * falcon_fwd_recurrent - the recurrent form, one token at a time (explainer
 * §3 "recurrent", O(d^2) per step).  Every variant, window >= 1, bf16 or fp32
 * inputs.
 *
 *   variant   falcon_variant
 *   window    B >= 1; must be 1 unless variant is FALCON_3 / FALCON_3A
 *   beta, beta_t, beta_kind   plasticity gain (scalar, per token, per channel)
 *   lambda    forgetting strength, finite, >= 0
 *   eps       normalizer floor, finite, >= 0 (eps = 0 with a zero key after
 *             the first step gives non-finite outputs)
 *   batch, heads, seqlen (L >= 1), dk, dv     sizes; dk, dv in {16,32,64,128}
 *   dtype     falcon_dtype of q, k, v, k_prev, beta_t
 *   q, k, v   inputs (device)
 *   k_prev    key carried from the previous call, or NULL (fresh sequence)
 *   S0        initial state, or NULL (zero).  S0 != NULL requires k_prev.
 *             window > 1 with S0 != NULL is unsupported here (the window
 *             history is carried by falcon_fwd_recurrent_ex).
 *   o         output [batch, heads, L, dv] float32 (must not alias inputs)
 *   S_out     final state, or NULL; may equal S0 (in-place carry)
 *   stream    hipStream_t or NULL
 * All pointers 16-byte aligned.
 */
int falcon_fwd_recurrent(int variant, int window, float beta, const void* beta_t,
                         int beta_kind, float lambda, float eps, int batch, int heads,
                         int seqlen, int dk, int dv, int dtype, const void* q,
                         const void* k, const void* v, const void* k_prev,
                         const float* S0, float* o, float* S_out, void* stream);

/*
 * falcon_fwd_chunk - the chunk-parallel form (explainer §3 "chunk-parallel";
 * 163.com section 02 (2): parallel inside a chunk, only the fixed-size state
 * crosses chunks).  Same arguments and results as falcon_fwd_recurrent plus
 *   chunk     requested tokens per chunk, in {16, 32, 64}; any L (a short last
 *             chunk is handled in place)
 * Restrictions (FALCON_ERR_UNSUPPORTED): dtype must be FALCON_BF16;
 * window <= 4, except FALCON_3A with gains shared by the value rows (scalar or
 * per-token beta), dk in {64, 128} and dv a multiple of 32: window <= 16.
 * window <= chunk (FALCON_ERR_INVALID_ARG otherwise).
 *   chunk is a tuning hint: each kernel family runs its own chunk length (32
 *   steps for window 1 with shared gains and dk 32 or 64; 16-step sub-chunks for
 *   windows 2..4 of the regression family; 64 for the inner-product family with
 *   shared gains; the requested length, halved until chunk * window <= 64 and
 *   at most 32 at dk 128, otherwise); the result does not depend on it beyond
 *   rounding.  A call of at most FALCON_MASKED_MAX_LEN (64) steps with window 1
 *   and gains shared by the value rows is one chunk; it runs the kernel of
 *   falcon_fwd_masked (the whole call as one masked system, exact for any decay).
 * The result equals the recurrence up to floating-point rounding (state
 * carried in float32, products on bf16 matrix cores with split-bf16 operands
 * where an operand is not an exact bf16 input) for every finite input: the
 * chunk algebra scales a chunk's unknowns by the decay products
 * g_t = prod (1 - eta_r lambda) over the chunk, and when some |g_t| leaves
 * [2^-100, 2^100] or some decay |1 - eta_t lambda| is below 2^-24 (strong
 * forgetting, eta_t lambda near 1 or above 2) the kernel recomputes that
 * (batch, head) chain exactly by the recurrence, in the same launch (slower:
 * one token at a time).
 */
int falcon_fwd_chunk(int variant, int window, float beta, const void* beta_t,
                     int beta_kind, float lambda, float eps, int batch, int heads,
                     int seqlen, int dk, int dv, int dtype, const void* q, const void* k,
                     const void* v, const void* k_prev, const float* S0, float* o,
                     float* S_out, int chunk, void* stream);

/*
 * falcon_decode_step - one token of the recurrent form for serving (explainer
 * §3, recurrent form for inference; 163.com section 01 read-after-write):
 *   x = k_prev, y = v, S <- update(S), o = S_new q, then k_prev <- k.
 * S [nseq, heads, dv, dk] float32 and k_prev [nseq, heads, dk] are updated in
 * place; q, k [nseq, heads, dk], v [nseq, heads, dv]; o [nseq, heads, dv]
 * float32; beta_t NULL, [nseq, heads] (FALCON_BETA_TOKEN) or
 * [nseq, heads, dv] (FALCON_BETA_CHANNEL, Falcon-2/2A).
 * Variants FALCON_1, FALCON_2, FALCON_1A, FALCON_2A (the sliding-window
 * variants need a carried history: FALCON_ERR_UNSUPPORTED).
 * k_prev must not alias k.
 */
int falcon_decode_step(int variant, float beta, const void* beta_t, int beta_kind,
                       float lambda, float eps, int nseq, int heads, int dk, int dv,
                       int dtype, float* S, void* k_prev, const void* q, const void* k,
                       const void* v, float* o, void* stream);

/*
 * Extended entry points: the same computations with a carried window history
 * and a choice of sample pairing.
 *
 * flags: 0, or FALCON_SAME_STEP - pair each value with the same step's key,
 *   x_t = k_t (explainer §1, the alternative alignment it warns against; the
 *   163.com article, section 01, explains why the default pairs v_t with
 *   k_{t-1}).  The carried key is then meaningless: k_prev must be NULL, and
 *   S0 needs no k_prev.  Other bits are invalid.
 *
 * Carried window history (Falcon-3/3A).  The window of step t holds the B
 * latest causal samples (explainer §2 variant table; 163.com section 02 (2)),
 * so when a sequence is split into calls the first B-1 steps of a call reach
 * samples of the previous one.  Besides S and k_prev the caller then carries
 * those samples:
 *   x_hist [batch, heads, B-1, dk], y_hist [batch, heads, B-1, dv], element
 *   type `dtype`: the samples (x_j, y_j) before step 1, oldest first, with
 *   x_j = k_{j-1} (x_j = k_j under FALCON_SAME_STEP) and y_j = v_j.  A zero row
 *   stands for a missing sample (it adds nothing to the normalizer or to the
 *   write), so a fresh sequence may start from zeros.
 *
 * falcon_fwd_recurrent_ex / falcon_fwd_chunk_ex - falcon_fwd_recurrent /
 * falcon_fwd_chunk with
 *   flags              as above
 *   x_hist, y_hist     the incoming history, or both NULL (none).  Non-NULL
 *                      requires window > 1, and k_prev unless FALCON_SAME_STEP.
 *   x_hist_out, y_hist_out   the B-1 latest samples after the call (same
 *                      shapes), or both NULL.  Requires window > 1.  Written
 *                      by a kernel enqueued after the main one, so they may
 *                      equal x_hist / y_hist exactly (in-place carry); any
 *                      other overlap with an argument is an error.
 * With window > 1, S0 != NULL requires the incoming history (the state of a
 * resumed sequence is meaningless without its window samples).
 */
#define FALCON_SAME_STEP 1
int falcon_fwd_recurrent_ex(int variant, int window, int flags, float beta, const void* beta_t,
                            int beta_kind, float lambda, float eps, int batch, int heads,
                            int seqlen, int dk, int dv, int dtype, const void* q,
                            const void* k, const void* v, const void* k_prev,
                            const float* S0, const void* x_hist, const void* y_hist,
                            float* o, float* S_out, void* x_hist_out, void* y_hist_out,
                            void* stream);
int falcon_fwd_chunk_ex(int variant, int window, int flags, float beta, const void* beta_t,
                        int beta_kind, float lambda, float eps, int batch, int heads,
                        int seqlen, int dk, int dv, int dtype, const void* q, const void* k,
                        const void* v, const void* k_prev, const float* S0,
                        const void* x_hist, const void* y_hist, float* o, float* S_out,
                        void* x_hist_out, void* y_hist_out, int chunk, void* stream);

/*
 * falcon_fwd_workspace_bytes - bytes of device workspace with which
 * falcon_fwd_chunk_ws runs the two-kernel form of the call; 0 where that form
 * does not apply (it applies to the regression family with a window of 2 or 4,
 * gains shared by the value rows, dk in {64, 128}, bf16 inputs).  Per
 * (batch, head) and 16-step sub-chunk one record of 12416 bytes: the
 * sub-chunk's folds of the chunk equations (the state-independent part of
 * every step), its decay products and a range flag.
 *
 * falcon_fwd_chunk_ws - falcon_fwd_chunk_ex with a caller workspace (device
 * memory, 16-byte aligned, overlapping no other argument; NULL: none).  With
 * workspace_bytes >= falcon_fwd_workspace_bytes(...) a first kernel prepares
 * every sub-chunk of every chain in parallel into the workspace and a second
 * runs only the sequential state part; otherwise the call runs exactly as
 * falcon_fwd_chunk_ex.  Results as falcon_fwd_chunk_ex (rounding aside);
 * errors as falcon_fwd_chunk_ex, and FALCON_ERR_INVALID_ARG for a misaligned
 * or overlapping workspace.
 */
unsigned long long falcon_fwd_workspace_bytes(int variant, int window, int beta_kind, int batch,
                                              int heads, int seqlen, int dk, int dv, int dtype);
int falcon_fwd_chunk_ws(int variant, int window, int flags, float beta, const void* beta_t,
                        int beta_kind, float lambda, float eps, int batch, int heads, int seqlen,
                        int dk, int dv, int dtype, const void* q, const void* k, const void* v,
                        const void* k_prev, const float* S0, const void* x_hist,
                        const void* y_hist, float* o, float* S_out, void* x_hist_out,
                        void* y_hist_out, void* workspace, unsigned long long workspace_bytes,
                        int chunk, void* stream);

/*
 * falcon_fwd_masked - the masked-parallel form (explainer of arXiv 2608.27763,
 * section 核心方法 §3: the recurrence unrolled under a causal mask into one
 * parallel system, the form for short sequences): the whole call is one masked
 * system.  The samples' Gram matrix X X^T and the key-query products X Q^T are
 * formed for the whole sequence at once; the causally masked, decay-weighted
 * unit-lower-triangular system over every (step, window sample) unknown is then
 * solved without carrying a dk-sized state from step to step, and no decay
 * product is divided by (any decay, however strong, is exact).  With window 1
 * and gains shared by the value rows (scalar or per-token beta) the system is
 * the same for every value row and is solved once, in 16-step blocks on the
 * matrix cores; per-channel gains and windows 2..8 solve it per value row by
 * forward substitution.
 * Arguments, results and errors as falcon_fwd_recurrent_ex (every variant,
 * window 1..8, bf16 or fp32 inputs, carried key, state and window history,
 * FALCON_SAME_STEP); in addition FALCON_ERR_UNSUPPORTED for
 * seqlen > FALCON_MASKED_MAX_LEN.
 */
#define FALCON_MASKED_MAX_LEN 64
int falcon_fwd_masked(int variant, int window, int flags, float beta, const void* beta_t,
                      int beta_kind, float lambda, float eps, int batch, int heads, int seqlen,
                      int dk, int dv, int dtype, const void* q, const void* k, const void* v,
                      const void* k_prev, const float* S0, const void* x_hist,
                      const void* y_hist, float* o, float* S_out, void* x_hist_out,
                      void* y_hist_out, void* stream);

/*
 * falcon_decode_step_ex - falcon_decode_step for every variant, with the
 * window history of Falcon-3/3A and the pairing flag:
 *   window    B in 1..8; > 1 only for FALCON_3 / FALCON_3A
 *   flags     0 or FALCON_SAME_STEP (then x = k, and k_prev must be NULL and
 *             is not updated)
 *   x_hist, y_hist   [nseq, heads, B-1, dk] / [nseq, heads, B-1, dv] (dtype),
 *             oldest first; required when window > 1, NULL when window == 1.
 * The window of the step is the history plus (x, y), x = k_prev (x = k under
 * FALCON_SAME_STEP), y = v.  S, k_prev and the history are updated in place:
 * the oldest sample is dropped and (x, y) appended, then k_prev <- k (prefix
 * pairing only).  beta_t as in falcon_decode_step
 * (per-channel gains only for Falcon-2/2A).  No argument may overlap another.
 */
int falcon_decode_step_ex(int variant, int window, int flags, float beta, const void* beta_t,
                          int beta_kind, float lambda, float eps, int nseq, int heads, int dk,
                          int dv, int dtype, float* S, void* k_prev, void* x_hist,
                          void* y_hist, const void* q, const void* k, const void* v, float* o,
                          void* stream);

/*
 * Backward pass of the chunk form (every variant; windows 1 to 8): gradients
 * of  sum_t <dO_t, o_t> + <dS_L, S_L> + <dk_last, k_last>  with respect to q, k,
 * v, the gains, k_prev and S0.  The pages present the chunk-parallel form as
 * the training form (explainer §3; 163.com section 02 (2)) but print no
 * gradients; these are the chain rule through the chunk equations (per value
 * row: the triangular solve over the (step, window slot) unknowns, its
 * transpose, the decay products), computed in fp32 with the chunk-start states
 * recomputed by a forward sweep.
 *
 * falcon_bwd_workspace_bytes - bytes of device workspace falcon_bwd_chunk needs:
 *   per (batch, head), per slice of R = min(dv, 32) value rows (a head's rows are
 *   split over dv / R workgroups) and per chunk of floor(16 / window) steps,
 *   fp32: the chunk-start state (R x dk), S0 x
 *   (16 x R) and the unknowns' Gram (16 x 16); with two or more slices also each
 *   slice's partial dq, dk (L x dk each), dk_prev (dk) and per-token dbeta (L),
 *   which a second kernel adds in slice order.  0 for invalid sizes or a window
 *   outside 1..8.
 *
 * falcon_bwd_chunk
 *   variant ... k_prev, S0, flags   as falcon_fwd_chunk_ex (flags 0 or
 *             FALCON_SAME_STEP); dk, dv in {16, 32, 64, 128}; dtype bf16 or fp32
 *   window    1, or 2..8 for FALCON_3 / FALCON_3A; a windowed call takes no
 *             start state (S0 must be NULL: its window history is not an input)
 *   dO        [batch, heads, L, dv] float32, gradient of o
 *   dS_L      [batch, heads, dv, dk] float32 gradient of the final state, or NULL
 *   dk_last   [batch, heads, dk] float32 gradient of k_last = k_L (the key a
 *             next call takes as k_prev), or NULL
 *   dq, dk_out, dv_out   [batch, heads, L, dk / dk / dv] float32 outputs
 *   dbeta_t   gradient of beta_t (float32, beta_t's shape), or NULL; must be
 *             NULL for a scalar beta (a scalar beta gets no gradient)
 *   dk_prev   [batch, heads, dk] float32, or NULL; needs k_prev
 *   dS0       [batch, heads, dv, dk] float32, or NULL; needs S0
 *   workspace, workspace_bytes   device scratch of at least
 *             falcon_bwd_workspace_bytes(..., window) bytes, 16-byte aligned
 * Outputs must not overlap each other, the inputs or the workspace.
 * Errors as elsewhere; FALCON_ERR_UNSUPPORTED for a window above 8, a
 * windowed start state, or a chain whose inputs or workspace records reach
 * 1 GiB: the kernel addresses a chain's buffers with 32-bit offsets.  The
 * records dominate: 4 * (R * dk + 16 * R + 256) bytes per chunk of
 * floor(16 / window) steps, so the limit is about 880 K steps at
 * dk = dv = 128, window 1, and about 110 K steps at window 8.
 * Range: the chunks of floor(16 / window) steps are scaled by their decay
 * products g_t = prod (1 - eta_r lambda); for a (batch, head) chain in which
 * some |g_t| leaves [2^-100, 2^100] or some |1 - eta_t lambda| is below 2^-24
 * (strong forgetting) the gradients are not computed: every output of that
 * chain is set to NaN (the forward entry points have an exact path for such
 * chains; the backward has none).
 */
unsigned long long falcon_bwd_workspace_bytes(int batch, int heads, int seqlen, int dk, int dv,
                                              int window);
int falcon_bwd_chunk(int variant, int window, int flags, float beta, const void* beta_t,
                     int beta_kind, float lambda, float eps, int batch, int heads, int seqlen,
                     int dk, int dv, int dtype, const void* q, const void* k, const void* v,
                     const void* k_prev, const float* S0, const float* dO, const float* dS_L,
                     const float* dk_last, float* dq, float* dk_out, float* dv_out,
                     float* dbeta_t, float* dk_prev, float* dS0, void* workspace,
                     unsigned long long workspace_bytes, void* stream);

/*
 * falcon_bwd_chunk_noalloc - falcon_bwd_chunk without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * device array of FALCON_BWD_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends; the call allocates nothing.  Arguments,
 * results and errors as falcon_bwd_chunk; in addition
 *   FALCON_ERR_UNSUPPORTED  falcon_bwd_workspace_bytes(...) of the call exceeds
 *                           FALCON_BWD_SCRATCH_BYTES (use falcon_bwd_chunk)
 *   FALCON_ERR_HIP          the array's device address could not be obtained
 * Every call on one GPU uses that GPU's array: calls that overlap in time on
 * one GPU (different streams or host threads) race and give wrong gradients;
 * calls in order on one stream are safe.
 */
#define FALCON_BWD_SCRATCH_BYTES (64ull << 20)
int falcon_bwd_chunk_noalloc(int variant, int window, int flags, float beta, const void* beta_t,
                             int beta_kind, float lambda, float eps, int batch, int heads,
                             int seqlen, int dk, int dv, int dtype, const void* q, const void* k,
                             const void* v, const void* k_prev, const float* S0, const float* dO,
                             const float* dS_L, const float* dk_last, float* dq, float* dk_out,
                             float* dv_out, float* dbeta_t, float* dk_prev, float* dS0,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FALCON_H */
