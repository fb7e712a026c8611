/*
 * specverify -- the verify step of speculative sampling on AMD Instinct
 * MI355X (gfx950), as a C ABI.
 *
 * The operation (cited by page title and section):
 *   "CS3602_FINAL_SpeDec", section 2 (perplexity test) and its proof: p is
 *   the target distribution, q the draft distribution; a guess x ~ q is
 *   accepted with probability min(1, p(x)/q(x)); at the first rejection the
 *   token is drawn from the residual p' = norm(max(0, p - q)), whose
 *   normaliser is 1 - beta with beta = sum_x min(p(x), q(x)); this makes the
 *   emitted token exactly p-distributed.
 *   "Text Generation via Speculative Sampling, KV Caching, and OpenVINO",
 *   section "Prepare speculative sampling", steps 3 and 4: one uniform draw per
 *   draft position, stop at the first rejection, and draw one extra token from
 *   the last target position when every guess was accepted; section "Prepare
 *   autoregressive sampling": softmax over the vocabulary, argmax decode
 *   (the greedy mode here).  spec_draft_sample draws the guesses themselves
 *   (step 1 of "Prepare speculative sampling", sampling in place of the
 *   argmax), and spec_token_likelihood scores given tokens under the
 *   speculative step (the perplexity check of "CS3602_FINAL_SpeDec").
 *
 * Conventions shared by the calls
 *   Batch layout (packed, ragged).  Sequence b has K_b >= 0 draft tokens.
 *   With cu_draft == NULL every K_b equals shape->max_draft; otherwise
 *   cu_draft is a DEVICE array of B+1 int32 prefix sums (cu_draft[0] = 0,
 *   cu_draft[b+1] - cu_draft[b] = K_b, cu_draft[B] = shape->total_draft).
 *   Target rows: sequence b owns rows cu_draft[b] + b + k for k = 0..K_b
 *   (K_b + 1 rows; row K_b is the extra-token position).  Draft rows:
 *   cu_draft[b] + k for k = 0..K_b-1.  draft_ids[cu_draft[b] + k] is the
 *   guess at position k.  Each row holds `vocab` logits, row-major, with
 *   row_stride elements between row starts.
 *
 *   Output tokens: out_tokens[cu_draft[b] + b + j] for j = 0..K_b holds the
 *   accepted guesses x_0..x_{n-1}, then the new token at j = n, then -1.
 *   out_num_accepted[b] = n (0 <= n <= K_b), or -1 when the sequence's
 *   cu_draft entries or draft ids are out of range (then its token slots are
 *   left untouched).
 *
 *   Memory.  Every pointer is device memory owned by the caller.  The
 *   library allocates nothing and keeps no state between calls; it reads
 *   the inputs, overwrites the outputs and uses `workspace` as scratch.
 *   Vectorised reads may touch bytes outside a row that share its 16-byte
 *   aligned blocks (never outside those blocks); the values read there are
 *   discarded.  Logit pointers must be aligned to their element size.
 *
 *   Execution.  Asynchronous on `stream` (NULL = the null stream); no host
 *   synchronisation inside the call.  Concurrent calls are safe when they
 *   use different workspaces and outputs.  Results are a pure function of
 *   (inputs, temperature, top_k, seed, offset): bit-identical across runs.
 *
 *   Workspace.  Call once with workspace == NULL: *workspace_bytes receives
 *   the size needed for this shape and mode and nothing is launched.  Then
 *   call with a device buffer of at least that many bytes (256-byte aligned).
 *
 *   Errors.  Argument checks are synchronous and happen before any launch:
 *   SV_ERR_INVALID_ARGUMENT (null or misaligned pointer, B < 1, V < 1,
 *   K < 0, total_draft inconsistent with B*K when cu_draft is NULL, stride
 *   < V, temperature not finite and > 0, or so small that log2(e) / T
 *   overflows fp32 (T below about 4.2e-39), top_k < 0 or > V),
 *   SV_ERR_UNSUPPORTED (V > SV_MAX_VOCAB, max_draft > SV_MAX_DRAFT),
 *   SV_ERR_WORKSPACE_TOO_SMALL, SV_ERR_HIP (a launch failed).  Data
 *   preconditions are the caller's: logits finite or -inf with at least one
 *   finite logit in each row's kept set, and |logit| * log2(e) / T finite in
 *   fp32; cu_draft monotone.  The kernels
 *   never read out of bounds when they are violated: a bad sequence reports
 *   num_accepted = -1.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(SPECVERIFY_BUILDING)
#define SV_API __attribute__((visibility("default")))
#else
#define SV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define SV_MAX_VOCAB (1 << 20)
#define SV_MAX_DRAFT 128

typedef enum {
    SV_OK = 0,
    SV_ERR_INVALID_ARGUMENT = 1,
    SV_ERR_UNSUPPORTED = 2,
    SV_ERR_WORKSPACE_TOO_SMALL = 3,
    SV_ERR_HIP = 4
} sv_status_t;

/* Logit element types.  Every type is widened exactly to fp32 on load and no
 * probability is ever formed in 16 bits ("CS3602_FINAL_SpeDec", problem
 * analysis, item 1: fp16 probabilities underflow).  SV_DTYPE_F16 is IEEE
 * binary16, the precision the pages' models ran in. */
typedef enum { SV_DTYPE_F32 = 0, SV_DTYPE_BF16 = 1, SV_DTYPE_F16 = 2 } sv_dtype_t;

typedef struct {
    int32_t batch;             /* B >= 1                                          */
    int32_t max_draft;         /* K, or the largest K_b when cu_draft != NULL     */
    int32_t total_draft;       /* sum_b K_b; must be B*K when cu_draft == NULL    */
    int32_t vocab;             /* V >= 1                                          */
    sv_dtype_t dtype;          /* element type of both logit tensors              */
    int64_t target_row_stride; /* elements between target rows, >= V             */
    int64_t draft_row_stride;  /* elements between draft rows, >= V              */
    const int32_t* cu_draft;   /* device [B+1] prefix sums of K_b, or NULL        */
} sv_shape_t;

/*
 * Speculative sampling verify.
 *   p_k = softmax(target row k / T) and q_k = softmax(draft row k / T), each
 *   restricted to its own top-k kept set when top_k > 0 (every id whose raw
 *   logit is >= the top_k-th largest, ties kept; top_k = 0 or V keeps all),
 *   then, when top_p < 1, to its own top-p nucleus: every id whose logit is
 *   >= tau_p, the largest logit value t for which the probability of
 *   {v : l_v >= t} reaches top_p (ties kept), renormalised.  Top-K and
 *   Top-P are the two filters the sampling helpers of "CS3602_FINAL_SpeDec"
 *   name (its module list; problem analysis, item 2).
 *   Position k accepts iff u_k < min(1, p_k(x_k) / q_k(x_k)) (q = 0 accepts
 *   iff p > 0), u_k = U(b, k, 0).  n = the first rejected position, or K_b.
 *   If n < K_b the new token is the first id (ascending) whose running sum
 *   of max(0, p_n - q_n) exceeds U(b, n, 1) times its total; otherwise it is
 *   the inverse-CDF draw of p_{K_b} with U(b, K_b, 2).
 *   U(b, pos, purpose) = (w >> 8) * 2^-24 where w is word 0 of
 *   Philox4x32-10 (Salmon et al., SC'11) with key (seed lo32, seed hi32)
 *   and counter (b, pos, purpose, offset).
 * Arguments
 *   target_logits [rows_t, stride] and draft_logits [rows_d, stride] in
 *   shape->dtype; draft_ids int32 [total_draft] in [0, V).
 *   temperature > 0, finite, and >= about 4.2e-39 (log2(e) / T must be a
 *   finite fp32).  top_k in [0, V].  top_p in (0, 1]; 1 is
 *   off.  top-p over full rows costs several extra reads of each row (a
 *   mass-weighted radix select); after top-k it works on the kept lists.
 *   out_tokens int32 [total_draft + B]; out_num_accepted int32 [B];
 *   out_probs (nullable) float [total_draft][2] = p_k(x_k), q_k(x_k) for
 *   every draft position; out_residual_mass (nullable) float [B] = the
 *   residual total sum_v max(0, p_n - q_n) = 1 - beta_n (0 if all accepted).
 */
SV_API sv_status_t spec_verify_sample(const sv_shape_t* shape,
                               const void* target_logits,
                               const void* draft_logits,
                               const int32_t* draft_ids,
                               float temperature,
                               int32_t top_k,
                               float top_p,
                               uint64_t seed,
                               uint32_t offset,
                               int32_t* out_tokens,
                               int32_t* out_num_accepted,
                               float* out_probs,
                               float* out_residual_mass,
                               void* workspace,
                               size_t* workspace_bytes,
                               hipStream_t stream);

/*
 * spec_verify_sample for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call, results and errors, with no workspace
 * argument.  Its scratch is one file-scope device array of
 * SV_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends; its address is taken once per device, on the first call
 * made with that device current.  The call allocates nothing.
 *   A shape and mode whose workspace (the size spec_verify_sample's query
 *   reports) exceeds SV_NOALLOC_SCRATCH_BYTES is rejected with
 *   SV_ERR_WORKSPACE_TOO_SMALL before anything is launched.
 *   Every call on one GPU shares that GPU's array and leaves the last call's
 *   contents in it (no call relies on them: every call writes what it
 *   reads).  Calls that overlap in time on one GPU race, on any streams:
 *   serialise them, or use spec_verify_sample with separate workspaces.
 */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

SV_API sv_status_t spec_verify_sample_noalloc(const sv_shape_t* shape,
                               const void* target_logits,
                               const void* draft_logits,
                               const int32_t* draft_ids,
                               float temperature,
                               int32_t top_k,
                               float top_p,
                               uint64_t seed,
                               uint32_t offset,
                               int32_t* out_tokens,
                               int32_t* out_num_accepted,
                               float* out_probs,
                               float* out_residual_mass,
                               hipStream_t stream);

/*
 * Verify with argmax draws, the variant the OpenVINO page implements
 * ("Text Generation via Speculative Sampling, KV Caching, and OpenVINO",
 * "Prepare speculative sampling", steps 3 and 4): the same probabilistic
 * acceptance test as spec_verify_sample (same uniforms U(b, k, 0)), but the
 * new token is the argmax (lowest id among equal maxima) of
 * max(0, p_n - q_n) at the first rejection n < K_b -- of p_n when that
 * residual has no positive entry -- and the argmax of p_{K_b} when every
 * guess is accepted.  Arguments, outputs and errors as for
 * spec_verify_sample; out_residual_mass is the residual's total as there.
 */
SV_API sv_status_t spec_verify_argmax(const sv_shape_t* shape,
                               const void* target_logits,
                               const void* draft_logits,
                               const int32_t* draft_ids,
                               float temperature,
                               int32_t top_k,
                               float top_p,
                               uint64_t seed,
                               uint32_t offset,
                               int32_t* out_tokens,
                               int32_t* out_num_accepted,
                               float* out_probs,
                               float* out_residual_mass,
                               void* workspace,
                               size_t* workspace_bytes,
                               hipStream_t stream);

/*
 * Greedy argmax-compare verify (the argmax rule of the autoregressive decode
 * on the OpenVINO page).  a_k = the lowest index among the maxima of target
 * row k; n = the first k < K_b with draft_ids[k] != a_k, or K_b; the tokens
 * are x_0..x_{n-1}, a_n, then -1.  Temperature and top-k do not change an
 * argmax, so they are not arguments.  Draft logits are not read.
 * Arguments as in spec_verify_sample; shape->draft_row_stride is ignored.
 */
SV_API sv_status_t spec_verify_greedy(const sv_shape_t* shape,
                               const void* target_logits,
                               const int32_t* draft_ids,
                               int32_t* out_tokens,
                               int32_t* out_num_accepted,
                               void* workspace,
                               size_t* workspace_bytes,
                               hipStream_t stream);

/*
 * Draft-side sampling, the step before verify: every guess x(b, k) ~ q_k.
 * The draft model proposes its K guesses one position at a time ("Text
 * Generation via Speculative Sampling, KV Caching, and OpenVINO", section
 * "Prepare speculative sampling", step 1, which takes the argmax); the
 * acceptance proof of "CS3602_FINAL_SpeDec", section 2, assumes each guess
 * is drawn from q, and that page's sampling helpers filter by top-K.
 *   q_k = softmax(draft row k / T) over its top-k kept set and top-p
 *   nucleus, exactly as in spec_verify_sample; x(b, k) = the first id (ascending) whose running sum
 *   of q_k exceeds U(b, k, 3), with U as in spec_verify_sample.
 * Arguments
 *   shape as for spec_verify_sample; target_row_stride is ignored.
 *   draft_logits [total_draft, draft_row_stride] in shape->dtype.
 *   temperature > 0 and finite; top_k in [0, V]; top_p in (0, 1].
 *   out_ids int32 [total_draft]: x(b, k) at cu_draft[b] + k.  A sequence
 *   whose cu_draft entries are out of range leaves its slots untouched; a
 *   row with no finite logit in its kept set yields -1.
 * Memory, execution, workspace and errors as for spec_verify_sample.
 */
SV_API sv_status_t spec_draft_sample(const sv_shape_t* shape,
                              const void* draft_logits,
                              float temperature,
                              int32_t top_k,
                              float top_p,
                              uint64_t seed,
                              uint32_t offset,
                              int32_t* out_ids,
                              void* workspace,
                              size_t* workspace_bytes,
                              hipStream_t stream);

/*
 * Per-token speculative likelihood, the quantity behind the perplexity
 * check of "CS3602_FINAL_SpeDec" (section 2's proof, used by that report's
 * problem analysis, item 1, to score speculative output without summing
 * over the vocabulary).  For position (b, k), k < K_b, with p = the target
 * row's and q = the draft row's softmax at temperature T (each over its
 * top-k kept set and top-p nucleus, exactly as in spec_verify_sample) and
 * y = tokens[r]:
 *   accept part  P(guess accepted, x = y) = q(y) min(1, p(y)/q(y)) = min(p(y), q(y))
 *   reject part  P(guess rejected, x = y) = (1 - beta) p'(y)       = p(y) - min(p(y), q(y))
 *   beta         = sum_v min(p(v), q(v))   (the position's acceptance mass)
 *   nll[b]       = -sum_k log(accept part + reject part)
 * The two parts add to p(y): one speculative step emits y with the target's
 * probability.
 * Arguments
 *   shape: batch, vocab, dtype, strides and cu_draft as for
 *   spec_verify_sample, but position (b, k) is row r = cu_draft[b] + k of
 *   BOTH tensors (total_draft rows each; max_draft, the largest K_b, has no
 *   upper limit here).
 *   target_logits [total_draft, target_row_stride], draft_logits
 *   [total_draft, draft_row_stride] in shape->dtype; tokens int32
 *   [total_draft].  temperature > 0 and finite; top_k in [0, V]; top_p in
 *   (0, 1].
 *   out_terms (nullable) float [total_draft][2] = accept part, reject part;
 *   out_beta (nullable) float [total_draft]; out_nll (nullable) double [B].
 *   At least one output must be non-NULL.  beta over full rows costs a
 *   second read of both rows; leave out_beta NULL when it is not needed.
 *   A token outside [0, V), or a row with no finite logit in its kept set,
 *   gives NaN parts (and NaN beta for such a row); p(y) = 0 gives an infinite
 *   nll.  A sequence whose cu_draft entries are out of range gets nll = NaN
 *   and leaves its other slots untouched.
 * Memory, execution, workspace and errors as for spec_verify_sample.
 */
SV_API sv_status_t spec_token_likelihood(const sv_shape_t* shape,
                              const void* target_logits,
                              const void* draft_logits,
                              const int32_t* tokens,
                              float temperature,
                              int32_t top_k,
                              float top_p,
                              float* out_terms,
                              float* out_beta,
                              double* out_nll,
                              void* workspace,
                              size_t* workspace_bytes,
                              hipStream_t stream);

/* A static, human-readable name for a status code. */
SV_API const char* spec_verify_status_string(sv_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
