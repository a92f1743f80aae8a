/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library.
 *
 * The layer: each head keeps a d_k x d_v state S (rows = key channels) and
 * every token updates it once with the gated delta rule
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *
 * (dimsnsums.com "GLM-5.3-FLASH" attention page, section "How can a layer
 * remember without rereading?": the update rule and the sentence that
 * defines its symbols; the same section fixes a 128x128 state per head that
 * each token updates once).  The output of token t is the read-out of the
 * post-update state, o_t = S_t^T q_t, with no scale (a convention: the page
 * prints only the update).  alpha_t holds one decay rate per key channel
 * (Diag(alpha_t) multiplies S from the left), beta_t one scalar per token
 * and head.
 *
 * Gate kinds (shape->gate):
 *  - KDA_GATE_CHANNEL: the KDA rule above, alpha [tokens][H][d_k].
 *  - KDA_GATE_HEAD: one decay rate per token and head, alpha [tokens][H]:
 *    Diag(alpha_t) = alpha_t I, the scalar-gated delta rule of the Gated
 *    DeltaNet layers that the ainewsfeed.tech page on the GLM-5.3-Flash
 *    configuration names (the pages print no formula for it; a scalar
 *    decay per head is the reading taken).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Tensor arguments are DEVICE pointers to contiguous, row-major arrays
 *    on the current HIP device, aligned to 16 bytes, except beta,
 *    cu_seqlens, accepted and a per-head alpha (KDA_GATE_HEAD), which need
 *    4 bytes (they are read one element at a time), and the workspace,
 *    which needs 256 bytes.  The same rule holds for every entry point.
 *    Layouts are token-major:
 *        q, k          [tokens][H][d_k]
 *        alpha         [tokens][H][d_k]  (KDA_GATE_CHANNEL)
 *                      [tokens][H]       (KDA_GATE_HEAD; 4-byte aligned)
 *        v, o          [tokens][H][d_v]
 *        beta          [tokens][H]
 *        state         [N][H][d_k][d_v]        (fp32)
 *    q, k, v are fp32 or bf16 (shape->qkv_dtype); alpha, beta, state and o
 *    are always fp32.
 *  - The caller owns every buffer, including the prefill workspace.  The
 *    library allocates no device memory at run time and never synchronises:
 *    every call only enqueues kernels on `stream` (a hipStream_t passed as
 *    void*; NULL = the default stream) and returns.  Its only global state
 *    is the static scratch of kda_prefill_noalloc (a device array per GPU)
 *    and that array's cached addresses.
 *    Calls on different streams may run concurrently.
 *  - Errors: every call returns a kda_status_t and never throws, aborts or
 *    prints.  Argument validation happens on the host before any HIP call,
 *    so an invalid call enqueues nothing.  KDA_ERR_LAUNCH reports a failed
 *    kernel launch (hipGetLastError); faults inside a kernel surface as HIP
 *    errors at the caller's next synchronisation, as for any HIP kernel.
 *  - Supported sizes: d_k == d_v in {16, 32, 64, 128}; H >= 1.
 *  - Device-side preconditions (not checked, a check would need a sync):
 *    0 <= alpha <= 1 (KDA_INPUT_FINAL); beta, q, k, v finite; cu_seqlens[0] == 0,
 *    non-decreasing, cu_seqlens[N] == total_tokens; outputs do not overlap
 *    inputs except where aliasing is stated below.  Non-finite inputs give
 *    non-finite outputs; they do not fault.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 5
#define KDA_CHUNK 64 /* prefill chunk length (tokens); not a semantic parameter */

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misaligned, inconsistent shape */
    KDA_ERR_UNSUPPORTED = 2,      /* valid but not built: d_k != d_v, d not in {16,32,64,128},
                                     prefill with 64 * H * d * 4 >= 2^31 (H > 65535 at d = 128),
                                     prefill and backward with (total_tokens + 64 N) H d/16
                                     >= 2^40 (about 4e9 tokens at H = 32, d = 128) */
    KDA_ERR_WORKSPACE_TOO_SMALL = 3,
    KDA_ERR_LAUNCH = 4            /* a kernel launch failed (HIP error) */
} kda_status_t;

typedef enum kda_dtype {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype_t;

/* Layout of alpha: one decay rate per key channel (KDA) or per head. */
typedef enum kda_gate {
    KDA_GATE_CHANNEL = 0, /* alpha [tokens][H][d_k] */
    KDA_GATE_HEAD = 1     /* alpha [tokens][H] */
} kda_gate_t;

/* What q, k, alpha and beta hold.
 *  - KDA_INPUT_FINAL: the values the update rule uses.
 *  - KDA_INPUT_PREACT: the layer's gate pre-activations and raw q, k; the
 *    library forms, per token and head, inside the kernels' load stage
 *        alpha = exp(-softplus(a)) = 1 / (1 + e^a)   from a in `alpha`
 *        beta  = sigmoid(b)        = 1 / (1 + e^-b)  from b in `beta`
 *        q <- q / max(||q||_2, 1e-12),  k <- k / max(||k||_2, 1e-12)
 *    (norms over the d_k key channels).  The attention page says each key
 *    channel decays at a learned, data-driven rate but prints no
 *    parameterisation; this one is the reading taken.  v is used as given. */
typedef enum kda_input_form {
    KDA_INPUT_FINAL = 0,
    KDA_INPUT_PREACT = 1
} kda_input_form_t;

/* Problem shape.  Dense batch: cu_seqlens == NULL, num_seqs sequences of
 * seq_len tokens each, sequence n owning tokens n*seq_len .. (n+1)*seq_len-1,
 * and total_tokens == num_seqs * seq_len.  Varlen batch: cu_seqlens != NULL,
 * seq_len ignored, total_tokens == cu_seqlens[num_seqs]. */
typedef struct kda_shape {
    int32_t num_seqs;     /* N >= 0 */
    int32_t seq_len;      /* tokens per sequence (dense batch only), >= 0 */
    int64_t total_tokens; /* >= 0 */
    int32_t num_heads;    /* H >= 1 */
    int32_t d_k;          /* key channels per head */
    int32_t d_v;          /* value channels per head (must equal d_k) */
    int32_t qkv_dtype;    /* kda_dtype_t of q, k, v */
    int32_t gate;         /* kda_gate_t: layout of alpha */
    int32_t input_form;   /* kda_input_form_t */
} kda_shape_t;

/* Version of this ABI (KDA_ABI_VERSION of the built library). */
int kda_abi_version(void);

/* Human-readable name of a status code; never NULL. */
const char *kda_status_string(kda_status_t status);

/* Recommended bytes of device workspace for kda_prefill of `shape` (written
 * to *bytes): a chunk table of 2N+1 int32 (each sequence's first chunk, the
 * total, and the sequences in the order the state pass takes them; padded to
 * 256 B), then one record
 * of chunk operands (108.5 KiB at d = 128) per head and per 64-token chunk,
 * for an upper bound on the batch's chunks, floor(total_tokens/64) + N.  It
 * depends on N, H, d and total_tokens only.  With it every chunk of the batch
 * is built in one pass (the fastest; the two phase entry points need it).
 *
 * kda_prefill also accepts less, down to the table plus H records (plus N H
 * d_k d_v floats when S_T is NULL and the batch needs more than one stripe):
 * it then runs in stripes of W consecutive chunks of the batch (sequence
 * after sequence), W = the records the workspace holds divided by H, and
 * hands each sequence's state from one stripe to the next through S_T.  So
 * the workspace need not grow with the context: a 2^20-token sequence at
 * H = 32, d = 128 runs in 1 GiB as well as in the recommended 58 GB.
 * Returns KDA_ERR_INVALID_ARGUMENT / KDA_ERR_UNSUPPORTED for a shape
 * kda_prefill would reject. */
kda_status_t kda_prefill_workspace_size(const kda_shape_t *shape, size_t *bytes);

/* Prefill (chunked): run the update over every token of every sequence and
 * write o for every token and, if S_T != NULL, the final state of every
 * sequence.
 *   q, k        [total_tokens][H][d_k]      fp32 or bf16 (qkv_dtype)
 *   v           [total_tokens][H][d_v]      same dtype
 *   alpha       [total_tokens][H][d_k]      fp32, per key channel, or
 *               [total_tokens][H]           per head (shape->gate)
 *   beta        [total_tokens][H]           fp32
 *   cu_seqlens  [N+1] int32 device array, or NULL for a dense batch
 *   S0          [N][H][d_k][d_v] fp32 initial states, or NULL for zeros
 *   o           [total_tokens][H][d_v] fp32 output
 *   S_T         [N][H][d_k][d_v] fp32 final states, or NULL to skip; may be
 *               the same pointer as S0 (in-place update)
 *   workspace   device scratch, 256-byte aligned: the recommended size of
 *               kda_prefill_workspace_size, or less down to the minimum
 *               given there (KDA_ERR_WORKSPACE_TOO_SMALL below it); its
 *               contents on entry do not matter and are clobbered
 * A zero-length sequence gets S_T[n] = S0[n] (zeros if S0 == NULL).
 * Sequences and heads are independent. */
kda_status_t kda_prefill(const kda_shape_t *shape,
                         const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta,
                         const int32_t *cu_seqlens,
                         const float *S0,
                         float *o, float *S_T,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/* The two phases of kda_prefill, for callers that schedule them separately
 * (e.g. phase 1 of the next batch on another stream while phase 2 of this
 * one runs).  They need a workspace that holds every chunk of the batch in
 * one stripe (the recommended size of kda_prefill_workspace_size always does;
 * one that would need stripes is KDA_ERR_WORKSPACE_TOO_SMALL), with which
 * kda_prefill(...) is exactly phase 1 followed by phase 2 on the same stream
 * with the same arguments.
 *
 * Phase 1 (fully parallel over chunks and heads): builds the per-sequence
 * chunk table and, for every 64-token chunk and head, the chunk-local
 * operands of the chunked form, into `workspace`.  Reads q, k, alpha, beta
 * and cu_seqlens. */
kda_status_t kda_prefill_chunk_local(const kda_shape_t *shape,
                                     const void *q, const void *k,
                                     const float *alpha, const float *beta,
                                     const int32_t *cu_seqlens,
                                     void *workspace, size_t workspace_bytes,
                                     void *stream);

/* Phase 2 (sequential over the chunks of each sequence, parallel over
 * sequences, heads and value columns): carries each state across its
 * sequence's chunks and writes o and S_T.  `workspace` must hold the result
 * of kda_prefill_chunk_local for the same shape, q, k, alpha, beta and
 * cu_seqlens, ordered before this call (same stream, or an event).
 * Arguments as for kda_prefill. */
kda_status_t kda_prefill_state_pass(const kda_shape_t *shape,
                                    const void *q, const void *k, const void *v,
                                    const float *alpha,
                                    const int32_t *cu_seqlens,
                                    const float *S0,
                                    float *o, float *S_T,
                                    void *workspace, size_t workspace_bytes,
                                    void *stream);

/* Prefill without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc).  Arguments, results and errors are those of
 * kda_prefill; the workspace is a static device array of the library,
 * KDA_NOALLOC_WORKSPACE_BYTES (128 MiB) on each GPU the library runs on,
 * held from the library's first use on that GPU until the process ends.
 *  - Any batch runs, in stripes when it needs more than the recommended
 *    workspace (as kda_prefill with a workspace of that size), provided the
 *    chunk table and H records (108.5 KiB each at d = 128: up to 1,208 heads)
 *    fit, and when S_T is NULL and the batch needs stripes, also the N H
 *    carried states (64 KiB each at d = 128: about 60 sequences at H = 32).
 *    Otherwise KDA_ERR_WORKSPACE_TOO_SMALL, before any HIP call.
 *  - The call allocates nothing: no hipMalloc, no allocating library call.
 *    Its first call on a device looks up the array's address there
 *    (hipGetSymbolAddress) and caches it.  The array used is the current
 *    device's, so a non-NULL stream must belong to the current device
 *    (hipStreamGetDevice); otherwise KDA_ERR_INVALID_ARGUMENT, nothing
 *    enqueued.
 *  - Every call on one GPU uses that GPU's one array, whose contents on
 *    entry do not matter.  Calls that overlap in time on the same GPU (two
 *    streams, or two host threads) race on it and give wrong results; order
 *    them (one stream, or events). */
#define KDA_NOALLOC_WORKSPACE_BYTES (128u << 20)
kda_status_t kda_prefill_noalloc(const kda_shape_t *shape,
                                 const void *q, const void *k, const void *v,
                                 const float *alpha, const float *beta,
                                 const int32_t *cu_seqlens,
                                 const float *S0,
                                 float *o, float *S_T,
                                 void *stream);

/* Decode: one new token for each of N sequences; every head state is read
 * once, advanced one step and written back in place.
 *   shape       num_seqs = N, seq_len must be 1, total_tokens must be N,
 *               no cu_seqlens
 *   q, k        [N][H][d_k]   fp32 or bf16 (qkv_dtype)
 *   v           [N][H][d_v]
 *   alpha       [N][H][d_k]   fp32 ([N][H] with KDA_GATE_HEAD)
 *   beta        [N][H]        fp32
 *   S           [N][H][d_k][d_v] fp32, updated in place
 *   o           [N][H][d_v]   fp32 output (must not overlap S) */
kda_status_t kda_decode_step(const kda_shape_t *shape,
                             const void *q, const void *k, const void *v,
                             const float *alpha, const float *beta,
                             float *S, float *o,
                             void *stream);

/* Several new tokens per sequence from the live state: speculative
 * verification of drafted tokens (the kongchang.com page "18B Active for
 * Just $0.045: How GLM-5.3-Flash Beat Claude with Hybrid Attention", section
 * "The Architecture Stack: How Linear and Sparse Interleave": one MTP draft
 * layer; drafted tokens checked in parallel, rejected ones rolled back), or plain multi-token
 * decode.  Each token is one step of the update rule, in order; the state
 * is read once and kept in registers across a sequence's tokens.
 *   shape       num_seqs = N, seq_len = k >= 1 tokens per sequence,
 *               total_tokens must be N * k, no cu_seqlens
 *   q, k        [N * k][H][d_k]   (sequence n owns rows n*k .. n*k+k-1)
 *   v           [N * k][H][d_v]
 *   alpha       [N * k][H][d_k] fp32 ([N * k][H] with KDA_GATE_HEAD)
 *   beta        [N * k][H]     fp32
 *   S           [N][H][d_k][d_v] fp32 live states
 *   o           [N * k][H][d_v] fp32 output for every token
 *   S_hist      [N][k][H][d_k][d_v] fp32, or NULL.  NULL: S is advanced in
 *               place by all k tokens.  Non-NULL: S is left unchanged and
 *               S_hist[n][t] receives the state after token t of sequence n
 *               (for kda_state_commit); it must not overlap S.
 * Gate kind and input form as for the other calls. */
kda_status_t kda_decode_tokens(const kda_shape_t *shape,
                               const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta,
                               float *S, float *o, float *S_hist,
                               void *stream);

/* After verification: for every sequence n with j = accepted[n] >= 1,
 * S[n] <- S_hist[n][min(j, k) - 1] (the state after its j accepted tokens);
 * j <= 0 leaves S[n] unchanged (every draft rejected).
 *   shape       num_seqs = N, seq_len = k (as passed to kda_decode_tokens),
 *               num_heads, d_k == d_v; the other fields are not used
 *   S           [N][H][d_k][d_v] fp32, updated
 *   S_hist      [N][k][H][d_k][d_v] fp32 from kda_decode_tokens
 *   accepted    [N] int32 device array */
kda_status_t kda_state_commit(const kda_shape_t *shape, float *S, const float *S_hist,
                              const int32_t *accepted, void *stream);

/* Speculative verification with rollback by recomputation instead of a
 * state history (the same passage as kda_decode_tokens).  kda_verify_tokens
 * gives the outputs of k tokens per sequence from the live state and writes
 * nothing else; kda_accept_tokens then advances the live state by the first
 * accepted[n] of those tokens (clamped to [0, k]; 0 leaves S[n] untouched),
 * running them again.  Per (sequence, head) a verify round reads the state
 * once and an accepting sequence reads and writes it once more, where
 * kda_decode_tokens with S_hist writes k states and kda_state_commit copies
 * one: no history buffer, and fewer state bytes per round.  Both give the
 * outputs and states that kda_decode_tokens (with S_hist) and
 * kda_state_commit give, bit for bit.
 *   shape, q, k, v, alpha, beta   as for kda_decode_tokens (the same token
 *                 rows for both calls of a round)
 *   S             [N][H][d_k][d_v] fp32 live states (read only in
 *                 kda_verify_tokens, updated in kda_accept_tokens)
 *   o             [N * k][H][d_v] fp32 output for every token (verify)
 *   accepted      [N] int32 device array (accept), 4-byte aligned
 * Gate kind and input form as for the other calls; a shape, pointer or
 * alignment the checks of kda_decode_tokens reject is rejected the same
 * way. */
kda_status_t kda_verify_tokens(const kda_shape_t *shape,
                               const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta,
                               const float *S, float *o, void *stream);
kda_status_t kda_accept_tokens(const kda_shape_t *shape,
                               const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta,
                               float *S, const int32_t *accepted, void *stream);

/* One round of the loop above in one pass over the state: S[n] advanced by
 * the first accepted[n] tokens of the previous round (q0 .. beta0, what
 * kda_accept_tokens would run), then the outputs of this round's tokens (q ..
 * beta, what kda_verify_tokens would give) from the advanced state, which S
 * keeps.  Equal, bit for bit, to kda_accept_tokens then kda_verify_tokens;
 * per (sequence, head) the state is read once and written once when
 * accepted[n] > 0.  Both rounds have the shape's k tokens per sequence.
 *   shape           as for kda_verify_tokens
 *   q0, k0, v0, alpha0, beta0, accepted   the previous round (as for
 *                   kda_accept_tokens)
 *   q, k, v, alpha, beta, o               this round (as for
 *                   kda_verify_tokens)
 *   S               [N][H][d_k][d_v] fp32 live states, updated */
kda_status_t kda_accept_verify_tokens(const kda_shape_t *shape,
                                      const void *q0, const void *k0, const void *v0,
                                      const float *alpha0, const float *beta0,
                                      const int32_t *accepted,
                                      const void *q, const void *k, const void *v,
                                      const float *alpha, const float *beta,
                                      float *S, float *o, void *stream);

/* Backward pass (training): gradients of L with respect to q, k, v, alpha,
 * beta and the initial states, given dL/do for every token (dO) and dL/dS_T
 * for every final state (dS_T, or NULL for zero).  It differentiates the
 * same update rule and read-out as kda_prefill, token by token in reverse:
 * with X = Diag(alpha_t) S_{t-1}, w = v_t - X^T k_t and G = dL/dS_t,
 *     dv_t = beta_t G^T k_t,  dbeta_t = (G^T k_t) . w,
 *     dk_t = beta_t (G w - X G^T k_t),  dq_t = S_t dO_t,
 *     dalpha_t = rowsum((G - beta_t k_t k_t^T G) * S_{t-1})  (summed over all
 *     entries with KDA_GATE_HEAD),
 *     dL/dS_{t-1} = Diag(alpha_t) (G - beta_t k_t k_t^T G) + q_{t-1} dO_{t-1}^T.
 * The states are recomputed from S0 (checkpoints in the workspace every 16
 * tokens at d <= 64; at d = 128 every 12 for bf16 inputs, every 8 for fp32
 * ones); nothing from a forward call is needed.
 *   shape, q, k, v, alpha, beta, cu_seqlens, S0  as for kda_prefill
 *                 (input_form must be KDA_INPUT_FINAL, else UNSUPPORTED)
 *   dO            [total_tokens][H][d_v] fp32
 *   dS_T          [N][H][d_k][d_v] fp32, or NULL (zero)
 *   dq, dk        [total_tokens][H][d_k] fp32 outputs
 *   dv            [total_tokens][H][d_v] fp32 output
 *   dalpha        alpha's layout, fp32 output
 *   dbeta         [total_tokens][H] fp32 output
 *   dS0           [N][H][d_k][d_v] fp32 output, or NULL to skip
 *   workspace     256-byte aligned.  kda_backward_workspace_size() gives the
 *                 recommended size: state checkpoints (floor(T/B) + N per
 *                 head, B the checkpoint interval above) and per-16-column
 *                 partial sums of dq, dk, dalpha, dbeta (4 (3 d + 1) (d/16)
 *                 T H bytes at most), linear in T.  A smaller workspace also
 *                 works: every sequence is then cut into pieces of L tokens
 *                 (L a multiple of 48, the largest that fits), a forward
 *                 sweep stores the state at each piece start and the pieces
 *                 run from last to first, handing dL/dS on; it needs the
 *                 piece-start states ((P-1) N H d_k d_v floats for P pieces
 *                 of the longest sequence, total_tokens for varlen), a carry
 *                 of N H d_k d_v floats and the checkpoints and partial sums
 *                 of one piece, and costs one more forward sweep.  The
 *                 results are bit-identical to the one-piece run.
 *                 KDA_ERR_WORKSPACE_TOO_SMALL when not even 48-token pieces
 *                 fit.
 * Outputs must not overlap inputs.  Results are deterministic (the partial
 * sums are added in a fixed order). */
kda_status_t kda_backward_workspace_size(const kda_shape_t *shape, size_t *bytes);
kda_status_t kda_backward(const kda_shape_t *shape,
                          const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta,
                          const int32_t *cu_seqlens, const float *S0,
                          const float *dO, const float *dS_T,
                          float *dq, float *dk, float *dv, float *dalpha, float *dbeta,
                          float *dS0,
                          void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
