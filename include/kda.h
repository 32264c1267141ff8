/*
 * kda.h -- C ABI of libkda: Kimi Delta Attention (KDA) forward on MI355X (gfx950).
 *
 * KDA is the gated delta rule with a per-channel (diagonal) forget gate.  Per
 * (sequence, head) chain the state S is d_k x d_v; for each token t:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * Source: KimiLinear article (intl.cloud.baidu.com), section 2.3 (update with a
 * per-dimension gate vector acting on the rows of the state) and section 2.1
 * (delta-rule erase and write).  The pages print the write term as v k^T; with
 * the gate on rows the state is d_k x d_v and the write is k v^T.  The read-out
 * o_t = S_t^T q_t (inclusive of token t, no scale, no normalisation, no output
 * gate) is not on the pages; it is the reading this library implements.
 * alpha_t = exp(log_alpha_t) is passed in log form.
 *
 * Conventions for every call:
 *  - All tensors are caller-owned DEVICE memory, contiguous and row-major with
 *    the shapes given below; base pointers must be 16-byte aligned, except beta
 *    and cu_seqlens, which need only their natural alignment.  The library never
 *    allocates, frees or retains a pointer, and keeps no global mutable state
 *    apart from the device scratch of kda_chunk_fwd_noalloc.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is
 *    the legacy default stream).  KDA_OK means "validated and enqueued".
 *  - Every argument check runs on the host before any HIP call; on error nothing
 *    is enqueued and no memory is touched.  Device-resident values (cu_seqlens,
 *    tensor contents) are not read by the host and are trusted: see the
 *    preconditions of each call.
 *  - Outputs must not alias inputs, except where a call says otherwise.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, bad size, misalignment */
    KDA_ERR_UNSUPPORTED = 2,      /* d_k or d_v not in {64, 128}, unknown dtype,
                                     or a batch beyond HIP's launch limits (a
                                     grid of 2^32 work-items or more)          */
    KDA_ERR_WORKSPACE = 3,        /* workspace smaller than the size query         */
    KDA_ERR_HIP = 4               /* a HIP launch reported an error                */
} kda_status_t;

/* Element types.  Calls take them as int32_t codes with these values (any
 * other value is refused with KDA_ERR_UNSUPPORTED). */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;

/* Version of this ABI; bumped on any incompatible change. */
int32_t kda_abi_version(void);

/* Static text for a status code (never NULL; "KDA_ERR_UNKNOWN" for any other value). */
const char *kda_status_string(int32_t status);

/* Text of the last KDA_ERR_HIP reported on the calling thread ("" if none). */
const char *kda_last_hip_error(void);

/*
 * Bytes of device workspace kda_chunk_fwd needs for these sizes (0 if none).
 * Arguments as for kda_chunk_fwd; num_seqs is the number of sequences (0 when
 * no cu_seqlens is given).  With fp32 I/O: none at d_k = 64 (one fused kernel);
 * at d_k = 128 the chunkwise fp32 forward keeps per chunk-head its fp32 record
 * (about 148 KiB), the chunk's start state and U (64 KiB and 32 KiB at
 * d_v = 128), and per token-head the input prologue's mapped q, k and log alpha
 * (about 1.5 KiB): about 5.3 KiB per token-head in all, 0 without tokens.
 * With bf16 I/O:
 *  - a packed batch (num_seqs > 0) at d_k = d_v = 128 runs one fused kernel per
 *    (sequence, head): the workspace holds the order in which the sequences
 *    are taken (int32 per sequence, rounded up to 256 bytes);
 *  - an equal-length batch at d_k = d_v = 128 may run either forward (plain KDA
 *    and the scalar gates run two passes, the other input variants the fused
 *    kernel), so the size covers
 *    both: the two-pass records (per chunk and head, the chunk's
 *    state-independent operands, about 1.4 KiB per token-head; a single
 *    sequence longer than 2048 / H chunks runs in segments of that many chunks,
 *    so at most 2048 chunk-heads, about 190 MB, plus an fp32 state of
 *    H x d_k x d_v; at d_k = 128 a single sequence of at least 16 chunks whose
 *    state pass has at most 128 workgroups (H <= 16 at d_v = 128, H <= 32 at
 *    d_v = 64) runs instead in segments of half its chunks, at most 1024
 *    chunk-heads each, with two record buffers and the same fp32 state) and
 *    the fused kernel's segment states (a chain too long for
 *    the parallelism of the GPU is cut into segments: a start state for each
 *    segment but the first, and an end state and a transition for each
 *    segment but the first and the last, d_k x d_v or d_k x d_k fp32 each,
 *    at most 48 MiB in all);
 *  - at d_k or d_v = 64 both kinds of batch run two passes (records as above).
 * The size depends only on the arguments, never on tensor contents.
 */
size_t kda_chunk_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k,
                                    int32_t d_v, int32_t num_seqs, int32_t io_dtype);

/*
 * kda_chunk_fwd -- chunkwise KDA forward over a batch of sequences (prefill).
 *
 * Computes, for every sequence and head, the per-token recurrence above, using
 * the chunkwise parallel form of section 3.1 of the KimiLinear article (chunks
 * of C = 64 tokens: intra-chunk interactions by matrix products, inter-chunk
 * contribution carried by the state) and the specialised DPLR / WY form named
 * in the Kimi Linear abstract (CoChat record): one decay-weighted key Gram block
 * per chunk and a unit-lower-triangular solve.  Results equal the per-token
 * recurrence up to rounding.
 *
 *   q, k        [B, T, H, d_k]  io_dtype
 *   v           [B, T, H, d_v]  io_dtype
 *   log_alpha   [B, T, H, d_k]  gate_dtype; precondition: finite and <= 0
 *   beta        [B, T, H]       gate_dtype; any finite value
 *   h0          [N, H, d_k, d_v] fp32 initial state per sequence, or NULL (zeros)
 *   cu_seqlens  device int32 [N+1] or NULL.  When given, B must be 1 and the
 *               batch is the packed concatenation of N = num_seqs sequences:
 *               sequence n covers tokens [cu_seqlens[n], cu_seqlens[n+1]).
 *               Precondition: cu_seqlens[0] = 0, non-decreasing, last = T.
 *               When NULL, N = B and num_seqs must be B (or 0, meaning B).
 *   o           [B, T, H, d_v]  io_dtype (out)
 *   h_T         [N, H, d_k, d_v] fp32 final state per sequence (out), or NULL.
 *               h_T may alias h0 exactly (same pointer): each sequence's h0 is
 *               read before its h_T is written.  A zero-length sequence gives
 *               h_T = h0 (or zeros).  h_T has the layout of decode's S, so a
 *               prefill can hand its state to kda_decode_step without a copy.
 *   d_k, d_v    each 64 or 128
 *   io_dtype    KDA_BF16 or KDA_F32; gate_dtype likewise
 *   workspace   device scratch of at least kda_chunk_fwd_workspace_size()
 *               bytes (may be NULL when that size is 0), 16-byte aligned,
 *               owned by the caller; its contents on entry do not matter and
 *               on return are unspecified.  Two calls in flight at once on
 *               different streams must not share one workspace.
 *
 * Numerics: the state and every accumulation are fp32.  With bf16 I/O the
 * products of chunk operands run on bf16 matrix cores with hi/lo-split (or
 * power-of-two-scaled fp16) operands where precision needs it; with fp32 I/O
 * they are split bf16 (d_k = 64) or fp32 on the fp32 matrix cores (d_k = 128).
 * o is rounded to io_dtype with round-to-nearest-even.  Accuracy is specified
 * for log_alpha >= -30 per token; smaller values act as a reset.
 * Deterministic: the same inputs give bitwise identical outputs.
 */
kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const void *log_alpha,
                           const void *beta, const float *h0, const int32_t *cu_seqlens,
                           int32_t num_seqs, void *o, float *h_T, int32_t B, int32_t T,
                           int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype,
                           int32_t gate_dtype, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).
 *
 * Arguments, layouts, preconditions and results as for kda_chunk_fwd, without
 * the workspace: the call uses a scratch array of 80 MiB that the library
 * holds on each device it runs on (from the loading of its code object until
 * the process ends; its address is looked up on the first call per device,
 * with that device current).  It never calls hipMalloc, hipFree or any
 * allocating routine.  The scratch is that of the CURRENT device, so `stream`
 * and every tensor must belong to it.
 *
 * With bf16 I/O at d_k = d_v = 128 every batch shape runs the fused kernel
 * (for packed batches and the input variants kda_chunk_fwd runs it too), whose
 * workspace never exceeds the scratch; results agree with kda_chunk_fwd to the
 * accuracy of either, and bitwise for packed batches.  The other calls run
 * the kernels of kda_chunk_fwd (bitwise its results) and are accepted while
 * their workspace (kda_chunk_fwd_workspace_size) fits the scratch: fp32 at
 * d_k = 64 needs none, fp32 at d_k = 128 and bf16 at d_k or d_v = 64 grow with
 * the batch.
 *
 * Errors: as kda_chunk_fwd; KDA_ERR_WORKSPACE when the call would need more
 * than the 80 MiB of scratch (bf16 at d = 64, or fp32 at d_k = 128, with a
 * large batch); KDA_ERR_HIP if the scratch's address cannot be
 * found.  Every call on one device shares that device's scratch and leaves its
 * contents behind (the forward reads none of it before writing it): calls that
 * overlap in time on one device -- on different streams, or from different
 * threads -- race and must not be issued; calls in order on one stream are safe.
 */
kda_status_t kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *log_alpha,
                                   const void *beta, const float *h0, const int32_t *cu_seqlens,
                                   int32_t num_seqs, void *o, float *h_T, int32_t B, int32_t T,
                                   int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype,
                                   int32_t gate_dtype, void *stream);

/*
 * kda_decode_step -- one recurrent KDA step for B resident states (decode).
 *
 * Applies the per-token update once to every (b, h) state in place and writes
 * the read-out: constant work per token with a fixed-size state and no history
 * (KimiLinear article, section 4.2).
 *
 *   q, k        [B, H, d_k]  io_dtype
 *   v           [B, H, d_v]  io_dtype
 *   log_alpha   [B, H, d_k]  gate_dtype; precondition: finite and <= 0
 *   beta        [B, H]       gate_dtype
 *   S           [B, H, d_k, d_v] fp32, read and overwritten in place
 *   o           [B, H, d_v]  io_dtype (out)
 *
 * S is streamed once (one read, one write per element).
 */
kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const void *log_alpha,
                             const void *beta, float *S, void *o, int32_t B, int32_t H,
                             int32_t d_k, int32_t d_v, int32_t io_dtype,
                             int32_t gate_dtype, void *stream);

/*
 * kda_chunk_fwd_prologue -- kda_chunk_fwd on raw projections (fused input
 * prologue).
 *
 * The KimiLinear article, section 3.2, keeps the chunkwise computation stable by
 * normalising the inputs and by constraining and reparameterising the gate
 * values.  This entry point takes the inputs before those maps and applies them
 * inside the kernels as the inputs are read, so no separate pass over q, k and
 * the gates is needed.  Per token and head:
 *
 *   q = q_raw / max(||q_raw||_2, 1e-6),   k likewise          (over d_k)
 *   log_alpha = max(-softplus(gate_pre), log_alpha_min)      (per channel)
 *   beta = sigmoid(beta_pre)
 *
 * then exactly the computation of kda_chunk_fwd.  Arguments, layouts, the
 * workspace (kda_chunk_fwd_workspace_size), ownership and errors are those of
 * kda_chunk_fwd, with q_raw, k_raw in place of q, k (io_dtype), gate_pre in
 * place of log_alpha and beta_pre in place of beta (gate_dtype; any finite
 * values).  log_alpha_min must be finite and <= 0, else
 * KDA_ERR_INVALID_ARGUMENT; the accuracy statement of kda_chunk_fwd applies
 * for log_alpha_min >= -30.
 */
kda_status_t kda_chunk_fwd_prologue(const void *q_raw, const void *k_raw, const void *v,
                                    const void *gate_pre, const void *beta_pre, float log_alpha_min,
                                    const float *h0, const int32_t *cu_seqlens, int32_t num_seqs,
                                    void *o, float *h_T, int32_t B, int32_t T, int32_t H, int32_t d_k,
                                    int32_t d_v, int32_t io_dtype, int32_t gate_dtype,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_decode_step_prologue -- kda_decode_step on raw projections: the maps of
 * kda_chunk_fwd_prologue applied to q_raw, k_raw [B, H, d_k], gate_pre
 * [B, H, d_k] and beta_pre [B, H], then exactly one kda_decode_step.  Same
 * arguments and errors as kda_decode_step; log_alpha_min as for
 * kda_chunk_fwd_prologue.
 */
kda_status_t kda_decode_step_prologue(const void *q_raw, const void *k_raw, const void *v,
                                      const void *gate_pre, const void *beta_pre, float log_alpha_min,
                                      float *S, void *o, int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                                      int32_t io_dtype, int32_t gate_dtype, void *stream);

/*
 * kda_gdn_chunk_fwd -- the scalar-gate members of the family through the same
 * path: Gated DeltaNet, one decay per token and head (KimiLinear article,
 * section 2.2), and DeltaNet, no decay (section 2.1), when log_alpha is NULL.
 * Computes exactly kda_chunk_fwd with every key channel's log_alpha[t, h, c]
 * equal to log_alpha[t, h] (or to 0); the gate is read once per token and head
 * instead of once per channel.  Arguments, workspace and errors as for
 * kda_chunk_fwd except:
 *
 *   log_alpha   [B, T, H] gate_dtype, aligned to its element size; finite and
 *               <= 0; or NULL for no decay
 */
kda_status_t kda_gdn_chunk_fwd(const void *q, const void *k, const void *v, const void *log_alpha,
                               const void *beta, const float *h0, const int32_t *cu_seqlens, int32_t num_seqs,
                               void *o, float *h_T, int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                               int32_t io_dtype, int32_t gate_dtype, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * kda_gdn_decode_step -- kda_decode_step with a scalar gate: log_alpha is
 * [B, H] (aligned to its element size) or NULL for no decay; every key channel
 * of a state decays by the same factor.  Otherwise as kda_decode_step.
 */
kda_status_t kda_gdn_decode_step(const void *q, const void *k, const void *v, const void *log_alpha,
                                 const void *beta, float *S, void *o, int32_t B, int32_t H, int32_t d_k,
                                 int32_t d_v, int32_t io_dtype, int32_t gate_dtype, void *stream);

/*
 * kda_chunk_fwd_decoupled -- KDA with the update strength split into an erase
 * strength b_t and a write strength w_t (per token and head):
 *
 *     S <- (I - b_t k_t k_t^T) Diag(alpha_t) S + w_t k_t v_t^T,   o_t = S^T q_t
 *
 * b_t = w_t = beta_t is kda_chunk_fwd.  The Kimi Linear CoChat record (section
 * "Claims other papers make about this one") cites a follow-up that unties the
 * single beta into erase and write gates; it gives no formula, and this is the
 * scalar reading of it.  Arguments, workspace and errors as for kda_chunk_fwd,
 * with b_erase in place of beta and
 *
 *   w_write     [B, T, H] gate_dtype, aligned to its element size; required
 *               (NULL is KDA_ERR_INVALID_ARGUMENT when there are tokens)
 */
kda_status_t kda_chunk_fwd_decoupled(const void *q, const void *k, const void *v, const void *log_alpha,
                                     const void *b_erase, const void *w_write, const float *h0,
                                     const int32_t *cu_seqlens, int32_t num_seqs, void *o, float *h_T, int32_t B,
                                     int32_t T, int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype,
                                     int32_t gate_dtype, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * kda_decode_step_decoupled -- one decode step of the same update: b_erase and
 * w_write are [B, H] gate_dtype (w_write required); otherwise as
 * kda_decode_step.
 */
kda_status_t kda_decode_step_decoupled(const void *q, const void *k, const void *v, const void *log_alpha,
                                       const void *b_erase, const void *w_write, float *S, void *o, int32_t B,
                                       int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype,
                                       int32_t gate_dtype, void *stream);

/*
 * Bytes of device workspace kda_chunk_bwd needs for these sizes (arguments as
 * for kda_chunk_bwd; 0 for invalid arguments).  The backward keeps, per
 * (chunk, head), in fp32: the chunk's decayed queries and keys, W, the UT
 * inverse, the intra-chunk score and Gram blocks and the decay scales (about
 * 130 KiB at d_k = 128), the state at the chunk's start and the state gradient
 * at its end (d_k x d_v each), and U and dU (64 x d_v each): about 330 KiB per
 * chunk-head at d_k = d_v = 128, i.e. about 5 KiB per token-head (about 11 GB
 * for 65,536 tokens x 32 heads, well inside 288 GB of HBM).  The size depends
 * only on the arguments.
 */
size_t kda_chunk_bwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k,
                                    int32_t d_v, int32_t num_seqs, int32_t io_dtype);

/*
 * kda_chunk_bwd -- gradients of kda_chunk_fwd, for training.
 *
 * The KimiLinear article presents the chunkwise form as what makes training on
 * long sequences efficient (sections 3 and 4.1) and notes that it only keeps a
 * chunk-sized score block per chunk for the backward pass (section 3.2).  The
 * gradient itself is that of the per-token recurrence above: for a scalar loss
 * L whose gradients with respect to o and h_T are grad_o and grad_hT, this
 * computes dL/dq, dL/dk, dL/dv, dL/dlog_alpha, dL/dbeta and dL/dh0.  It runs in
 * chunks of 64 tokens: the state-independent chunk operands in parallel, one
 * forward pass and one reverse pass over the chunks for the states and state
 * gradients at chunk boundaries, then the per-chunk gradients in parallel.
 *
 *   q, k, v, log_alpha, beta, h0, cu_seqlens, num_seqs, B, T, H, d_k, d_v,
 *   io_dtype, gate_dtype    the forward's inputs, as for kda_chunk_fwd
 *   H               at most 65,535 (KDA_ERR_UNSUPPORTED above)
 *   grad_o          [B, T, H, d_v]  io_dtype
 *   grad_hT         [N, H, d_k, d_v] fp32, or NULL (L does not depend on h_T)
 *   grad_q, grad_k  [B, T, H, d_k]  io_dtype (out)
 *   grad_v          [B, T, H, d_v]  io_dtype (out)
 *   grad_log_alpha  [B, T, H, d_k]  gate_dtype (out)
 *   grad_beta       [B, T, H]       gate_dtype (out)
 *   grad_h0         [N, H, d_k, d_v] fp32 (out), or NULL (not wanted); given
 *                   also when h0 is NULL (the gradient at a zero state).  A
 *                   zero-length sequence gives grad_h0 = grad_hT (or zeros).
 *   workspace       at least kda_chunk_bwd_workspace_size() bytes, 16-byte
 *                   aligned, caller-owned; contents on entry do not matter.
 *
 * Outputs must not alias inputs or one another.  Numerics: every product and
 * accumulation is fp32 (fp32 matrix cores); outputs are rounded to their dtype
 * with round-to-nearest-even.  Range: any finite log_alpha <= 0.  A chunk in
 * which some key channel decays by more than about e^-159 in total (sum of
 * log_alpha over the chunk below about -159) is outside the fp32 range of the
 * anchored chunk factors and is computed exactly instead: the decay between
 * each pair of its tokens is formed directly (a factor at most 1), more slowly
 * but to the same accuracy.  Deterministic: no atomics; the same inputs give
 * bitwise identical outputs.
 */
kda_status_t kda_chunk_bwd(const void *q, const void *k, const void *v, const void *log_alpha,
                           const void *beta, const float *h0, const int32_t *cu_seqlens,
                           int32_t num_seqs, const void *grad_o, const float *grad_hT,
                           void *grad_q, void *grad_k, void *grad_v, void *grad_log_alpha,
                           void *grad_beta, float *grad_h0, int32_t B, int32_t T, int32_t H,
                           int32_t d_k, int32_t d_v, int32_t io_dtype,
                           int32_t gate_dtype, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * Bytes of device workspace kda_chunk_bwd_prologue needs (arguments as for
 * kda_chunk_bwd_workspace_size; 0 for invalid arguments): that of
 * kda_chunk_bwd plus six fp32 [B*T*H, d_k] buffers and four fp32 [B*T*H]
 * buffers (about 3 KiB more per token-head at d_k = 128).
 */
size_t kda_chunk_bwd_prologue_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k,
                                             int32_t d_v, int32_t num_seqs, int32_t io_dtype);

/*
 * kda_chunk_bwd_prologue -- gradients of kda_chunk_fwd_prologue with respect
 * to its raw inputs.  The maps of the input prologue are applied in a pass of
 * their own into fp32 workspace buffers (q/max(||q||, eps), k likewise,
 * max(-softplus(gate_pre), log_alpha_min), sigmoid(beta_pre)); the gradients
 * of kda_chunk_bwd are taken at those fp32 values; a last pass applies the
 * chain rule back through the maps:
 *     grad_q_raw = (dq_hat - q_hat (q_hat . dq_hat)) / ||q||   (dq_hat / eps when ||q|| <= eps),
 *     grad_gate_pre = -sigmoid(gate_pre) dlog_alpha where the floor does not bind, else 0,
 *     grad_beta_pre = beta (1 - beta) dbeta.
 * Arguments, numerics, range and errors as for kda_chunk_bwd, with the raw
 * inputs and log_alpha_min as for kda_chunk_fwd_prologue, the gradients of the
 * raw inputs in place of those of q, k, log_alpha, beta (same layouts and
 * dtypes), and a workspace of kda_chunk_bwd_prologue_workspace_size() bytes.
 */
kda_status_t kda_chunk_bwd_prologue(const void *q_raw, const void *k_raw, const void *v,
                                    const void *gate_pre, const void *beta_pre, float log_alpha_min,
                                    const float *h0, const int32_t *cu_seqlens, int32_t num_seqs,
                                    const void *grad_o, const float *grad_hT, void *grad_q_raw,
                                    void *grad_k_raw, void *grad_v, void *grad_gate_pre,
                                    void *grad_beta_pre, float *grad_h0, int32_t B, int32_t T,
                                    int32_t H, int32_t d_k, int32_t d_v, int32_t io_dtype,
                                    int32_t gate_dtype, void *workspace, size_t workspace_bytes,
                                    void *stream);

/*
 * kda_chunk_bwd_decoupled -- gradients of kda_chunk_fwd_decoupled (separate
 * erase strength b and write strength w per token and head):
 *
 *     S <- (I - b_t k_t k_t^T) Diag(alpha_t) S + w_t k_t v_t^T,   o_t = S^T q_t
 *
 * For a scalar loss with gradients grad_o, grad_hT as for kda_chunk_bwd, this
 * computes dL/dq, dL/dk, dL/dv, dL/dlog_alpha, dL/db, dL/dw and dL/dh0 in the
 * same kernels: the erase strength enters the triangular system and the
 * erase term, the write strength the written values.  Arguments, workspace
 * (kda_chunk_bwd_workspace_size), numerics, range and errors as for
 * kda_chunk_bwd, with b_erase in place of beta and
 *
 *   w_write        [B, T, H] gate_dtype, aligned to its element size; required
 *   grad_b_erase   [B, T, H] gate_dtype (out), in place of grad_beta
 *   grad_w_write   [B, T, H] gate_dtype (out), aligned to its element size; required
 *
 * With w_write equal to b_erase, grad_b_erase + grad_w_write is kda_chunk_bwd's
 * grad_beta (each part rounded on its own).
 */
kda_status_t kda_chunk_bwd_decoupled(const void *q, const void *k, const void *v, const void *log_alpha,
                                     const void *b_erase, const void *w_write, const float *h0,
                                     const int32_t *cu_seqlens, int32_t num_seqs, const void *grad_o,
                                     const float *grad_hT, void *grad_q, void *grad_k, void *grad_v,
                                     void *grad_log_alpha, void *grad_b_erase, void *grad_w_write,
                                     float *grad_h0, int32_t B, int32_t T, int32_t H, int32_t d_k,
                                     int32_t d_v, int32_t io_dtype, int32_t gate_dtype,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace kda_gdn_chunk_bwd needs (arguments as for
 * kda_chunk_bwd_workspace_size; 0 for invalid arguments): the same as
 * kda_chunk_bwd's.
 */
size_t kda_gdn_chunk_bwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k,
                                        int32_t d_v, int32_t num_seqs, int32_t io_dtype);

/*
 * kda_gdn_chunk_bwd -- gradients of kda_gdn_chunk_fwd: Gated DeltaNet (one
 * decay per token and head, KimiLinear article section 2.2) or DeltaNet (no
 * decay, section 2.1) when log_alpha is NULL.  The scalar gate is the
 * per-channel gate of kda_chunk_bwd with every channel equal to it, so by the
 * chain rule its gradient is the sum over the key channels of the per-channel
 * gradient; the kernels of kda_chunk_bwd read the gate once per (token, head)
 * and take that sum per (token, head) in a fixed order.  Arguments, workspace,
 * numerics, range and errors as for kda_chunk_bwd except:
 *
 *   log_alpha       [B, T, H] gate_dtype, aligned to its element size; or NULL
 *                   for no decay
 *   grad_log_alpha  [B, T, H] gate_dtype (out), aligned to its element size;
 *                   required when log_alpha is given, ignored when it is NULL
 *   workspace       at least kda_gdn_chunk_bwd_workspace_size() bytes
 */
kda_status_t kda_gdn_chunk_bwd(const void *q, const void *k, const void *v, const void *log_alpha,
                               const void *beta, const float *h0, const int32_t *cu_seqlens,
                               int32_t num_seqs, const void *grad_o, const float *grad_hT,
                               void *grad_q, void *grad_k, void *grad_v, void *grad_log_alpha,
                               void *grad_beta, float *grad_h0, int32_t B, int32_t T, int32_t H,
                               int32_t d_k, int32_t d_v, int32_t io_dtype,
                               int32_t gate_dtype, void *workspace, size_t workspace_bytes,
                               void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
