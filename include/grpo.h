/*
 * grpo.h - C ABI of the MI355X (gfx950) chunked GRPO log-probability and loss library.
 *
 * The library computes, from a model's final hidden states H[T, D] and the lm_head
 * weight W[V, D], the per-token log-probability of each target token, the GRPO
 * per-token objective and its gradient with respect to H, chunk by chunk over the
 * flattened token stream, so that the [T, V] logit tensor never exists in memory.
 *
 * Sources (page titles as printed on the pages):
 *  [P4] "Reinforcement Learning GRPO mit 7x laengerem Kontext" (Unsloth docs):
 *       section "Chunking der abgeflachten Sequenzlaenge" (Eq. 1-3: the batch and
 *       context axes are flattened and cut into chunks, logit memory bounded by one
 *       chunk), the call of chunked_hidden_states_selective_log_softmax (hidden
 *       states, lm_head, completion ids, temperature; chunked logits upcast to
 *       float32), and section "Auslagern von Aktivierungen fuer Log-Softmax" (the
 *       forward keeps no logits; the backward recomputes the chunk and
 *       back-propagates the incoming gradient).
 *  [P2] "Unsloth internals", section "The relationship to TRL": group-relative
 *       advantages, clipped surrogate objective, KL-to-reference term.
 *  [P3] "You can now train reasoning models with 5GB VRAM thanks to Unsloth",
 *       section "Under the Hood": reverse KL; ratio exp(q - q_old) times the
 *       advantage broadcast over the tokens of a sequence.
 *  [P1] "Unsloth GRPO Implementation: How It Accelerates Reinforcement Learning
 *       Training", section "Corrected Hyperparameters for GRPO Stability":
 *       beta = 0.001.
 *  [P2] also describes the fused, chunked cross-entropy that the same chunked
 *       log-softmax serves for supervised fine-tuning.
 *
 * Conventions shared by every entry point:
 *  - Pointers are device pointers unless marked [host].  `stream` is a
 *    hipStream_t passed as void* (NULL = the null stream).  Every call only
 *    enqueues work on `stream`; none synchronizes the host (except the timer
 *    read-out and grpo_offload_destroy), none allocates device memory, and none keeps a
 *    pointer after it returns ([host] arrays are read during the call, into kernel
 *    arguments; the pinned H_host of the offload calls is the exception: the GPU's copies
 *    read or write it asynchronously, like device memory, so it lives until their work is done).
 *    The caller owns every buffer, including the workspace.
 *  - Row-major layouts: H[T, D], W[V, D] (the nn.Linear [out, in] layout), dH[T, D].
 *    Row t of H predicts targets[t]; the caller applies any causal shift.
 *  - Sequences are contiguous runs of the flattened stream given by cu_seqlens;
 *    groups are consecutive runs of `group_size` sequences (prompt-major).
 *  - Every host-checkable error is reported before anything is enqueued and leaves
 *    every output untouched.  A failed launch returns GRPO_E_HIP.
 *  - A target outside [0, V) yields NaN logp / token_loss for that token (and a
 *    NaN loss if its weight is non-zero), a zero dH row, and no out-of-bounds access.
 *  - Calls keep no global state and may run concurrently on different streams with
 *    different workspaces; grpo_loss_fwd_bwd_static is the exception (its workspace is one
 *    array per device, see there).
 */
#ifndef GRPO_MI355X_H
#define GRPO_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GRPO_OK = 0,
  GRPO_E_NULL = 1,        /* a required pointer is NULL */
  GRPO_E_SHAPE = 2,       /* a size is out of range or cu_seqlens is inconsistent */
  GRPO_E_VALUE = 3,       /* a scalar is out of range or not finite */
  GRPO_E_WORKSPACE = 4,   /* workspace missing, too small or misaligned */
  GRPO_E_UNSUPPORTED = 5, /* dtype, alignment or divisibility this build does not handle */
  GRPO_E_HIP = 6,         /* the HIP runtime reported an error */
  GRPO_E_SCRATCH = 7      /* the call needs more than grpo_loss_fwd_bwd_static's static scratch */
} grpo_status;

typedef enum { GRPO_BF16 = 0, GRPO_F32 = 1 } grpo_dtype;            /* element type of H, W, dH */
typedef enum { GRPO_AGG_SEQ_MEAN = 0, GRPO_AGG_TOKEN_MEAN = 1 } grpo_agg;
typedef enum { GRPO_STD_UNBIASED = 0, GRPO_STD_POPULATION = 1 } grpo_std;

/* Problem shape.  T >= 0 tokens, D >= 1 hidden size (multiple of 8 for bf16, of 4 for
 * fp32, at most 2^20), V >= 1 vocabulary size, chunk_tokens >= 1 tokens per chunk.  T, V
 * and chunk_tokens are below 2^31.
 * Logits ([P4], the arguments of the chunked call: logit_scale_multiply,
 * logit_scale_divide, logit_softcapping, temperature; item 3 after it): with
 * x = H[t] . W[v] and s = logit_scale_multiply / logit_scale_divide,
 *   z = s x / temperature                                (logit_softcapping == 0)
 *   z = c tanh(s x / c) / temperature,  c = logit_softcapping  (> 0).
 * temperature > 0 and finite; the three logit arguments are finite and >= 0, and 0 means
 * "not used" (a factor of 1, no cap), so a zero-initialized tail gives plain logits.
 * keep_chunk_logits (0 or 1; bf16 only) selects how the loss calls (grpo_loss_fwd_bwd,
 * grpo_ce_loss_fwd_bwd) form the probabilities of their backward: 0, the pages' method
 * ([P4] "Auslagern von Aktivierungen fuer Log-Softmax"), recomputes the chunk's logits with
 * a second GEMM; 1 keeps them from the forward GEMM, as d = z - (max over a 256-entry
 * vocabulary tile) in fp16, in the buffer the probabilities occupy anyway (no extra
 * memory), and turns them into probabilities in place: 4 D V instead of 6 D V flop per
 * token.  logp, token_loss and the loss are bitwise the same either way; dH differs by the
 * fp16 rounding of d (relative error at most 2^-11 |d| per probability).
 * dh_fp32 (0 or 1) selects dH's element type for bf16 inputs: 0 writes dH as bf16 (rounded to
 * nearest even, a relative error of up to 2^-9 per element), from probabilities rounded to
 * bf16; 1 writes it as fp32 and keeps each entry of the backward's P - onehot as a bf16 pair
 * hi + lo (lo = the rounding residual of hi, about 16 significant bits together), read by a
 * dH GEMM twice as long over the vocabulary: per-row relative error ~1e-5 instead of ~1e-3.
 * fp32 inputs always give fp32 dH (dh_fp32 is ignored). */
typedef struct {
  int64_t T;
  int64_t D;
  int64_t V;
  int64_t chunk_tokens;
  int32_t dtype;       /* grpo_dtype */
  float temperature;
  float logit_scale_multiply;
  float logit_scale_divide;
  float logit_softcapping;
  int32_t keep_chunk_logits;
  int32_t dh_fp32;     /* 0 or 1: dH is written as fp32 [T, D] for bf16 inputs (see below) */
} grpo_shape;

/* GRPO objective parameters ([P2], [P3], [P1]).  The ratio is clipped to
 * [1 - clip_eps_low, 1 + clip_eps_high]; 0 <= clip_eps_low < 1, clip_eps_high >= 0;
 * beta >= 0 weights the k3 reverse-KL term; agg is a grpo_agg. */
typedef struct {
  float clip_eps_low;
  float clip_eps_high;
  float beta;
  int32_t agg;
} grpo_loss_params;

/* Kernel classes that a grpo_timer can time (events around each launch). */
typedef enum {
  GRPO_K_TARGET_LOGIT = 0, /* z[t, y_t] by a row dot product */
  GRPO_K_LOGITS_LSE = 1,   /* MFMA logits GEMM with online max / sum-exp epilogue */
  GRPO_K_MERGE = 2,        /* merge of the vocabulary tiles' partials; GRPO per-token terms */
  GRPO_K_PROBS = 3,        /* recompute GEMM writing softmax probabilities */
  GRPO_K_DH_GEMM = 4,      /* MFMA GEMM dH = (g/tau) (W[y] - P W) */
  GRPO_K_DH_REDUCE = 5,    /* fixed-order sum of split-vocabulary dH partials */
  GRPO_K_TOKEN_INDEX = 6,  /* sequence index, per-sequence token counts and weights */
  GRPO_K_LOSS_FINALIZE = 7,/* fixed-order fp64 sum of the per-token loss terms */
  GRPO_K_ADVANTAGES = 8,
  GRPO_K_FRAG_COPY = 9,    /* fragment-major copy of a chunk's hidden states (bf16 path) */
  GRPO_K_TRANSPOSE_W = 10, /* fragment-major W^T for the dH GEMM (bf16, when it fits) */
  GRPO_K_PROBS_KEPT = 11,  /* probabilities from the kept logits, in place (keep_chunk_logits) */
  GRPO_K_ONEHOT_FIX = 12,  /* exact target entries of the backward's P' - onehot matrix */
  GRPO_K_HT_COPY = 13,     /* tokens' operand of the dW GEMM (bf16, when dW is requested) */
  GRPO_K_DW_GEMM = 14,     /* MFMA GEMM dW (+)= Gx^T H per chunk */
  GRPO_K_W_COPY = 15,      /* fragment-major W for the logits GEMMs (bf16, when it fits) */
  GRPO_K_QT_BAND = 16,     /* one vocabulary band of the dW GEMM's operand (P' - onehot)^T (bf16) */
  GRPO_K_COUNT = 17
} grpo_kernel_id;

typedef struct grpo_timer grpo_timer; /* opaque, owned by the caller */

/* with_backward flag of grpo_workspace_bytes / grpo_plan_info: the backward reads H from
 * pinned host memory (grpo_logp_bwd_offload), with 1 (no dW) or 2 (dW). */
#define GRPO_WS_HOST_H 4

/* Bytes of workspace that grpo_logp_fwd (with_backward = 0), the backward entry points
 * (with_backward = 1) or the backward entry points given a dW output (with_backward = 2)
 * need for this shape and num_seqs sequences; 1 | GRPO_WS_HOST_H and 2 | GRPO_WS_HOST_H:
 * grpo_logp_bwd_offload, whose workspace also holds two buffers of chunk_tokens rows of H.
 * Returns 0 for an invalid shape or with_backward.  Bounded by chunk_tokens * V * 4 (one chunk's fp32 logits) plus
 * O(T + chunk_tokens * (V / 128 + D)) bytes of per-token state.  For bf16 the workspace
 * may also hold fragment-major copies of W^T (for the dH GEMM) and of W (for the logits
 * GEMMs), about D * V * 2 bytes each, and the backward may run over slices of a chunk's
 * tokens (not with dW): the library takes the largest of these layouts that keeps the
 * total within chunk_tokens * V * 4 (grpo_plan_info reports the choice).  With dh_fp32 the
 * probabilities take two bf16 halves (twice the room), and the backward runs in token slices
 * without the copies when nothing else fits.  Without room for the whole W^T copy (bf16, no
 * dh_fp32, no dW, chunks of at least 2048 tokens) the rest of the bound holds one band of it:
 * each backward pass transposes W band by band of the vocabulary into that room, and the dH
 * GEMM accumulates over the bands. */
size_t grpo_workspace_bytes(const grpo_shape* shape, int64_t num_seqs, int with_backward);

/* The workspace layout behind grpo_workspace_bytes for the same arguments (host only, no
 * HIP call): info[0] = how the dH GEMM reads W^T: 0 transposing W tiles in registers, 1 from a
 * fragment-major copy made once per call, n >= 2 from n vocabulary bands of that copy made in
 * each backward pass (consecutive passes walk the bands in opposite orders and reuse the band
 * that is already in place); info[1] = 1 if
 * the logits GEMMs read a fragment-major copy of W, info[2] = tokens per backward slice
 * (>= the chunk's tokens when the backward of a chunk runs in one pass; 0 without the
 * backward), info[3] = workspace bytes.  GRPO_E_NULL if info is NULL, GRPO_E_VALUE for an
 * invalid with_backward; the shape errors of grpo_workspace_bytes otherwise (info untouched). */
grpo_status grpo_plan_info(const grpo_shape* shape, int64_t num_seqs, int with_backward, int64_t info[4]);

/* Per-token log-probabilities of the targets ([P4]: chunked hidden-state selective
 * log-softmax): logp[t] = z[t, y_t] - logsumexp_v z[t, v], z = H W^T / temperature,
 * fp32 accumulation of bf16 (or fp32) products.
 *   H [T, D], W [V, D] of shape->dtype, 16-byte aligned; targets int32 [T];
 *   logp fp32 [T] (written); lse fp32 [T] (written when not NULL);
 *   workspace of grpo_workspace_bytes(shape, 1, 0) bytes, 256-byte aligned;
 *   timer may be NULL.
 * logp is bitwise independent of chunk_tokens and equal to the logp that
 * grpo_loss_fwd_bwd computes for the same inputs. */
grpo_status grpo_logp_fwd(const grpo_shape* shape, const void* H, const void* W,
                          const int32_t* targets, float* logp, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream, grpo_timer* timer);

/* Group-relative advantages ([P2]): for group k = sequences [k G, (k + 1) G),
 * adv[i] = (r_i - mean) / (std + eps), std unbiased or population per std_mode;
 * a group of size 1, or whose rewards are all equal, gets 0.  Computed in fp64.
 *   rewards fp32 [num_seqs]; adv fp32 [num_seqs] (written).
 * num_seqs must be a positive multiple of group_size; eps >= 0 and finite. */
grpo_status grpo_advantages(const float* rewards, int64_t num_seqs, int64_t group_size,
                            int32_t std_mode, float eps, float* adv, void* stream);

/* GRPO loss over the flattened stream and its gradient with respect to H
 * ([P2], [P3], [P4] "Auslagern von Aktivierungen fuer Log-Softmax"):
 *   rho_t  = exp(logp_t - old_logp_t)
 *   surr_t = min(rho_t A_s(t), clip(rho_t, 1 - eps_low, 1 + eps_high) A_s(t))
 *   d_t    = ref_logp_t - logp_t,  k3_t = exp(d_t) - d_t - 1
 *   l_t    = -(surr_t - beta k3_t)
 *   loss   = sum_t w_t l_t   with w_t = mask_t / (S * L_s(t)) (seq mean; L_i = unmasked
 *            tokens of sequence i) or w_t = mask_t / sum(mask) (token mean)
 *   dH_t   = g_t (z'_t,y W[y_t] - sum_v softmax(z_t)_v z'_t,v W[v]),  z' = dz/dx
 *            (= s / temperature without a softcap),
 *            g_t = w_t (-(rho A if rho A <= clip(rho) A else 0) + beta (1 - exp(d_t)))
 * Arguments:
 *   cu_seqlens [host] int32 [num_seqs + 1]: cu[0] = 0, non-decreasing, cu[S] = T.
 *   mask uint8 [T] (NULL = every token counts); old_logp, ref_logp fp32 [T]
 *   (ref_logp may be NULL only when beta == 0); adv fp32 [num_seqs].
 *   loss fp64 [1] (written); logp, token_loss fp32 [T] (written when not NULL;
 *   token_loss holds l_t, unweighted); dH [T, D] of shape->dtype (fp32 with dh_fp32) (overwritten;
 *   masked tokens get +0 rows); dW fp32 [V, D], 16-byte aligned (NULL = not computed;
 *   bf16 only; else GRPO_E_UNSUPPORTED): the
 *   gradient with respect to W, dW = sum_t (dL/dx_t)^T H_t with x_t = H_t W^T, overwritten
 *   (accumulated over the chunks in fixed order; for a full fine-tune, where the lm_head is
 *   trained: under LoRA it is frozen), one more 2 D V flop GEMM per token;
 *   workspace of grpo_workspace_bytes(shape, S, 1) bytes (S, 2 with dW).
 * The loss is summed in fp64 in a fixed token order, so it is bitwise independent
 * of chunk_tokens, as are logp and token_loss. */
grpo_status grpo_loss_fwd_bwd(const grpo_shape* shape, const grpo_loss_params* params,
                              const void* H, const void* W, const int32_t* targets,
                              const int32_t* cu_seqlens, int64_t num_seqs, const uint8_t* mask,
                              const float* old_logp, const float* ref_logp, const float* adv,
                              double* loss, float* logp, float* token_loss, void* dH, float* dW,
                              void* workspace, size_t workspace_bytes, void* stream,
                              grpo_timer* timer);

/* grpo_loss_fwd_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments and
 * results, without the workspace.  The call uses a workspace array compiled into the library,
 * one copy per device, GRPO_STATIC_SCRATCH_BYTES (256 MiB) each, held from the library's load
 * until the process ends; it calls no hipMalloc, hipFree or allocating routine.
 *   The call must fit: grpo_workspace_bytes(shape, num_seqs, 1) (2 with dW) <= 256 MiB, else
 *   GRPO_E_SCRATCH before anything is enqueued (e.g. the Qwen3-8B shape, V = 151936, fits with
 *   chunk_tokens = 256, not with 8192).
 *   The current device must be the device of `stream` and of the buffers.
 *   Every call on one device shares that device's array: calls that overlap in time on one
 *   device (different streams, or host threads) race and give undefined results; calls
 *   queued on one stream are ordered and safe.  Nothing in the array needs to start at zero.
 *   The first call on a device looks the array's device address up (hipGetSymbolAddress) and
 *   keeps it; that lookup is the only HIP call besides the launches and hipGetDevice. */
#define GRPO_STATIC_SCRATCH_BYTES ((size_t)256 << 20)
grpo_status grpo_loss_fwd_bwd_static(const grpo_shape* shape, const grpo_loss_params* params,
                                     const void* H, const void* W, const int32_t* targets,
                                     const int32_t* cu_seqlens, int64_t num_seqs, const uint8_t* mask,
                                     const float* old_logp, const float* ref_logp, const float* adv,
                                     double* loss, float* logp, float* token_loss, void* dH, float* dW,
                                     void* stream, grpo_timer* timer);

/* Backward of grpo_logp_fwd ([P4] "Auslagern von Aktivierungen fuer Log-Softmax": the
 * forward keeps only the per-token log-sum-exp; the backward recomputes each chunk's logits
 * and applies the incoming gradient of the log-probabilities):
 *   dH_t = grad_logp_t (z'_t,y W[y_t] - sum_v softmax(z_t)_v z'_t,v W[v]),  z' = dz/dx,
 * the gradient of sum_t grad_logp_t * logp_t with respect to H.  Any loss written on top of
 * the log-probabilities (other GRPO variants, other aggregations) back-propagates through it.
 *   H, W, targets, shape as for grpo_logp_fwd; lse fp32 [T]: the log-sum-exp grpo_logp_fwd
 *   returned for the same H, W and temperature; grad_logp fp32 [T] (dL/dlogp; 0 for tokens
 *   that do not contribute); dH [T, D] of shape->dtype (fp32 with dh_fp32) (overwritten; +0 rows where
 *   grad_logp is 0 or the target is outside [0, V)); dW fp32 [V, D] as for
 *   grpo_loss_fwd_bwd (NULL = not computed); workspace of grpo_workspace_bytes(shape, 1, 1)
 *   bytes (1, 2 with dW). */
grpo_status grpo_logp_bwd(const grpo_shape* shape, const void* H, const void* W, const int32_t* targets,
                          const float* lse, const float* grad_logp, void* dH, float* dW,
                          void* workspace, size_t workspace_bytes, void* stream, grpo_timer* timer);

/* Host offload of the hidden states that the split forward / backward keeps ([P4]
 * "Auslagern von Aktivierungen fuer Log-Softmax": the activations of the chunked log-softmax
 * are moved off the GPU outside the model's forward, and the hint there: this pays only when
 * the hidden states are processed in pieces, as here, chunk by chunk).  grpo_logp_fwd_offload
 * copies H into pinned host memory while its logits GEMMs run; grpo_logp_bwd_offload reads H
 * back from there one chunk at a time, so the backward holds two chunks of H on the GPU
 * instead of all of it.  The copies run on a stream of the offload context, ordered against
 * `stream` by its events; a context serves one call at a time.
 *   grpo_offload_create: a copy stream (default priority) and events on the current device;
 *     *out owned by the caller.  grpo_offload_destroy: waits for the context's copies, then
 *     releases it (GRPO_E_NULL for NULL); the caller first lets the work of the calls that used
 *     it complete (the events they recorded on their streams belong to the context). */
typedef struct grpo_offload grpo_offload; /* opaque, owned by the caller */
grpo_status grpo_offload_create(grpo_offload** out);
grpo_status grpo_offload_destroy(grpo_offload* offload);

/* grpo_logp_fwd, and H [T, D] copied to H_host [host, pinned: hipHostMalloc or equivalent,
 * T * D elements of shape->dtype] on the context's copy stream, which starts after the work
 * enqueued on `stream` before this call (that produced H) and runs beside the call's GEMMs;
 * `stream` then waits for the copy, so H_host is complete when the call's work on `stream` is
 * (H may be freed after that).  offload: a context of grpo_offload_create (GRPO_E_NULL if
 * NULL).  GRPO_E_VALUE if H_host is not pinned host memory. */
grpo_status grpo_logp_fwd_offload(const grpo_shape* shape, const void* H, const void* W,
                                  const int32_t* targets, float* logp, float* lse, void* H_host,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  grpo_timer* timer, grpo_offload* offload);

/* grpo_logp_bwd with H in pinned host memory: before each chunk's backward its rows are copied
 * into one of two workspace buffers on the context's copy stream (the next chunk's copy runs
 * while this chunk's GEMMs read the other buffer); results bitwise equal to grpo_logp_bwd's.
 *   H_host [host, pinned] [T, D] of shape->dtype; the rest as for grpo_logp_bwd; workspace of
 *   grpo_workspace_bytes(shape, 1, 1 | GRPO_WS_HOST_H) bytes (2 | GRPO_WS_HOST_H with dW);
 *   offload as for grpo_logp_fwd_offload.  GRPO_E_VALUE if H_host is not pinned host memory. */
grpo_status grpo_logp_bwd_offload(const grpo_shape* shape, const void* H_host, const void* W,
                                  const int32_t* targets, const float* lse, const float* grad_logp,
                                  void* dH, float* dW, void* workspace, size_t workspace_bytes,
                                  void* stream, grpo_timer* timer, grpo_offload* offload);

/* Chunked cross-entropy, forward and backward ([P2] "Unsloth internals", the fused, chunked
 * cross-entropy: the loss over the vocabulary without the [T, V] logits or their gradient):
 *   loss = -(1/N) sum_t mask_t logp_t,  N = sum_t mask_t  (loss = 0 and dH = 0 when N = 0),
 *   dH   = the grpo_logp_bwd of g_t = -mask_t / N.
 *   mask uint8 [T] (NULL = every token counts); loss fp64 [1] (written, summed in fp64 in a
 *   fixed token order); logp, token_loss fp32 [T] (written when not NULL; token_loss holds
 *   -logp_t); dH [T, D] of shape->dtype (fp32 with dh_fp32) (overwritten); dW fp32 [V, D] as for
 *   grpo_loss_fwd_bwd (NULL = not computed); workspace of grpo_workspace_bytes(shape, 1, 1)
 *   bytes (1, 2 with dW).  A counted token whose target is outside [0, V)
 *   makes the loss NaN; its dH row is +0. */
grpo_status grpo_ce_loss_fwd_bwd(const grpo_shape* shape, const void* H, const void* W,
                                 const int32_t* targets, const uint8_t* mask, double* loss,
                                 float* logp, float* token_loss, void* dH, float* dW,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 grpo_timer* timer);

/* Human-readable name of a status code (static storage). */
const char* grpo_status_string(grpo_status status);

/* Test hook: the per-token sequence id, chunk id (t / chunk_tokens) and position within
 * the sequence, exactly as the loss kernels derive them.  cu_seqlens [host] as for
 * grpo_loss_fwd_bwd; seq_id, chunk_id, pos int32 [T] device outputs; the workspace
 * needs (num_seqs + 1) * 4 bytes rounded up to 256. */
grpo_status grpo_debug_token_index(const int32_t* cu_seqlens, int64_t num_seqs, int64_t T,
                                   int64_t chunk_tokens, int32_t* seq_id, int32_t* chunk_id,
                                   int32_t* pos, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Kernel timing for measurement.  A timer holds `capacity` event pairs; a call that
 * receives a timer records an event pair around every kernel launch it makes until
 * the timer is full (launches beyond capacity are counted in `dropped`).
 * grpo_timer_read waits for the recorded events and returns the summed duration and
 * launch count of one kernel class.  Timers are not thread-safe. */
grpo_status grpo_timer_create(int32_t capacity, grpo_timer** out);
grpo_status grpo_timer_destroy(grpo_timer* timer);
grpo_status grpo_timer_reset(grpo_timer* timer);
grpo_status grpo_timer_read(grpo_timer* timer, int32_t kernel_id, double* total_ms,
                            int64_t* launches, int64_t* dropped);

/* Library version string. */
const char* grpo_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GRPO_MI355X_H */
