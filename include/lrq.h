/*
 * lrq.h -- C ABI of liblrq: the fused attention-input projection of a LoRA-adapted
 * transformer layer, on AMD Instinct MI355X (gfx950).
 *
 *   out = RoPE( W_qkv . h + b + (alpha / r) . B (A . h) ),   h = RMSNorm(x) . gamma
 *
 * for every token row of x, computed in one pass per token tile: neither the
 * normalised activations h nor the rank-r intermediate A . h is written to memory.
 *
 * Where the operation is defined (web pages on Liger-Kernel, cited by title and section):
 *  - RMSNorm (mean of squares over the hidden size, eps inside the square root, then
 *    times the norm weight) and the projection with bias before the rotary step:
 *    "Liger-Kernel底层优化：新一代内核级推理加速引擎深度解析", fused-kernel pseudocode,
 *    Step 1 (RMSNorm) and Step 2 (QKV Projection).
 *  - The chain normalise -> project to q, k, v -> rotate q and k (v is not rotated), which
 *    the fused kernel replaces: "Swift-All一文详解：如何用Liger-Kernel提升训练效率",
 *    section 2.2 (1), RMSNorm + Rotary Embedding + Attention QKV fusion.
 *  - LoRA: frozen projection plus up(down(x)), with down A [r, d_in] and up B [d_out, r]:
 *    "Liger-Kernel内核级优化：GPU利用率飙升至90%以上", section on why conventional
 *    fine-tuning stalls (the y = Wx + B(Ax) formula and its unfused two-step form);
 *    rank r, alpha and the q/k/v target modules are the LoRA configuration fields shown
 *    on the same pages.  The scale alpha / r is the standard LoRA scale (the formula on the
 *    pages prints none).
 *  - RoPE: rotate-half (GPT-NeoX) pairing -- the pseudocode's frequency index is the
 *    feature index modulo head_dim / 2 -- with omega_i = theta^(-2i/D), i < D/2, angle
 *    pos * omega_i, pair (y[i], y[i + D/2]) -> (a cos - b sin, b cos + a sin).  The rest of
 *    that pseudocode's rotation (it pairs k with v) is not used.
 *  - Backward with recomputation instead of stored activations: "Liger-Kernel内核级优化",
 *    system architecture and workflow section (backward also fused, with recompute).
 *
 * Layouts (all row-major, dense):
 *   x, dx      [T, d]            activations (dtype)
 *   gamma      [d]               RMSNorm weight (dtype)
 *   w_qkv      [N, d]            N = (Hq + 2 Hkv) * D; rows are the q heads, then the k heads,
 *                                then the v heads; each head's D rows are contiguous
 *   bias       [N]               optional (dtype)
 *   lora_a[t]  [r, d]            down projection of target t (t = 0 q, 1 k, 2 v)
 *   lora_b[t]  [N_t, r]          up projection; N_q = Hq * D, N_k = N_v = Hkv * D
 *   positions  [T] int32         absolute RoPE position of each token, >= 0
 *   out, y, dy [T, N]            q | k | v column blocks
 *   d_lora_a[t] [r, d], d_lora_b[t] [N_t, r]   float32 gradients
 * Every array pointer must be 16-byte aligned.
 *
 * Ownership: every pointer is a device pointer owned by the caller; the library keeps no
 * reference after a call returns.  Work is enqueued asynchronously on `stream` (a
 * hipStream_t; NULL = the null stream) and nothing is synchronised.  The library allocates
 * no device memory; scratch space is the caller's `workspace` of at least
 * lrq_workspace_size() bytes, 256-byte aligned (LRQ_ERR_UNSUPPORTED otherwise), used only
 * until the enqueued work ends; its contents before a call do not matter.
 * Calls that share a workspace must be ordered on one stream.
 *
 * Errors: every entry point validates its arguments on the host before enqueuing
 * anything; on error nothing is launched and a message is kept for lrq_last_error()
 * (per thread).
 *   LRQ_ERR_INVALID_ARG  malformed descriptor or a required pointer is NULL (see below)
 *   LRQ_ERR_UNSUPPORTED  well-formed but outside what the kernels cover (alignment,
 *                        rank > LRQ_MAX_LORA_RANK, a forced variant that cannot run)
 *   LRQ_ERR_HIP          a HIP call failed (message holds the HIP error string)
 * Positions are not range-checked on the device; a negative position is rotated by a
 * negative angle.
 */
#ifndef LRQ_H_
#define LRQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LRQ_ABI_VERSION 5
#define LRQ_MAX_LORA_RANK 64

typedef enum lrq_status {
  LRQ_OK = 0,
  LRQ_ERR_INVALID_ARG = 1,
  LRQ_ERR_UNSUPPORTED = 2,
  LRQ_ERR_HIP = 3
} lrq_status;

/* Element type of x, gamma, w_qkv, bias, lora_a, lora_b, out, y, dy and dx.  Arithmetic
 * is float32 throughout for LRQ_F32; for LRQ_BF16 the matrix products take bfloat16
 * operands with float32 accumulation, and the row statistics, bias, LoRA scale and
 * rotation are applied in float32 before one round-to-nearest-even store. */
typedef enum lrq_dtype { LRQ_F32 = 0, LRQ_BF16 = 1 } lrq_dtype;

enum { LRQ_TARGET_Q = 1, LRQ_TARGET_K = 2, LRQ_TARGET_V = 4 };

/* Storage of the frozen W_qkv (lrq_desc.weight_format). */
typedef enum lrq_weight_format {
  LRQ_WEIGHT_DENSE = 0, /* [N, d] in the call's dtype */
  LRQ_WEIGHT_NF4 = 1    /* QLoRA base: 4-bit NormalFloat blocks, see lrq_quantize_nf4 */
} lrq_weight_format;

/* Kernel families; LRQ_VARIANT_AUTO lets the library choose. */
typedef enum lrq_variant {
  LRQ_VARIANT_AUTO = 0,
  LRQ_VARIANT_GENERIC = 1, /* any shape, fp32 or bf16, scalar FMA tiles */
  LRQ_VARIANT_TILED = 2,   /* bf16, head_dim 128: MFMA tiles for many tokens */
  LRQ_VARIANT_DECODE = 3   /* bf16, head_dim 128: few tokens, streams W from HBM */
} lrq_variant;

typedef struct lrq_desc {
  int64_t n_tokens;      /* T >= 0; T == 0 is a no-op                                 */
  int64_t d_model;       /* d >= 1                                                    */
  int32_t n_q_heads;     /* Hq >= 1                                                   */
  int32_t n_kv_heads;    /* Hkv >= 1, Hq % Hkv == 0                                   */
  int32_t head_dim;      /* D >= 2, even                                              */
  int32_t dtype;         /* lrq_dtype                                                 */
  float eps;             /* RMSNorm epsilon, finite and >= 0, added to the mean square */
  float rope_theta;      /* RoPE base, finite and > 0                                 */
  int32_t lora_rank;     /* r; 1..LRQ_MAX_LORA_RANK when lora_targets != 0            */
  float lora_alpha;      /* LoRA alpha (finite); the update is scaled by alpha / r    */
  uint32_t lora_targets; /* OR of LRQ_TARGET_*; 0 = no adapters                       */
  int32_t has_bias;      /* 0 or 1                                                    */
  int32_t variant;       /* lrq_variant; LRQ_VARIANT_AUTO (0) normally                 */
  /* LoRA dropout (training).  The LoRA configurations on the pages carry a dropout rate
   * ("Swift-All一文详解：如何用Liger-Kernel提升训练效率", section 3.2, SftArguments; the
   * LoRAConfig in the usage section of "Liger-Kernel底层优化：新一代内核级推理加速引擎深度解析").
   * The library's reading: each adapter's input is h * keep_t / (1 - p) with its own keep
   * mask per target t (the frozen projection sees h itself), which makes the adapter scale
   * alpha / r / (1 - p).  Feature j of token row i is kept for target t (0 q, 1 k, 2 v) iff
   * word j % 4 of Philox4x32-10 (Salmon et al., SC 2011) on the counter
   * (j / 4, i, t, dropout_offset) under the key (low, high 32 bits of dropout_seed) is
   * >= floor(lora_dropout * 2^32), the rate taken as this float32 value.  Rows are the
   * call's own token indices 0 .. T-1.  A backward call with the same seed and offset
   * regenerates the forward's masks.  0 turns dropout off (bit-identical to no dropout);
   * the decode family does not run dropout (AUTO picks another family; forcing it fails
   * with UNSUPPORTED).  Inference callers leave these fields 0. */
  float lora_dropout;      /* p, finite, 0 <= p < 1                                   */
  uint32_t dropout_offset; /* per-call counter word (e.g. the training step)         */
  uint64_t dropout_seed;   /* generator key                                           */
  /* lrq_weight_format of w_qkv.  With LRQ_WEIGHT_NF4 every entry point takes w_qkv as the
   * buffer that lrq_quantize_nf4 writes (lrq_nf4_weight_size bytes), d must be a multiple of
   * 64, and the decode family is not used (AUTO picks another one; forcing it fails with
   * UNSUPPORTED).  Everything else of the call is unchanged. */
  int32_t weight_format;
} lrq_desc;

/* Forward: out = RoPE(W h + b + (alpha/r) B (A h)), h = x * inv_rms(x) * gamma.
 *   lora_a / lora_b: arrays of 3 pointers (q, k, v); entries of non-targets are ignored
 *   and may be NULL, and the arrays themselves may be NULL when lora_targets == 0.
 *   bias is ignored (may be NULL) when has_bias == 0.
 * INVALID_ARG when: desc is NULL; T < 0; d < 1; Hq < 1; Hkv < 1; Hq % Hkv != 0; D < 2
 *   or odd; dtype unknown; eps < 0 or not finite; theta <= 0 or not finite; lora_targets
 *   has bits other than q|k|v; targets set with r < 1 or alpha not finite; has_bias not
 *   0/1; variant unknown; lora_dropout not finite or outside [0, 1); weight_format unknown; x, gamma, w_qkv, positions or out NULL (T > 0); bias NULL with
 *   has_bias; a target's lora_a / lora_b NULL; workspace_bytes below
 *   lrq_workspace_size(desc, 0) or workspace NULL when that size is > 0. */
lrq_status lrq_forward(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                       const void* bias, const void* const* lora_a, const void* const* lora_b,
                       const int32_t* positions, void* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Destination of a forward call's keys and values in a key/value cache.  The rotated k and
 * the (unrotated) v that the projection produces are what the attention step after it reads:
 * "Liger-Kernel底层优化：新一代内核级推理加速引擎深度解析" shows the decoder layer's op
 * sequence (normalise, project to q, k, v, rotate, attention), lists a fused attention
 * kernel with KV-cache handling next to the fused norm/QKV/RoPE kernel, and mentions paged
 * KV-cache management in serving engines.  The pages define no cache layout, so this one is
 * the library's: one row per cached token, which covers a contiguous cache (slot = position)
 * and a paged one flattened to [num_blocks * block_size] rows (slot = the caller's mapping
 * of the token's page and offset).
 *   k_cache, v_cache  [num_slots, Hkv * D]  dtype of the call, 16-byte aligned
 *   slots             [T] int32             cache row of token t
 * Tokens with slots[t] < 0 or >= num_slots are not written (padding).  Two tokens with the
 * same valid slot: which one's row lands is unspecified.  Rows that no token names are left
 * as they were.  The caches are owned by the caller, like every other buffer. */
typedef struct {
  void* k_cache;
  void* v_cache;
  const int32_t* slots;
  int64_t num_slots;  /* >= 0; 0 writes nothing */
} lrq_kv_cache;

/* lrq_forward, and in the same call k_cache[slots[t]] = out[t, Hq*D : (Hq+Hkv)*D] and
 * v_cache[slots[t]] = out[t, (Hq+Hkv)*D : N], bit for bit the values written to out.  The
 * decode family stores the cache rows from the same epilogues that store out; the other
 * families copy them from out in one more pass on the stream.  kv == NULL behaves as
 * lrq_forward.  Same INVALID_ARG rules as lrq_forward, plus num_slots < 0, or k_cache,
 * v_cache or slots NULL (T > 0); UNSUPPORTED for a cache or slots pointer that is not
 * 16-byte aligned. */
lrq_status lrq_forward_kv(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                          const void* bias, const void* const* lora_a, const void* const* lora_b,
                          const int32_t* positions, void* out, const lrq_kv_cache* kv, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Backward of the forward above with W, gamma and bias frozen.  Given dy = dL/d(out),
 * writes dx = dL/dx (dtype) and, for every target t, d_lora_a[t] = dL/dA_t and
 * d_lora_b[t] = dL/dB_t (float32, overwritten, not accumulated).  h and A h are
 * recomputed from x.  `y` must be the forward output for the same inputs (it provides the
 * row statistic <dy, y - R b> that the RMSNorm backward needs without a second pass).
 * Same INVALID_ARG rules as lrq_forward, plus y, dy, dx NULL (T > 0) or a target's
 * d_lora_a / d_lora_b NULL.  With T == 0 the LoRA gradients are set to zero. */
lrq_status lrq_backward(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                        const void* bias, const void* const* lora_a, const void* const* lora_b,
                        const int32_t* positions, const void* y, const void* dy, void* dx,
                        float* const* d_lora_a, float* const* d_lora_b, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Bytes of workspace the call needs (0 if none); 0 for an invalid descriptor. */
size_t lrq_workspace_size(const lrq_desc* desc, int for_backward);

/* ---- Prepared frozen weights.  In the fine-tuning setting the pages describe, the projection
 * weights and the norm weight are frozen and only the LoRA factors train ("Liger-Kernel内核级优化：
 * GPU利用率飙升至90%以上", section on why conventional fine-tuning stalls: W stays fixed, A and B
 * are learned).  The MFMA families read W in layouts derived from (W, gamma) alone: the forward
 * multiplies by W' = bf16(W * gamma) [N, d] (gamma scales the K dimension of the product, so it
 * is folded into the weights), the backward by W^T [d, N].  Without preparation every call
 * rebuilds them in its workspace; lrq_prepare_weights builds them once into a caller buffer that
 * later calls reuse for as long as W and gamma stay unchanged.
 *
 * Bytes of the prepared buffer for descriptors of this shape and dtype (n_tokens and the LoRA
 * fields do not matter): the forward layout, plus the backward one when for_backward != 0.
 * 0 when no family that would run uses one (float32, shapes only the generic family covers),
 * or for an invalid descriptor. */
size_t lrq_prepared_size(const lrq_desc* desc, int for_backward);

/* Writes the prepared layouts of (gamma, w_qkv) into `prepared` (device memory, 256-byte
 * aligned, at least lrq_prepared_size(desc, for_backward) bytes, owned by the caller), enqueued
 * on `stream`.  A no-op returning LRQ_OK when that size is 0.  INVALID_ARG for an invalid
 * descriptor, NULL gamma / w_qkv / prepared, or a buffer below the size; UNSUPPORTED for
 * misaligned pointers. */
lrq_status lrq_prepare_weights(const lrq_desc* desc, int for_backward, const void* gamma, const void* w_qkv,
                               void* prepared, size_t prepared_bytes, void* stream);

/* lrq_forward_kv with prepared weights: the same operation and results, bit for bit, as the
 * call without them (the layouts hold the same values).  prepared == NULL behaves exactly as
 * lrq_forward_kv; kv may be NULL.  The kernel family chosen for the call reads `prepared` when
 * it uses a prepared layout (the tiled family) and ignores it otherwise.  It must hold the
 * output of lrq_prepare_weights for the same shape, gamma and w_qkv (not checked: stale or
 * foreign contents give wrong results); w_qkv and gamma are still required, since other
 * families and the adapters' fold read them.  The workspace may be as small as
 * lrq_workspace_size_prepared(desc, 0).  Adds to lrq_forward_kv's errors: INVALID_ARG when
 * prepared_bytes is below the layout the family reads; UNSUPPORTED for a prepared pointer that
 * is not 256-byte aligned. */
lrq_status lrq_forward_prepared(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                                const void* prepared, size_t prepared_bytes, const void* bias,
                                const void* const* lora_a, const void* const* lora_b, const int32_t* positions,
                                void* out, const lrq_kv_cache* kv, void* workspace, size_t workspace_bytes,
                                void* stream);

/* lrq_backward with prepared weights (prepared with for_backward != 0); same results bit for
 * bit, same rules as lrq_forward_prepared; the workspace may be as small as
 * lrq_workspace_size_prepared(desc, 1). */
lrq_status lrq_backward_prepared(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                                 const void* prepared, size_t prepared_bytes, const void* bias,
                                 const void* const* lora_a, const void* const* lora_b, const int32_t* positions,
                                 const void* y, const void* dy, void* dx, float* const* d_lora_a,
                                 float* const* d_lora_b, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of a call that passes prepared weights (<= lrq_workspace_size). */
size_t lrq_workspace_size_prepared(const lrq_desc* desc, int for_backward);

/* ---- For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  lrq_forward_prepared with no workspace
 * argument: the scratch the call needs comes from an array the library holds on each GPU
 * (LRQ_NOALLOC_SCRATCH_BYTES, part of its device code, kept until the process ends); the call
 * runs on the current device (the stream must belong to it) and allocates nothing.  The
 * tiled family needs the scratch only for the adapters' folded A rows when weights are
 * prepared (without prepared weights its W' does not fit and the call is refused); the decode
 * family keeps its per-call intermediates there.  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race and give wrong results
 * (in the decode family, whose blocks hand data to each other through the scratch, a call can
 * then also wait up to about a second before giving up); order them.  No part of the scratch
 * needs to start at zero: every call writes what it reads.  Same results, bit for bit, as lrq_forward_prepared; same errors, plus UNSUPPORTED
 * when the call needs more than LRQ_NOALLOC_SCRATCH_BYTES of scratch (lrq_workspace_size or
 * lrq_workspace_size_prepared tells how much), and LRQ_ERR_HIP if the array's device address
 * cannot be looked up. */
#define LRQ_NOALLOC_SCRATCH_BYTES (16u << 20)
lrq_status lrq_forward_noalloc(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                               const void* prepared, size_t prepared_bytes, const void* bias,
                               const void* const* lora_a, const void* const* lora_b, const int32_t* positions,
                               void* out, const lrq_kv_cache* kv, void* stream);

/* The kernel family lrq_forward (for_backward = 0) or lrq_backward (1) would run for this
 * descriptor (an lrq_variant value), or -1 when the descriptor is invalid or the forced
 * variant cannot run.  Host-only; enqueues nothing. */
int lrq_select_variant(const lrq_desc* desc, int for_backward);

/* Static name of a status code ("LRQ_OK", ...). */
const char* lrq_status_string(lrq_status status);

/* Message describing the last error returned on the calling thread ("" if none). */
const char* lrq_last_error(void);

/* ---- QLoRA base: W_qkv as NF4 blocks.
 * The pages name QLoRA among the fine-tuning settings these kernels serve ("Liger-Kernel内核级
 * 优化：GPU利用率飙升至90%以上", opening section; "Swift-All一文详解：如何用Liger-Kernel提升训练
 * 效率", section 2.3, the QLoRA row of the table; "Liger-Kernel底层优化：新一代内核级推理加速引擎
 * 深度解析", system-integration section) without defining a stored format.  The library's
 * format is the QLoRA paper's 4-bit NormalFloat (Dettmers et al., NeurIPS 2023): its published
 * 16-value code book L, blocks of 64 consecutive weights of a row of W [N, d], one float32
 * scale per block (the block's largest magnitude), no second-level quantisation.  A weight is
 * L[code] * scale.  Buffer: codes [N][d / 2] bytes (weight k of a row in the low nibble of byte
 * k / 2 for even k, the high nibble for odd k), then the scales [N][d / 64] float32 at the
 * codes' size rounded up to 256 bytes.  Buffers made elsewhere in this layout are accepted. */

/* Bytes of the NF4 buffer of desc's W_qkv (0 for an invalid desc or d % 64 != 0). */
size_t lrq_nf4_weight_size(const lrq_desc* desc);

/* Quantise W_qkv [N, d] (desc's dtype, dense) into the NF4 buffer w_nf4 (16-byte aligned,
 * nf4_bytes >= lrq_nf4_weight_size(desc)), on the device.  Per block: y = w / absmax in
 * float32 (correctly rounded); the code is the number of midpoints (L_i + L_{i+1}) / 2
 * (float32) that y exceeds, so exact ties take the lower level; an all-zero block gets code 7
 * (L[7] = 0) and scale 0.  desc->weight_format is ignored here.
 * INVALID_ARG: invalid desc, NULL pointers, buffer too small; UNSUPPORTED: d % 64 != 0 or
 * misaligned pointers. */
lrq_status lrq_quantize_nf4(const lrq_desc* desc, const void* w_qkv, void* w_nf4, size_t nf4_bytes,
                            void* stream);

/* ---- Attention over the key/value cache: the step after the projection.
 * "Liger-Kernel底层优化：新一代内核级推理加速引擎深度解析" lists a fused attention kernel with
 * KV-cache handling next to the fused norm/QKV/RoPE kernel; its decoder-layer op sequence
 * computes scaled_dot_product_attention(q, k, v) from the rotated q, k and v.  The library's
 * readings: softmax(q.k * scale) v per query head, scale = 1/sqrt(D) unless given; query head h
 * reads kv head h / (Hq / Hkv); causal with the queries as the last q_len tokens of their
 * sequence (query i, 0-based among the sequence's queries, sees keys 0 .. kv_len - q_len + i),
 * or non-causal (every key).  Keys and values are rows of the caches lrq_forward_kv writes,
 * named per sequence by a slot list in token order (a contiguous cache, or a paged one
 * flattened to rows); queries are rows of the projection's output (its first Hq * D columns).
 * Sequence b: query rows q_indptr[b] .. q_indptr[b+1] of q and out, keys
 * kv_slots[kv_indptr[b] .. kv_indptr[b+1]].  Device arrays; the library reads them as given:
 * slots outside [0, num_slots) read as zero vectors, rows past max_q_len of a sequence are not
 * computed, and a query with no visible key (kv_len < q_len) gets a zero row. */
typedef struct lrq_attn_desc {
  int32_t n_seqs;      /* sequences, >= 0 (0: no-op)                                    */
  int32_t n_q_heads;   /* Hq >= 1                                                       */
  int32_t n_kv_heads;  /* Hkv >= 1, Hq % Hkv == 0                                       */
  int32_t head_dim;    /* D; 128 is supported                                           */
  int32_t dtype;       /* LRQ_BF16 (q, caches, out); scores and softmax in float32      */
  int32_t max_q_len;   /* >= every sequence's query count; (max_q_len * Hq/Hkv + 127) / 128 <= 65535 */
  int64_t ld_q;        /* elements between rows of q, >= Hq * D, multiple of 8          */
  int64_t num_slots;   /* rows of each cache, >= 0                                      */
  float scale;         /* softmax scale, finite and >= 0; 0 means 1/sqrt(D)             */
  int32_t causal;      /* 1 causal, 0 not                                               */
} lrq_attn_desc;

/* out [T_q, Hq * D] bf16 = attention of the queries over their cached keys and values.
 * q, k_cache, v_cache, out 16-byte aligned; the index arrays int32.  No workspace.
 * INVALID_ARG: NULL desc, negative counts, heads invalid, ld_q < Hq * D, scale invalid, causal
 * not 0/1, NULL pointers (n_seqs > 0 and max_q_len > 0); UNSUPPORTED: head_dim != 128, dtype
 * not bf16, ld_q % 8 != 0, misaligned pointers, too many query rows per sequence. */
lrq_status lrq_attention(const lrq_attn_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* q_indptr, const int32_t* kv_indptr, const int32_t* kv_slots, void* out,
                         void* stream);

/* LRQ_ABI_VERSION of the loaded library. */
int lrq_abi_version(void);

/* ---- LoRA-adapted SwiGLU MLP, the fused MLP the pages list beside the fused norm/QKV/RoPE
 * kernel: "Swift-All一文详解：如何用Liger-Kernel提升训练效率", section 2.2 (2) (Linear ->
 * SwiGLU -> Linear fused end to end for LLaMA-family FFNs, without storing the intermediate
 * activations); "Liger-Kernel内核级优化：GPU利用率飙升至90%以上", section "内核融合" (a LoRA
 * linear, frozen W plus up(down(x)), with SiLU fused into its last step);
 * "Liger-Kernel底层优化：新一代内核级推理加速引擎深度解析", fused-kernel list (fused MLP with
 * SwiGLU; gate_proj / up_proj / down_proj).  Per token row h:
 *   g = W_g h + s B_g (A_g h),   u = W_u h + s B_u (A_u h),   a = SiLU(g) * u,
 *   y = W_d a + s B_d (A_d a),   SiLU(z) = z / (1 + exp(-z)),  s = alpha / r,
 * each adapter present when its target bit is set.  bf16 operands, fp32 accumulation; g and u
 * stay on chip, a is rounded once to bf16 (the workspace holds it: a full down projection
 * needs whole rows of a), y once.  Layouts (row-major): h, out [T, d]; w_gate, w_up [F, d];
 * w_down [d, F]; lora_a = {A_g [r, d], A_u [r, d], A_d [r, F]}, lora_b = {B_g [F, r],
 * B_u [F, r], B_d [d, r]}.  Same ownership, stream and error rules as lrq_forward; covered
 * shapes: bf16, d % 256 == 0, d_ff % 128 == 0, rank <= 32 (UNSUPPORTED otherwise). */
enum { LRQ_MLP_GATE = 1, LRQ_MLP_UP = 2, LRQ_MLP_DOWN = 4 };

typedef struct lrq_mlp_desc {
  int64_t n_tokens;      /* T >= 0; T == 0 is a no-op                                  */
  int64_t d_model;       /* d                                                           */
  int64_t d_ff;          /* F, the intermediate size                                    */
  int32_t dtype;         /* lrq_dtype (LRQ_BF16)                                        */
  int32_t lora_rank;     /* r; 1..32 when lora_targets != 0                             */
  float lora_alpha;      /* the update is scaled by alpha / r                           */
  uint32_t lora_targets; /* OR of LRQ_MLP_*; 0 = no adapters                            */
} lrq_mlp_desc;

/* Bytes of workspace lrq_mlp_forward needs (T * d_ff * 2); 0 for an invalid descriptor. */
size_t lrq_mlp_workspace_size(const lrq_mlp_desc* desc);

/* out = down(SiLU(gate(h)) * up(h)).  INVALID_ARG for a malformed descriptor, a NULL required
 * pointer (h, the three weights and out when T > 0; a target's lora_a / lora_b), or a workspace
 * below lrq_mlp_workspace_size; UNSUPPORTED for an uncovered shape, float32, or misalignment. */
lrq_status lrq_mlp_forward(const lrq_mlp_desc* desc, const void* h, const void* w_gate, const void* w_up,
                           const void* w_down, const void* const* lora_a, const void* const* lora_b, void* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Measurement hook (not part of the operator).  While enabled, every lrq_forward /
 * lrq_backward call records a pair of HIP events on the caller's stream around the call's
 * dominant kernel: the fused tile kernel of the tiled forward, the streaming kernel of the
 * decode forward, the dh/dx product of the tiled backward, the single kernel of the
 * generic family, the fused gate/up/SwiGLU kernel of lrq_mlp_forward and the attention
 * kernel of lrq_attention (both as forwards).  Enabling (or disabling) discards what was recorded.  Events are created
 * on demand (at most 4096 pairs per direction) and kept until the process ends.  Not
 * thread-safe: meant for one benchmarking thread.  Always LRQ_OK. */
lrq_status lrq_kernel_timing(int enable);

/* Mean duration in milliseconds of the dominant kernel over the forward (for_backward = 0)
 * or backward (1) calls recorded since the hook was enabled, and their number; waits for
 * the recorded events.  INVALID_ARG when mean_ms or count is NULL; LRQ_ERR_HIP if an event
 * query fails.  count = 0 and mean 0 when nothing was recorded. */
lrq_status lrq_kernel_time_ms(int for_backward, double* mean_ms, int* count);

#ifdef __cplusplus
}
#endif

#endif /* LRQ_H_ */
