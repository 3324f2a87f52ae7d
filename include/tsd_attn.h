/*
 * tsd_attn.h -- C ABI of the MI355X (gfx950) scaled dot-product attention
 * forward pass and its multi-head layer.
 *
 * Operations (definitions from the pages; the pages' names):
 *
 *   attn_fwd  O = softmax(Q K^T * scale + M) V, per (batch, head).
 *             "04. Self-Attention：Transformer 的核心计算", section 四
 *             (four stages: scores, scaling by 1/sqrt(d_k), row softmax,
 *             weighted sum) and section 七 (the mask M is added before the
 *             softmax; masked positions get weight 0). Padding mask: the
 *             "attention-mechanism" page, section 掩码 (padded positions are
 *             set to -inf as well).
 *
 *   attn_fwd_ex  attn_fwd with grouped K/V heads and the per-row
 *             log-sum-exp. "Self-Attention 机制", section
 *             MHA -> MQA -> GQA -> MLA: every heads/kv_heads query heads
 *             share one K/V head (kv_heads = heads: plain multi-head,
 *             kv_heads = 1: one shared K/V head). The log-sum-exp is the log
 *             of the softmax denominator of each row, from which any weight
 *             of the pages' attention matrix A is exp(s_ij - lse_i).
 *
 *   mha_fwd   Y = Concat(head_1..head_h) W_O, head_i = Attention of the
 *             i-th d_k-wide column block of X W_Q, X W_K, X W_V, with the
 *             three projections fused into one GEMM against
 *             W_QKV = [W_Q | W_K | W_V].
 *             "Self-Attention 机制", sections 五步计算 (fused W_QKV) and
 *             维度全程跟踪 (split into heads, transpose, concat, W_O);
 *             "04. Self-Attention", section 八 (MultiHead formula).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The
 *    library allocates no device memory, keeps no pointer after it
 *    returns, and never synchronises: work is enqueued on `stream`
 *    (a hipStream_t; NULL = the default stream) and the call returns at
 *    once. Buffers must stay alive until the stream has passed the work.
 *  - A call enqueues kernel launches only (no memset, copy or host
 *    callback), so it can be captured into a HIP graph on `stream` and
 *    replayed; a replay reads and writes the buffers the captured call
 *    named (attn_fwd and mha_fwd replays are tested against eager calls).
 *  - Tensors are dense, row-major, and 16-byte aligned. Outputs must not
 *    overlap inputs.
 *  - Errors are reported only through the return code; nothing aborts and
 *    no exception crosses the ABI. Argument checks run on the host before
 *    any HIP call, so an ATTN_EINVAL/ATTN_EUNSUPPORTED call has no side
 *    effect. attn_last_error() gives a message for the calling thread's
 *    last failure.
 */
#ifndef TSD_ATTN_H
#define TSD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define TSD_API __attribute__((visibility("default")))
#else
#define TSD_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_EINVAL = 1,       /* null pointer, bad size, misaligned pointer, non-finite scale */
    ATTN_EUNSUPPORTED = 2, /* well-formed but outside the supported set below */
    ATTN_EHIP = 3          /* a HIP launch failed; see attn_last_error() */
} attn_status_t;

typedef enum {
    ATTN_MASK_NONE = 0,
    ATTN_MASK_CAUSAL = 1,  /* key j hidden from query i when j > i (diagonal visible) */
    ATTN_MASK_PADDING = 2, /* key j hidden from every query of batch b when j >= valid_lens[b] */
    ATTN_MASK_CAUSAL_PADDING = 3 /* hidden when either rule hides it: visible iff j <= i and j < valid_lens[b]
                                    (the decoder's masked self-attention over a padded batch) */
} attn_mask_kind_t;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/*
 * attn_fwd -- scaled dot-product attention forward.
 *
 *   Q          [batch, heads, seq_q, head_dim]   in_dtype
 *   K, V       [batch, heads, seq_k, head_dim]   in_dtype   (d_v = d_k = head_dim)
 *   mask_kind  attn_mask_kind_t
 *   valid_lens device int32 [batch]; read only for ATTN_MASK_PADDING and
 *              ATTN_MASK_CAUSAL_PADDING (may be NULL otherwise). Values are
 *              clamped to [0, seq_k] on the device.
 *   scale      multiplies Q K^T; finite and >= 0 (the pages use 1/sqrt(d_k)).
 *   O          [batch, heads, seq_q, head_dim]   out_dtype
 *
 * A query row with no visible key (valid_lens[b] == 0) gets O = 0.
 * Masked keys get weight exactly 0: their K and V values never reach O.
 * The [seq_q, seq_k] score matrix is never written to memory.
 *
 * Supported set (else ATTN_EUNSUPPORTED):
 *   in_dtype BF16: head_dim 64 or 128; out_dtype BF16 or F32; products in
 *                  bf16 with float32 accumulation, softmax in float32.
 *   in_dtype F32:  head_dim 16, 32, 64 or 128; out_dtype F32; all float32.
 *   ATTN_MASK_CAUSAL and ATTN_MASK_CAUSAL_PADDING require seq_q == seq_k.
 *   batch*heads, seq_q, seq_k < 2^31; seq_q, seq_k may be 0 (nothing to do).
 */
TSD_API attn_status_t attn_fwd(const void *Q, const void *K, const void *V, int32_t mask_kind, const int32_t *valid_lens,
                       float scale, void *O, int32_t batch, int32_t heads, int32_t seq_q, int32_t seq_k,
                       int32_t head_dim, int32_t in_dtype, int32_t out_dtype, void *stream);

/*
 * attn_fwd_ex -- attn_fwd with grouped K/V heads and an optional per-row
 * log-sum-exp output. attn_fwd(...) is attn_fwd_ex(..., lse = NULL, ...,
 * kv_heads = heads, ...).
 *
 *   K, V       [batch, kv_heads, seq_k, head_dim]; query head h of batch b
 *              reads K/V head h / (heads / kv_heads) of batch b, i.e.
 *              consecutive query heads form a group.
 *   kv_heads   >= 1 and divides heads (else ATTN_EINVAL).
 *   lse        NULL, or device float32 [batch, heads, seq_q], 4-byte
 *              aligned, not overlapping any other tensor: receives
 *              ln sum_j exp(scale * q_i . k_j) over the visible keys j of
 *              each query row (natural log; -inf for a row without a
 *              visible key). With bf16 inputs the sum is that of the
 *              bf16-rounded weights the kernel applies to V.
 *
 * Every other argument, the errors and the supported set are those of
 * attn_fwd.
 */
TSD_API attn_status_t attn_fwd_ex(const void *Q, const void *K, const void *V, int32_t mask_kind,
                          const int32_t *valid_lens, float scale, void *O, float *lse, int32_t batch,
                          int32_t heads, int32_t kv_heads, int32_t seq_q, int32_t seq_k, int32_t head_dim,
                          int32_t in_dtype, int32_t out_dtype, void *stream);

/*
 * attn_weights -- the attention weights themselves, A = softmax(scale Q K^T
 * + M) row by row, for short key sequences: the second result of the
 * pages' attention functions (the "attention-mechanism" page, section
 * 最小实现, returns (output, A); "多模态大模型学习笔记（十四）" section 2.3
 * returns the weights too). The attention kernels never form A (at long
 * sequences it is the n x n matrix that tiling avoids, "Self-Attention
 * 机制" section 瓶颈); this call computes it where it is small.
 *
 *   Q          [batch, heads, seq_q, head_dim]      dtype
 *   K          [batch, kv_heads, seq_k, head_dim]   dtype (grouped heads as in attn_fwd_ex)
 *   mask_kind, valid_lens, scale: as for attn_fwd_ex
 *   A          device float32 [batch, heads, seq_q, seq_k], 4-byte aligned, written;
 *              masked weights are exactly 0, each row with a visible key sums to 1
 *              (rounding aside), a row without one is all zeros
 *   dtype      ATTN_BF16 or ATTN_F32; scores and softmax in float32
 *
 * Supported set: seq_k <= 1024, head_dim 1..256 (else ATTN_EUNSUPPORTED);
 * the causal masks need seq_q == seq_k. Errors as for attn_fwd.
 */
TSD_API attn_status_t attn_weights(const void *Q, const void *K, int32_t mask_kind, const int32_t *valid_lens,
                           float scale, float *A, int32_t batch, int32_t heads, int32_t kv_heads, int32_t seq_q,
                           int32_t seq_k, int32_t head_dim, int32_t dtype, void *stream);

/*
 * attn_bwd -- gradients of attn_fwd_ex's O with respect to Q, K and V.
 * The pages give no backward algorithm; this is the chain rule through
 * the forward stages ("04. Self-Attention", section 四), the weights
 * recomputed from the forward's log-sum-exp:
 *   P_ij = exp(scale q_i.k_j - lse_i) (0 where masked), dV_j = sum_i P_ij dO_i,
 *   dS_ij = P_ij (dO_i.v_j - dO_i.O_i), dQ_i = scale sum_j dS_ij k_j,
 *   dK_j = scale sum_i dS_ij q_i (grouped K/V heads: summed over the group).
 *
 *   Q, O, dO   [batch, heads, seq_q, head_dim]     bf16
 *   K, V       [batch, kv_heads, seq_k, head_dim]  bf16
 *   lse        [batch, heads, seq_q] float32, as written by attn_fwd_ex for
 *              the same inputs, mask and scale
 *   mask_kind, valid_lens, scale, kv_heads: as for attn_fwd_ex
 *   dQ         [batch, heads, seq_q, head_dim]     bf16, written
 *   dK, dV     [batch, kv_heads, seq_k, head_dim]  bf16, written
 *   workspace  device scratch of attn_bwd_workspace_bytes(batch, heads,
 *              seq_q) bytes, 256-byte aligned (holds, per query row, dO_i . O_i
 *              and lse_i in base 2, each head's rows padded to a multiple of 64)
 *
 * Outputs and workspace must not overlap inputs or each other. Supported
 * set: bf16, head_dim 64 or 128 (else ATTN_EUNSUPPORTED); the causal masks
 * need seq_q == seq_k. P and dS are rounded to bf16 for the matrix
 * products, accumulation is float32.
 */
TSD_API attn_status_t attn_bwd(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                       const float *lse, int32_t mask_kind, const int32_t *valid_lens, float scale, void *dQ,
                       void *dK, void *dV, int32_t batch, int32_t heads, int32_t kv_heads, int32_t seq_q,
                       int32_t seq_k, int32_t head_dim, int32_t dtype, void *workspace, size_t workspace_bytes,
                       void *stream);

/* attn_bwd_workspace_bytes -- workspace attn_bwd needs (0 for bad sizes). */
TSD_API size_t attn_bwd_workspace_bytes(int32_t batch, int32_t heads, int32_t seq_q);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * or training loops, harnesses that forbid allocation). Same arguments,
 * results, supported set and errors as attn_bwd, minus the workspace: the
 * per-row terms go to a scratch array the library holds in each GPU's
 * memory from load until the process ends, attn_bwd_noalloc_max_scratch_bytes()
 * bytes (8 MiB), i.e. batch * heads * (seq_q rounded up to 64) <= 2^20 rows
 * (the B1 H32 N32768 workload exactly); larger sizes return ATTN_EINVAL
 * before any HIP call. The call allocates nothing (no hipMalloc, no
 * allocating library routine) and does not synchronise. Every call on a
 * GPU shares that GPU's one scratch array: calls that overlap in time on
 * one GPU (other streams, other threads) race and must be serialised by
 * the caller; calls on one stream are ordered and safe. Nothing carries
 * over between calls (each writes every scratch value it reads).
 */
TSD_API attn_status_t attn_bwd_noalloc(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                               const float *lse, int32_t mask_kind, const int32_t *valid_lens, float scale,
                               void *dQ, void *dK, void *dV, int32_t batch, int32_t heads, int32_t kv_heads,
                               int32_t seq_q, int32_t seq_k, int32_t head_dim, int32_t dtype, void *stream);

/* attn_bwd_noalloc_max_scratch_bytes -- the size of attn_bwd_noalloc's scratch array (8 MiB). */
TSD_API size_t attn_bwd_noalloc_max_scratch_bytes(void);

/*
 * mha_workspace_bytes -- device workspace mha_fwd needs for these sizes:
 * Q, K, V split into heads ([3, batch, h, seq, d_model/h]) plus the
 * concatenated head outputs ([batch, seq, d_model]), in bf16. Returns 0
 * for sizes mha_fwd would reject.
 */
TSD_API size_t mha_workspace_bytes(int32_t batch, int32_t seq, int32_t d_model, int32_t h, int32_t dtype);

/*
 * mha_fwd -- multi-head self-attention layer, no bias, no mask.
 *
 *   X        [batch, seq, d_model]          dtype
 *   W_qkv    [d_model, 3*d_model]           dtype; column blocks W_Q | W_K | W_V,
 *            head i owns columns [i*d_k, (i+1)*d_k) of each block
 *   W_o      [d_model, d_model]             dtype; Y = C W_o
 *   h        number of heads; d_k = d_model / h; scale 1/sqrt(d_k)
 *   O        [batch, seq, d_model]          dtype (the layer output Y)
 *   workspace, workspace_bytes: device scratch of at least
 *            mha_workspace_bytes(batch, seq, d_model, h, dtype) bytes,
 *            256-byte aligned, owned by the caller.
 *
 * Runs three kernels on `stream`: projection GEMM (its epilogue writes the
 * head-split layout), attention (its epilogue writes the concatenated
 * layout), output GEMM. Intermediates are rounded to bf16.
 *
 * Supported set: dtype BF16; d_model % h == 0; d_k in {64, 128};
 * d_model % 64 == 0; batch*seq < 2^31.
 */
TSD_API attn_status_t mha_fwd(const void *X, const void *W_qkv, const void *W_o, int32_t h, void *O, int32_t batch,
                      int32_t seq, int32_t d_model, int32_t dtype, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * mha_cross_workspace_bytes -- device workspace mha_cross_fwd needs: Q split
 * into heads ([batch, h, seq_q, d_k]), K and V split into heads ([2, batch,
 * h, seq_kv, d_k]) and the concatenated head outputs ([batch, seq_q,
 * d_model]), bf16. Returns 0 for sizes mha_cross_fwd would reject.
 */
TSD_API size_t mha_cross_workspace_bytes(int32_t batch, int32_t seq_q, int32_t seq_kv, int32_t d_model, int32_t h,
                                 int32_t dtype);

/*
 * mha_cross_fwd -- multi-head cross-attention layer, no bias: the queries
 * come from one sequence, the keys and values from another
 * ("多模态大模型学习笔记（十四）" section 4: in the decoder's cross-attention
 * Q is the decoder's, K and V the encoder's; "Transformer 详解" section
 * 编码器、解码器与因果掩码). Q = Xq W_Q, [K | V] = Xkv [W_K | W_V], heads
 * split and concatenated as in mha_fwd, Y = C W_o.
 *
 *   Xq       [batch, seq_q, d_model]        dtype
 *   Xkv      [batch, seq_kv, d_model]       dtype (may be NULL when seq_kv = 0)
 *   W_qkv    [d_model, 3*d_model]           the same weight layout as mha_fwd
 *   W_o      [d_model, d_model]
 *   h        number of heads; d_k = d_model / h; scale 1/sqrt(d_k)
 *   mask_kind ATTN_MASK_NONE, or ATTN_MASK_PADDING with valid_lens (device
 *            int32 [batch]): keys j >= valid_lens[b] of the key sequence are
 *            hidden (clamped to [0, seq_kv]); a row without a visible key is 0.
 *            The causal masks are defined for self-attention only:
 *            ATTN_EUNSUPPORTED.
 *   O        [batch, seq_q, d_model]        dtype
 *   workspace, workspace_bytes: device scratch of at least
 *            mha_cross_workspace_bytes(...) bytes, 256-byte aligned.
 *
 * Runs four kernels on `stream`: the query projection and the key/value
 * projection (both writing the head-split layout), attention (writing the
 * concatenated layout), the output projection. Intermediates are bf16.
 * Supported set and errors as for mha_fwd.
 */
TSD_API attn_status_t mha_cross_fwd(const void *Xq, const void *Xkv, const void *W_qkv, const void *W_o, int32_t h,
                            int32_t mask_kind, const int32_t *valid_lens, void *O, int32_t batch, int32_t seq_q,
                            int32_t seq_kv, int32_t d_model, int32_t dtype, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Static description of a status code. */
TSD_API const char *attn_status_string(int32_t status);

/* Message for the calling thread's most recent failed call ("" if none). */
TSD_API const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TSD_ATTN_H */
