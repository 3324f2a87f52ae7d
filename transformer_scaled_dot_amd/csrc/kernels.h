// Host-side launchers shared between the kernels and the C ABI layer.
// Every launcher assumes its arguments were validated by the C ABI layer
// (shapes, alignment, supported set) and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsd {

// Bit 0: causal (key j hidden from query i when j > i); bit 1: padding (keys j >= valid_lens[b] hidden).
enum MaskKind { kMaskNone = 0, kMaskCausal = 1, kMaskPadding = 2, kMaskCausalPadding = 3 };
constexpr bool mask_causal(int m) { return (m & kMaskCausal) != 0; }
constexpr bool mask_padding(int m) { return (m & kMaskPadding) != 0; }

// Grouped K/V heads and the optional per-row log-sum-exp of one attention call: query head h of batch b
// reads K/V head b * kv_heads + h / group (group = H / kv_heads); lse, when not null, receives
// ln sum_j exp(s_ij) over the visible scaled scores of each query row, [B,H,Nq] float32 (-inf for a row
// without a visible key).
struct AttnHeads {
    int kv_heads;
    int group;
    float *lse;
};

enum OutLayout { kOutBHND = 0, kOutBNHD = 1 };  // [B,H,N,D] or concatenated heads [B,N,H*D]

// bf16 attention, head_dim 64 or 128, output bf16 (out_f32 = 0) or f32.
hipError_t launch_attn_bf16(const void *Q, const void *K, const void *V, int mask, const int32_t *valid_lens,
                            float scale, void *O, int out_f32, int out_layout, int B, int H, int Nq, int Nk, int D,
                            AttnHeads heads, hipStream_t stream);

// f32 attention, head_dim 16, 32, 64 or 128, output f32, layout [B,H,N,D].
hipError_t launch_attn_f32(const float *Q, const float *K, const float *V, int mask, const int32_t *valid_lens,
                           float scale, float *O, int B, int H, int Nq, int Nk, int D, AttnHeads heads,
                           hipStream_t stream);

// bf16 attention backward, head_dim 64 or 128: dQ [B,H,Nq,D], dK and dV [B,Hkv,Nk,D] (bf16) from Q, K, V,
// the forward's O and per-row log-sum-exp lse ([B,H,Nq] float32) and dO; work: float32 scratch of
// 2 * B * H * (Nq rounded up to 64) values.
hipError_t launch_attn_bwd_bf16(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                                const float *lse, int mask, const int32_t *valid_lens, float scale, void *dQ, void *dK,
                                void *dV, int B, int H, int Hkv, int Nq, int Nk, int D, float *work,
                                hipStream_t stream);

// The attention weights A = softmax(Q K^T * scale + M) as float32 [B,H,Nq,Nk], for Nk <= kAttnWeightsMaxKeys;
// Q [B,H,Nq,D] and K [B,Hkv,Nk,D] bf16 (bf16 = 1) or float32, D in 1..256.
constexpr int kAttnWeightsMaxKeys = 1024;
hipError_t launch_attn_weights(const void *Q, const void *K, int mask, const int32_t *valid_lens, float scale,
                               float *A, int bf16, int B, int H, int Nq, int Nk, int D, AttnHeads heads,
                               hipStream_t stream);

// Compute units of the current device (cached per device): the size of persistent grids.
int device_cu_count();

// C = A[M,K] * B[K,N] in bf16 with f32 accumulation, bf16 output.
// Plain epilogue: C row-major [M,N].
hipError_t launch_gemm_bf16(const void *A, const void *Bm, void *C, int M, int N, int K, hipStream_t stream);

// Projection epilogue: column n of the [M = batch*seq, 3*d_model] product is
// written to qkv[which][b][head][t][c] with which = n / d_model,
// head = (n % d_model) / dk, c = n % dk, b = m / seq, t = m % seq.
hipError_t launch_gemm_bf16_qkv_split(const void *X, const void *Wqkv, void *qkv, int batch, int seq, int d_model,
                                      int heads, hipStream_t stream);

// The same head-split epilogue for the columns [0, n_cols) of a weight with row stride ldw (W may point into
// a wider matrix): out[which][b][head][t][c] with which = n / d_model, so n_cols = d_model gives Q alone
// and n_cols = 2 d_model (W at the W_K block) gives K and V.
hipError_t launch_gemm_bf16_heads(const void *X, const void *W, int ldw, void *out, int batch, int seq, int n_cols,
                                  int d_model, int heads, hipStream_t stream);


}  // namespace tsd
