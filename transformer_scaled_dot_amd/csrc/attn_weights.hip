// The attention weight matrix A = softmax(Q K^T * scale + M) itself, for
// short key sequences: the second result of the pages' attention functions
// (the "attention-mechanism" page, section 最小实现, returns the output and
// the weights; "多模态大模型学习笔记（十四）" section 2.3 returns attn_weights).
// The attention kernels never form A -- at long sequences it is the n x n
// matrix that tiling exists to avoid ("Self-Attention 机制", section 瓶颈) --
// so this separate kernel computes it where it is small.
//
// One wavefront per query row: lane l holds the scaled scores of keys
// l, l + 64, ... (up to 16 per lane: N_k <= 1024), the row max and the sum of
// the exponentials are wavefront reductions, and every row is written as
// contiguous float32. Masked keys (causal j > i; padding j >= valid_len) get
// weight exactly 0; a row with no visible key is all zeros. Inputs bf16 or
// float32, head_dim 1..256, grouped K/V heads as in the forward.
#include "kernels.h"

#include <math.h>

namespace tsd {
namespace {

constexpr int kMaxKeysPerLane = kAttnWeightsMaxKeys / 64;

template <bool BF16>
__device__ __forceinline__ float load_elem(const void *p, size_t i)
{
    if constexpr (BF16)
        return __uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
    else
        return ((const float *)p)[i];
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <bool BF16, int MASK>
__global__ __launch_bounds__(256) void attn_weights_kernel(const void *__restrict__ Q, const void *__restrict__ K,
                                                           const int32_t *__restrict__ valid_lens, float scale,
                                                           float *__restrict__ A, int H, int Nq, int Nk, int D,
                                                           long long rows, AttnHeads hd)
{
    __shared__ float qs[4][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long row = (long long)blockIdx.x * 4 + wave;  // flat (b, h, i)
    if (row >= rows) return;                                 // wave-uniform
    const long long bh = row / Nq;
    const int i = (int)(row - bh * Nq);
    const int b = (int)(bh / H), h = (int)(bh - (long long)b * H);
    int kv_len = Nk;
    if (mask_padding(MASK)) {
        const int L = valid_lens[b];
        kv_len = L < 0 ? 0 : (L > Nk ? Nk : L);
    }
    const int last = mask_causal(MASK) ? min(i, kv_len - 1) : kv_len - 1;  // visible keys: j <= last
    for (int c = lane; c < D; c += 64) qs[wave][c] = load_elem<BF16>(Q, (size_t)row * D + c);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const size_t kvh = (size_t)b * hd.kv_heads + h / hd.group;
    float s[kMaxKeysPerLane];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < kMaxKeysPerLane; ++t) {
        const int j = lane + 64 * t;
        s[t] = -INFINITY;
        if (j <= last) {
            const size_t kb = (kvh * Nk + j) * (size_t)D;
            float dot = 0.f;
            for (int c = 0; c < D; ++c) dot = fmaf(qs[wave][c], load_elem<BF16>(K, kb + c), dot);
            s[t] = dot * scale;
            mx = fmaxf(mx, s[t]);
        }
    }
    mx = wave_max(mx);
    float z = 0.f;
#pragma unroll
    for (int t = 0; t < kMaxKeysPerLane; ++t) {
        s[t] = lane + 64 * t <= last ? expf(s[t] - mx) : 0.f;
        z += s[t];
    }
    z = wave_sum(z);
    const float inv = z > 0.f ? 1.f / z : 0.f;
    float *out = A + (size_t)row * Nk;
#pragma unroll
    for (int t = 0; t < kMaxKeysPerLane; ++t) {
        const int j = lane + 64 * t;
        if (j < Nk) out[j] = s[t] * inv;
    }
}

template <bool BF16>
hipError_t dispatch(const void *Q, const void *K, int mask, const int32_t *vl, float scale, float *A, int B, int H,
                    int Nq, int Nk, int D, AttnHeads hd, hipStream_t s)
{
    const long long rows = (long long)B * H * Nq;
    if (rows <= 0) return hipSuccess;
    const long long grid = (rows + 3) / 4;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 g((unsigned)grid), blk(256);
    switch (mask) {
    case kMaskCausal:
        hipLaunchKernelGGL((attn_weights_kernel<BF16, kMaskCausal>), g, blk, 0, s, Q, K, vl, scale, A, H, Nq, Nk, D,
                           rows, hd);
        break;
    case kMaskPadding:
        hipLaunchKernelGGL((attn_weights_kernel<BF16, kMaskPadding>), g, blk, 0, s, Q, K, vl, scale, A, H, Nq, Nk, D,
                           rows, hd);
        break;
    case kMaskCausalPadding:
        hipLaunchKernelGGL((attn_weights_kernel<BF16, kMaskCausalPadding>), g, blk, 0, s, Q, K, vl, scale, A, H, Nq,
                           Nk, D, rows, hd);
        break;
    default:
        hipLaunchKernelGGL((attn_weights_kernel<BF16, kMaskNone>), g, blk, 0, s, Q, K, vl, scale, A, H, Nq, Nk, D,
                           rows, hd);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_weights(const void *Q, const void *K, int mask, const int32_t *valid_lens, float scale,
                               float *A, int bf16, int B, int H, int Nq, int Nk, int D, AttnHeads hd,
                               hipStream_t stream)
{
    if (Nk < 1 || Nk > kAttnWeightsMaxKeys || D < 1 || D > 256) return hipErrorInvalidValue;
    if (bf16) return dispatch<true>(Q, K, mask, valid_lens, scale, A, B, H, Nq, Nk, D, hd, stream);
    return dispatch<false>(Q, K, mask, valid_lens, scale, A, B, H, Nq, Nk, D, hd, stream);
}

}  // namespace tsd
