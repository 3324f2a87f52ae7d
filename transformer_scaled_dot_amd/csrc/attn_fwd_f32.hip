// Scaled dot-product attention forward, float32 throughout (the accuracy
// path; not tuned for speed).
//
// Same definition as the bf16 kernel ("04. Self-Attention：Transformer 的核心
// 计算" section 四, masks of its section 七 and of the "attention-mechanism"
// page, section 掩码), computed with float32 FMAs and expf. Keys are read
// through LDS tiles of 32 and folded into the row state one key at a time
// with the online softmax recurrence of "Self-Attention 机制", section
// Online Softmax: m_j = max(m_{j-1}, s_j),
// l_j = l_{j-1} e^{m_{j-1} - m_j} + e^{s_j - m_j}, and the output row
// follows the same rescaling.
//
// One workgroup = 16 query rows of one head; 16 lanes per row, each lane
// owning D/16 interleaved columns (lane c of a row owns columns c, c+16, ...).
#include "kernels.h"

#include <math.h>

namespace tsd {
namespace {

constexpr int kRows = 16;      // query rows per workgroup
constexpr int kKeyTile = 32;   // keys per LDS tile

template <int D, int MASK>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K,
                                                           const float *__restrict__ V,
                                                           const int32_t *__restrict__ valid_lens, float scale,
                                                           float *__restrict__ O, int H, int Nq, int Nk,
                                                           int num_qtiles, AttnHeads hd)
{
    constexpr int CPL = D / 16;  // columns per lane
    __shared__ float Ks[kKeyTile][D + 1];
    __shared__ float Vs[kKeyTile][D + 1];

    const int tid = threadIdx.x, row = tid >> 4, sub = tid & 15;
    const int bh = blockIdx.x / num_qtiles, qt = blockIdx.x % num_qtiles;
    const int b = bh / H;
    const int q0 = qt * kRows;
    const int qrow = q0 + row;

    int kv_len = Nk;
    if (mask_padding(MASK)) {
        const int L = valid_lens[b];
        kv_len = L < 0 ? 0 : (L > Nk ? Nk : L);
    }
    int kv_end = kv_len;
    if (mask_causal(MASK)) kv_end = min(kv_len, q0 + kRows);

    const size_t kvh = (size_t)b * hd.kv_heads + (bh - b * H) / hd.group;
    const float *Kh = K + kvh * Nk * D;
    const float *Vh = V + kvh * Nk * D;
    float q[CPL], o[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        q[e] = qrow < Nq ? Q[((size_t)bh * Nq + qrow) * D + sub + 16 * e] : 0.f;
        o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    for (int k0 = 0; k0 < kv_end; k0 += kKeyTile) {
        const int nk = min(kKeyTile, kv_end - k0);
        for (int i = tid; i < kKeyTile * D; i += 256) {
            const int j = i / D, c = i % D;
            const bool ok = j < nk;
            Ks[j][c] = ok ? Kh[(size_t)(k0 + j) * D + c] : 0.f;
            Vs[j][c] = ok ? Vh[(size_t)(k0 + j) * D + c] : 0.f;
        }
        __syncthreads();
        for (int j = 0; j < nk; ++j) {
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) part = fmaf(q[e], Ks[j][sub + 16 * e], part);
            // sum over the 16 lanes of this row
            part += __shfl_xor(part, 8, 16);
            part += __shfl_xor(part, 4, 16);
            part += __shfl_xor(part, 2, 16);
            part += __shfl_xor(part, 1, 16);
            const int key = k0 + j;
            const bool vis = key < kv_len && (!mask_causal(MASK) || key <= qrow);
            if (vis) {
                const float s = part * scale;
                const float m_new = fmaxf(m, s);
                const float alpha = expf(m - m_new);  // 0 while m is still -inf
                const float p = expf(s - m_new);
                l = l * alpha + p;
#pragma unroll
                for (int e = 0; e < CPL; ++e) o[e] = fmaf(p, Vs[j][sub + 16 * e], o[e] * alpha);
                m = m_new;
            }
        }
        __syncthreads();
    }

    if (qrow < Nq) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) O[((size_t)bh * Nq + qrow) * D + sub + 16 * e] = o[e] * inv;
        // log of the softmax denominator: m is the row max of the scaled scores, l = sum exp(s - m)
        if (hd.lse && sub == 0) hd.lse[(size_t)bh * Nq + qrow] = l > 0.f ? m + logf(l) : -INFINITY;
    }
}

template <int D, int MASK>
hipError_t launch(const float *Q, const float *K, const float *V, const int32_t *vl, float scale, float *O, int B,
                  int H, int Nq, int Nk, AttnHeads hd, hipStream_t s)
{
    const int num_qtiles = (Nq + kRows - 1) / kRows;
    const long long grid = (long long)num_qtiles * B * H;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, MASK>), dim3((unsigned)grid), dim3(256), 0, s, Q, K, V, vl, scale, O,
                       H, Nq, Nk, num_qtiles, hd);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch(const float *Q, const float *K, const float *V, int mask, const int32_t *vl, float scale,
                    float *O, int B, int H, int Nq, int Nk, AttnHeads hd, hipStream_t s)
{
    switch (mask) {
    case kMaskCausal: return launch<D, kMaskCausal>(Q, K, V, vl, scale, O, B, H, Nq, Nk, hd, s);
    case kMaskPadding: return launch<D, kMaskPadding>(Q, K, V, vl, scale, O, B, H, Nq, Nk, hd, s);
    case kMaskCausalPadding: return launch<D, kMaskCausalPadding>(Q, K, V, vl, scale, O, B, H, Nq, Nk, hd, s);
    default: return launch<D, kMaskNone>(Q, K, V, vl, scale, O, B, H, Nq, Nk, hd, s);
    }
}

}  // namespace

hipError_t launch_attn_f32(const float *Q, const float *K, const float *V, int mask, const int32_t *valid_lens,
                           float scale, float *O, int B, int H, int Nq, int Nk, int D, AttnHeads hd,
                           hipStream_t stream)
{
    switch (D) {
    case 16: return dispatch<16>(Q, K, V, mask, valid_lens, scale, O, B, H, Nq, Nk, hd, stream);
    case 32: return dispatch<32>(Q, K, V, mask, valid_lens, scale, O, B, H, Nq, Nk, hd, stream);
    case 64: return dispatch<64>(Q, K, V, mask, valid_lens, scale, O, B, H, Nq, Nk, hd, stream);
    case 128: return dispatch<128>(Q, K, V, mask, valid_lens, scale, O, B, H, Nq, Nk, hd, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace tsd
