// Scaled dot-product attention forward, bf16 inputs, gfx950 MFMA.
//
// Computes O = softmax(Q K^T * scale + M) V per (batch, head) -- the four
// stages of "04. Self-Attention：Transformer 的核心计算" section 四 with the
// mask of its section 七 (causal) and of the "attention-mechanism" page,
// section 掩码 (padding) -- without ever forming the [N_q, N_k] score
// matrix in memory. Keys are consumed in tiles of 64 and the row softmax
// is carried across tiles by the running (max, sum) pair of the online
// softmax recurrence ("Self-Attention 机制", section Softmax 的数值稳定性与
// Online Softmax): when the running max moves from m to m', the partial
// sum and the partial output are rescaled by e^{m - m'}.
//
// Work decomposition (one workgroup = WAVES wavefronts = WAVES*32 query
// rows of one head; each wave owns 32 query rows):
//   * Q^T stays in registers as the B operand of v_mfma_f32_32x32x16_bf16.
//   * K and V tiles (64 keys) are staged through LDS, double buffered: the
//     global loads of tile t+1 are in flight while tile t is computed.
//   * S^T = K Q^T: the accumulator puts one query per lane (lane % 32) and
//     16 keys per lane, so the row max/sum are 32 in-lane values plus one
//     exchange with the other half-wave (v_permlane32_swap).
//   * P^T goes straight from the S accumulator (rounded to bf16) into the
//     B operand of O^T += V^T P^T: the MFMA's k index is mapped onto keys in
//     the order the accumulator holds them, and V^T operands are read from
//     the row-major V tile with ds_read_b64_tr_b16 in that same order.
//   * O^T also has one query per lane, so the e^{m - m'} rescale is one
//     scalar per lane; it is skipped when no row of the wave changed max.
//   * Causal: key tiles above a wave's diagonal are skipped, tiles crossing
//     it are masked; workgroups are issued longest-first.
#include "device_common.h"
#include "kernels.h"

#include <math.h>

namespace tsd {
namespace {

constexpr int kBlockN = 64;  // keys per LDS tile

template <int D>
struct AttnLds {
    static constexpr int kStrideK = D + 8;   // K row pitch (elements): rows shift by 4 banks
    static constexpr int kStrideV = D + 16;  // V row pitch: 4 rows of one tr-read hit disjoint banks
    static constexpr int kTile = kBlockN * kStrideK + kBlockN * kStrideV;
};

template <int D, int MASK, bool OUT_F32, int OLAYOUT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ valid_lens, float c_log2, void *__restrict__ Out, int H, int Nq, int Nk,
    int num_qtiles, int BH)
{
    constexpr int BM = WAVES * 32;
    constexpr int NT = WAVES * 64;
    constexpr int KS = D / 16;  // k-steps of the Q K^T contraction
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    constexpr int SK = AttnLds<D>::kStrideK, SV = AttnLds<D>::kStrideV, TILE = AttnLds<D>::kTile;
    constexpr int CH = kBlockN * D / 8 / NT;  // 16-byte chunks per thread per tensor per tile
    static_assert(kBlockN * D / 8 % NT == 0, "tile must split evenly over the workgroup");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5, g16 = lane >> 4, i16 = lane & 15;

    // q-tile-major order: the q-tiles of one head are BH ids apart, which
    // lands them on the same XCD (and L2) when BH is a multiple of 8
    const int id = blockIdx.x;
    const int bh = id % BH;
    int qt = id / BH;
    if (MASK == kMaskCausal) qt = num_qtiles - 1 - qt;
    const int b = bh / H;
    const int q0 = qt * BM;

    int kv_len = Nk;
    if (MASK == kMaskPadding) {
        const int L = valid_lens[b];
        kv_len = L < 0 ? 0 : (L > Nk ? Nk : L);
    }
    int kv_end = kv_len;
    if (MASK == kMaskCausal) kv_end = min(kv_len, q0 + BM);
    const int ntiles = (kv_end + kBlockN - 1) / kBlockN;

    const uint16_t *Kh = K + (size_t)bh * Nk * D;
    const uint16_t *Vh = V + (size_t)bh * Nk * D;

    // Q^T as B operands: lane holds Q[qrow][ks*16 + hf*8 .. +7]
    const int qrow = q0 + wave * 32 + l32;
    bf16x8 qreg[KS];
    {
        const bool ok = qrow < Nq;
        const uint16_t *qp = Q + ((size_t)bh * Nq + (ok ? qrow : 0)) * D + hf * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = ok ? *(const u32x4 *)(qp + ks * 16) : u32x4{0u, 0u, 0u, 0u};
            qreg[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    f32x16 acc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // global -> registers for one tile; keys at or past kv_end are never
    // visible to any row of this workgroup and are not read (zero fill)
    u32x4 kreg[CH], vreg[CH];
    auto load_tile = [&](int t) {
        const int k0 = t * kBlockN;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * NT;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            const int key = k0 + row;
            if (key < kv_end) {
                kreg[i] = *(const u32x4 *)(Kh + (size_t)key * D + col);
                vreg[i] = *(const u32x4 *)(Vh + (size_t)key * D + col);
            } else {
                kreg[i] = u32x4{0u, 0u, 0u, 0u};
                vreg[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t *Ks = smem + buf * TILE;
        uint16_t *Vs = Ks + kBlockN * SK;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * NT;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            *(u32x4 *)(Ks + row * SK + col) = kreg[i];
            *(u32x4 *)(Vs + row * SV + col) = vreg[i];
        }
    };

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    const int qmin_w = q0 + wave * 32, qmax_w = qmin_w + 31;
    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) load_tile(t + 1);
        const int k0 = t * kBlockN;
        const uint16_t *Ks = smem + (t & 1) * TILE;
        const uint16_t *Vs = Ks + kBlockN * SK;
        const bool skip = (MASK == kMaskCausal) && (k0 > qmax_w);
        if (!skip) {
            const bool need_mask =
                (k0 + kBlockN > kv_len) || (MASK == kMaskCausal && k0 + kBlockN - 1 > qmin_w);

            // ---- S^T = K Q^T (64 keys x 32 queries per wave) ----
            f32x16 s[2];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[jb][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const bf16x8 a = *(const bf16x8 *)(Ks + (jb * 32 + l32) * SK + ks * 16 + hf * 8);
                    s[jb] = mfma32x32x16(a, qreg[ks], s[jb]);
                }

            // ---- mask: key j of this lane's row is hidden when j >= kv_len or (causal) j > qrow ----
            if (need_mask) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + jb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
                        const bool vis = key < kv_len && (MASK != kMaskCausal || key <= qrow);
                        if (!vis) s[jb][r] = -INFINITY;
                    }
            }

            // ---- online softmax update (base 2, scale folded into c_log2) ----
            float mx = -INFINITY;
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
            mx = half_swap_max(mx);
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float mc = m_use * c_log2;
            const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_use) * c_log2);
            float lsum = 0.f;
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = fast_exp2(fmaf(s[jb][r], c_log2, -mc));
                    if (need_mask) p = (s[jb][r] == -INFINITY) ? 0.f : p;
                    s[jb][r] = p;
                    lsum += p;
                }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int i = 0; i < DB; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
            }

            // ---- P (bf16) as B operands, 16 keys per MFMA ----
            bf16x8 pb[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int jb = c >> 1, r0 = (c & 1) * 8;
                u32x4 w;
                w[0] = pack_bf16x2(s[jb][r0 + 0], s[jb][r0 + 1]);
                w[1] = pack_bf16x2(s[jb][r0 + 2], s[jb][r0 + 3]);
                w[2] = pack_bf16x2(s[jb][r0 + 4], s[jb][r0 + 5]);
                w[3] = pack_bf16x2(s[jb][r0 + 6], s[jb][r0 + 7]);
                pb[c] = __builtin_bit_cast(bf16x8, w);
            }

            // ---- O^T += V^T P^T ----
            // MFMA k slot hf*8 + t of chunk c is key c*16 + (t/4)*8 + hf*4 + t%4,
            // the order in which the S accumulator holds the keys
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int key_lo = c * 16 + hf * 4 + (i16 >> 2);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int col = db * 32 + (g16 & 1) * 16 + 4 * (i16 & 3);
                    const bf16x8 a = lds_tr_pair(Vs + key_lo * SV + col, Vs + (key_lo + 8) * SV + col);
                    acc[db] = mfma32x32x16(a, pb[c], acc[db]);
                }
            }
        }
        if (t + 1 < ntiles) store_tile((t + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l (0 for a row with no visible key) ----
    const float l_tot = half_swap_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < Nq) {
        size_t row_off;
        if (OLAYOUT == kOutBHND) {
            row_off = ((size_t)bh * Nq + qrow) * D;
        } else {
            const int hh = bh % H;
            row_off = (((size_t)b * Nq + qrow) * H + hh) * D;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = db * 32 + rg * 8 + hf * 4;
                const float v0 = acc[db][rg * 4 + 0] * inv, v1 = acc[db][rg * 4 + 1] * inv;
                const float v2 = acc[db][rg * 4 + 2] * inv, v3 = acc[db][rg * 4 + 3] * inv;
                if (OUT_F32) {
                    *(f32x4 *)((float *)Out + row_off + d0) = f32x4{v0, v1, v2, v3};
                } else {
                    *(u32x2 *)((uint16_t *)Out + row_off + d0) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                }
            }
    }
}

template <int D, int MASK, bool OUT_F32, int OLAYOUT>
hipError_t launch_variant(const void *Q, const void *K, const void *V, const int32_t *valid_lens, float scale,
                          void *O, int B, int H, int Nq, int Nk, hipStream_t stream)
{
    constexpr int WAVES = 4, BM = WAVES * 32;
    const int BH = B * H;
    const int num_qtiles = (Nq + BM - 1) / BM;
    const long long grid = (long long)num_qtiles * BH;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float c_log2 = scale * 1.4426950408889634f;  // exp(x) = exp2(x * log2(e))
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, MASK, OUT_F32, OLAYOUT, WAVES>), dim3((unsigned)grid),
                       dim3(WAVES * 64), 0, stream, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                       valid_lens, c_log2, O, H, Nq, Nk, num_qtiles, BH);
    return hipGetLastError();
}

template <int D, int MASK>
hipError_t dispatch_out(const void *Q, const void *K, const void *V, const int32_t *vl, float scale, void *O,
                        int out_f32, int out_layout, int B, int H, int Nq, int Nk, hipStream_t s)
{
    if (out_layout == kOutBNHD) {
        if (out_f32) return launch_variant<D, MASK, true, kOutBNHD>(Q, K, V, vl, scale, O, B, H, Nq, Nk, s);
        return launch_variant<D, MASK, false, kOutBNHD>(Q, K, V, vl, scale, O, B, H, Nq, Nk, s);
    }
    if (out_f32) return launch_variant<D, MASK, true, kOutBHND>(Q, K, V, vl, scale, O, B, H, Nq, Nk, s);
    return launch_variant<D, MASK, false, kOutBHND>(Q, K, V, vl, scale, O, B, H, Nq, Nk, s);
}

template <int D>
hipError_t dispatch_mask(const void *Q, const void *K, const void *V, int mask, const int32_t *vl, float scale,
                         void *O, int out_f32, int out_layout, int B, int H, int Nq, int Nk, hipStream_t s)
{
    switch (mask) {
    case kMaskCausal: return dispatch_out<D, kMaskCausal>(Q, K, V, vl, scale, O, out_f32, out_layout, B, H, Nq, Nk, s);
    case kMaskPadding: return dispatch_out<D, kMaskPadding>(Q, K, V, vl, scale, O, out_f32, out_layout, B, H, Nq, Nk, s);
    default: return dispatch_out<D, kMaskNone>(Q, K, V, vl, scale, O, out_f32, out_layout, B, H, Nq, Nk, s);
    }
}

}  // namespace

hipError_t launch_attn_bf16(const void *Q, const void *K, const void *V, int mask, const int32_t *valid_lens,
                            float scale, void *O, int out_f32, int out_layout, int B, int H, int Nq, int Nk, int D,
                            hipStream_t stream)
{
    if (D == 128)
        return dispatch_mask<128>(Q, K, V, mask, valid_lens, scale, O, out_f32, out_layout, B, H, Nq, Nk, stream);
    if (D == 64)
        return dispatch_mask<64>(Q, K, V, mask, valid_lens, scale, O, out_f32, out_layout, B, H, Nq, Nk, stream);
    return hipErrorInvalidValue;
}

}  // namespace tsd
