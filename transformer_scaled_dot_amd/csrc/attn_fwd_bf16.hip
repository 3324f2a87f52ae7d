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

#include <type_traits>

namespace tsd {
namespace {

constexpr int kBlockN = 64;  // keys per LDS tile

// LDS tiles are dense [64 keys][D] bf16 with the 16-byte chunks of each row
// XOR-swizzled: element (r, e) lives at r*D + 8*((e/8) ^ swz(r)) + e%8.
// The swizzle makes both reads conflict-free at the 2-cycle minimum:
//  - K reads (16 B per lane, 16 consecutive rows, same column chunk) land
//    on 16 distinct bank groups;
//  - V transposed reads (8 rows x 64 B per wave) spread over all banks.
template <int D>
__device__ __forceinline__ int swz(int r)
{
    if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);  // 16 chunks per 256-byte row
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);         // 8 chunks per 128-byte row
}

template <int D>
__device__ __forceinline__ int swz_off(int r, int e)
{
    return r * D + ((((e >> 3) ^ swz<D>(r))) << 3) + (e & 7);
}

// Per-lane LDS byte offsets used by every tile (buffer and key-chunk offsets
// are added as instruction immediates).
template <int D>
struct TileAddrs {
    uint32_t k[D / 16];      // K read (A operand of S^T) for k-step ks, key block 0
    uint32_t v[D / 32][2];   // V transposed read for output block db, rows +0 / +8, key chunk 0
};

template <int D>
__device__ __forceinline__ TileAddrs<D> tile_addrs(int lane)
{
    const int l32 = lane & 31, hf = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
    TileAddrs<D> a;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) a.k[ks] = 2 * swz_off<D>(l32, ks * 16 + hf * 8);
    const int row = hf * 4 + (i16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const int col = db * 32 + (g16 & 1) * 16 + 4 * (i16 & 3);
        a.v[db][0] = 2 * swz_off<D>(row, col);
        a.v[db][1] = 2 * swz_off<D>(row + 8, col);
    }
    return a;
}

template <int OFF>
__device__ __forceinline__ bf16x8 lds_read_b128(const uint8_t *base, uint32_t addr)
{
    return *(const bf16x8 *)(base + addr + OFF);
}

// One 64-key tile for one wave (32 query rows): S^T = K Q^T, mask, online
// softmax update, O^T += V^T P^T. KOFF/VOFF: byte offsets of the K and V
// tiles in LDS (compile-time, so they fold into instruction immediates).
template <int D, int MASK, int KOFF, int VOFF>
__device__ __forceinline__ void attend_tile(const uint8_t *lds, const TileAddrs<D> &ad, const bf16x8 (&qreg)[D / 16],
                                            f32x16 (&acc)[D / 32], float &m_run, float &l_run, float c_log2,
                                            int k0, int kv_len, int qrow, int lane, bool need_mask)
{
    constexpr int KS = D / 16, DB = D / 32;
    const int hf = lane >> 5;

    // ---- S^T = K Q^T (64 keys x 32 queries); K operands fetched one k-step ahead ----
    f32x16 s[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[jb][r] = 0.f;
    bf16x8 ka[2][2];
    ka[0][0] = *(const bf16x8 *)(lds + ad.k[0] + KOFF);
    ka[0][1] = *(const bf16x8 *)(lds + ad.k[0] + KOFF + 32 * D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        if (ks + 1 < KS) {
            ka[nxt][0] = *(const bf16x8 *)(lds + ad.k[ks + 1] + KOFF);
            ka[nxt][1] = *(const bf16x8 *)(lds + ad.k[ks + 1] + KOFF + 32 * D * 2);
        }
        s[0] = mfma32x32x16(ka[cur][0], qreg[ks], s[0]);
        s[1] = mfma32x32x16(ka[cur][1], qreg[ks], s[1]);
    }

    // ---- mask: key j hidden from this lane's row when j >= kv_len or (causal) j > qrow ----
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

    // ---- online softmax (base 2; scale * log2(e) folded into c_log2 > 0, so a
    //      masked score -inf gives exactly exp2(-inf) = 0) ----
    float mx = s[0][0];
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
            const float p = fast_exp2(fmaf(s[jb][r], c_log2, -mc));
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

    // ---- P in bf16 as B operands, 16 keys per MFMA ----
    bf16x8 pb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int jb = c >> 1, r0 = (c & 1) * 8;
        u32x4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = pack_bf16x2(s[jb][r0 + 2 * u], s[jb][r0 + 2 * u + 1]);
        pb[c] = __builtin_bit_cast(bf16x8, w);
    }

    // ---- O^T += V^T P^T ----
    // MFMA k slot hf*8 + t of chunk c is key c*16 + (t/4)*8 + hf*4 + t%4, the
    // order in which the S accumulator holds the keys; a transposed read of
    // rows c*16 + hf*4 + (0..3) (+8) gives exactly those 8 keys per column.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint8_t *p0 = lds + ad.v[db][0] + VOFF + c * 16 * D * 2;
            const uint8_t *p1 = lds + ad.v[db][1] + VOFF + c * 16 * D * 2;
            const bf16x8 a = lds_tr_pair((const uint16_t *)p0, (const uint16_t *)p1);
            acc[db] = mfma32x32x16(a, pb[c], acc[db]);
        }
    }
}

template <int D, int MASK, bool OUT_F32, int OLAYOUT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ valid_lens, float c_log2, void *__restrict__ Out, int H, int Nq, int Nk,
    int num_qtiles, int BH)
{
    constexpr int BM = WAVES * 32;
    constexpr int KS = D / 16;  // k-steps of the Q K^T contraction
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    constexpr int TILE_B = kBlockN * D * 2;                     // bytes of one K (or V) tile
    constexpr int CPR = D / 8;                                  // 16-byte chunks per row
    constexpr int CH = kBlockN * CPR / (WAVES * 64);            // chunk loads per lane per tensor per tile
    static_assert(kBlockN * CPR % (WAVES * 64) == 0, "tile must split evenly over the workgroup");
    static_assert(4 * TILE_B <= 65536, "buffer offsets must fit LDS instruction immediates");
    // buffer 0 = [K | V] at bytes [0, 2*TILE_B), buffer 1 at [2*TILE_B, 4*TILE_B)
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * TILE_B];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;

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

    // Global -> LDS without registers: DMA j of this wave fills the 64
    // consecutive LDS chunks [(j*WAVES + wave)*64, +64) of a tile; lane i
    // fetches the global chunk that the swizzle puts in slot i. The per-lane
    // byte offset within the tile's rows is fixed; the tile's first key moves
    // the (uniform) base pointer. Rows at or past kv_end are never visible to
    // this workgroup: they are not read; the last valid row is fetched in
    // their place (its weight is exactly 0).
    uint32_t voff[CH];
    int drow[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = (j * WAVES + wave) * 64 + lane;
        const int r = c / CPR, x = c % CPR;
        drow[j] = r;
        voff[j] = (uint32_t)(r * D + ((x ^ swz<D>(r)) << 3)) * 2;
    }
    const uint32_t lds0 = lds_addr(smem);
    auto issue_tile = [&](int t, uint32_t buf_off) {
        const int k0 = t * kBlockN;
        const uint16_t *kb = Kh + (size_t)k0 * D;
        const uint16_t *vb = Vh + (size_t)k0 * D;
        const bool tail = k0 + kBlockN > kv_end;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            uint32_t off = voff[j];
            if (tail) {
                const int r = min(drow[j], kv_end - 1 - k0);
                off = off - (uint32_t)(drow[j] - r) * (D * 2);
            }
            const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + buf_off + (j * WAVES + wave) * 1024);
            lds_dma16(dst, kb, off);
            lds_dma16(dst + TILE_B, vb, off);
        }
    };

    const TileAddrs<D> ad = tile_addrs<D>(lane);
    if (ntiles > 0) issue_tile(0, 0);
    wait_vmcnt0();
    __syncthreads();

    const int qmin_w = q0 + wave * 32, qmax_w = qmin_w + 31;
    auto step = [&](int t, auto buf) {
        constexpr int B = decltype(buf)::value;
        if (t + 1 < ntiles) issue_tile(t + 1, (B ^ 1) * 2 * TILE_B);
        const int k0 = t * kBlockN;
        const bool skip = (MASK == kMaskCausal) && (k0 > qmax_w);
        if (!skip) {
            const bool need_mask =
                (k0 + kBlockN > kv_len) || (MASK == kMaskCausal && k0 + kBlockN - 1 > qmin_w);
            attend_tile<D, MASK, B * 2 * TILE_B, B * 2 * TILE_B + TILE_B>(smem, ad, qreg, acc, m_run, l_run, c_log2,
                                                                          k0, kv_len, qrow, lane, need_mask);
        }
        wait_vmcnt0();
        __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
        step(t, std::integral_constant<int, 0>());
        if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>());
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
    // exp(x) = exp2(x * log2(e)). The kernel needs c_log2 > 0 so that masked
    // scores (-inf) map to weight 0 without a select; below 1e-30 every
    // visible exp2 argument rounds to 0 anyway, which is the scale = 0 result.
    const float c_log2 = fmaxf(scale * 1.4426950408889634f, 1e-30f);
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
