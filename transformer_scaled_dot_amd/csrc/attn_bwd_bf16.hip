// Scaled dot-product attention backward, bf16 inputs, gfx950 MFMA.
//
// The gradients of O = softmax(Q K^T * scale + M) V with respect to Q, K and V, given dO, the forward's
// output O and its per-row log-sum-exp lse. The pages motivate gradients ("04. Self-Attention", section
// 四 stage 2) but give no backward algorithm; this is the chain rule through the forward stages, with the
// weights recomputed from lse instead of stored:
//   P_ij  = exp(scale * q_i . k_j - lse_i)   (0 where the mask hides j from i)
//   dV_j  = sum_i P_ij dO_i
//   dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i),  D_i = dO_i . O_i  (= sum_j P_ij dP_ij: the softmax Jacobian's row term)
//   dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
// Two kernels, dQ first:
//   attn_bwd_dq:    one workgroup per 256 query rows of one (batch, head), 32 rows per wave; it walks the
//                   key tiles like the forward: S^T = K Q^T and dP^T = V dO^T with one query per lane, then
//                   dQ^T += K^T dS^T. It also writes the row terms D_i and lse_i * log2(e) (0 for a row
//                   without a visible key) into the caller's workspace, each head's rows padded to a multiple
//                   of 64 with zeros, so that the dK/dV kernel fetches whole 64-row tiles of them;
//   attn_bwd_dkdv:  one workgroup per 128 keys of one (batch, K/V head): 8 waves, two per SIMD, each
//                   owning 32 keys and one 32-row half of every query tile; it walks the query tiles (of
//                   every query head of the K/V head's group) and keeps partial dK and dV in registers:
//                   S = Q K^T and dP = dO V^T with one key per lane, then dV^T += dO^T P and
//                   dK^T += Q^T dS with P and dS taken straight from those accumulators; the two halves
//                   are added through LDS at the end.
// Both main kernels use the forward's tile layout and contractions (attn_tiles.h); Q/dO (dK/dV kernel) or
// K/V (dQ kernel) tiles of 64 rows go to LDS by DMA, double buffered. P and dS are rounded to bf16 for the
// MFMAs, products accumulate in float32.
#include "attn_tiles.h"
#include "device_common.h"
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace tsd {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Rows of the wave's 32-row block (this lane's row, 8 bf16 of each 16-wide k-step) as B operands; rows at
// or past n read as zero.
template <int D>
__device__ __forceinline__ void load_rows_b(const uint16_t *__restrict__ base, int row, int n, int hf,
                                            bf16x8 (&reg)[1][D / 16])
{
    const bool ok = row < n;
    const uint16_t *p = base + (size_t)(ok ? row : 0) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 v = ok ? *(const u32x4 *)(p + ks * 16) : u32x4{0u, 0u, 0u, 0u};
        reg[0][ks] = __builtin_bit_cast(bf16x8, v);
    }
}

// P or dS of one 64 x 32 accumulator pair packed as the four 16-row B operands of accumulate_pv.
__device__ __forceinline__ void pack_operands(const f32x16 (&x)[2], bf16x8 (&pb)[1][4])
{
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int jb = c >> 1, r0 = (c & 1) * 8;
        u32x4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = pack_bf16x2(x[jb][r0 + 2 * u], x[jb][r0 + 2 * u + 1]);
        pb[0][c] = __builtin_bit_cast(bf16x8, w);
    }
}

// DMA of one 64-row tile (rows r0 .. r0 + 63 of a [n, D] bf16 matrix) into LDS at slot_off, rows at or past
// n replaced by row n - 1 (their results are masked). voff/drow: this lane's chunk offsets within a tile.
template <int D, int CH, int WAVES>
__device__ __forceinline__ void issue_tile(uint32_t lds0, const uint16_t *src, int r0, int n, uint32_t slot_off,
                                           const uint32_t (&voff)[CH], const int (&drow)[CH], int wave)
{
    const uint16_t *base = src + (size_t)r0 * D;
    const bool tail = r0 + kBlockN > n;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        uint32_t off = voff[j];
        if (tail) {
            const int r = min(drow[j], n - 1 - r0);
            off = off - (uint32_t)(drow[j] - r) * (D * 2);
        }
        lds_dma16(__builtin_amdgcn_readfirstlane(lds0 + slot_off + (j * WAVES + wave) * 1024), base, off);
    }
}

template <int D, int WAVES>
struct TileDma {
    static constexpr int CPR = D / 8;
    static constexpr int CH = kBlockN * CPR / (WAVES * 64);
    static_assert(kBlockN * CPR % (WAVES * 64) == 0, "tile must split evenly over the workgroup");
    uint32_t voff[CH];
    int drow[CH];
    __device__ TileDma(int wave, int lane)
    {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = (j * WAVES + wave) * 64 + lane;
            const int r = c / CPR, x = c % CPR;
            drow[j] = r;
            voff[j] = (uint32_t)(r * D + ((x ^ swz<D>(r)) << 3)) * 2;
        }
    }
};

// acc^T += T_blk^T P_blk: the two 16-row chunks of 32-row block blk of the tile at OFF, read transposed,
// times the two B operands packed from a 32 x 32 accumulator whose rows are that block's rows.
template <int D, int OFF>
__device__ __forceinline__ void accumulate_block(const uint8_t *lds, const TileAddrs<D> &ad, int blk,
                                                 const bf16x8 (&pb)[2], f32x16 (&acc)[D / 32])
{
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
        const uint32_t c_off = (uint32_t)(2 * blk + cl) * 16 * D * 2;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const uint8_t *p0 = lds + ad.v[db][0] + OFF + c_off;
            const uint8_t *p1 = lds + ad.v[db][1] + OFF + c_off;
            const bf16x8 a = lds_tr_pair((const uint16_t *)p0, (const uint16_t *)p1);
            acc[db] = mfma32x32x16(a, pb[cl], acc[db]);
        }
    }
}

__device__ __forceinline__ void pack_block(const f32x16 &x, bf16x8 (&pb)[2])
{
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
        u32x4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = pack_bf16x2(x[cl * 8 + 2 * u], x[cl * 8 + 2 * u + 1]);
        pb[cl] = __builtin_bit_cast(bf16x8, w);
    }
}

// dK and dV for 128 keys of one (batch, K/V head). 8 waves, two per SIMD: wave w owns keys
// (w % 4) * 32 .. +31 of the block and query rows (w / 4) * 32 .. +31 of every 64-row query tile; the
// two waves of a key group add their partial dK and dV through LDS at the end.
template <int D, int MASK>
__global__ __launch_bounds__(512) void attn_bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ dO, const float *__restrict__ lse2, const float *__restrict__ delta,
    const int32_t *__restrict__ valid_lens, float c_log2, float scale, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, int H, int Hkv, int group, int Nq, int Nq_pad, int Nk, int num_kblocks)
{
    constexpr int WAVES = 8, DB = D / 32, TILE_B = kBlockN * D * 2;
    // Q slots 0, 1; dO slots 0, 1; the block's 128 V and K rows (two tiles each, read as B operands); then per slot the
    // tile's 64 values of lse * log2(e) and of D. After the loop the first 4 tiles hold the partial
    // accumulators being added.
    __shared__ __attribute__((aligned(16))) uint8_t smem[8 * TILE_B + 2 * 512];
    constexpr int QS0 = 0, QS1 = TILE_B, GS0 = 2 * TILE_B, GS1 = 3 * TILE_B, VB = 4 * TILE_B, KB = 6 * TILE_B;
    constexpr int LS0 = 8 * TILE_B, LS1 = LS0 + 512;
    static_assert(4 * 64 * 16 * DB * 4 <= 4 * TILE_B, "the reduction area must fit in the tile slots");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int kg = wv & 3, qh = wv >> 2;
    // key block major: every head's first key block, then every head's second, ... With the causal mask
    // the first blocks see the most query tiles, so the longest workgroups are dispatched first
    const int BHkv = (int)(gridDim.x / num_kblocks);
    const int kbk = blockIdx.x / BHkv, bk = blockIdx.x % BHkv;
    const int b = bk / Hkv, hk = bk % Hkv;
    const int kwg0 = kbk * 128, key = kwg0 + kg * 32 + l32;

    int kv_len = Nk;
    if (mask_padding(MASK)) {
        const int L = valid_lens[b];
        kv_len = L < 0 ? 0 : (L > Nk ? Nk : L);
    }

    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.f;

    const TileAddrs<D> ad = tile_addrs<D>(lane);
    const TileDma<D, WAVES> dma(wave, lane);
    const uint32_t lds0 = lds_addr(smem);
    const uint32_t blk_off = (uint32_t)qh * 32 * D * 2;
    // query tiles that can see one of these keys: causal rows below the first key see none of them
    const int nqt = (Nq + kBlockN - 1) / kBlockN;
    const int t0 = mask_causal(MASK) ? min(kwg0 / kBlockN, nqt) : 0;
    const int per_head = kwg0 < kv_len ? nqt - t0 : 0;
    const int n = group * per_head;
    const int h0 = hk * group;

    // the tiles in walking order: (query head, tile) = (h0 + u / per_head, t0 + u % per_head), followed by
    // counters rather than divided out per step
    auto advance = [&](int &bh, int &t) {
        if (++t == nqt) {
            t = t0;
            ++bh;
        }
    };
    auto issue = [&](int bh, int t, uint32_t qs, uint32_t gs, uint32_t ls) {
        issue_tile<D, TileDma<D, WAVES>::CH, WAVES>(lds0, Q + (size_t)bh * Nq * D, t * kBlockN, Nq, qs, dma.voff,
                                                    dma.drow, wave);
        issue_tile<D, TileDma<D, WAVES>::CH, WAVES>(lds0, dO + (size_t)bh * Nq * D, t * kBlockN, Nq, gs, dma.voff,
                                                    dma.drow, wave);
        // the tile's 64 padded rows of lse * log2(e) (wave 0) and of D (wave 1), 16 bytes per lane
        const size_t r0 = (size_t)bh * Nq_pad + (size_t)t * kBlockN;
        if (wv < 2 && lane < 16)
            lds_dma16(lds0 + ls + wv * 256, (wv == 0 ? lse2 : delta) + r0, (uint32_t)lane * 16);
    };
    // the block's K and V rows (rows past Nk repeat row Nk - 1; those keys are masked)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const uint16_t *src = (x == 0 ? K : V) + (size_t)bk * Nk * D;
        const uint32_t dst = x == 0 ? KB : VB;
        issue_tile<D, TileDma<D, WAVES>::CH, WAVES>(lds0, src, kwg0, Nk, dst, dma.voff, dma.drow, wave);
        if (kwg0 + kBlockN < Nk)
            issue_tile<D, TileDma<D, WAVES>::CH, WAVES>(lds0, src, kwg0 + kBlockN, Nk, dst + TILE_B, dma.voff,
                                                        dma.drow, wave);
    }
    // this wave's 32 K and V rows inside them: B operands read with the same lane addresses as a tile's rows
    const uint32_t kv_sub = (uint32_t)(kg >> 1) * TILE_B + (uint32_t)(kg & 1) * 32 * D * 2;
    const uint32_t v_off = VB + kv_sub, k_off = KB + kv_sub;
    int t_c = t0;                          // query tile of the next step
    int bh_f = b * H + h0, t_f = t0;       // (query head, tile) fetched next
    if (n > 0) {
        issue(bh_f, t_f, QS0, GS0, LS0);
        advance(bh_f, t_f);
    }
    wait_vmcnt0();
    __syncthreads();
    auto step = [&](int u, auto parity) {
        constexpr int P = decltype(parity)::value;
        constexpr int QS = P ? QS1 : QS0, GS = P ? GS1 : GS0, LS = P ? LS1 : LS0;
        if (u + 1 < n) {
            issue(bh_f, t_f, P ? QS0 : QS1, P ? GS0 : GS1, P ? LS0 : LS1);
            advance(bh_f, t_f);
        }
        const int t = t_c;
        if (++t_c == nqt) t_c = t0;
        // S = Q K^T and dP = dO V^T for this wave's 32 query rows: one key per lane
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 aq = *(const bf16x8 *)(smem + ad.k[ks] + QS + blk_off);
            const bf16x8 kb = *(const bf16x8 *)(smem + ad.k[ks] + k_off);
            const bf16x8 ag = *(const bf16x8 *)(smem + ad.k[ks] + GS + blk_off);
            const bf16x8 vb = *(const bf16x8 *)(smem + ad.k[ks] + v_off);
            s = mfma32x32x16(aq, kb, s);
            dp = mfma32x32x16(ag, vb, dp);
        }
        // every (row, key) pair of the wave's 32 x 32 block visible (the common case): no per-element test
        const int qlo = t * kBlockN + qh * 32, klast = kwg0 + kg * 32 + 31;
        const bool all_vis = qlo + 31 < Nq && klast < kv_len && (!mask_causal(MASK) || klast <= qlo);
        if (all_vis) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int qo = qh * 32 + g * 8 + hf * 4;  // offset of the lane's 4 rows in the tile
                const f32x4 l4 = *(const f32x4 *)(smem + LS + qo * 4);
                const f32x4 d4 = *(const f32x4 *)(smem + LS + 256 + qo * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = g * 4 + e;
                    const float p = fast_exp2(fmaf(s[r], c_log2, -l4[e]));
                    s[r] = p;
                    dp[r] = p * (dp[r] - d4[e]);
                }
            }
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int qo = qh * 32 + g * 8 + hf * 4;
                const f32x4 l4 = *(const f32x4 *)(smem + LS + qo * 4);
                const f32x4 d4 = *(const f32x4 *)(smem + LS + 256 + qo * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int q = t * kBlockN + qo + e, r = g * 4 + e;
                    const bool vis = q < Nq && key < kv_len && (!mask_causal(MASK) || key <= q);
                    const float p = fast_exp2(fmaf(s[r], c_log2, -l4[e]));
                    s[r] = vis ? p : 0.f;
                    dp[r] = vis ? p * (dp[r] - d4[e]) : 0.f;
                }
            }
        }
        bf16x8 pb[2], sb[2];
        pack_block(s, pb);
        pack_block(dp, sb);
        accumulate_block<D, GS>(smem, ad, qh, pb, dv);  // dV^T += dO^T P
        accumulate_block<D, QS>(smem, ad, qh, sb, dk);  // dK^T += Q^T dS
        wait_vmcnt0();
        __syncthreads();
    };
    for (int u = 0; u < n; u += 2) {
        step(u, std::integral_constant<int, 0>());
        if (u + 1 < n) step(u + 1, std::integral_constant<int, 1>());
    }
    // add the second query half's partial sums into the first's, through LDS (16-byte chunks, lanes
    // contiguous), dK then dV; then the first half stores
    f32x4 *red = (f32x4 *)smem;
    auto reduce = [&](f32x16 (&acc)[DB]) {
        if (qh == 1) {
#pragma unroll
            for (int i = 0; i < DB * 4; ++i)
                red[(kg * DB * 4 + i) * 64 + lane] =
                    f32x4{acc[i / 4][(i % 4) * 4], acc[i / 4][(i % 4) * 4 + 1], acc[i / 4][(i % 4) * 4 + 2],
                          acc[i / 4][(i % 4) * 4 + 3]};
        }
        __syncthreads();
        if (qh == 0) {
#pragma unroll
            for (int i = 0; i < DB * 4; ++i) {
                const f32x4 x = red[(kg * DB * 4 + i) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i / 4][(i % 4) * 4 + e] += x[e];
            }
        }
        __syncthreads();
    };
    reduce(dk);
    reduce(dv);
    if (qh == 0) {
        // dV = acc, dK = scale * acc, rows = keys of this (batch, K/V head)
        store_rows<D, false, kOutBHND, false>(dv, 1.f, key, bk, Hkv, Nk, b, hf, dV);
        store_rows<D, false, kOutBHND, false>(dk, 1.f / scale, key, bk, Hkv, Nk, b, hf, dK);
    }
}

// dQ for 256 query rows of one (batch, head): 8 waves of 32 rows, two per SIMD.
template <int D, int MASK>
__global__ __launch_bounds__(512) void attn_bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ O, const uint16_t *__restrict__ dO, const float *__restrict__ lse,
    float *__restrict__ lse2, float *__restrict__ delta, const int32_t *__restrict__ valid_lens, float c_log2,
    float scale, uint16_t *__restrict__ dQ, int H, int Hkv, int group, int Nq, int Nq_pad, int Nk, int num_qtiles,
    int BH)
{
    constexpr int WAVES = 8, ROWS = WAVES * 32, DB = D / 32, TILE_B = kBlockN * D * 2;
    __shared__ __attribute__((aligned(16))) uint8_t smem[4 * TILE_B];  // K slots 0, 1; V slots 0, 1
    constexpr int KS0 = 0, KS1 = TILE_B, VS0 = 2 * TILE_B, VS1 = 3 * TILE_B;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int bh = blockIdx.x % BH;
    int qt = blockIdx.x / BH;
    if (mask_causal(MASK)) qt = num_qtiles - 1 - qt;  // longest first
    const int b = bh / H, h = bh % H;
    const size_t kvbh = (size_t)b * Hkv + h / group;
    const int q0 = qt * ROWS, qrow = q0 + wave * 32 + l32;

    int kv_len = Nk;
    if (mask_padding(MASK)) {
        const int L = valid_lens[b];
        kv_len = L < 0 ? 0 : (L > Nk ? Nk : L);
    }
    int kv_end = kv_len;
    if (mask_causal(MASK)) kv_end = min(kv_len, q0 + ROWS);
    const int ntiles = (kv_end + kBlockN - 1) / kBlockN;

    bf16x8 qreg[1][D / 16], greg[1][D / 16];
    load_rows_b<D>(Q + (size_t)bh * Nq * D, qrow, Nq, hf, qreg);
    load_rows_b<D>(dO + (size_t)bh * Nq * D, qrow, Nq, hf, greg);
    // The row terms: D_i = dO_i . O_i (this lane's half of every 16-wide k-step, plus the other half from the
    // lane 32 away, which holds the same row) and lse_i * log2(e), 0 for a row without a visible key, so that
    // its masked scores give exp2(-inf) = 0 rather than -inf - (-inf). They go to the workspace for the dK/dV
    // kernel, which runs after this one, with zeros for the rows from Nq up to Nq_pad.
    float d_row, l2_row = 0.f;
    {
        float acc = 0.f;
        if (qrow < Nq) {
            const uint16_t *orow = O + ((size_t)bh * Nq + qrow) * D + hf * 8;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const u32x4 o = *(const u32x4 *)(orow + ks * 16);
                const u32x4 g = __builtin_bit_cast(u32x4, greg[0][ks]);
#pragma unroll
                for (int w = 0; w < 4; ++w) acc += bf16_lo(o[w]) * bf16_lo(g[w]) + bf16_hi(o[w]) * bf16_hi(g[w]);
            }
            const float l = lse[(size_t)bh * Nq + qrow];
            l2_row = isinf(l) ? 0.f : l * kLog2e;
        }
        d_row = half_swap_sum(acc);
        if (hf == 0 && qrow < Nq_pad) {
            delta[(size_t)bh * Nq_pad + qrow] = d_row;
            lse2[(size_t)bh * Nq_pad + qrow] = l2_row;
        }
    }

    f32x16 dq[1][DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[0][i][r] = 0.f;

    const TileAddrs<D> ad = tile_addrs<D>(lane);
    const TileDma<D, WAVES> dma(wave, lane);
    const uint32_t lds0 = lds_addr(smem);
    const uint16_t *Kh = K + kvbh * Nk * D, *Vh = V + kvbh * Nk * D;
    if (ntiles > 0) {
        issue_tile<D, TileDma<D, WAVES>::CH, WAVES>(lds0, Kh, 0, kv_end, KS0, dma.voff, dma.drow, wave);
        issue_tile<D, TileDma<D, WAVES>::CH, WAVES>(lds0, Vh, 0, kv_end, VS0, dma.voff, dma.drow, wave);
    }
    wait_vmcnt0();
    __syncthreads();
    auto step = [&](int t, auto parity) {
        constexpr int P = decltype(parity)::value;
        constexpr int KS = P ? KS1 : KS0, VS = P ? VS1 : VS0;
        if (t + 1 < ntiles) {
            issue_tile<D, TileDma<D, WAVES>::CH, WAVES>(lds0, Kh, (t + 1) * kBlockN, kv_end, P ? KS0 : KS1, dma.voff, dma.drow,
                                          wave);
            issue_tile<D, TileDma<D, WAVES>::CH, WAVES>(lds0, Vh, (t + 1) * kBlockN, kv_end, P ? VS0 : VS1, dma.voff, dma.drow,
                                          wave);
        }
        // S^T = K Q^T and dP^T = V dO^T: one query per lane, rows = keys
        f32x16 s[1][2], dp[1][2];
        scores<D, 1, KS>(smem, ad, qreg, s);
        scores<D, 1, VS>(smem, ad, greg, dp);
        // a tile whose keys every row of the wave sees needs no mask
        const int klast = t * kBlockN + kBlockN - 1;
        if (!(klast < kv_len && (!mask_causal(MASK) || klast <= q0 + __builtin_amdgcn_readfirstlane(wave) * 32)))
            mask_scores<MASK>(s[0], t * kBlockN, kv_len, qrow, hf);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[0][jb][r], c_log2, -l2_row));
                dp[0][jb][r] = p * (dp[0][jb][r] - d_row);
            }
        bf16x8 sb[1][4];
        pack_operands(dp[0], sb);
        accumulate_pv<D, 1, KS>(smem, ad, sb, dq);  // dQ^T += K^T dS^T
        wait_vmcnt0();
        __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
        step(t, std::integral_constant<int, 0>());
        if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>());
    }
    store_rows<D, false, kOutBHND, false>(dq[0], 1.f / scale, qrow, bh, H, Nq, b, hf, dQ);
}

template <int D, int MASK>
hipError_t launch_bwd(const void *Q, const void *K, const void *V, const void *O, const void *dO, const float *lse,
                      const int32_t *vl, float scale, void *dQ, void *dK, void *dV, int B, int H, int Hkv, int Nq,
                      int Nk, float *work, hipStream_t s)
{
    const long long BH = (long long)B * H;
    const int Nq_pad = (Nq + kBlockN - 1) / kBlockN * kBlockN;
    float *lse2 = work, *delta = work + BH * Nq_pad;
    const int group = H / Hkv;
    // scale = 0 must still send masked scores (-inf) to weight 0: -inf * 0 would be NaN in the dQ kernel's
    // exponent, so the factor is held above 0 (every score below 1e-30 in magnitude then weighs as 0 does)
    const float c_log2 = fmaxf(scale * kLog2e, 1e-30f);
    // dQ first: it also writes the row terms the dK/dV kernel reads
    const int num_qtiles = (Nq + 255) / 256;
    const long long g2 = (long long)num_qtiles * B * H;
    if (g2 > 0)
        hipLaunchKernelGGL((attn_bwd_dq_kernel<D, MASK>), dim3((unsigned)g2), dim3(512), 0, s, (const uint16_t *)Q,
                           (const uint16_t *)K, (const uint16_t *)V, (const uint16_t *)O, (const uint16_t *)dO, lse,
                           lse2, delta, vl, c_log2, scale, (uint16_t *)dQ, H, Hkv, group, Nq, Nq_pad, Nk, num_qtiles,
                           B * H);
    const int num_kblocks = (Nk + 127) / 128;
    const long long g1 = (long long)num_kblocks * B * Hkv;
    if (g1 > 0)
        hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, MASK>), dim3((unsigned)g1), dim3(512), 0, s, (const uint16_t *)Q,
                           (const uint16_t *)K, (const uint16_t *)V, (const uint16_t *)dO, lse2, delta, vl, c_log2,
                           scale, (uint16_t *)dK, (uint16_t *)dV, H, Hkv, group, Nq, Nq_pad, Nk, num_kblocks);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_bwd(const void *Q, const void *K, const void *V, const void *O, const void *dO, const float *lse,
                        int mask, const int32_t *vl, float scale, void *dQ, void *dK, void *dV, int B, int H, int Hkv,
                        int Nq, int Nk, float *delta, hipStream_t s)
{
    switch (mask) {
    case kMaskCausal:
        return launch_bwd<D, kMaskCausal>(Q, K, V, O, dO, lse, vl, scale, dQ, dK, dV, B, H, Hkv, Nq, Nk, delta, s);
    case kMaskPadding:
        return launch_bwd<D, kMaskPadding>(Q, K, V, O, dO, lse, vl, scale, dQ, dK, dV, B, H, Hkv, Nq, Nk, delta, s);
    case kMaskCausalPadding:
        return launch_bwd<D, kMaskCausalPadding>(Q, K, V, O, dO, lse, vl, scale, dQ, dK, dV, B, H, Hkv, Nq, Nk, delta,
                                                 s);
    default:
        return launch_bwd<D, kMaskNone>(Q, K, V, O, dO, lse, vl, scale, dQ, dK, dV, B, H, Hkv, Nq, Nk, delta, s);
    }
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                                const float *lse, int mask, const int32_t *valid_lens, float scale, void *dQ, void *dK,
                                void *dV, int B, int H, int Hkv, int Nq, int Nk, int D, float *delta,
                                hipStream_t stream)
{
    if (D == 128)
        return dispatch_bwd<128>(Q, K, V, O, dO, lse, mask, valid_lens, scale, dQ, dK, dV, B, H, Hkv, Nq, Nk, delta,
                                 stream);
    if (D == 64)
        return dispatch_bwd<64>(Q, K, V, O, dO, lse, mask, valid_lens, scale, dQ, dK, dV, B, H, Hkv, Nq, Nk, delta,
                                stream);
    return hipErrorInvalidValue;
}

}  // namespace tsd
