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
// Two kernels, one tile design:
//   * attn_fwd_qb2_kernel (128-wide heads; 64-wide ones when the grid of
//     256-row items covers every CU): persistent, one workgroup per CU of 4
//     wavefronts (one per SIMD) of 64 query rows; each workgroup runs a fixed
//     list of 256-row items, head-major per XCD. Its tile loop is one
//     generated inline-asm statement (gen_qb2_tile.py).
//   * attn_fwd_bf16_kernel (64-wide heads on smaller grids): C++ with MFMA
//     builtins, 32 query rows per wave and two waves per SIMD; 4 waves of
//     one 128-row block, or 8 waves that split the block's key tiles in two
//     halves when even the 4-wave grid leaves CUs idle.
// Shared by both:
//   * Q^T stays in registers as the B operand of v_mfma_f32_32x32x16_bf16.
//   * K and V tiles (64 keys) go HBM -> LDS by DMA (no staging registers),
//     double buffered, while the previous tile is computed.
//   * Software pipeline per wave: the MFMAs of S(t+1) are issued together
//     with the exponentials of S(t), then P(t).V(t) is accumulated.
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
//     it are masked; long and short items alternate so that every
//     workgroup gets the same number of tile steps.
#include "attn_sched.h"
#include "attn_tiles.h"
#include "device_common.h"
#include "kernels.h"

#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

namespace tsd {
namespace {

constexpr float kRescaleSlack = 8.f;    // log2 units the reference max may lag the true max

// Online softmax of one tile of scores of one query block, base 2 (scale *
// log2(e) folded into c_log2 > 0, so a masked score -inf gives exactly
// exp2(-inf) = 0). The reference max mc_run (already scaled) only moves
// when the tile's max exceeds it by more than kRescaleSlack: exponents stay
// <= the slack, P <= 2^slack is still exact up to rounding, and the rescale
// of O and l by e^{m - m'} is needed on few tiles.
//
// Part 1: the tile's max, the new reference, and the factor alpha that O and
// l must be multiplied by before this tile is added (1 when the reference
// did not move). Returns the reference to subtract in the exponents.
__device__ __forceinline__ float softmax_ref(const f32x16 (&s)[2], float &mc_run, float &l_run, float c_log2,
                                             float &alpha, bool &upd)
{
    float mx = s[0][0];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
    mx = half_swap_max(mx);
    const float tmax = mx * c_log2;
    upd = tmax > mc_run + kRescaleSlack;
    const float mc_new = upd ? tmax : mc_run;
    alpha = !upd ? 1.f : (mc_run == -INFINITY ? 0.f : fast_exp2(mc_run - mc_new));
    mc_run = mc_new;
    l_run *= alpha;
    return (mc_new == -INFINITY) ? 0.f : mc_new;
}

// Part 2: P = exp2(s * c_log2 - mref) rounded to bf16 -- the B operands of
// the P.V MFMAs, 16 keys each -- and the row sum of those same rounded values
// into l_run, so that the weights applied to V sum to exactly l (a dominant
// weight's rounding then cancels in O / l instead of showing up in O).
__device__ __forceinline__ void softmax_exp(f32x16 (&s)[2], bf16x8 (&pb)[4], float mref, float c_log2, float &l_run)
{
    float lsum[2] = {0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int jb = c >> 1, r0 = (c & 1) * 8;
        u32x4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float p0 = fast_exp2(fmaf(s[jb][r0 + 2 * u], c_log2, -mref));
            const float p1 = fast_exp2(fmaf(s[jb][r0 + 2 * u + 1], c_log2, -mref));
            w[u] = pack_bf16x2(p0, p1);
            lsum[u & 1] = add_bf16x2(w[u], lsum[u & 1]);
        }
        pb[c] = __builtin_bit_cast(bf16x8, w);
    }
    l_run += lsum[0] + lsum[1];
}

// Log-sum-exp of one query row, written by the lanes of the first half-wave: the weights were
// P = exp2(s * scale * log2(e) - mc) and l = sum P, so ln sum_j exp(s_j * scale) = ln(2) * (mc + log2(l))
// (-inf for a row without a visible key, l = 0).
__device__ __forceinline__ void store_lse(float *__restrict__ lse, float l, float mc, int qrow, int bh, int Nq,
                                          int hf)
{
    if (hf == 0 && qrow < Nq)
        lse[(size_t)bh * Nq + qrow] = l > 0.f ? (mc + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// O = O_acc / l for one block of 32 query rows, as bf16, staged through a 32-row LDS area of the wave (32 * D * 2
// bytes) so that every store writes whole rows (64 / (D / 8) rows per instruction) instead of 16 bytes per row.
// The stores go through a buffer descriptor that covers exactly the block's rows below Nq, so rows past Nq are
// dropped by the range check (no per-row branch). The area's 16-byte chunks are XOR-swizzled by row so that both
// the 8-byte writes and the 16-byte reads spread over the banks.
// pk[db] holds the block's 16 values of the lane, already divided by the row sum, as bf16 pairs.
template <int D, int OLAYOUT>
__device__ __forceinline__ void store_rows_bf16_staged(const u32x8 (&pk)[D / 32], int row0, int bh, int H, int Nq,
                                                       int b, int lane, uint8_t *stage, void *__restrict__ Out)
{
    constexpr int CPR = D / 8, RPR = 64 / CPR, ROWB = D * 2;
    // computed here rather than kept from the kernel's start: the lane-dependent addresses would otherwise
    // be hoisted out of the workgroup's item loop and held across the tile loop, which has no registers
    // to spare
    asm volatile("" : "+v"(lane));
    const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int c = db * 4 + rg;
            const u32x2 v = {pk[db][rg * 2], pk[db][rg * 2 + 1]};
            *(u32x2 *)(stage + l32 * ROWB + ((c ^ (l32 & (CPR - 1))) << 4) + hf * 8) = v;
        }
    // the wave's LDS operations complete in order: keep the compiler from moving the reads up
    asm volatile("" ::: "memory");
    row0 = __builtin_amdgcn_readfirstlane(row0);
    const int stride = (OLAYOUT == kOutBHND ? D : H * D) * 2;  // bytes from one output row to the next
    const size_t first = OLAYOUT == kOutBHND ? ((size_t)bh * Nq + row0) * D : (((size_t)b * Nq + row0) * H + bh % H) * D;
    const int nrows = min(32, Nq - row0);
    const int nbytes = nrows > 0 ? (nrows - 1) * stride + D * 2 : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((uint16_t *)Out + first, (short)0, nbytes, 0x20000);
#pragma unroll
    for (int i = 0; i < 32 / RPR; ++i) {
        const int r = i * RPR + lane / CPR, cc = lane % CPR;
        const u32x4 d = *(const u32x4 *)(stage + r * ROWB + ((cc ^ (r & (CPR - 1))) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(d, rs, r * stride + cc * 16, 0, 0);
    }
    asm volatile("" ::: "memory");
}

// The C++ kernel (64-wide heads): one query block of 32 rows per wave, two waves per SIMD.
template <int D, int QB>
struct AttnTraits {
    static constexpr int kWavesPerEU = 2;
};

// KSPLIT = 2: the workgroup's waves form two sets of WAVES / 2, each set running the same query rows over
// one half of the key tiles (for grids too small to give every SIMD two waves otherwise); the halves' online
// softmax states (reference max, sum, partial output) are merged through LDS at the end.
template <int D, int QB, int MASK, bool OUT_F32, int OLAYOUT, int WAVES, int KSPLIT>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(
    AttnTraits<D, QB>::kWavesPerEU, AttnTraits<D, QB>::kWavesPerEU))) void attn_fwd_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ valid_lens, float c_log2, void *__restrict__ Out, int H, int Nq, int Nk,
    int num_qtiles, int BH, AttnHeads hd)
{
    static_assert(QB == 1, "one query block per wave");
    static_assert(KSPLIT == 1 || KSPLIT == 2, "one or two key halves");
    constexpr int RB = WAVES / KSPLIT; // waves per key half = 32-row blocks per workgroup
    constexpr int RW = QB * 32;        // query rows per wave
    constexpr int BM = RB * RW;        // query rows per workgroup
    constexpr int KS = D / 16;         // k-steps of the Q K^T contraction
    constexpr int DB = D / 32;         // 32-row blocks of O^T
    constexpr int TILE_B = kBlockN * D * 2;                     // bytes of one K (or V) tile
    constexpr int CPR = D / 8;                                  // 16-byte chunks per row
    constexpr int CH = kBlockN * CPR / (RB * 64);               // DMA chunks per lane per tensor per tile
    static_assert(kBlockN * CPR % (RB * 64) == 0, "tile must split evenly over the waves of a key half");
    static_assert(4 * TILE_B <= 65536, "LDS offsets must fit instruction immediates");
    // LDS bytes, per key half: [K slot 0 | K slot 1 | V slot 0 | V slot 1]; tile i uses slot i % 2
    constexpr int HALF_B = 4 * TILE_B;
    __shared__ __attribute__((aligned(16))) uint8_t smem[KSPLIT * HALF_B];
    constexpr int KSLOT0 = 0, KSLOT1 = TILE_B, VSLOT0 = 2 * TILE_B, VSLOT1 = 3 * TILE_B;

    const int tid = threadIdx.x, lane = tid & 63;
    // kh: the wave's key half; wave: its 32-row block within the workgroup
    const int kh = __builtin_amdgcn_readfirstlane((tid >> 6) / RB), wave = (tid >> 6) % RB;
    const int l32 = lane & 31, hf = lane >> 5;

    // q-tile-major order: the q-tiles of one head are BH ids apart, which
    // lands them on the same XCD (and L2) when BH is a multiple of 8
    const int id = blockIdx.x;
    const int bh = id % BH;
    int qt = id / BH;
    if (mask_causal(MASK)) qt = num_qtiles - 1 - qt;
    const int b = bh / H;
    const int q0 = qt * BM;

    int kv_len = Nk;
    if (mask_padding(MASK)) {
        const int L = valid_lens[b];
        kv_len = L < 0 ? 0 : (L > Nk ? Nk : L);
    }
    int kv_end = kv_len;
    if (mask_causal(MASK)) kv_end = min(kv_len, q0 + BM);
    const int ntiles = (kv_end + kBlockN - 1) / kBlockN;

    const size_t kvh = (size_t)b * hd.kv_heads + (bh - b * H) / hd.group;
    const uint16_t *Kh = K + kvh * Nk * D;
    const uint16_t *Vh = V + kvh * Nk * D;

    // Q^T as B operands: lane holds Q[qrow][ks*16 + hf*8 .. +7]
    const int qmin_w = q0 + wave * RW, qmax_w = qmin_w + RW - 1;
    int qrow[QB];
    bf16x8 qreg[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        qrow[qb] = qmin_w + qb * 32 + l32;
        const bool ok = qrow[qb] < Nq;
        const uint16_t *qp = Q + ((size_t)bh * Nq + (ok ? qrow[qb] : 0)) * D + hf * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = ok ? *(const u32x4 *)(qp + ks * 16) : u32x4{0u, 0u, 0u, 0u};
            qreg[qb][ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    f32x16 acc[QB][DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qb][i][r] = 0.f;
    float mc_run[QB], l_run[QB];  // running (scaled, base-2) reference max and row sum
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mc_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
    }

    TileAddrs<D> ad = tile_addrs<D>(lane);
    if constexpr (KSPLIT > 1) {
        // the second key half's slots: its base folded into the address registers (slot offsets stay
        // instruction immediates)
        const uint32_t hb = (uint32_t)__builtin_amdgcn_readfirstlane(kh * HALF_B);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint32_t x = ad.k[ks] + hb;
            asm volatile("" : "+v"(x));
            ad.k[ks] = x;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                uint32_t x = ad.v[db][h2] + hb;
                asm volatile("" : "+v"(x));
                ad.v[db][h2] = x;
            }
    }

    // DMA j of this wave fills the 64 consecutive LDS chunks
    // [(j*WAVES + wave)*64, +64) of a tile; lane i fetches the global chunk
    // that the swizzle puts in slot i. Rows at or past kv_end are never
    // visible to this workgroup: they are not read; the last valid row is
    // fetched in their place (its weight is exactly 0).
    const uint32_t lds0 = lds_addr(smem);
    uint32_t voff[CH];
    int drow[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = (j * RB + wave) * 64 + lane;
        const int r = c / CPR, x = c % CPR;
        drow[j] = r;
        voff[j] = (uint32_t)(r * D + ((x ^ swz<D>(r)) << 3)) * 2;
    }
    auto issue = [&](const uint16_t *src, int t, uint32_t slot_off) {
        const int k0 = t * kBlockN;
        const uint16_t *base = src + (size_t)k0 * D;
        const bool tail = k0 + kBlockN > kv_end;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            uint32_t off = voff[j];
            if (tail) {
                const int r = min(drow[j], kv_end - 1 - k0);
                off = off - (uint32_t)(drow[j] - r) * (D * 2);
            }
            lds_dma16(__builtin_amdgcn_readfirstlane(lds0 + kh * HALF_B + slot_off + (j * RB + wave) * 1024), base,
                      off);
        }
    };

    // tiles this wave computes: causal rows <= qmax_w see no key past qmax_w
    const int ntiles_w = mask_causal(MASK) ? min(ntiles, qmax_w / kBlockN + 1) : ntiles;
    auto needs_mask = [&](int t) {
        const int k0 = t * kBlockN;
        return (k0 + kBlockN > kv_len) || (mask_causal(MASK) && k0 + kBlockN - 1 > qmin_w);
    };

    // Online-softmax bookkeeping for one tile whose scores are in `cur`:
    // mask, move the reference max, rescale O when any row of the wave needs
    // it; returns the reference per query block in mref.
    auto prepare = [&](int t, f32x16(&cur)[QB][2], float (&mref)[QB]) {
        if (needs_mask(t)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) mask_scores<MASK>(cur[qb], t * kBlockN, kv_len, qrow[qb], hf);
        }
        float alpha[QB];
        bool upd = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            bool u;
            mref[qb] = softmax_ref(cur[qb], mc_run[qb], l_run[qb], c_log2, alpha[qb], u);
            upd = upd || u;
        }
        if (__builtin_amdgcn_ballot_w64(upd)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int i = 0; i < DB; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[qb][i][r] *= alpha[qb];
                }
    };

    // This wave's key half: tiles [tb, te) of the workgroup's ntiles (all of them without a split); nsteps
    // steps for every wave (the halves differ by at most one tile), each ending in the same barrier.
    const int nt0 = KSPLIT == 1 ? ntiles : (ntiles + 1) / 2;
    const int tb = kh == 0 ? 0 : nt0, te = kh == 0 ? nt0 : ntiles;
    const int nh = te - tb;                                  // tiles this half fetches
    const int nwh = min(max(ntiles_w - tb, 0), nh);           // tiles of the half this wave computes
    const int nsteps = nt0;
    {
        // Software pipeline: iteration t reads K(t+1) and V(t) from LDS while
        // the DMA fills K(t+2) and V(t+1); the MFMAs of S(t+1) are issued in
        // the same basic block as the exponentials of S(t). (t: the tile's index within the half.)
        f32x16 sa[QB][2], sb[QB][2];
        if (nsteps > 0) {
            if (nh > 0) issue(Kh, tb, KSLOT0);
            wait_vmcnt0();
            __syncthreads();
            if (nh > 1) issue(Kh, tb + 1, KSLOT1);
            if (nh > 0) issue(Vh, tb, VSLOT0);
            if (nwh > 0) scores<D, QB, KSLOT0>(smem, ad, qreg, sa);
            wait_vmcnt0();
            __syncthreads();
        }
        auto step = [&](int t, auto parity, f32x16(&cur)[QB][2], f32x16(&nxt)[QB][2]) {
            constexpr int P = decltype(parity)::value;  // t % 2
            constexpr int KNEXT = P ? KSLOT0 : KSLOT1;  // K(t+1) lives in slot (t+1)%2
            constexpr int VCUR = P ? VSLOT1 : VSLOT0;   // V(t) in slot t%2
            if (t + 2 < nh) issue(Kh, tb + t + 2, P ? KSLOT1 : KSLOT0);
            if (t + 1 < nh) issue(Vh, tb + t + 1, P ? VSLOT0 : VSLOT1);
            if (t < nwh) {
                float mref[QB];
                prepare(tb + t, cur, mref);
                bf16x8 pb[QB][4];
                // S(t+1) also on the wave's last tile (one set of MFMAs whose result is never read): a
                // branch here would leave the compiler two versions of the O accumulator to reconcile
                scores<D, QB, KNEXT>(smem, ad, qreg, nxt);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) softmax_exp(cur[qb], pb[qb], mref[qb], c_log2, l_run[qb]);
                accumulate_pv<D, QB, VCUR>(smem, ad, pb, acc);
            }
            wait_vmcnt0();
            __syncthreads();
        };
        for (int t = 0; t < nsteps; t += 2) {
            step(t, std::integral_constant<int, 0>(), sa, sb);
            if (t + 1 < nsteps) step(t + 1, std::integral_constant<int, 1>(), sb, sa);
        }
    }

    if constexpr (KSPLIT > 1) {
        // Merge the halves, row by row (lane by lane: both halves hold the same rows and output columns in
        // the same lanes). With references m_a, m_b: m = max, each half scaled by exp2(m_x - m) (0 for a half
        // without a visible key), O = O_a s_a + O_b s_b, l = l_a s_a + l_b s_b. The second half's state goes
        // through LDS (the tile slots are free: the last step ended in a barrier).
        constexpr int NV = DB * 16 + 2;
        float *part = (float *)smem + wave * (NV * 64);
        if (kh == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) part[(db * 16 + r) * 64 + lane] = acc[0][db][r];
            part[(NV - 2) * 64 + lane] = mc_run[0];
            part[(NV - 1) * 64 + lane] = l_run[0];
        }
        __syncthreads();
        if (kh == 1) return;
        const float mb = part[(NV - 2) * 64 + lane], lb = part[(NV - 1) * 64 + lane];
        const float m = fmaxf(mc_run[0], mb);
        const float sa = mc_run[0] == -INFINITY ? 0.f : fast_exp2(mc_run[0] - m);
        const float sb = mb == -INFINITY ? 0.f : fast_exp2(mb - m);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[0][db][r] = acc[0][db][r] * sa + part[(db * 16 + r) * 64 + lane] * sb;
        l_run[0] = l_run[0] * sa + lb * sb;
        mc_run[0] = m;
    }

    // ---- epilogue: O = O_acc / l (0 for a row with no visible key) ----
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) store_rows<D, OUT_F32, OLAYOUT>(acc[qb], l_run[qb], qrow[qb], bh, H, Nq, b, hf, Out);
    if (hd.lse) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) store_lse(hd.lse, half_swap_sum(l_run[qb]), mc_run[qb], qrow[qb], bh, Nq, hf);
    }
}

#include "attn_qb2_tile.inc"
#include "attn_qb2_tile_d64.inc"

// Row max of one query block's 64 scores of a tile (both half-waves).
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2])
{
    float mx = s[0][0];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
    return half_swap_max(mx);
}

// ---------------------------------------------------------------------------
// 128- and 64-wide heads, 64 query rows per wave (two blocks of 32), 4 waves per
// workgroup, one wave per SIMD. Every K or V operand read from LDS feeds two
// MFMAs, which halves the LDS bytes per MFMA against 32-row waves. The whole
// tile loop of a wave -- S(t+1) MFMAs, the exponentials of S(t), the
// P(t).V(t) and row-sum MFMAs, the row max of S(t+1), the DMA of later K/V
// tiles, masking, reference max and rescale of O -- is one inline-asm
// statement with a fixed schedule (generated by gen_qb2_tile.py), since a
// single wave per SIMD has no partner wave to hide its latencies.
//
// The grid is persistent: one workgroup per CU, each taking work items
// (256 query rows of one (batch, head)) in a fixed order. For the causal mask
// items are ranked heaviest first and dealt out boustrophedon-wise (even
// rounds in workgroup order, odd rounds reversed by groups of 8 so that a
// workgroup keeps its XCD), which gives every workgroup the same number of
// tiles when the ranks split evenly; each workgroup starts its list at a
// different item so that item boundaries are spread in time. The next item's
// Q rows are fetched into LDS while the current item runs, and the tile
// loop's fetches run on past the item's last tile into the next item's first
// K/V tiles (tiles take slots of parity (t + off) % 2, off carried from item
// to item). Outputs go out as whole rows through an LDS staging area.
// LDS: K0 K1 V0 V1, the four waves' Q rows, 32 rows of staging per wave
// (160 KiB for 128-wide heads, 80 KiB for 64-wide ones).
//
// Registers: O, Q^T, the row sums and an all-ones operand in AGPRs, the two
// score buffers, P and the operand staging in VGPRs, at the physical
// registers the asm names.
struct Qb2Item {
    int valid, bh, b, kvh, q0, kv_len, kv_end, ntiles;
};

// The parameters of the item (bh, query block qt of the schedule's order); valid = false: no item.
template <int MASK>
__device__ __forceinline__ Qb2Item qb2_item(bool valid, int bh, int qt, int num_qtiles, int H, int Nk,
                                            const int32_t *__restrict__ valid_lens, const AttnHeads &hd)
{
    constexpr int BM = 256;
    Qb2Item it{};
    it.valid = valid;
    if (!it.valid) return it;
    it.bh = bh;
    if (mask_causal(MASK)) qt = num_qtiles - 1 - qt;
    it.b = it.bh / H;
    it.kvh = it.b * hd.kv_heads + (it.bh - it.b * H) / hd.group;
    it.q0 = qt * BM;
    it.kv_len = Nk;
    if (mask_padding(MASK)) {
        const int L = valid_lens[it.b];
        it.kv_len = L < 0 ? 0 : (L > Nk ? Nk : L);
    }
    it.kv_end = it.kv_len;
    if (mask_causal(MASK)) it.kv_end = min(it.kv_len, it.q0 + BM);
    it.ntiles = (it.kv_end + kBlockN - 1) / kBlockN;
    // wave-uniform by construction; say so, so that they stay in SGPRs
    it.bh = __builtin_amdgcn_readfirstlane(it.bh);
    it.b = __builtin_amdgcn_readfirstlane(it.b);
    it.kvh = __builtin_amdgcn_readfirstlane(it.kvh);
    it.q0 = __builtin_amdgcn_readfirstlane(it.q0);
    it.kv_len = __builtin_amdgcn_readfirstlane(it.kv_len);
    it.kv_end = __builtin_amdgcn_readfirstlane(it.kv_end);
    it.ntiles = __builtin_amdgcn_readfirstlane(it.ntiles);
    return it;
}

template <int D, int MASK, bool OUT_F32, int OLAYOUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_fwd_qb2_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ valid_lens, float c_log2, void *__restrict__ Out, int H, int Nq, int Nk,
    int num_qtiles, int BH, AttnHeads hd)
{
    constexpr int QB = 2, WAVES = 4, RW = 64;
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int TILE_B = kBlockN * D * 2;
    constexpr int CPR = D / 8;
    constexpr int CH = kBlockN * CPR / (WAVES * 64);
    static_assert(kBlockN * CPR % (WAVES * 64) == 0, "tile must split evenly over the workgroup");
    // K0 K1 V0 V1 (the tile loop's slots), then the Q rows of the four waves (the next item's while the
    // current item's loop runs its last tiles)
    constexpr int STAGE_W = 32 * D * 2;  // per wave: 32 output rows (the last item's epilogue)
    __shared__ __attribute__((aligned(256))) uint8_t smem[8 * TILE_B + WAVES * STAGE_W];
    constexpr int KSLOT0 = 0, KSLOT1 = TILE_B, VSLOT0 = 2 * TILE_B, VSLOT1 = 3 * TILE_B, QSLOT = 4 * TILE_B;
    constexpr int STAGE = 8 * TILE_B;  // the waves' output staging areas (bf16 output)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int G = gridDim.x, w = blockIdx.x;
    const int num_items = num_qtiles * BH;

    const TileAddrs<D> ad = tile_addrs<D>(lane);
    const uint32_t lds0 = lds_addr(smem);
    // lane's row of each 1 KiB DMA chunk and its byte offset (16-byte chunks XOR-swizzled)
    auto dma_row = [&](int j) { return ((j * WAVES + wave) * 64 + lane) / CPR; };
    uint32_t voff[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int r = dma_row(j), x = ((j * WAVES + wave) * 64 + lane) % CPR;
        voff[j] = (uint32_t)(r * D + ((x ^ swz<D>(r)) << 3)) * 2;
    }
    // LDS byte addresses of the operand reads (the tile offsets are instruction immediates)
    uint32_t kaddr[KS], vaddr[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kaddr[ks] = lds0 + ad.k[ks];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        vaddr[db][0] = lds0 + ad.v[db][0];
        vaddr[db][1] = lds0 + ad.v[db][1];
    }

    const uint32_t lbw = __builtin_amdgcn_readfirstlane(lds0 + wave * 1024);
    // wave-uniform values go to the asm in SGPRs
    auto u = [](int x) { return (int32_t)__builtin_amdgcn_readfirstlane(x); };
    // 64 rows [r0, r0 + 64) of a [rows, D] matrix (r_end >= 1 rows) into an LDS tile slot (swizzled like
    // every tile); rows at or past r_end repeat row r_end - 1, so nothing past the matrix is read. The
    // offsets are taken from the first fetched row, r_base <= every fetched row, so none is negative
    // (the whole tile may lie past r_end: the rows of a last partial Q tile).
    auto issue = [&](const uint16_t *mat, int r0, int r_end, uint32_t slot_off) {
        const int r_base = min(r0, r_end - 1);
        const uint16_t *base = mat + (size_t)r_base * D;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            // voff[j] = lane's tile row * (D * 2) + its (swizzled) chunk's byte offset in the row
            const int row = min(r0 + (int)(voff[j] / (D * 2)), r_end - 1);
            const uint32_t off = (voff[j] % (D * 2)) + (uint32_t)(row - r_base) * (D * 2);
            lds_dma16(lbw + slot_off + j * WAVES * 1024, base, off);
        }
    };
    // first tiles of an item whose slots take parity off: K(0), K(1), V(0). The tile loop fetches no row at
    // or past kv_end; the other V slot is read (with weight 0) before the item's own fetches have written
    // such rows, so it holds zeros rather than what LDS held before. (Each wave fetches a quarter of every
    // tile.)
    auto first_tiles = [&](const Qb2Item &it, int off) {
#pragma unroll
        for (int i = 0; i < TILE_B / (16 * 256); ++i)
            *(u32x4 *)(smem + VSLOT0 + (1 - off) * TILE_B + (i * 256 + tid) * 16) = u32x4{0u, 0u, 0u, 0u};
        if (it.ntiles > 0) {
            const uint16_t *Kh = K + (size_t)it.kvh * Nk * D, *Vh = V + (size_t)it.kvh * Nk * D;
            issue(Kh, 0, it.kv_end, KSLOT0 + off * TILE_B);
            if (it.ntiles > 1) issue(Kh, kBlockN, it.kv_end, KSLOT0 + (1 - off) * TILE_B);
            issue(Vh, 0, it.kv_end, VSLOT0 + off * TILE_B);
        }
    };
    // the item's Q rows (the four waves' 64-row blocks) into the Q slots, each block through a buffer
    // descriptor that covers its rows below Nq: rows past Nq (a last partial block) read as zeros
    auto q_tiles = [&](const Qb2Item &it) {
        const uint16_t *Qh = Q + ((size_t)it.bh * Nq + it.q0) * D;
#pragma unroll
        for (int qw = 0; qw < WAVES; ++qw) {
            const int rows = __builtin_amdgcn_readfirstlane(min(max(Nq - it.q0 - qw * RW, 0), RW));
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void *)(Qh + (size_t)qw * RW * D), (short)0, rows * D * 2, 0x20000);
#pragma unroll
            for (int j = 0; j < CH; ++j) lds_dma16_rsrc(rs, lbw + QSLOT + qw * TILE_B + j * WAVES * 1024, voff[j]);
        }
    };

    int k = 0, off = 0;
    const bool by_heads = qb2_heads_schedule(G, BH, num_qtiles);
    // the workgroup's j-th item
    auto item = [&](int j) {
        int bh = 0, qt = 0;
        bool valid;
        if (by_heads) {
            valid = qb2_sched_heads(w, j, G, BH, num_qtiles, bh, qt);
        } else {
            const int p = qb2_sched(w, j, G, num_items);
            valid = p < num_items;
            qt = p / BH;
            bh = p - qt * BH;
        }
        return qb2_item<MASK>(valid, bh, qt, num_qtiles, H, Nk, valid_lens, hd);
    };
    // Q^T of this wave's rows from its Q slot into the AGPRs the tile loop names, and O = 0 (qb2_init; the slot
    // offset is computed there so that the KS addresses are not held across the tile loop)
    bf16x8 qreg[QB][KS];
    f32x16 acc[QB][DB];
    Qb2Item cur = item(0);
    if (!cur.valid) return;
    q_tiles(cur);
    first_tiles(cur, 0);
    wait_vmcnt0();
    __syncthreads();
    {
        uint32_t wq = QSLOT + wave * TILE_B;
        asm volatile("" : "+v"(wq));
        uint32_t qa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = kaddr[ks] + wq;
        if constexpr (D == 128) qb2_init(acc, qreg, qa);
        else qb2_init_d64(acc, qreg, qa);
    }
    // bf16 output: the tile loop of each later item starts with the turn, which packs the previous item's
    // output rows while the new item's first scores are computed (turn = 1); the parameters of those rows
    constexpr int OSTRIDE = (OLAYOUT == kOutBHND ? D : 0) * 2;  // BNHD: H * D * 2, below
    const uint32_t ostride = OSTRIDE ? OSTRIDE : (uint32_t)H * D * 2;
    int32_t turn = 0;
    float inv[QB] = {0.f, 0.f};
    uint64_t ob = 0;
    uint32_t ob_bytes = 0;
    for (;;) {
        const Qb2Item nxt = item(++k);
        const int qmin_w = cur.q0 + wave * RW, qmax_w = qmin_w + RW - 1;
        int32_t lim[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            // a visible key of row qrow satisfies key <= lim; the asm compares the key's
            // offset within the tile (lane half included) against lim - tile start
            const int qrow = qmin_w + qb * 32 + l32;
            lim[qb] = (mask_causal(MASK) ? min(qrow, cur.kv_len - 1) : cur.kv_len - 1) - hf * 4;
        }
        const int ntiles_w = mask_causal(MASK) ? min(cur.ntiles, qmax_w / kBlockN + 1) : cur.ntiles;
        // The tiles of this wave that need a mask: from the tile crossing kv_len on (masked after their
        // scores, out of line, against key <= lim), or, causal, the wave's diagonal tile, which starts at
        // the wave's first row (a multiple of 64) and is masked inside its step. Causal rows past Nk are
        // past Nq: not stored. With the padding mask as well, the diagonal tile keeps its in-step mask
        // only when no key before its end (or before Nk) is past kv_len; otherwise every tile from the
        // one crossing kv_len on takes the general mask, which applies both rules.
        int t_mask = cur.kv_len / kBlockN, t_diag = 0x7fffffff;
        if (mask_causal(MASK) &&
            (!mask_padding(MASK) || cur.kv_len >= min(Nk, (qmin_w / kBlockN + 1) * kBlockN))) {
            t_mask = 0x7fffffff;
            t_diag = qmin_w / kBlockN;
        }
        const uint64_t kh = (uint64_t)(K + (size_t)cur.kvh * Nk * D), vh = (uint64_t)(V + (size_t)cur.kvh * Nk * D);
        const Qb2Item &nn = nxt.valid ? nxt : cur;  // a valid address even when there is no next item
        const uint64_t nkh = (uint64_t)(K + (size_t)nn.kvh * Nk * D), nvh = (uint64_t)(V + (size_t)nn.kvh * Nk * D);
        // the next item's Q rows, fetched into the Q slots by the loop once every wave has read this item's
        const uint64_t nq = (uint64_t)(Q + ((size_t)nn.bh * Nq + nn.q0) * D);
        const int nq_rows = nxt.valid ? Nq - nxt.q0 : 0;
        float l_run[QB] = {0.f, 0.f}, mc0 = -INFINITY, mc1 = -INFINITY;
        if constexpr (D == 128)
            qb2_loop(acc, qreg, kaddr, vaddr, voff, lim[0], lim[1], c_log2, l_run[0], l_run[1], mc0, mc1,
                 u(0), u(cur.ntiles), u(ntiles_w), u(t_mask), u(cur.kv_end), u((uint32_t)kh),
                 u((uint32_t)(kh >> 32)), u((uint32_t)vh), u((uint32_t)(vh >> 32)), lbw, u(off),
                 u((uint32_t)nkh), u((uint32_t)(nkh >> 32)), u((uint32_t)nvh), u((uint32_t)(nvh >> 32)),
                 u(nxt.valid ? nxt.kv_end : 0), u(t_diag), u(turn), inv[0], inv[1], u((uint32_t)ob),
                 u((uint32_t)(ob >> 32)), u(ob_bytes), u(ostride), u(QSLOT + wave * TILE_B),
                 u(lds0 + QSLOT + wave * TILE_B), u((uint32_t)nq), u((uint32_t)(nq >> 32)), u(nq_rows));
        else
            qb2_loop_d64(acc, qreg, kaddr, vaddr, voff, lim[0], lim[1], c_log2, l_run[0], l_run[1], mc0, mc1,
                 u(0), u(cur.ntiles), u(ntiles_w), u(t_mask), u(cur.kv_end), u((uint32_t)kh),
                 u((uint32_t)(kh >> 32)), u((uint32_t)vh), u((uint32_t)(vh >> 32)), lbw, u(off),
                 u((uint32_t)nkh), u((uint32_t)(nkh >> 32)), u((uint32_t)nvh), u((uint32_t)(nvh >> 32)),
                 u(nxt.valid ? nxt.kv_end : 0), u(t_diag), u(turn), inv[0], inv[1], u((uint32_t)ob),
                 u((uint32_t)(ob >> 32)), u(ob_bytes), u(ostride), u(QSLOT + wave * TILE_B),
                 u(lds0 + QSLOT + wave * TILE_B), u((uint32_t)nq), u((uint32_t)(nq >> 32)), u(nq_rows));
        if (hd.lse) {
            store_lse(hd.lse, l_run[0], mc0, cur.q0 + wave * RW + l32, cur.bh, Nq, hf);
            store_lse(hd.lse, l_run[1], mc1, cur.q0 + wave * RW + 32 + l32, cur.bh, Nq, hf);
        }
        // the row sums come from an MFMA over all 64 lanes: each lane holds its row's whole sum
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) inv[qb] = l_run[qb] > 0.f ? __builtin_amdgcn_rcpf(l_run[qb]) : 0.f;
        if constexpr (OUT_F32) {
            mfma_fence_a8(acc);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                store_rows<D, OUT_F32, OLAYOUT, false>(acc[qb], l_run[qb], cur.q0 + wave * RW + qb * 32 + l32, cur.bh,
                                                       H, Nq, cur.b, hf, Out);
        } else if (!nxt.valid) {
            // the last item's rows: O / l packed straight from the O registers, then staged and stored
            u32x8 pk[QB][DB];
            if constexpr (D == 128) qb2_out_bf16(acc, inv[0], inv[1], pk);
            else qb2_out_bf16_d64(acc, inv[0], inv[1], pk);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                store_rows_bf16_staged<D, OLAYOUT>(pk[qb], cur.q0 + wave * RW + qb * 32, cur.bh, H, Nq, cur.b, lane,
                                                   smem + STAGE + wave * STAGE_W, Out);
        } else {
            // this item's rows, written by the next item's turn: the wave's 64 rows from row0, those below Nq
            const int row0 = cur.q0 + wave * RW;
            const size_t first = OLAYOUT == kOutBHND ? ((size_t)cur.bh * Nq + row0) * D
                                                     : (((size_t)cur.b * Nq + row0) * H + cur.bh % H) * D;
            const int nrows = min(RW, Nq - row0);
            ob = (uint64_t)((uint16_t *)Out + first);
            ob_bytes = nrows > 0 ? (uint32_t)(nrows - 1) * ostride + D * 2 : 0u;
            turn = 1;
        }
        if (!nxt.valid) break;
        // The loop's last steps fetched the next item's K(0), K(1), V(0) into the slots of parity
        // (off + ntiles) % 2 and ended with a barrier after they (and the next Q rows) had arrived. With
        // fewer than two tiles it did not (K(0) of the next item would have been due before this item's
        // first step): fetch them here and wait for them (and for the Q rows).
        const int off_next = (off + cur.ntiles) & 1;
        if (cur.ntiles < 2) {
            first_tiles(nxt, off_next);
            wait_vmcnt0();
            __syncthreads();
        }
        if constexpr (OUT_F32) {
            uint32_t wq = QSLOT + wave * TILE_B;
            asm volatile("" : "+v"(wq));
            uint32_t qa[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[ks] = kaddr[ks] + wq;
            if constexpr (D == 128) qb2_init(acc, qreg, qa);
            else qb2_init_d64(acc, qreg, qa);
        }
        cur = nxt;
        off = off_next;
    }
}

// The C++ MFMA kernel (32 * QB query rows per wave, WAVES waves per workgroup) on its grid of query tiles.
template <int D, int QB, int MASK, bool OUT_F32, int OLAYOUT, int WAVES, int KSPLIT = 1>
hipError_t launch_cpp(const void *Q, const void *K, const void *V, const int32_t *valid_lens, float c_log2, void *O,
                      int B, int H, int Nq, int Nk, AttnHeads hd, hipStream_t stream)
{
    constexpr int BM = WAVES / KSPLIT * 32 * QB;
    const int BH = B * H;
    const int num_qtiles = (Nq + BM - 1) / BM;
    const long long grid = (long long)num_qtiles * BH;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, QB, MASK, OUT_F32, OLAYOUT, WAVES, KSPLIT>), dim3((unsigned)grid),
                       dim3(WAVES * 64), 0, stream, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                       valid_lens, c_log2, O, H, Nq, Nk, num_qtiles, BH, hd);
    return hipGetLastError();
}

template <int D, int MASK, bool OUT_F32, int OLAYOUT>
hipError_t launch_variant(const void *Q, const void *K, const void *V, const int32_t *valid_lens, float scale,
                          void *O, int B, int H, int Nq, int Nk, AttnHeads hd, hipStream_t stream)
{
    // exp(x) = exp2(x * log2(e)). The kernels need c_log2 > 0 so that masked
    // scores (-inf) map to weight 0 without a select; below 1e-30 every
    // visible exp2 argument rounds to 0 anyway, which is the scale = 0 result.
    const float c_log2 = fmaxf(scale * 1.4426950408889634f, 1e-30f);
    if constexpr (D == 128) {
        // 64 query rows per wave: the whole register file, one wave per SIMD, 4 per workgroup; a persistent
        // grid of at most one workgroup per CU over 256-row work items
        const int BH = B * H;
        const int num_qtiles = (Nq + 255) / 256;
        const long long grid = (long long)num_qtiles * BH;
        if (grid <= 0) return hipSuccess;
        if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((attn_fwd_qb2_kernel<D, MASK, OUT_F32, OLAYOUT>),
                           dim3((unsigned)std::min<long long>(grid, device_cu_count())), dim3(256), 0, stream,
                           (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, valid_lens, c_log2, O, H,
                           Nq, Nk, num_qtiles, BH, hd);
        return hipGetLastError();
    } else {
        static_assert(D == 64, "head_dim 64 or 128");
        // smaller grids: the C++ kernel with 4 waves of 128 rows, which give every SIMD two waves when their
        // grid has more workgroups than CUs; smaller still, each workgroup's keys split over two sets of 4 waves
        const int cus = device_cu_count();
        const long long g8 = (long long)((Nq + 255) / 256) * B * H, g4 = (long long)((Nq + 127) / 128) * B * H;
        if (g8 >= cus) {
            // 256-row work items cover every CU: the persistent kernel with the generated tile loop (64 rows per
            // wave, one wave per SIMD), as for 128-wide heads
            if (g8 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((attn_fwd_qb2_kernel<D, MASK, OUT_F32, OLAYOUT>), dim3((unsigned)cus), dim3(256), 0,
                               stream, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, valid_lens,
                               c_log2, O, H, Nq, Nk, (Nq + 255) / 256, B * H, hd);
            return hipGetLastError();
        }
        if (g4 <= cus)
            return launch_cpp<D, 1, MASK, OUT_F32, OLAYOUT, 8, 2>(Q, K, V, valid_lens, c_log2, O, B, H, Nq, Nk, hd,
                                                                 stream);
        return launch_cpp<D, 1, MASK, OUT_F32, OLAYOUT, 4>(Q, K, V, valid_lens, c_log2, O, B, H, Nq, Nk, hd, stream);
    }
}

template <int D, int MASK>
hipError_t dispatch_out(const void *Q, const void *K, const void *V, const int32_t *vl, float scale, void *O,
                        int out_f32, int out_layout, int B, int H, int Nq, int Nk, AttnHeads hd, hipStream_t s)
{
    if (out_layout == kOutBNHD) {
        if (out_f32) return launch_variant<D, MASK, true, kOutBNHD>(Q, K, V, vl, scale, O, B, H, Nq, Nk, hd, s);
        return launch_variant<D, MASK, false, kOutBNHD>(Q, K, V, vl, scale, O, B, H, Nq, Nk, hd, s);
    }
    if (out_f32) return launch_variant<D, MASK, true, kOutBHND>(Q, K, V, vl, scale, O, B, H, Nq, Nk, hd, s);
    return launch_variant<D, MASK, false, kOutBHND>(Q, K, V, vl, scale, O, B, H, Nq, Nk, hd, s);
}

template <int D>
hipError_t dispatch_mask(const void *Q, const void *K, const void *V, int mask, const int32_t *vl, float scale,
                         void *O, int out_f32, int out_layout, int B, int H, int Nq, int Nk, AttnHeads hd,
                         hipStream_t s)
{
    switch (mask) {
    case kMaskCausal:
        return dispatch_out<D, kMaskCausal>(Q, K, V, vl, scale, O, out_f32, out_layout, B, H, Nq, Nk, hd, s);
    case kMaskPadding:
        return dispatch_out<D, kMaskPadding>(Q, K, V, vl, scale, O, out_f32, out_layout, B, H, Nq, Nk, hd, s);
    case kMaskCausalPadding:
        return dispatch_out<D, kMaskCausalPadding>(Q, K, V, vl, scale, O, out_f32, out_layout, B, H, Nq, Nk, hd, s);
    default: return dispatch_out<D, kMaskNone>(Q, K, V, vl, scale, O, out_f32, out_layout, B, H, Nq, Nk, hd, s);
    }
}

}  // namespace

// Compute units of the current device (cached per device): the persistent grid's size.
int device_cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_attn_bf16(const void *Q, const void *K, const void *V, int mask, const int32_t *valid_lens,
                            float scale, void *O, int out_f32, int out_layout, int B, int H, int Nq, int Nk, int D,
                            AttnHeads hd, hipStream_t stream)
{
    if (D == 128)
        return dispatch_mask<128>(Q, K, V, mask, valid_lens, scale, O, out_f32, out_layout, B, H, Nq, Nk, hd, stream);
    if (D == 64)
        return dispatch_mask<64>(Q, K, V, mask, valid_lens, scale, O, out_f32, out_layout, B, H, Nq, Nk, hd, stream);
    return hipErrorInvalidValue;
}

}  // namespace tsd
