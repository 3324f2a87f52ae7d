// Tile operations shared by the attention kernels (forward and backward): the swizzled LDS layout of
// [64 rows][D] bf16 tiles, the per-lane LDS addresses, the two MFMA contractions over a tile and the
// row store. They compute, with v_mfma_f32_32x32x16_bf16:
//   scores:        S^T = T R^T  -- T a 64-row tile in LDS, R 32 * QB rows held in registers; the
//                  accumulator has one R row per lane (lane % 32) and 16 T rows per lane;
//   accumulate_pv: A^T += T^T P^T -- P^T taken straight from such an accumulator (rounded to bf16) as the
//                  B operand, the MFMA's k index mapped onto T rows in the order the accumulator holds
//                  them, T^T read from the row-major tile with ds_read_b64_tr_b16 in that same order.
#pragma once

#include "device_common.h"
#include "kernels.h"

#include <math.h>

namespace tsd {
namespace {

constexpr int kBlockN = 64;            // rows per LDS tile (keys in the forward)

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

// S^T = K Q^T for one 64-key tile and QB blocks of 32 queries: s[qb][jb]
// holds keys jb*32.. of query block qb. KOFF: byte offset of the K tile in
// LDS (compile-time, folded into immediates).
template <int D, int QB, int KOFF>
__device__ __forceinline__ void scores(const uint8_t *lds, const TileAddrs<D> &ad, const bf16x8 (&qreg)[QB][D / 16],
                                       f32x16 (&s)[QB][2])
{
    constexpr int KS = D / 16;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[qb][jb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 k0 = *(const bf16x8 *)(lds + ad.k[ks] + KOFF);
        const bf16x8 k1 = *(const bf16x8 *)(lds + ad.k[ks] + KOFF + 32 * D * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            s[qb][0] = mfma32x32x16(k0, qreg[qb][ks], s[qb][0]);
            s[qb][1] = mfma32x32x16(k1, qreg[qb][ks], s[qb][1]);
        }
    }
}

// Hide the scores of keys that this lane's query row must not see:
// j >= kv_len, or (causal) j > qrow.
template <int MASK>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[2], int k0, int kv_len, int qrow, int hf)
{
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + jb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
            const bool vis = key < kv_len && (!mask_causal(MASK) || key <= qrow);
            if (!vis) s[jb][r] = -INFINITY;
        }
}

// O^T += V^T P^T for one tile and QB query blocks. VOFF: byte offset of the
// V tile in LDS. MFMA k slot hf*8 + t of chunk c is key
// c*16 + (t/4)*8 + hf*4 + t%4, the order in which the S accumulator holds
// the keys; a transposed read of rows c*16 + hf*4 + (0..3) (+8) gives
// exactly those 8 keys per column.
template <int D, int QB, int VOFF>
__device__ __forceinline__ void accumulate_pv(const uint8_t *lds, const TileAddrs<D> &ad, const bf16x8 (&pb)[QB][4],
                                              f32x16 (&acc)[QB][D / 32])
{
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const uint8_t *p0 = lds + ad.v[db][0] + VOFF + c * 16 * D * 2;
            const uint8_t *p1 = lds + ad.v[db][1] + VOFF + c * 16 * D * 2;
            const bf16x8 a = lds_tr_pair((const uint16_t *)p0, (const uint16_t *)p1);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32x32x16(a, pb[qb][c], acc[qb][db]);
        }
    }
}

// O = O_acc / l for one block of 32 query rows (0 for a row with no
// visible key), rounded to the output type and stored as [B,H,N,D] or as
// the head concat [B,N,H,D]. L_HALVES: each half-wave holds the row sum of
// its own keys (else l_run is already the row's whole sum).
template <int D, bool OUT_F32, int OLAYOUT, bool L_HALVES = true>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[D / 32], float l_run, int qrow, int bh, int H, int Nq,
                                           int b, int hf, void *__restrict__ Out)
{
    const float l_tot = L_HALVES ? half_swap_sum(l_run) : l_run;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow >= Nq) return;
    size_t row_off;
    if (OLAYOUT == kOutBHND) {
        row_off = ((size_t)bh * Nq + qrow) * D;
    } else {
        const int hh = bh % H;
        row_off = (((size_t)b * Nq + qrow) * H + hh) * D;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
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

}  // namespace
}  // namespace tsd
