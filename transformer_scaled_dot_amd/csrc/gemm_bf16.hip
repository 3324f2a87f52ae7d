// bf16 GEMMs of the multi-head layer on gfx950 MFMA: the fused projection
// X W_QKV ("Self-Attention 机制", section 五步计算: W_Q, W_K, W_V concatenated
// into one d x 3d matrix, one GEMM, then split) with an epilogue that writes
// the per-head layout of section 维度全程跟踪 directly, and the output
// projection C W_O.
//
// C = A[M,K] * B[K,N], both row-major, f32 accumulation. Each wave computes
// the transposed block D^T = B^T A^T with v_mfma_f32_32x32x16_bf16 so that
// an accumulator lane holds one output ROW and four consecutive columns per
// register group: stores are 8 contiguous bytes per lane. The B^T operand is
// read from the row-major B tile with ds_read_b64_tr_b16, the A^T operand
// with plain 16-byte LDS reads. Tiles are 128 x BN x BK with 2 x 2 waves and a double-buffered LDS
// stage: 128 x 128 x 32 on grids of at least two workgroups per CU, else 128 x 64 x 64 where K allows.
#include "device_common.h"
#include "kernels.h"

#include <type_traits>

#ifndef TSD_GEMM_NARROW_BK
#define TSD_GEMM_NARROW_BK 64
#endif

namespace tsd {
namespace {

constexpr int kBM = 128, kBK = 32;  // kBK: the smallest k-step, the granularity K must have

enum Epilogue { kEpiPlain = 0, kEpiQkvSplit = 1 };

struct QkvShape {
    int batch, seq, d_model, heads, dk;
};

template <int BN, int BK, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ Bm,
                                                        uint16_t *__restrict__ C, int M, int N, int Kd, QkvShape qs)
{
    constexpr int TM = kBM / 2, TN = BN / 2;  // per-wave tile
    constexpr int MB = TM / 32, NB = TN / 32;
    constexpr int SA = BK + 8;    // A row pitch (elements): 16-byte reads of 16 rows hit disjoint banks
    constexpr int SB = BN + 16;    // B row pitch
    constexpr int ACH = kBM * BK / 8 / 256;  // 16-byte chunks per thread
    constexpr int BCH = BK * BN / 8 / 256;
    static_assert(ACH >= 1 && BCH >= 1, "");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * SA];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BK * SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;

    const int ntn = N / BN;
    const int tn = blockIdx.x % ntn, tm = blockIdx.x / ntn;
    const int m0 = tm * kBM, n0 = tn * BN;

    u32x4 areg[ACH], breg[BCH];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int c = tid + i * 256;
            const int row = c / (BK / 8), col = (c % (BK / 8)) * 8;
            const int m = m0 + row;
            areg[i] = m < M ? *(const u32x4 *)(A + (size_t)m * Kd + k0 + col) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int c = tid + i * 256;
            const int row = c / (BN / 8), col = (c % (BN / 8)) * 8;
            breg[i] = *(const u32x4 *)(Bm + (size_t)(k0 + row) * N + n0 + col);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int c = tid + i * 256;
            const int row = c / (BK / 8), col = (c % (BK / 8)) * 8;
            *(u32x4 *)(&As[buf][row * SA + col]) = areg[i];
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int c = tid + i * 256;
            const int row = c / (BN / 8), col = (c % (BN / 8)) * 8;
            *(u32x4 *)(&Bs[buf][row * SB + col]) = breg[i];
        }
    };

    f32x16 acc[NB][MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.f;

    const int nk = Kd / BK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) load((kt + 1) * BK);
        const uint16_t *as = As[kt & 1];
        const uint16_t *bs = Bs[kt & 1];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 bop[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                bop[mb] = *(const bf16x8 *)(as + (wm * TM + mb * 32 + l32) * SA + kk * 16 + hf * 8);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                // lane j of a 16-lane group addresses row (j/4), columns 4*(j%4).. of its 16-column strip
                const int krow = kk * 16 + hf * 8 + (i16 >> 2);
                const int col = wn * TN + nb * 32 + (g16 & 1) * 16 + 4 * (i16 & 3);
                const bf16x8 aop = lds_tr_pair(bs + krow * SB + col, bs + (krow + 4) * SB + col);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mfma32x32x16(aop, bop[mb], acc[nb][mb]);
            }
        }
        if (kt + 1 < nk) store((kt + 1) & 1);
        __syncthreads();
    }

    // acc[nb][mb][r]: row m = m0 + wm*TM + mb*32 + l32,
    //                 col n = n0 + wn*TN + nb*32 + (r/4)*8 + hf*4 + r%4
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + wm * TM + mb * 32 + l32;
        if (m >= M) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int n = n0 + wn * TN + nb * 32 + rg * 8 + hf * 4;
                const u32x2 v = {pack_bf16x2(acc[nb][mb][rg * 4 + 0], acc[nb][mb][rg * 4 + 1]),
                                 pack_bf16x2(acc[nb][mb][rg * 4 + 2], acc[nb][mb][rg * 4 + 3])};
                size_t off;
                if (EPI == kEpiPlain) {
                    off = (size_t)m * N + n;
                } else {
                    // [which][b][head][t][c]: 4 consecutive columns never cross a head
                    const int which = n / qs.d_model, rem = n % qs.d_model;
                    const int hh = rem / qs.dk, c = rem % qs.dk;
                    const int bb = m / qs.seq, t = m % qs.seq;
                    off = ((((size_t)which * qs.batch + bb) * qs.heads + hh) * qs.seq + t) * qs.dk + c;
                }
                *(u32x2 *)(C + off) = v;
            }
    }
}

template <int EPI>
hipError_t launch(const void *A, const void *Bm, void *C, int M, int N, int K, QkvShape qs, hipStream_t stream)
{
    if (M <= 0) return hipSuccess;
    const long long mt = (M + kBM - 1) / kBM;
    // 128-wide tiles when they still give the chip two workgroups per CU
    const bool wide = (N % 128 == 0) && mt * (N / 128) >= 512;
    const long long grid = mt * (wide ? N / 128 : N / 64);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    auto go = [&](auto bn, auto bk) {
        hipLaunchKernelGGL((gemm_bf16_kernel<decltype(bn)::value, decltype(bk)::value, EPI>), dim3((unsigned)grid),
                           dim3(256), 0, stream, (const uint16_t *)A, (const uint16_t *)Bm, (uint16_t *)C, M, N, K, qs);
    };
    // narrow grids (fewer workgroups, each waiting on its global loads once per k-step) take deeper k-steps
    // where K allows: fewer load round trips and barriers, more products between them
    constexpr int NBK = TSD_GEMM_NARROW_BK;
    if (wide)
        go(std::integral_constant<int, 128>(), std::integral_constant<int, 32>());
    else if (K % NBK == 0)
        go(std::integral_constant<int, 64>(), std::integral_constant<int, NBK>());
    else
        go(std::integral_constant<int, 64>(), std::integral_constant<int, 32>());
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const void *A, const void *Bm, void *C, int M, int N, int K, hipStream_t stream)
{
    if (N % 64 != 0 || K % kBK != 0) return hipErrorInvalidValue;
    return launch<kEpiPlain>(A, Bm, C, M, N, K, QkvShape{0, 1, 1, 1, 1}, stream);
}

hipError_t launch_gemm_bf16_qkv_split(const void *X, const void *Wqkv, void *qkv, int batch, int seq, int d_model,
                                      int heads, hipStream_t stream)
{
    const int N = 3 * d_model;
    if (N % 64 != 0 || d_model % kBK != 0 || d_model % heads != 0) return hipErrorInvalidValue;
    const QkvShape qs{batch, seq, d_model, heads, d_model / heads};
    return launch<kEpiQkvSplit>(X, Wqkv, qkv, batch * seq, N, d_model, qs, stream);
}

}  // namespace tsd
