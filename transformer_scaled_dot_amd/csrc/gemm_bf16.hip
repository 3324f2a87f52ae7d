// bf16 GEMMs of the multi-head layer on gfx950 MFMA: the fused projection
// X W_QKV ("Self-Attention 机制", section 五步计算: W_Q, W_K, W_V concatenated
// into one d x 3d matrix, one GEMM, then split) with an epilogue that writes
// the per-head layout of section 维度全程跟踪 directly, and the output
// projection C W_O.
//
// C = A[M,K] * B[K,N], both row-major, f32 accumulation, bf16 output. Each
// wave computes its block of the transposed product, C^T = B^T A^T, with
// v_mfma_f32_32x32x16_bf16: the B^T operand (32 columns of B x 16 k) comes
// from the row-major B tile by ds_read_b64_tr_b16, the A^T operand is 16
// contiguous bytes of an A row, and an accumulator lane holds one output row.
//
// Workgroup tile BM x BN x 64 (k), WM x WN waves of (BM/WM) x (BN/WN). The A
// and B tiles go HBM -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4, no
// staging registers), STAGES deep: the tile of k-step kt + STAGES - 1 is
// fetched while k-step kt computes, and one barrier per k-step publishes the
// tiles and frees the oldest buffer. Rows of a tile are stored with their
// 16-byte chunks XOR-swizzled (the attention kernels' tile swizzle), so the
// row reads of A and the transposed reads of B are bank-conflict free.
//
// Epilogue: each wave writes its bf16 block into LDS (swizzled) and reads it
// back as whole 128-byte row segments, so every global store instruction
// writes full cache lines: row-major C (plain), or the head-split layout
// [which][b][head][t][c] (projection; a 64-column segment never crosses a
// head since d_k is a multiple of 64).
//
// Workgroups take tiles XCD by XCD (workgroup w runs on XCD w % 8): each
// XCD's workgroups cover a contiguous run of row-major tiles, i.e. a few
// row blocks of A against all of B, which stay in that XCD's L2.
#include "attn_tiles.h"
#include "device_common.h"
#include "kernels.h"

#include <type_traits>

namespace tsd {
namespace {

constexpr int kGBK = 64;  // k per step; K must be a multiple

enum Epilogue { kEpiPlain = 0, kEpiQkvSplit = 1 };

struct QkvShape {
    int batch, seq, d_model, heads, dk;
};

// byte offset of element (r, e) in a swizzled tile of rows of W bf16 (W = 64 or 128)
template <int W>
__device__ __forceinline__ uint32_t gsw(int r, int e)
{
    return 2u * (uint32_t)swz_off<W>(r, e);
}

template <int BM, int BN, int WM, int WN, int STAGES, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(const uint16_t *__restrict__ A,
                                                                const uint16_t *__restrict__ Bm,
                                                                uint16_t *__restrict__ C, int M, int N, int Kd, int ldb,
                                                                int tiles_n, int xcd_chunk, QkvShape qs)
{
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    constexpr int MB = TM / 32, NB = TN / 32;
    constexpr int A_BYTES = BM * kGBK * 2, B_BYTES = kGBK * BN * 2, STAGE = A_BYTES + B_BYTES;
    constexpr int A_DMA = A_BYTES / 1024 / NW, B_DMA = B_BYTES / 1024 / NW;  // 1 KiB DMA instructions per wave
    constexpr int A_RPK = 1024 / (kGBK * 2), B_RPK = 1024 / (BN * 2);        // tile rows per KiB
    constexpr int B_CPR = BN / 8;                                            // 16-byte chunks per B row
    static_assert(A_DMA * 1024 * NW == A_BYTES && B_DMA * 1024 * NW == B_BYTES, "tiles must split over the waves");
    static_assert(BN == 64 || BN == 128, "B rows are swizzled as 64- or 128-wide tiles");
    static_assert(MB >= 1 && NB >= 1 && TN % 32 == 0, "");
    static_assert(NW * TM * TN * 2 <= STAGES * STAGE, "epilogue staging must fit in the stage buffers");
    __shared__ __attribute__((aligned(16))) uint8_t smem[STAGES * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
    const int wm = wave / WN, wn = wave % WN;

    // the workgroup's tile: a contiguous run of row-major tiles per XCD
    const int b = blockIdx.x;
    const int t = xcd_chunk > 0 ? (b % 8) * xcd_chunk + b / 8 : b;
    const int tm = t / tiles_n, tn = t - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;

    // DMA: lane's LDS chunk of each 1 KiB block and the global offset it fetches (relative to the tile's
    // row 0, k 0); rows of A past M repeat row M - 1 (their products are never stored)
    uint32_t a_off[A_DMA], b_off[B_DMA];
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
        const int blk = j * NW + wave, r = blk * A_RPK + lane / 8, cp = lane % 8;
        const int c = cp ^ swz<64>(r);
        a_off[j] = (uint32_t)min(r, M - 1 - m0) * (uint32_t)Kd * 2u + (uint32_t)c * 16u;
    }
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) {
        const int blk = j * NW + wave, r = blk * B_RPK + lane / B_CPR, cp = lane % B_CPR;
        const int c = cp ^ swz<BN>(r);
        b_off[j] = (uint32_t)r * (uint32_t)ldb * 2u + (uint32_t)c * 16u;
    }
    const uint32_t lds0 = lds_addr(smem);
    const uint32_t lwave = __builtin_amdgcn_readfirstlane(lds0 + wave * 1024);
    const uint16_t *Ab = A + (size_t)m0 * Kd, *Bb = Bm + n0;
    auto fetch = [&](int kt, int buf) {
        const uint16_t *ak = Ab + kt * kGBK, *bk = Bb + (size_t)kt * kGBK * ldb;
#pragma unroll
        for (int j = 0; j < A_DMA; ++j) lds_dma16(lwave + buf * STAGE + j * NW * 1024, ak, a_off[j]);
#pragma unroll
        for (int j = 0; j < B_DMA; ++j) lds_dma16(lwave + buf * STAGE + A_BYTES + j * NW * 1024, bk, b_off[j]);
    };

    // operand read addresses within a stage (k-substep kk and the block index are immediates)
    uint32_t ra[MB], rb[NB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) ra[mb] = gsw<64>(wm * TM + mb * 32 + l32, hf * 8);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int krow = hf * 8 + (i16 >> 2), col = wn * TN + nb * 32 + (g16 & 1) * 16 + 4 * (i16 & 3);
        rb[nb][0] = A_BYTES + gsw<BN>(krow, col);
        rb[nb][1] = A_BYTES + gsw<BN>(krow + 4, col);
    }

    f32x16 acc[NB][MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.f;

    const int nk = Kd / kGBK;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) fetch(s, s);
    for (int kt = 0; kt < nk; ++kt) {
        // this wave's fetches of step kt are done (those of the later steps may still run), then every wave's
        if (kt + STAGES - 2 < nk) {
            if constexpr (STAGES == 3) __builtin_amdgcn_s_waitcnt(0x0F70 | ((A_DMA + B_DMA) & 15) |
                                                                  (((A_DMA + B_DMA) >> 4) << 14));
            else wait_vmcnt0();
        } else {
            wait_vmcnt0();
        }
        __syncthreads();
        if (kt + STAGES - 1 < nk) fetch(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
        const uint8_t *st = smem + (kt % STAGES) * STAGE;
#pragma unroll
        for (int kk = 0; kk < kGBK / 16; ++kk) {
            bf16x8 aop[NB], bop[MB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                aop[nb] = lds_tr_pair((const uint16_t *)(st + rb[nb][0] + kk * 16 * BN * 2),
                                      (const uint16_t *)(st + rb[nb][1] + kk * 16 * BN * 2));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                bop[mb] = *(const bf16x8 *)(st + (ra[mb] ^ (uint32_t)(kk * 32)));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mfma32x32x16(aop[nb], bop[mb], acc[nb][mb]);
        }
    }

    // epilogue: the wave's TM x TN block, bf16, through LDS as whole row segments
    __syncthreads();  // every wave is done reading the stage buffers
    constexpr int RB = TN * 2, CPRW = TN / 8;  // staging row bytes, 16-byte chunks per row
    uint8_t *stg = smem + wave * (TM * RB);
    auto stg_off = [&](int r, int c) { return (uint32_t)(r * RB + ((c ^ (r % CPRW)) << 4)); };
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                // acc[nb][mb][rg*4 + i]: row mb*32 + l32, column nb*32 + rg*8 + hf*4 + i of the wave's block
                const u32x2 v = {pack_bf16x2(acc[nb][mb][rg * 4 + 0], acc[nb][mb][rg * 4 + 1]),
                                 pack_bf16x2(acc[nb][mb][rg * 4 + 2], acc[nb][mb][rg * 4 + 3])};
                *(u32x2 *)(stg + stg_off(mb * 32 + l32, nb * 4 + rg) + hf * 8) = v;
            }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    constexpr int RPI = 64 / CPRW;  // rows per read instruction
    const int gcol = n0 + wn * TN;  // first column of the wave's block
    size_t seg_base = 0;
    if constexpr (EPI == kEpiQkvSplit) {
        const int which = gcol / qs.d_model, rem = gcol - which * qs.d_model;
        const int hh = rem / qs.dk, cc = rem - hh * qs.dk;
        seg_base = (((size_t)which * qs.batch) * qs.heads + hh) * (size_t)qs.seq * qs.dk + cc;
    }
#pragma unroll
    for (int i = 0; i < TM / RPI; ++i) {
        const int r = i * RPI + lane / CPRW, c = lane % CPRW;
        const u32x4 v = *(const u32x4 *)(stg + r * RB + (((c ^ (r % CPRW))) << 4));
        const int m = m0 + wm * TM + r;
        if (m < M) {
            size_t off;
            if constexpr (EPI == kEpiPlain) {
                off = (size_t)m * N + gcol + c * 8;
            } else {
                const int bb = m / qs.seq, tt = m - bb * qs.seq;
                off = seg_base + ((size_t)bb * qs.heads * qs.seq + tt) * qs.dk + c * 8;
            }
            *(u32x4 *)(C + off) = v;
        }
    }
}

template <int EPI>
hipError_t launch(const void *A, const void *Bm, int ldb, void *C, int M, int N, int K, QkvShape qs,
                  hipStream_t stream)
{
    if (M <= 0) return hipSuccess;
    const int cus = device_cu_count();
    auto go = [&](auto bm, auto bn, auto wmc, auto wnc, auto stages) {
        constexpr int BM = decltype(bm)::value, BN = decltype(bn)::value;
        constexpr int WM = decltype(wmc)::value, WN = decltype(wnc)::value, ST = decltype(stages)::value;
        const long long tiles_m = (M + BM - 1) / BM, tiles_n = N / BN, grid = tiles_m * tiles_n;
        if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const int chunk = grid % 8 == 0 ? (int)(grid / 8) : 0;
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, ST, EPI>), dim3((unsigned)grid), dim3(WM * WN * 64), 0,
                           stream, (const uint16_t *)A, (const uint16_t *)Bm, (uint16_t *)C, M, N, K, ldb,
                           (int)tiles_n, chunk, qs);
        return hipGetLastError();
    };
    using I = std::integral_constant<int, 0>;
    (void)sizeof(I);
    // 128 x 128 tiles while they give every CU at least two, else 128 x 64
    const long long t128 = (long long)((M + 127) / 128) * (N / 128);
    if (N % 128 == 0 && t128 >= 2LL * cus)
        return go(std::integral_constant<int, 128>(), std::integral_constant<int, 128>(),
                  std::integral_constant<int, 2>(), std::integral_constant<int, 2>(),
                  std::integral_constant<int, 2>());
    return go(std::integral_constant<int, 128>(), std::integral_constant<int, 64>(), std::integral_constant<int, 2>(),
              std::integral_constant<int, 2>(), std::integral_constant<int, 2>());
}

}  // namespace

hipError_t launch_gemm_bf16(const void *A, const void *Bm, void *C, int M, int N, int K, hipStream_t stream)
{
    if (N % 64 != 0 || K % kGBK != 0) return hipErrorInvalidValue;
    return launch<kEpiPlain>(A, Bm, N, C, M, N, K, QkvShape{0, 1, 1, 1, 1}, stream);
}

hipError_t launch_gemm_bf16_heads(const void *X, const void *W, int ldw, void *out, int batch, int seq, int n_cols,
                                  int d_model, int heads, hipStream_t stream)
{
    if (d_model % 64 != 0 || d_model % heads != 0 || (d_model / heads) % 64 != 0 || n_cols % d_model != 0 ||
        ldw < n_cols || ldw % 8 != 0)
        return hipErrorInvalidValue;
    const QkvShape qs{batch, seq, d_model, heads, d_model / heads};
    return launch<kEpiQkvSplit>(X, W, ldw, out, batch * seq, n_cols, d_model, qs, stream);
}

hipError_t launch_gemm_bf16_qkv_split(const void *X, const void *Wqkv, void *qkv, int batch, int seq, int d_model,
                                      int heads, hipStream_t stream)
{
    return launch_gemm_bf16_heads(X, Wqkv, 3 * d_model, qkv, batch, seq, 3 * d_model, d_model, heads, stream);
}

}  // namespace tsd
