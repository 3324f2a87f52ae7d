// Measurement support: the shader clock and the matrix-instruction rate the GPU sustains when every SIMD
// issues nothing but bf16 32x32x16 MFMAs on pseudo-random operands, for the benchmark's report (the
// chip's power management lowers the clock under a data-carrying matrix load well below where it runs for
// operands of zero). Not part of the attention path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tsd {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// integer finaliser of a 32-bit hash (an xorshift-multiply mix): operands whose bits change from lane to lane
__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return x;
}

__device__ __forceinline__ __bf16 operand(uint32_t h)
{
    return (__bf16)(((float)(h & 0xffffu) - 32768.0f) * (1.0f / 16384.0f));  // uniform in [-2, 2)
}

__global__ __launch_bounds__(256) void clock_probe_kernel(uint64_t *out, uint64_t wall_ticks)
{
    bf16x8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t h = mix32((blockIdx.x * 256u + threadIdx.x) * 64u + j * 8u + e);
            a[j][e] = operand(h);
            b[j][e] = operand(h >> 16);
        }
    f32x16 acc[4] = {};
    uint64_t n = 0, r;
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    do {  // ends: the wall-clock counter only grows
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c)  // four independent accumulators keep the matrix pipe full
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + c) & 3], b[(j + 3 * c) & 3], acc[c], 0, 0, 0);
        n += 16;
        r = __builtin_amdgcn_s_memrealtime();
    } while (r - r0 < wall_ticks);
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    if (threadIdx.x == 0) {
        out[3 * blockIdx.x] = t1 - t0;
        out[3 * blockIdx.x + 1] = r - r0;
        // a NaN sum is impossible for these operands; the test keeps the products from being optimised away
        out[3 * blockIdx.x + 2] = n + (s != s ? 1 : 0);
    }
}

}  // namespace

hipError_t launch_clock_probe(uint64_t *out, int blocks, int spin_us, hipStream_t stream)
{
    hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(256), 0, stream, out, (uint64_t)spin_us * 100u);
    return hipGetLastError();
}

}  // namespace tsd
