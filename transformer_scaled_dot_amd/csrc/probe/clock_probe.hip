// Measurement support for the benchmark, built into its own library (libtsd_probe.so) and not part of the
// attention library or its C ABI: the shader clock and the matrix-instruction rate the GPU sustains when
// every SIMD issues nothing but bf16 32x32x16 MFMAs on pseudo-random operands (the chip's power management
// lowers the clock under a data-carrying matrix load well below where it runs for operands of zero).
//
//   int tsd_probe_clock(uint64_t *out, int32_t blocks, int32_t spin_us, void *stream)
//
// One workgroup of four waves (one per SIMD) per block spins for spin_us microseconds of wall time and
// writes, per workgroup, (shader-clock ticks, 100 MHz wall-clock ticks, MFMAs per wave) to out[3 * blocks]
// (device memory, 8-byte aligned). Returns 0 when launched, 1 for a null or misaligned out or a count out
// of range (blocks 1..65536, spin_us 1..100000), 3 when the launch fails.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

extern "C" __attribute__((visibility("default"))) int tsd_probe_clock(uint64_t *out, int32_t blocks, int32_t spin_us,
                                                                      void *stream)
{
    if (!out || ((uintptr_t)out & 7u) || blocks < 1 || blocks > 65536 || spin_us < 1 || spin_us > 100000) return 1;
    hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out,
                       (uint64_t)spin_us * 100u);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
