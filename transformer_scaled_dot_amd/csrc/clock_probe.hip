// Measurement support: the shader clock the GPU sustains while its matrix pipes are busy (s_memtime ticks
// against the 100 MHz s_memrealtime counter), for the benchmark's report. Not part of the attention path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tsd {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void clock_probe_kernel(uint64_t *out, uint64_t wall_ticks)
{
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)0.0f;
        b[e] = (__bf16)0.0f;
    }
    f32x16 acc = {};
    uint64_t r;
    do {  // ends: the wall-clock counter only grows
#pragma unroll
        for (int i = 0; i < 16; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        r = __builtin_amdgcn_s_memrealtime();
    } while (r - r0 < wall_ticks);
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = t1 - t0;
        out[2 * blockIdx.x + 1] = r - r0 + (acc[0] != 0.f ? 1 : 0);  // acc is 0: keeps the MFMAs, adds nothing
    }
}

}  // namespace

hipError_t launch_clock_probe(uint64_t *out, int blocks, int spin_us, hipStream_t stream)
{
    hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(256), 0, stream, out, (uint64_t)spin_us * 100u);
    return hipGetLastError();
}

}  // namespace tsd
