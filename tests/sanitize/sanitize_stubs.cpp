// Stand-ins for the kernel launchers (transformer_scaled_dot_amd/csrc/kernels.h) in the sanitizer build of
// the host code: every launch "fails", so that the C ABI's argument checks run without device code or a GPU.
#include "kernels.h"

namespace tsd {

hipError_t launch_attn_bf16(const void *, const void *, const void *, int, const int32_t *, float, void *, int, int,
                            int, int, int, int, int, AttnHeads, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_attn_f32(const float *, const float *, const float *, int, const int32_t *, float, float *, int,
                           int, int, int, int, AttnHeads, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_attn_weights(const void *, const void *, int, const int32_t *, float, float *, int, int, int, int,
                               int, int, AttnHeads, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_attn_bwd_bf16(const void *, const void *, const void *, const void *, const void *, const float *,
                                int, const int32_t *, float, void *, void *, void *, int, int, int, int, int, int,
                                float *, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_gemm_bf16(const void *, const void *, void *, int, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemm_bf16_qkv_split(const void *, const void *, void *, int, int, int, int, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_gemm_bf16_heads(const void *, const void *, int, void *, int, int, int, int, int, hipStream_t)
{
    return hipErrorNoDevice;
}
int device_cu_count() { return 256; }

}  // namespace tsd
