// Device-side building blocks for gfx950 (CDNA4): vector types, bf16 MFMA,
// LDS transpose reads and cross-half wavefront exchange.
//
// Lane layouts used throughout (wave64, l = lane, l32 = l % 32, hf = l / 32):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A operand: lane holds A[l32][hf*8 + t], t = 0..7
//     B operand: lane holds B[hf*8 + t][l32]
//     D (16 f32): lane holds D[(r/4)*8 + hf*4 + r%4][l32], r = 0..15
//   ds_read_b64_tr_b16 (per group of 16 lanes, i = l % 16):
//     element t of lane i = the 16-bit word at (address of lane 4t + i/4) + (i%4)
//     so 16 lanes that address a 4-row x 16-column block (4 words each) get
//     one column each: lane i <- column i, rows 0..3.
//   v_permlane32_swap(x, x): lanes < 32 get (x[l], x[l+32]), lanes >= 32 get
//     (x[l-32], x[l]); max/sum of the pair combines a value with the same
//     lane of the other half.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// >= 19 wait states after a 16-pass MFMA wrote these AGPR accumulators (inline asm outside the compiler's
// hazard tracking), before anything else reads or writes them.
__device__ __forceinline__ void mfma_fence_a8(f32x16 (&x)[2][4])
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4"
                 : "+a"(x[0][0]), "+a"(x[0][1]), "+a"(x[0][2]), "+a"(x[0][3]), "+a"(x[1][0]), "+a"(x[1][1]),
                   "+a"(x[1][2]), "+a"(x[1][3]));
}

__device__ __forceinline__ void mfma_fence_a8(f32x16 (&x)[2][2])
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+a"(x[0][0]), "+a"(x[0][1]), "+a"(x[1][0]), "+a"(x[1][1]));
}

// Two transposed 4x4 reads make one 8-element MFMA operand.
__device__ __forceinline__ bf16x8 lds_tr_pair(const uint16_t *lo, const uint16_t *hi)
{
    i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)lo);
    i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)hi);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, c);
}

// max / sum of a value with the same lane of the other 32-lane half
__device__ __forceinline__ float half_swap_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + lo + hi of a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)):
// sums exactly the rounded values that feed the P.V MFMA
__device__ __forceinline__ float add_bf16x2(uint32_t packed, float acc)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

// Asynchronous 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4):
// lane i reads base + voff (bytes) and writes LDS bytes
// [lds + 16*i, lds + 16*i + 16). `lds` and `base` must be wave-uniform.
// Completion is tracked by vmcnt only: wait with s_waitcnt vmcnt(0) before a
// barrier that publishes the data. Written as inline asm so that the
// compiler, which cannot tell which LDS buffer a DMA targets, does not
// serialise unrelated LDS reads behind it. M0 is set here and is not used by
// compiler-generated code in the kernels that call this; the s_nop covers
// the M0-write -> LDS-DMA hazard.
__device__ __forceinline__ void lds_dma16(uint32_t lds, const void *base, uint32_t voff)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

// LDS byte address of a __shared__ object (the M0 / ds address space).
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes per lane from a range-checked buffer (byte offset voff) into LDS at lds + 16 * lane.
__device__ __forceinline__ void lds_dma16_rsrc(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(uintptr_t)lds, 16, voff, 0,
                                             0, 0);
}

__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // s_waitcnt vmcnt(0)

}  // namespace tsd
