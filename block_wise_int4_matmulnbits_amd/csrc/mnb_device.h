// Device helpers shared by the gfx950 GEMV kernels (lane-split dot2 kernel
// and MFMA tile kernel).  Internal header: HIP device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mnb {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Weights, scales and zero points are read exactly once per call: stream
// them with nontemporal loads (on gfx950 this raised a read-only probe from
// 6.4 to 7.1 TB/s).
#ifndef MNB_NT_LOADS
#define MNB_NT_LOADS 1
#endif
template <typename T>
__device__ __forceinline__ T stream_load(const T* p)
{
    if constexpr (MNB_NT_LOADS) return __builtin_nontemporal_load(p);
    else return *p;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t w, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a),
                                  __builtin_bit_cast(half2_t, w), c, false);
}

// bf16 bits -> fp16 bits, round to nearest even through the exact fp32 value.
__device__ __forceinline__ uint32_t bf16_to_f16(uint32_t b)
{
    const _Float16 h = (_Float16)__uint_as_float(b << 16);
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v)
{
    return bf16_to_f16(v & 0xFFFFu) | (bf16_to_f16(v >> 16) << 16);
}

// fp16 bits -> bf16 bits: exact widening to fp32, then RNE on the bit
// pattern; NaN becomes a quiet NaN with its sign.
__device__ __forceinline__ uint16_t f16_to_bf16(uint16_t h)
{
    uint32_t u = __float_as_uint((float)__builtin_bit_cast(_Float16, h));
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// v_and_or_b32 (x & mask) | orv in one VALU op.  gfx9 VOP3 takes no literal
// constants, so the mask comes from an SGPR and the or-value from a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t orv)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(orv));
    return r;
}

}  // namespace mnb
