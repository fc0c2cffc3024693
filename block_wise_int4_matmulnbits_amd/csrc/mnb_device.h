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

// Two bf16 -> two fp16, round to nearest even: the exact fp32 values of
// both halves, then one packed RNE conversion (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v)
{
    typedef float float2_t __attribute__((ext_vector_type(2)));
    const float2_t f = {__uint_as_float(v << 16), __uint_as_float(v & 0xFFFF0000u)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, half2_t));
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

// The unpack below relies on v_and_or_b32 ((x & mask) | orv in one VALU op).
// gfx9 VOP3 takes no literal and at most one SGPR, so the compiler forms it
// only when orv sits in a VGPR.  A constant built from a runtime zero that
// the compiler cannot see through (a kernel argument, always 0) stays in a
// VGPR; no inline assembly is needed, which keeps every instruction visible
// to the compiler's hazard checks (an MFMA still writing a register that a
// later instruction reuses).
__device__ __forceinline__ uint32_t vgpr_constant(uint32_t c, uint32_t zero)
{
    return c | ((uint32_t)threadIdx.x & zero);
}

// Packed fp16 a + b and a * b + c (one rounding each; exact where used).
__device__ __forceinline__ uint32_t hadd2(uint32_t a, uint32_t b)
{
    const half2_t r = __builtin_bit_cast(half2_t, a) + __builtin_bit_cast(half2_t, b);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t hfma2(uint32_t a, uint32_t b, uint32_t c)
{
    const half2_t r = __builtin_bit_cast(half2_t, a) * __builtin_bit_cast(half2_t, b) +
                      __builtin_bit_cast(half2_t, c);
    return __builtin_bit_cast(uint32_t, r);
}

// Nibble pairs of one dword x as exact fp16 pairs q - z.  (x & mask) lands in
// the low mantissa bits of two fp16 numbers of exponent 2^10:
//   mask 0x000F000F: 1024 + q  ->  + (-(1024 + z))       = q - z
//   mask 0x00F000F0: 1024 + 16q -> * 1/16 + (-(64 + z))  = q - z
// zneg1 = -(1024+z) and zfma = -(64+z) in both halves.
struct ZeroPoint {
    uint32_t zneg1, zfma;
};

__device__ __forceinline__ ZeroPoint zero_point_pairs(uint32_t z)
{
    const uint32_t zz = z | (z << 16);
    return ZeroPoint{0xE400E400u | zz, 0xD400D400u | (zz << 4)};
}

// magic: the fp16 pair (1024, 1024), 0x64006400, held in a VGPR (see
// vgpr_constant).
__device__ __forceinline__ void unpack_dword(uint32_t x, ZeroPoint zp, uint32_t magic,
                                             uint32_t (&pr)[4])
{
    const uint32_t sixteenth = 0x2C002C00u;  // fp16 pair (1/16, 1/16)
    const uint32_t y = x >> 8;
    pr[0] = hadd2((x & 0x000F000Fu) | magic, zp.zneg1);            // (q0-z, q4-z)
    pr[1] = hfma2((x & 0x00F000F0u) | magic, sixteenth, zp.zfma);  // (q1-z, q5-z)
    pr[2] = hadd2((y & 0x000F000Fu) | magic, zp.zneg1);            // (q2-z, q6-z)
    pr[3] = hfma2((y & 0x00F000F0u) | magic, sixteenth, zp.zfma);  // (q3-z, q7-z)
}

// 4x4 transpose of dwords across the four 16-lane rows of a wave: before,
// row g holds (r0..r3) = dwords 0..3 of block 4t+g; after, r_i holds dword g
// of block 4t+i in row g (the MFMA operand layout: lane j+16g supplies
// k = 8g..8g+7).
__device__ __forceinline__ void transpose_rows(uint32_t (&r)[4])
{
    const auto s02 = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
    const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    r[0] = s01[0];
    r[1] = s01[1];
    r[2] = s23[0];
    r[3] = s23[1];
}

// Raw buffer resources (gfx9 layout: 48-bit base, no stride, num_records
// bytes, word 3 = 0x00020000).  Loads at offsets >= num_records return 0,
// which the kernels use for ragged blocks and columns past the end.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;
constexpr int kNontemporal = MNB_NT_LOADS ? 2 : 0;   // cache-policy bits of the load

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes)
{
    const int n = bytes >= kOutOfRange ? (int)kOutOfRange : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRsrcWord3);
}

}  // namespace mnb
