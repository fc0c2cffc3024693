// Device helpers shared by the gfx950 GEMV kernels.  Internal header: HIP
// device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mnb {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
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

// Two values -> one fp16 pair, round to nearest even (v_cvt_pk_f16_f32):
// the fp32 values are exact (bf16 halves widened by a shift or a mask).
__device__ __forceinline__ uint32_t f16_pair(float lo, float hi)
{
    typedef float float2_t __attribute__((ext_vector_type(2)));
    const float2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, half2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// One 16-byte piece of eight activations a0..a7 (fp16, or bf16 rounded to
// fp16 RNE) as four fp16 pairs in the order the unpack yields the weights:
// (a0,a4) (a1,a5) (a2,a6) (a3,a7) for natural weights, (a0,a1) (a2,a3)
// (a4,a5) (a6,a7) for the even/odd layout.  bf16 halves are widened one by
// one and each pair is built by its own packed conversion, so the reorder
// costs nothing (three operations per pair); fp16 halves are reordered with
// one byte permute (v_perm_b32) per pair.
__device__ __forceinline__ u32x4 f16_pairs(u32x4 v, int a_bf16, int eo_pairs)
{
    const uint32_t x = v[0], y = v[1], z = v[2], w = v[3];   // (a0,a1) (a2,a3) (a4,a5) (a6,a7)
    if (a_bf16) {
        if (eo_pairs)
            return u32x4{f16_pair(bf16_lo(x), bf16_hi(x)), f16_pair(bf16_lo(y), bf16_hi(y)),
                         f16_pair(bf16_lo(z), bf16_hi(z)), f16_pair(bf16_lo(w), bf16_hi(w))};
        return u32x4{f16_pair(bf16_lo(x), bf16_lo(z)), f16_pair(bf16_hi(x), bf16_hi(z)),
                     f16_pair(bf16_lo(y), bf16_lo(w)), f16_pair(bf16_hi(y), bf16_hi(w))};
    }
    if (eo_pairs) return v;
    // v_perm_b32 picks bytes 0-3 from its second operand, 4-7 from its first.
    return u32x4{__builtin_amdgcn_perm(z, x, 0x05040100u), __builtin_amdgcn_perm(z, x, 0x07060302u),
                 __builtin_amdgcn_perm(w, y, 0x05040100u), __builtin_amdgcn_perm(w, y, 0x07060302u)};
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

// The same pairs for z = nib + zdef from two constants of the launch
// (zero_point_pairs(zdef)): the fields are z*0x00010001 and z*0x00100010
// added to the constants' bit patterns, with no carries, since z <= 15 only
// fills the bits the constants leave clear.  Two v_mad_u32_u24 per block.
__device__ __forceinline__ ZeroPoint zero_point_pairs(uint32_t nib, ZeroPoint base)
{
    return ZeroPoint{nib * 0x00010001u + base.zneg1, nib * 0x00100010u + base.zfma};
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

// Activations of one 32-weight block (four 16-byte pieces of fp16 or bf16,
// k = 0..31) as fp16 pairs in the order the unpack yields the weights.
__device__ __forceinline__ void activation_pairs(const u32x4 (&raw)[4], int a_bf16, int eo_pairs,
                                                 uint32_t (&act)[16])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 o = f16_pairs(raw[i], a_bf16, eo_pairs);
#pragma unroll
        for (int e = 0; e < 4; ++e) act[4 * i + e] = o[e];
    }
}

// v plus the value of lane (i - 4n) mod 16 of its 16-lane row (n = 1, 2):
// lanes that share i mod 4 (one column of a 4x4x4 product) stay together.
template <int CTRL>
__device__ __forceinline__ float row_ror_add(float v)
{
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sums over the 16 lane groups (of four lanes) of a wave of four values
// per lane, rows 0-3 of the column lane i = lane % 4 holds.  The rows are
// paired so that each exchange serves two of them: v_permlane32_swap of
// rows 0 and 1 (and of rows 2 and 3) plus one add leaves each row summed
// over the two 32-lane halves, in the lower half for the first row and the
// upper for the second; v_permlane16_swap of those two results plus one add
// sums over the 16-lane rows of each half; two rotations inside each 16-lane
// row sum its four lane groups.  Every lane of 16-lane row h ends with the
// total of row quad_total_row(h) = 0, 2, 1, 3 (h = 0..3) for its column.
// Eight VALU operations for four rows (one row at a time took six each);
// each row's total is ((h0 + h2) + (h1 + h3)) over the 16-lane rows, then
// the lane groups in rotation order, whatever the other rows hold.
__device__ __forceinline__ float quad_totals(float r0, float r1, float r2, float r3)
{
    auto halves = [](float x, float y) {
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
        return __uint_as_float(h[0]) + __uint_as_float(h[1]);
    };
    const float a = halves(r0, r1), b = halves(r2, r3);
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    float t = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    t = row_ror_add<0x124>(t);   // row_ror:4
    return row_ror_add<0x128>(t);   // row_ror:8
}
__device__ __forceinline__ int quad_total_row(int h) { return ((h & 1) << 1) | (h >> 1); }

__device__ __forceinline__ half4_t as_half4(uint32_t lo, uint32_t hi)
{
    return __builtin_bit_cast(half4_t, (uint32_t __attribute__((ext_vector_type(2)))){lo, hi});
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

// A resource of fewer than kOutOfRange bytes (no clamp, no 64-bit compare).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_small(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

}  // namespace mnb
