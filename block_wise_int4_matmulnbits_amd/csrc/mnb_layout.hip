// Stored-layout conversion of packed INT4 weights: the natural layout and
// the offline odd/even nibble interleave of the second page (pull request
// "PORT-1 (offline bias+interleave)", opening paragraph and "Method").
//
// Within a 32-bit word (8 consecutive weights k0..k7 of a row, little
// endian), the natural layout keeps k_p in nibble p; the even/odd layout
// keeps k_{2(p mod 4) + p/4} in nibble p (k0 k2 k4 k6 low, k1 k3 k5 k7
// high).  Each thread converts one word; in-place conversion is safe.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb.h"
#include "mnb_internal.h"

namespace mnb {
namespace {

// Nibble p of the result is nibble from(p) of x.
template <bool TO_EVEN_ODD>
__device__ __forceinline__ uint32_t permute_nibbles(uint32_t x)
{
    uint32_t y = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        // natural -> even/odd: nibble p takes k = 2(p%4) + p/4;
        // even/odd -> natural: nibble k takes position 4(k%2) + k/2.
        const int from = TO_EVEN_ODD ? 2 * (p % 4) + p / 4 : 4 * (p % 2) + p / 2;
        y |= ((x >> (4 * from)) & 0xFu) << (4 * p);
    }
    return y;
}

template <int MODE>   // 0 copy, 1 natural -> even/odd, 2 even/odd -> natural
__global__ __launch_bounds__(256) void mnb_repack_kernel(const uint32_t* src, uint32_t* dst, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) {
        const uint32_t x = src[i];
        dst[i] = MODE == 0 ? x : permute_nibbles<MODE == 1>(x);
    }
}

}  // namespace

int launch_repack(const uint8_t* src, int src_layout, uint8_t* dst, int dst_layout, int64_t words,
                  void* stream)
{
    if (words <= 0) return 0;
    const int mode = src_layout == dst_layout ? 0 : dst_layout == MNB_LAYOUT_EVEN_ODD ? 1 : 2;
    if (mode == 0 && src == dst) return 0;
    const int64_t want = (words + 255) / 256;
    const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
    const void* fn = mode == 0   ? reinterpret_cast<const void*>(mnb_repack_kernel<0>)
                     : mode == 1 ? reinterpret_cast<const void*>(mnb_repack_kernel<1>)
                                 : reinterpret_cast<const void*>(mnb_repack_kernel<2>);
    const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);
    void* args[] = {&s, &d, &words};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
    return (int)e;
}

}  // namespace mnb
