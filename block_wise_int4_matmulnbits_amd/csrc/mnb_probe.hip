// Read-only HBM streaming probe for gfx950: the attainable read bandwidth
// the GEMV's roofline fraction is read against.  Grid-stride 16-byte loads,
// U loads in flight per thread, one xor word written per thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ __launch_bounds__(256) void read_probe(const u32x4* __restrict__ p, size_t n16,
                                                  uint32_t* __restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" int mnb_probe_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups,
                              int unroll, void* stream)
{
    if (!buf || !sink || bytes % 16 || workgroups < 1) return -1;
    const u32x4* p = static_cast<const u32x4*>(buf);
    const size_t n16 = bytes / 16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 g(workgroups), b(256);
    switch (unroll) {
    case 1: hipLaunchKernelGGL((read_probe<1, false>), g, b, 0, s, p, n16, sink); break;
    case 2: hipLaunchKernelGGL((read_probe<2, false>), g, b, 0, s, p, n16, sink); break;
    case 4: hipLaunchKernelGGL((read_probe<4, false>), g, b, 0, s, p, n16, sink); break;
    case 8: hipLaunchKernelGGL((read_probe<8, false>), g, b, 0, s, p, n16, sink); break;
    case -1: hipLaunchKernelGGL((read_probe<1, true>), g, b, 0, s, p, n16, sink); break;
    case -2: hipLaunchKernelGGL((read_probe<2, true>), g, b, 0, s, p, n16, sink); break;
    case -4: hipLaunchKernelGGL((read_probe<4, true>), g, b, 0, s, p, n16, sink); break;
    case -8: hipLaunchKernelGGL((read_probe<8, true>), g, b, 0, s, p, n16, sink); break;
    default: return -1;
    }
    return (int)hipGetLastError();
}
