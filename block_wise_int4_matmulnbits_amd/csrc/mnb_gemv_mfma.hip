// Row-batched INT4 MatMulNBits GEMV on the matrix cores of gfx950 (CDNA4).
//
//   y[r][n] = sum_k a[r][k] * (q[n][k] - z[n][k/32]) * s[n][k/32],  2 <= m <= 8
//
// Same operation and epilogue as the lane-split kernel (onnx-genai pull
// request "perf(cuda): let the split-K decode GEMV store bf16 directly",
// opening paragraphs and the paragraph on matmul_nbits_store_narrowed; pull
// request "PORT-1 (offline bias+interleave)", "Why the premise fails here",
// item 1).  With several rows the dot products dominate the VALU work of
// the lane-split kernel (four v_dot2 per eight weights per row), so here they
// go to v_mfma_f32_16x16x32_f16 and the VALU only unpacks weights.
//
// Work decomposition.  A wave owns a tile of 16 output columns: lane l
// handles column c0 + (l % 16) and lane group g = l / 16.  The waves of a
// workgroup split the K range of the tile into contiguous stretches of
// quads (4 blocks = 128 k); at the end their partial tiles are added in a
// fixed order through LDS.  Activations (m rows) are converted to fp16,
// permuted into the unpack's pair order and staged in LDS once per
// workgroup (in K chunks when m*K*2 bytes do not fit).
//
// Per quad, lane (j, g) loads the 16 bytes of block 4t+g of its column, so a
// column's four lanes read 64 contiguous bytes.  Two v_permlane32_swap and
// two v_permlane16_swap transpose the 4x4 dwords across the lane groups, after
// which group g holds dword g of each block of the quad: the B operand layout
// of the MFMA (lane j+16g supplies k = 8g..8g+7 of column j).  The nibbles of
// a dword become exact fp16 pairs q-z as in the lane-split kernel (one
// v_and_or_b32 and one packed fp16 add or fma per pair), the activations of
// the same eight k come from LDS in the same order, and one MFMA per block
// gives the block's 16x16 product (rows m..15 are zero).  The block scale is
// applied to the fp32 result rows: acc += D * s.  Products stay exact; the
// summation order is fixed by (m, K, waves, chunk) only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb.h"
#include "mnb_device.h"
#include "mnb_internal.h"

namespace mnb {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct MfmaParams {
    const uint16_t* A;       // [m][K]
    const uint8_t* B;        // [N][K/2]
    const uint16_t* scales;  // [N][nb]
    const uint8_t* zp;       // [N][zb] or null
    uint16_t* out;           // [m][N]
    int64_t N;
    int32_t K, nb, zb;
    int32_t chunk_blocks;    // blocks of K staged in LDS per pass (multiple of 4)
    int32_t chunks;          // passes over K
    int32_t a_bf16, out_bf16;
};

// 4x4 transpose of dwords across the four 16-lane rows: before, row g holds
// (r0..r3) = dwords 0..3 of block 4t+g; after, r_i holds dword g of block
// 4t+i in row g.
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

// Global loads of one quad for one lane.
struct Quad {
    u32x4 w;          // 16 bytes: block 4t+g of this lane's column
    uint32_t s[4];    // fp16 scales of blocks 4t..4t+3 of the column
    uint32_t z;       // zero-point nibbles of blocks 4t..4t+3 (4 x 4 bits)
};

template <int M>
__global__ __launch_bounds__(512) void mnb_gemv_mfma_kernel(MfmaParams p)
{
    constexpr int RR = M < 4 ? M : 4;       // result rows 4g .. 4g+RR-1 per lane
    __shared__ float red[8][RR][64];        // per-wave partial tiles
    extern __shared__ uint4 a_lds[];        // [M][chunk_blocks][4] permuted fp16 A

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, W = (int)(blockDim.x >> 6);
    const int j = lane & 15, g = lane >> 4;
    const int nb = p.nb, kcb = p.chunk_blocks;
    const int64_t ntiles = (p.N + 15) / 16;
    const uint32_t row_bytes = (uint32_t)p.K / 2;

    // Stage rows 0..M-1, blocks b_lo .. b_lo+nbc-1 of A into LDS, converted
    // to fp16 and permuted to (a0,a4),(a1,a5),(a2,a6),(a3,a7) per 8 k.
    auto stage = [&](int b_lo, int nbc) {
        const int per_row = nbc * 4;
        const int n16 = M * per_row;
        for (int u = tid; u < n16; u += (int)blockDim.x) {
            const int r = u / per_row;
            const int rem = u - r * per_row;
            const int b = rem >> 2, gg = rem & 3;
            const uint4 v = *reinterpret_cast<const uint4*>(
                p.A + (int64_t)r * p.K + 32 * (int64_t)(b_lo + b) + 8 * gg);
            uint32_t x = v.x, y = v.y, z = v.z, w = v.w;
            if (p.a_bf16) {
                x = bf16x2_to_f16x2(x);
                y = bf16x2_to_f16x2(y);
                z = bf16x2_to_f16x2(z);
                w = bf16x2_to_f16x2(w);
            }
            uint4 o;
            o.x = (x & 0xFFFFu) | (z << 16);       // (a0,a4)
            o.y = (x >> 16) | (z & 0xFFFF0000u);   // (a1,a5)
            o.z = (y & 0xFFFFu) | (w << 16);       // (a2,a6)
            o.w = (y >> 16) | (w & 0xFFFF0000u);   // (a3,a7)
            a_lds[(r * kcb + b) * 4 + gg] = o;
        }
    };

    // Queue the loads of the quad that starts at global block blk0.
    auto issue = [&](Quad& q, int64_t col, bool col_ok, int blk0) {
        q.w = u32x4{0, 0, 0, 0};
        q.s[0] = q.s[1] = q.s[2] = q.s[3] = 0;
        q.z = 0x8888u;
        if (!col_ok) return;
        const int bw = blk0 + g;
        if (bw < nb)
            q.w = stream_load(reinterpret_cast<const u32x4*>(p.B + col * row_bytes + 16 * (uint32_t)bw));
        const uint16_t* srow = p.scales + col * nb;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (blk0 + i < nb) q.s[i] = stream_load(srow + blk0 + i);
        if (p.zp) {
            const uint8_t* zrow = p.zp + col * p.zb;
            const int zi = blk0 >> 1;
            uint32_t z0 = stream_load(zrow + zi);
            uint32_t z1 = zi + 1 < p.zb ? (uint32_t)stream_load(zrow + zi + 1) : 0x88u;
            q.z = z0 | (z1 << 8);
        }
    };

    // Unpack, MFMA and scale the four blocks of a quad.  rel = quad start
    // relative to the staged chunk, nbc = blocks in the chunk.
    auto compute = [&](const Quad& q, int rel, int nbc, float (&acc)[RR]) {
        uint32_t r[4] = {q.w[0], q.w[1], q.w[2], q.w[3]};
        transpose_rows(r);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 av = make_uint4(0, 0, 0, 0);
            if (j < M && rel + i < nbc) av = a_lds[(j * kcb + rel + i) * 4 + g];
            uint32_t bq[4];
            unpack_dword(r[i], zero_point_pairs((q.z >> (4 * i)) & 0xFu), bq);
            const uint32_t b0 = bq[0], b1 = bq[1], b2 = bq[2], b3 = bq[3];
            const u32x4 bv = {b0, b1, b2, b3};
            const u32x4 aw = {av.x, av.y, av.z, av.w};
            const float4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(half8_t, aw), __builtin_bit_cast(half8_t, bv),
                float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)q.s[i]);
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) acc[rr] = fmaf(d[rr], sf, acc[rr]);
        }
    };

    bool staged = false;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t col = tile * 16 + j;
        const bool col_ok = col < p.N;
        float acc[RR];
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) acc[rr] = 0.f;

        for (int ch = 0; ch < p.chunks; ++ch) {
            const int b_lo = ch * kcb;
            const int nbc = min(kcb, nb - b_lo);
            const int nq = (nbc + 3) / 4;
            const int q0 = wv * nq / W, q1 = (wv + 1) * nq / W;
            Quad qa, qb;
            if (q0 < q1) issue(qa, col, col_ok, b_lo + 4 * q0);   // before the staging wait
            if (!staged) {
                __syncthreads();
                stage(b_lo, nbc);
                __syncthreads();
                staged = p.chunks == 1;
            }
            for (int t = q0; t < q1;) {
                if (t + 1 < q1) issue(qb, col, col_ok, b_lo + 4 * (t + 1));
                compute(qa, 4 * t, nbc, acc);
                if (++t >= q1) break;
                if (t + 1 < q1) issue(qa, col, col_ok, b_lo + 4 * (t + 1));
                compute(qb, 4 * t, nbc, acc);
                ++t;
            }
        }

        // Fixed-order sum of the waves' partial tiles, epilogue, store.
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) red[wv][rr][lane] = acc[rr];
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                float v = red[0][rr][lane];
                for (int w = 1; w < W; ++w) v += red[w][rr][lane];
                const int row = 4 * g + rr;
                if (row < M && col_ok) {
                    const _Float16 h = (_Float16)v;            // fp32 -> fp16, RNE
                    uint16_t bits = __builtin_bit_cast(uint16_t, h);
                    if (p.out_bf16) bits = f16_to_bf16(bits);  // fp16 -> bf16, RNE
                    p.out[(int64_t)row * p.N + col] = bits;
                }
            }
        }
        __syncthreads();   // red and a_lds are reused by the next tile
    }
}

typedef void (*MfmaFn)(MfmaParams);

MfmaFn lookup_mfma(int64_t m)
{
    switch (m) {
    case 1: return mnb_gemv_mfma_kernel<1>;
    case 2: return mnb_gemv_mfma_kernel<2>;
    case 3: return mnb_gemv_mfma_kernel<3>;
    case 4: return mnb_gemv_mfma_kernel<4>;
    case 5: return mnb_gemv_mfma_kernel<5>;
    case 6: return mnb_gemv_mfma_kernel<6>;
    case 7: return mnb_gemv_mfma_kernel<7>;
    case 8: return mnb_gemv_mfma_kernel<8>;
    }
    return nullptr;
}

size_t mfma_lds_bytes(int64_t m, const mnb_plan& plan)
{
    return (size_t)m * (size_t)plan.chunk_blocks * 64;
}

}  // namespace

int launch_mfma(const GemvArgs& a, const mnb_plan& plan, void* stream)
{
    MfmaFn fn = lookup_mfma(a.m);
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    MfmaParams p;
    p.A = static_cast<const uint16_t*>(a.A);
    p.B = a.B;
    p.scales = a.scales;
    p.zp = a.zp;
    p.out = static_cast<uint16_t*>(a.out);
    p.N = a.N;
    p.K = (int32_t)a.K;
    p.nb = (int32_t)(a.K / 32);
    p.zb = (p.nb + 1) / 2;
    p.chunk_blocks = plan.chunk_blocks;
    p.chunks = plan.k_chunks;
    p.a_bf16 = a.a_bf16;
    p.out_bf16 = a.out_bf16;
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn),
                                   dim3((unsigned)plan.workgroups),
                                   dim3((unsigned)plan.threads_per_wg), args,
                                   mfma_lds_bytes(a.m, plan), static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
    return (int)e;
}

int mfma_workgroups_per_cu(int64_t m, const mnb_plan& plan)
{
    MfmaFn fn = lookup_mfma(m);
    if (!fn) return 0;
    return occupancy(reinterpret_cast<const void*>(fn), plan.threads_per_wg,
                     mfma_lds_bytes(m, plan));
}

int mfma_kernel_info(int64_t m, const mnb_plan& plan, mnb_kernel_info* info)
{
    MfmaFn fn = lookup_mfma(m);
    if (!fn) return -1;
    hipFuncAttributes attr;
    hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(fn));
    if (e != hipSuccess) return (int)e;
    info->vgprs = attr.numRegs;
    info->sgprs = 0;
    info->lds_bytes = (int32_t)(attr.sharedSizeBytes + mfma_lds_bytes(m, plan));
    info->max_threads = attr.maxThreadsPerBlock;
    info->wgs_per_cu = mfma_workgroups_per_cu(m, plan);
    return 0;
}

}  // namespace mnb
