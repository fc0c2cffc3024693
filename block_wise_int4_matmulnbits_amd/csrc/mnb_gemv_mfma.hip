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
    uint32_t zero;           // always 0 (see vgpr_constant)
    int32_t a_bf16, out_bf16;
};

// Quads of weights in flight per wave: a ring of P register sets, refilled
// as each is consumed, so a wave keeps P*1 KB of weights (plus scales and
// zero points) in flight instead of one quad.
template <bool VEC>
constexpr int kRing = VEC ? 8 : 4;

// Registers of one quad for one lane.
struct Quad {
    u32x4 w;          // 16 bytes: block 4t+g of this lane's column
    uint32_t s[4];    // fp16 scales of blocks 4t..4t+3 (VEC: two words, s[0..1])
    uint32_t z[2];    // zero-point bytes 2t, 2t+1 (VEC: one 16-bit word, z[0])
};

// VEC: scales of a quad read as one 8-byte load and its zero points as one
// 2-byte load (K/32 a multiple of 4, scales 8-byte and zero points 2-byte
// aligned); otherwise one load per scale and per zero-point byte.
template <int M, bool VEC>
__global__ __launch_bounds__(512) void mnb_gemv_mfma_kernel(MfmaParams p)
{
    constexpr int RR = M < 4 ? M : 4;       // result rows 4g .. 4g+RR-1 per lane
    constexpr int P = kRing<VEC>;
    __shared__ float red[8][RR][64];        // per-wave partial tiles
    extern __shared__ uint4 a_lds[];        // [chunk_blocks][M][4] permuted fp16 A

    const int tid = threadIdx.x;
    const int lane = tid & 63, W = (int)(blockDim.x >> 6);
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int j = lane & 15, g = lane >> 4;
    const int nb = p.nb, kcb = p.chunk_blocks;
    const int64_t ntiles = (p.N + 15) / 16;
    const uint32_t row_bytes = (uint32_t)p.K / 2;
    const uint32_t zdef = p.zp ? 0u : 8u;   // zero point 8 when none are given
    const uint32_t magic = vgpr_constant(0x64006400u, p.zero);   // fp16 pair (1024, 1024)

    // Stage rows 0..M-1, blocks b_lo .. b_lo+nbc-1 of A into LDS, converted
    // to fp16 and permuted to (a0,a4),(a1,a5),(a2,a6),(a3,a7) per 8 k.
    // Eight 16-byte loads per thread go out before any is converted.
    auto stage = [&](int b_lo, int nbc) {
        constexpr int U = 8;
        const int n16 = M * nbc * 4;
        const int step = (int)blockDim.x;
        for (int u0 = tid; u0 < n16; u0 += U * step) {
            uint4 v[U];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int u = u0 + i * step;
                v[i] = make_uint4(0, 0, 0, 0);
                if (u < n16) {
                    const int b = u / (4 * M);
                    const int r = (u >> 2) - b * M, gg = u & 3;
                    v[i] = *reinterpret_cast<const uint4*>(
                        p.A + (int64_t)r * p.K + 32 * (int64_t)(b_lo + b) + 8 * gg);
                }
            }
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int u = u0 + i * step;
                if (u >= n16) break;
                uint32_t x = v[i].x, y = v[i].y, z = v[i].z, w = v[i].w;
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
                a_lds[u] = o;                          // [b][r][gg]
            }
        }
        // Zeros after a ragged last block, up to the quad boundary, so the
        // unconditional operand reads of the last quad stay finite.
        const int tail = ((nbc + 3) & ~3) * M * 4;
        for (int u = n16 + tid; u < tail; u += step) a_lds[u] = make_uint4(0, 0, 0, 0);
    };

    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t col0 = tile * 16;
        const int64_t col = col0 + j;
        const bool col_ok = col < p.N;
        const uint32_t ncols = (uint32_t)(p.N - col0 < 16 ? p.N - col0 : 16);
        // Buffer resources over the tile's 16 column rows; loads past their
        // end (columns past N, blocks past K, quads past this wave's range,
        // absent zero points) return zeros without touching memory, so every
        // load is issued unconditionally and the wait counts stay exact.
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B + col0 * row_bytes, (uint64_t)ncols * row_bytes);
        const __amdgpu_buffer_rsrc_t rS = make_rsrc(p.scales + col0 * nb, (uint64_t)ncols * nb * 2);
        const __amdgpu_buffer_rsrc_t rZ =
            make_rsrc(p.zp ? p.zp + col0 * p.zb : p.B, p.zp ? (uint64_t)ncols * p.zb : 0);
        const uint32_t wbase = (uint32_t)j * row_bytes + 16 * (uint32_t)g;
        const uint32_t sbase = (uint32_t)j * (uint32_t)nb * 2;
        const uint32_t zbase = (uint32_t)j * (uint32_t)p.zb;

        // Queue the loads of quad t (blocks 4t..4t+3 of K) if `live`.
        auto issue = [&](Quad& q, int t, bool live) {
            const uint32_t b = 4 * (uint32_t)t;
            q.w = __builtin_amdgcn_raw_buffer_load_b128(
                rB, live && b + g < (uint32_t)nb ? wbase + 16 * b : kOutOfRange, 0, kNontemporal);
            if constexpr (VEC) {
                const u32x2 sv = __builtin_amdgcn_raw_buffer_load_b64(
                    rS, live ? sbase + 2 * b : kOutOfRange, 0, kNontemporal);
                q.s[0] = sv[0];
                q.s[1] = sv[1];
                q.z[0] = __builtin_amdgcn_raw_buffer_load_b16(
                    rZ, live ? zbase + b / 2 : kOutOfRange, 0, kNontemporal);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    q.s[i] = __builtin_amdgcn_raw_buffer_load_b16(
                        rS, live && b + i < (uint32_t)nb ? sbase + 2 * (b + i) : kOutOfRange, 0,
                        kNontemporal);
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    q.z[i] = __builtin_amdgcn_raw_buffer_load_b8(
                        rZ, live && b / 2 + i < (uint32_t)p.zb ? zbase + b / 2 + i : kOutOfRange, 0,
                        kNontemporal);
            }
        };

        // Unpack, MFMA and scale the four blocks of a quad.  rel = quad start
        // relative to the staged chunk.  Rows j >= M of the A operand read
        // row 0 (their products land in result rows that are never
        // stored), so every operand read is unconditional; the four reads,
        // unpacks and MFMAs go out before the scaling, which waits on them.
        const int jr = j < M ? j : 0;
        auto compute = [&](const Quad& q, int rel, float (&acc)[RR]) {
            uint32_t r[4] = {q.w[0], q.w[1], q.w[2], q.w[3]};
            transpose_rows(r);
            const uint32_t zw = VEC ? q.z[0] : ((q.z[0] & 0xFFu) | ((q.z[1] & 0xFFu) << 8));
            uint4 av[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = a_lds[((rel + i) * M + jr) * 4 + g];
            float4_t d[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t bq[4];
                unpack_dword(r[i], zero_point_pairs(((zw >> (4 * i)) & 0xFu) | zdef), magic, bq);
                const u32x4 bv = {bq[0], bq[1], bq[2], bq[3]};
                const u32x4 aw = {av[i].x, av[i].y, av[i].z, av[i].w};
                d[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(half8_t, aw), __builtin_bit_cast(half8_t, bv),
                    float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t sw = VEC ? (i < 2 ? q.s[0] : q.s[1]) >> (16 * (i & 1)) : q.s[i];
                const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)(sw & 0xFFFFu));
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) acc[rr] = fmaf(d[i][rr], sf, acc[rr]);
            }
        };

        float acc[RR];
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) acc[rr] = 0.f;

        for (int ch = 0; ch < p.chunks; ++ch) {
            const int b_lo = ch * kcb;
            const int nbc = min(kcb, nb - b_lo);
            const int nq = (nbc + 3) / 4;
            const int q0 = wv * nq / W, q1 = (wv + 1) * nq / W;
            const int T0 = b_lo / 4;         // first quad of the chunk (kcb % 4 == 0)
            Quad ring[P];
            // The ring fills before the staging wait.
#pragma unroll
            for (int s = 0; s < P; ++s) issue(ring[s], T0 + q0 + s, q0 + s < q1);
            // Activations: staged once per workgroup when K fits one chunk,
            // else chunk by chunk (after every wave is done with the last).
            if (p.chunks > 1 || tile == (int64_t)blockIdx.x) {
                __syncthreads();
                stage(b_lo, nbc);
                __syncthreads();
            }
            for (int t = q0; t < q1; t += P) {
#pragma unroll
                for (int s = 0; s < P; ++s) {
                    if (t + s < q1) compute(ring[s], 4 * (t + s), acc);
                    issue(ring[s], T0 + t + s + P, t + s + P < q1);
                }
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

template <bool VEC>
MfmaFn lookup_mfma_vec(int64_t m)
{
    switch (m) {
    case 1: return mnb_gemv_mfma_kernel<1, VEC>;
    case 2: return mnb_gemv_mfma_kernel<2, VEC>;
    case 3: return mnb_gemv_mfma_kernel<3, VEC>;
    case 4: return mnb_gemv_mfma_kernel<4, VEC>;
    case 5: return mnb_gemv_mfma_kernel<5, VEC>;
    case 6: return mnb_gemv_mfma_kernel<6, VEC>;
    case 7: return mnb_gemv_mfma_kernel<7, VEC>;
    case 8: return mnb_gemv_mfma_kernel<8, VEC>;
    }
    return nullptr;
}

// The vectorised quad loads need K/32 % 4 == 0 and aligned scale and
// zero-point rows; the kernel variant is chosen per call.
bool mfma_vec_ok(int64_t K, const void* scales, const void* zp)
{
    return (K / 32) % 4 == 0 && ((uintptr_t)scales & 7) == 0 && ((uintptr_t)zp & 1) == 0;
}

MfmaFn lookup_mfma(int64_t m, bool vec)
{
    return vec ? lookup_mfma_vec<true>(m) : lookup_mfma_vec<false>(m);
}

size_t mfma_lds_bytes(int64_t m, const mnb_plan& plan)
{
    return (size_t)m * (size_t)plan.chunk_blocks * 64;
}

}  // namespace

int launch_mfma(const GemvArgs& a, const mnb_plan& plan, void* stream)
{
    MfmaFn fn = lookup_mfma(a.m, mfma_vec_ok(a.K, a.scales, a.zp));
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
    p.zero = 0;
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
    MfmaFn fn = lookup_mfma(m, true);
    if (!fn) return 0;
    return occupancy(reinterpret_cast<const void*>(fn), plan.threads_per_wg,
                     mfma_lds_bytes(m, plan));
}

int mfma_kernel_info(int64_t m, const mnb_plan& plan, mnb_kernel_info* info)
{
    MfmaFn fn = lookup_mfma(m, true);
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
