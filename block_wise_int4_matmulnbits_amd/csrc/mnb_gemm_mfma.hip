// Prefill INT4 MatMulNBits (m > 8 rows) on the matrix cores of gfx950.
//
//   y[r][n] = sum_k a[r][k] * (q[n][k] - z[n][k/32]) * s[n][k/32]
//
// The same operation, arithmetic and epilogue as the decode kernels
// (onnx-genai pull request "perf(cuda): let the split-K decode GEMV store
// bf16 directly", opening paragraphs and the paragraph on
// matmul_nbits_store_narrowed; pull request "PORT-1 (offline
// bias+interleave)", "Why the premise fails here", item 1): weights enter
// the products as exact fp16 integers q - z, each 32-weight block's fp32
// product is scaled by its fp16 scale in fp32, the fp32 sum is rounded to
// fp16 once and, for bf16 output, narrowed to bf16 in the same kernel.
// The first page names a row-batched path without the narrowing store as
// the next step; this is that path with the store.
//
// Work decomposition.  A workgroup of four waves owns an output tile of
// 16*RT rows by 64 columns; wave w owns columns 16w .. 16w+15 of it and all
// RT row tiles, so each weight it unpacks feeds RT MFMAs.  K is walked one
// quad (4 blocks, 128 k) at a time:
//   - activations of the quad (16*RT rows x 128 k) are loaded by all 256
//     threads, converted to fp16, permuted into the unpack's pair order and
//     written to one of two LDS buffers ([block][row][16-byte piece], so the
//     operand reads of a wave are 1 KB contiguous);
//   - lane (j, g) loads block 4t+g of column j (16 bytes) with the quad's 4
//     scales (8 bytes) and zero points (2 bytes); two v_permlane32_swap and
//     two v_permlane16_swap put dword g of every block of the quad in row g
//     (the B operand layout), and the nibbles become exact fp16 pairs q - z;
//   - per block and row tile one v_mfma_f32_16x16x32_f16 (A rows from LDS,
//     B = the unpacked block), whose fp32 result is scaled by the block's
//     scale into the row tile's accumulators.
// Weight loads run three quads ahead of use, activation loads two.  The
// summation order of an output depends only on K: equal inputs give equal
// bits for any M, N and grid.
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

struct GemmParams {
    const uint16_t* A;       // [M][K]
    const uint8_t* B;        // [N][K/2]
    const uint16_t* scales;  // [N][nb]
    const uint8_t* zp;       // [N][zb] or null
    uint16_t* out;           // [M][N]
    int64_t M, N;
    int32_t K, nb, zb;
    uint32_t zero;           // always 0 (see vgpr_constant)
    int32_t a_bf16, out_bf16;
};

constexpr int kGemmWaves = 4;      // waves per workgroup (64 output columns)
constexpr int kGemmRing = 3;       // weight quads in flight per wave

struct WQuad {
    u32x4 w;          // 16 bytes: block 4t+g of this lane's column
    uint32_t s[4];    // fp16 scales of blocks 4t..4t+3 (VEC: two words)
    uint32_t z[2];    // zero-point bytes 2t, 2t+1 (VEC: one 16-bit word)
};

template <int RT, bool VEC>
__global__ __launch_bounds__(256) void mnb_gemm_mfma_kernel(GemmParams p)
{
    constexpr int MT = 16 * RT;              // rows per workgroup tile
    constexpr int QA = 16 * MT;              // 16-byte pieces of activations per quad
    constexpr int P = kGemmRing;
    extern __shared__ uint4 a_lds[];         // [2][4 blocks][MT rows][4 pieces]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int j = lane & 15, g = lane >> 4;
    const int nb = p.nb;
    const int nq = (nb + 3) / 4;
    const uint32_t row_bytes = (uint32_t)p.K / 2;
    const uint32_t zdef = p.zp ? 0u : 8u;    // zero point 8 when none are given
    const uint32_t magic = vgpr_constant(0x64006400u, p.zero);
    const int64_t tiles_m = (p.M + MT - 1) / MT;
    const int64_t tiles_n = (p.N + 63) / 64;

    // Eight activations to fp16 (bf16 rounded to nearest even), permuted
    // into the unpack's pair order.
    auto to_pairs = [&](uint4 v) {
        uint32_t x = v.x, y = v.y, z = v.z, w = v.w;
        if (p.a_bf16) {
            x = bf16x2_to_f16x2(x);
            y = bf16x2_to_f16x2(y);
            z = bf16x2_to_f16x2(z);
            w = bf16x2_to_f16x2(w);
        }
        uint4 o;
        o.x = (x & 0xFFFFu) | (z << 16);          // (a0,a4)
        o.y = (x >> 16) | (z & 0xFFFF0000u);      // (a1,a5)
        o.z = (y & 0xFFFFu) | (w << 16);          // (a2,a6)
        o.w = (y >> 16) | (w & 0xFFFF0000u);      // (a3,a7)
        return o;
    };

    for (int64_t tile = blockIdx.x; tile < tiles_m * tiles_n; tile += gridDim.x) {
        // Consecutive workgroups share a row block (its activations stay in
        // L2) and walk the column blocks.
        const int64_t tm = tile / tiles_n, tn = tile - tm * tiles_n;
        const int64_t r0 = tm * MT;
        const int64_t col0 = tn * 64 + 16 * wv;   // this wave's 16 columns
        const int64_t left = p.N - col0;
        const uint32_t ncols = left <= 0 ? 0u : (uint32_t)(left < 16 ? left : 16);
        const int64_t cb = left <= 0 ? 0 : col0;
        // Buffer resources over the wave's 16 column rows; loads past their
        // end (columns past N, blocks past K, quads past K, absent zero
        // points) return zeros without touching memory.
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B + cb * row_bytes, (uint64_t)ncols * row_bytes);
        const __amdgpu_buffer_rsrc_t rS = make_rsrc(p.scales + cb * nb, (uint64_t)ncols * nb * 2);
        const __amdgpu_buffer_rsrc_t rZ =
            make_rsrc(p.zp ? p.zp + cb * p.zb : p.B, p.zp ? (uint64_t)ncols * p.zb : 0);
        const uint32_t wbase = (uint32_t)j * row_bytes + 16 * (uint32_t)g;
        const uint32_t sbase = (uint32_t)j * (uint32_t)nb * 2;
        const uint32_t zbase = (uint32_t)j * (uint32_t)p.zb;

        auto issue = [&](WQuad& q, int t) {
            const bool live = t < nq;
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

        // Activations of quad t: thread tid holds pieces tid + 256 s, piece e
        // = (block * MT + row) * 4 + piece16 (zeros past M and past K).
        auto fetch_a = [&](uint4 (&v)[RT], int t) {
#pragma unroll
            for (int s = 0; s < RT; ++s) {
                const int e = tid + 256 * s;
                const int br = e >> 2, piece = e & 3;
                const int i = br / MT, row = br - i * MT;
                const int64_t r = r0 + row;
                const int b = 4 * t + i;
                v[s] = make_uint4(0, 0, 0, 0);
                if (t < nq && r < p.M && b < nb)
                    v[s] = *reinterpret_cast<const uint4*>(p.A + r * p.K + 32 * (int64_t)b + 8 * piece);
            }
        };
        auto store_a = [&](const uint4 (&v)[RT], int buf) {
#pragma unroll
            for (int s = 0; s < RT; ++s) a_lds[buf * QA + tid + 256 * s] = to_pairs(v[s]);
        };

        float acc[RT][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[rt][rr] = 0.f;

        // Unpack the quad's four blocks, one MFMA per block and row tile,
        // scale the block products into the accumulators.
        auto compute = [&](const WQuad& q, int buf) {
            uint32_t r[4] = {q.w[0], q.w[1], q.w[2], q.w[3]};
            transpose_rows(r);
            const uint32_t zw = VEC ? q.z[0] : ((q.z[0] & 0xFFu) | ((q.z[1] & 0xFFu) << 8));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t bq[4];
                unpack_dword(r[i], zero_point_pairs(((zw >> (4 * i)) & 0xFu) | zdef), magic, bq);
                const u32x4 bv = {bq[0], bq[1], bq[2], bq[3]};
                const uint32_t sw = VEC ? (i < 2 ? q.s[0] : q.s[1]) >> (16 * (i & 1)) : q.s[i];
                const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)(sw & 0xFFFFu));
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const uint4 av = a_lds[buf * QA + ((i * MT + rt * 16 + j) * 4 + g)];
                    const u32x4 aw = {av.x, av.y, av.z, av.w};
                    const float4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(half8_t, aw), __builtin_bit_cast(half8_t, bv),
                        float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) acc[rt][rr] = fmaf(d[rr], sf, acc[rt][rr]);
                }
            }
        };

        WQuad ring[P];
#pragma unroll
        for (int s = 0; s < P; ++s) issue(ring[s], s);
        uint4 av[RT];
        fetch_a(av, 0);
        __syncthreads();                  // the previous tile's readers are done
        store_a(av, 0);
        fetch_a(av, 1);
        for (int t0 = 0; t0 < nq; t0 += P) {
#pragma unroll
            for (int s = 0; s < P; ++s) {
                const int t = t0 + s;
                if (t < nq) {
                    // Buffer t&1 is complete, and every wave is done with
                    // buffer (t+1)&1 (it held quad t-1).
                    __syncthreads();
                    if (t + 1 < nq) store_a(av, (t + 1) & 1);
                    fetch_a(av, t + 2);
                    compute(ring[s], t & 1);
                }
                issue(ring[s], t + P);
            }
        }

        // Epilogue: fp32 -> fp16 (RNE), optionally -> bf16 (RNE), store.
        const int64_t col = col0 + j;
        if (col < p.N) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int64_t row = r0 + rt * 16 + 4 * g + rr;
                    if (row < p.M) {
                        const _Float16 h = (_Float16)acc[rt][rr];
                        uint16_t bits = __builtin_bit_cast(uint16_t, h);
                        if (p.out_bf16) bits = f16_to_bf16(bits);
                        p.out[row * p.N + col] = bits;
                    }
                }
        }
    }
}

typedef void (*GemmFn)(GemmParams);

template <bool VEC>
GemmFn lookup_gemm_vec(int rt)
{
    switch (rt) {
    case 1: return mnb_gemm_mfma_kernel<1, VEC>;
    case 2: return mnb_gemm_mfma_kernel<2, VEC>;
    case 4: return mnb_gemm_mfma_kernel<4, VEC>;
    case 8: return mnb_gemm_mfma_kernel<8, VEC>;
    }
    return nullptr;
}

GemmFn lookup_gemm(int rt, bool vec)
{
    return vec ? lookup_gemm_vec<true>(rt) : lookup_gemm_vec<false>(rt);
}

bool gemm_vec_ok(int64_t K, const void* scales, const void* zp)
{
    return (K / 32) % 4 == 0 && ((uintptr_t)scales & 7) == 0 && ((uintptr_t)zp & 1) == 0;
}

}  // namespace

size_t gemm_lds_bytes(const mnb_plan& plan)
{
    return (size_t)2 * 4 * 16 * plan.row_tiles * 4 * 16;
}

int launch_gemm(const GemvArgs& a, const mnb_plan& plan, void* stream)
{
    GemmFn fn = lookup_gemm(plan.row_tiles, gemm_vec_ok(a.K, a.scales, a.zp));
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    GemmParams p;
    p.A = static_cast<const uint16_t*>(a.A);
    p.B = a.B;
    p.scales = a.scales;
    p.zp = a.zp;
    p.out = static_cast<uint16_t*>(a.out);
    p.M = a.m;
    p.N = a.N;
    p.K = (int32_t)a.K;
    p.nb = (int32_t)(a.K / 32);
    p.zb = (p.nb + 1) / 2;
    p.zero = 0;
    p.a_bf16 = a.a_bf16;
    p.out_bf16 = a.out_bf16;
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn),
                                   dim3((unsigned)plan.workgroups), dim3(64 * kGemmWaves), args,
                                   gemm_lds_bytes(plan), static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
    return (int)e;
}

int gemm_workgroups_per_cu(const mnb_plan& plan)
{
    GemmFn fn = lookup_gemm(plan.row_tiles, true);
    if (!fn) return 0;
    return occupancy(reinterpret_cast<const void*>(fn), 64 * kGemmWaves, gemm_lds_bytes(plan));
}

int gemm_kernel_info(const mnb_plan& plan, mnb_kernel_info* info)
{
    GemmFn fn = lookup_gemm(plan.row_tiles, true);
    if (!fn) return -1;
    hipFuncAttributes attr;
    hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(fn));
    if (e != hipSuccess) return (int)e;
    info->vgprs = attr.numRegs;
    info->sgprs = 0;
    info->lds_bytes = (int32_t)(attr.sharedSizeBytes + gemm_lds_bytes(plan));
    info->max_threads = attr.maxThreadsPerBlock;
    info->wgs_per_cu = gemm_workgroups_per_cu(plan);
    return 0;
}

}  // namespace mnb
