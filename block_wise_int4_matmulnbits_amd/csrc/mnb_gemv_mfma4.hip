// Row-batched INT4 MatMulNBits GEMV (a few rows) on the 4x4x4 matrix
// product of gfx950, v_mfma_f32_4x4x4_16b_f16.
//
//   y[r][n] = sum_k a[r][k] * (q[n][k] - z[n][k/32]) * s[n][k/32]
//
// The operation, arithmetic and epilogue are those of the lane-split kernel
// (onnx-genai pull request "perf(cuda): let the split-K decode GEMV store
// bf16 directly", opening paragraphs and the paragraph on
// matmul_nbits_store_narrowed; pull request "PORT-1 (offline
// bias+interleave)", "Why the premise fails here", item 1): fp16 (or bf16
// rounded to fp16) activations, exact products a * (q - z) summed in fp32
// per 32-weight block, the block's fp16 scale applied by one fp32 FMA, one
// fp16 rounding of the total and, for bf16 output, the narrowing to bf16.
//
// Why this shape.  With several rows the lane-split kernel spends four
// v_dot2 per eight weights per row; one v_mfma_f32_4x4x4_16b_f16 does the
// work of eight of them in about two of their issue slots.  The instruction
// is sixteen independent 4x4x4 products, one per group of four lanes: lane
// 4b+i supplies row i of block b's A operand (four k) and column i of its B
// operand, and receives column i of the 4x4 result (register r = row r).
//
// Work decomposition.  A workgroup of W waves owns a contiguous range of
// column quads and walks it NC quads at a time.  Lane (g, i) of a wave (group
// g = lane / 4) holds column 4n + i of each quad n and, as the A side, rows i
// and 4 + i of the activations.  Wave w owns the 16 BPL consecutive K blocks
// from 16 BPL w, and its group g the blocks 16 BPL w + 16 j + g (j < BPL);
// together the waves cover all of K in one pass (where K does not fill W
// waves of BPL, the later waves take three blocks of four: see the kernel).
// The lane's activations are loaded once (under the plan's a_via_lds a row
// at a time, 1 KB per load, and handed to their lanes through a
// wave-private LDS buffer), converted to fp16,
// permuted into the unpack's pair order and kept in VGPRs.  Per block and column the lane loads its 16 bytes of
// weights (the four lanes of a group read four columns, the sixteen groups
// of a wave 256 contiguous bytes of each).  A wave's scales and zero points
// of a column are one contiguous run, read as whole dwords (full lines, any
// alignment of the arrays) and handed to the lanes through a small
// wave-private LDS stage: one 2- and one 1-byte load per lane and block had
// cost a load-only copy of this kernel 1.9 us on the down projection.  The
// lane unpacks its weights to the exact fp16 integers q - z, and per row
// quad eight chained MFMAs give the block's exact 4 x 4 product, which one
// FMA per row scales into the lane's fp32 accumulators.  Partial sums meet through a
// fixed tree inside the wave (rows paired through v_permlane32_swap and
// v_permlane16_swap, then two DPP row rotations) and a wave-ordered sum in
// LDS, so the summation order depends only on (K, W, BPL).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb.h"
#include "mnb_device.h"
#include "mnb_internal.h"

namespace mnb {
namespace {

struct Mfma4Params {
    const uint16_t* A;       // [m][K]
    const uint8_t* B;        // [N][K/2]
    const uint16_t* scales;  // [N][nb]
    const uint8_t* zp;       // [N][zb] or null
    uint16_t* out;           // [m][N]
    int64_t N;
    int32_t m, K, nb, zb;
    uint32_t zero;           // always 0 (see vgpr_constant)
    int32_t a_bf16, out_bf16;
    int32_t waves_hi;        // four blocks per lane group: waves [0, waves_hi) take
                             // four, the others three (see the kernel)
    int32_t eo_pairs;        // weights in the even/odd nibble layout: the unpack
                             // yields (k, k+1) pairs, activations keep their order
};

// Per wave of an XP variant: an LDS buffer through which the activations
// reach their lanes (four rows of 65 16-byte pieces); the launch gives
// waves_per_wg of them as dynamic LDS.
constexpr int kXposePieces = 4 * 65;
constexpr size_t kXposeBytesPerWave = kXposePieces * 16;

// RQ row quads (m <= 4 * RQ), BPL blocks per lane group, NC column quads per
// tile; XP: activations loaded a row at a time and passed through LDS (below),
// else each lane loads its own row and block directly.  The tile loop is straight-line code, two tiles per pass: each wave
// leaves its totals of the pass's two tiles in LDS, and one barrier, the
// sums over waves and another barrier close the pass.
template <int BPL, int NC>
constexpr int stage_dwords()   // a wave's LDS stage of one tile's scale and zero-point dwords
{
    return 64 * ((4 * NC * (8 * BPL + 1) + 63) / 64 + (4 * NC * (2 * BPL + 1) + 63) / 64);
}

// The wave's work (see the kernel): blocks B0 + 16 j + g of K (j < BPL) for
// every tile of the workgroup.  part: [2][8][NV] per-wave totals of a pass's
// two tiles, shared by all waves; st: this wave's stage.
template <int RQ, int BPL, int NC, bool XP>
__device__ __forceinline__ void mfma4_wave(const Mfma4Params& p, const uint32_t B0, float* const part,
                                           uint32_t* const st)
{
    constexpr int NV = 16 * NC * RQ;        // results of one tile (columns x rows)
    constexpr int NCOL = 4 * NC;            // columns of a tile
    constexpr int DS = 8 * BPL + 1;         // dwords covering a wave's 16 BPL scales of a column
    constexpr int DZ = 2 * BPL + 1;         // dwords covering its 16 BPL zero-point nibbles
    constexpr int SD = (NCOL * DS + 63) / 64;   // scale dwords loaded per lane and tile
    constexpr int ZD = (NCOL * DZ + 63) / 64;   // zero-point dwords loaded per lane and tile
    extern __shared__ u32x4 xpose_lds[];            // kXposePieces per wave

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int W = (int)(blockDim.x >> 6);
    const int qi = lane & 3, g = lane >> 2;
    const uint32_t nb = (uint32_t)p.nb, zb = (uint32_t)p.zb;
    const uint32_t row_bytes = (uint32_t)p.K / 2;
    // The wave owns the 16 BPL consecutive blocks from B0; lane group g takes
    // blocks B0 + 16 j + g (j < BPL), so each load instruction of a wave reads
    // 256 contiguous bytes of each of four columns, and a wave's scales (and
    // zero points) of a column are one contiguous run.
    const int zshift = (g & 1) * 4;         // block parity == group parity (B0 even)
    const uint32_t zdef = p.zp ? 0u : 8u;   // zero point 8 when none are given
    const ZeroPoint zbase = zero_point_pairs(zdef);
    const uint32_t magic = vgpr_constant(0x64006400u, p.zero);   // fp16 pair (1024, 1024)

    // Column quads [q_first, q_stop) of this workgroup.
    const int64_t nq = (p.N + 3) / 4;
    const int64_t q_first = nq * blockIdx.x / gridDim.x;
    const int64_t q_stop = nq * (blockIdx.x + 1) / gridDim.x;
    const int64_t c_stop = 4 * q_stop < p.N ? 4 * q_stop : p.N;

    // Activations: rows 4 rq + qi of this group's blocks B0 + 16 j + g; rows
    // past m and blocks past K load zeros.  With XP, load i of row quad rq
    // and block group j reads row 4 rq + i over the wave's 16 blocks B0 +
    // 16 j .. B0 + 16 j + 15, 1 KB contiguous (lane l takes piece l % 4 of
    // block l / 4), and the pieces reach their lanes through LDS below.
    // The direct loads (16 bytes of four rows per lane, 64 bytes apart)
    // take 2-4 times as many cache lines per load, which leaves the staging
    // slower from three rows up on long K or many columns (down projection
    // m = 3, 4 and 8: 12.5, 13.6 and 18.3 us direct against 11.5, 11.9 and
    // 15.7 with XP); the plan's a_via_lds selects XP.
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, (uint64_t)p.m * (uint64_t)p.K * 2);
    u32x4 raw[RQ][BPL][4];
#pragma unroll
    for (int rq = 0; rq < RQ; ++rq)
#pragma unroll
        for (int j = 0; j < BPL; ++j) {
            if constexpr (XP) {
                const uint32_t b = B0 + 16 * (uint32_t)j + (uint32_t)(lane >> 2);
                const uint32_t base = 64 * (B0 + 16 * (uint32_t)j) + 16 * (uint32_t)lane;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    raw[rq][j][i] = __builtin_amdgcn_raw_buffer_load_b128(
                        rA, b < nb ? (uint32_t)(4 * rq + i) * (uint32_t)p.K * 2 + base : kOutOfRange, 0, 0);
            } else {
                const uint32_t b = B0 + 16 * (uint32_t)j + (uint32_t)g;
                const uint32_t base = (uint32_t)(4 * rq + qi) * (uint32_t)p.K * 2 + 64 * b;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    raw[rq][j][i] = __builtin_amdgcn_raw_buffer_load_b128(rA, b < nb ? base + 16 * i : kOutOfRange, 0, 0);
            }
        }

    struct Tile {
        u32x4 w[NC][BPL];
        uint32_t sd[SD];   // whole dwords covering the wave's scales of the tile's columns
        uint32_t zd[ZD];   // and its zero points
    };
    // Scales and zero points are read as whole dwords from 4-byte-aligned
    // resource bases (ms, mz: how far the arrays start past such a boundary;
    // tiles advance the bases by multiples of 4 bytes, so these stay fixed).
    // Lane L loads dword L % D of column L / D of the tile's runs (D = DS or
    // DZ), in full lines rather than one 2- or 1-byte load per block.
    const uint32_t ms = (uint32_t)((uintptr_t)p.scales & 3);
    const uint32_t mz = p.zp ? (uint32_t)((uintptr_t)p.zp & 3) : 0u;
    uint32_t ow[NC][BPL], osd[SD], ozd[ZD];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const uint32_t col = (uint32_t)(4 * n + qi);
#pragma unroll
        for (int j = 0; j < BPL; ++j) {
            const uint32_t b = B0 + 16 * (uint32_t)j + (uint32_t)g;
            ow[n][j] = b < nb ? col * row_bytes + 16 * b : kOutOfRange;
        }
    }
#pragma unroll
    for (int k = 0; k < SD; ++k) {
        const uint32_t item = 64 * (uint32_t)k + (uint32_t)lane, c = item / DS, kk = item % DS;
        osd[k] = c < NCOL ? ((ms + c * nb * 2 + B0 * 2) & ~3u) + 4 * kk : kOutOfRange;
    }
#pragma unroll
    for (int k = 0; k < ZD; ++k) {
        const uint32_t item = 64 * (uint32_t)k + (uint32_t)lane, c = item / DZ, kk = item % DZ;
        ozd[k] = c < NCOL ? ((mz + c * zb + B0 / 2) & ~3u) + 4 * kk : kOutOfRange;
    }
    // Blocks of this lane group past K: their weights and activations load
    // zeros, but the bytes the scale dwords bring for them lie past the
    // column's scales (the next column's, or past the array for the last
    // column, where they may hold anything), so their scale is taken as 0:
    // a product of 0 and a NaN or infinity read there would poison the sum.
    bool in_k[BPL];
#pragma unroll
    for (int j = 0; j < BPL; ++j) in_k[j] = B0 + 16 * (uint32_t)j + (uint32_t)g < nb;
    // Where this lane finds its own scale and zero point of column 4n + qi,
    // block B0 + 16 j + g, in the wave's stage (bytes; + 32 j and + 8 j).
    uint32_t sread[NC], zread[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const uint32_t c = (uint32_t)(4 * n + qi);
        sread[n] = 4 * c * DS + ((ms + c * nb * 2 + B0 * 2) & 3u) + 2 * (uint32_t)g;
        zread[n] = 4 * (64 * SD + c * DZ) + ((mz + c * zb + B0 / 2) & 3u) + (uint32_t)g / 2;
    }

    // Loads of the next tile of this workgroup (NC column quads).  Tiles are
    // issued in column order, so the bases of the three buffer resources
    // advance by fixed strides and the columns left count down; the
    // resources end at the workgroup's last column (zeros past it, without
    // touching memory), and a tile past q_stop gets empty ones.
    const uint8_t* next_B = p.B + 4 * q_first * (int64_t)row_bytes;
    const uint8_t* next_S = reinterpret_cast<const uint8_t*>(p.scales + 4 * q_first * (int64_t)nb) - ms;
    const uint8_t* next_Z = p.zp ? p.zp + 4 * q_first * (int64_t)zb - mz : p.B;
    int64_t left = c_stop - 4 * q_first;
    auto issue = [&](Tile& t) {
        const uint32_t ncols = left <= 0 ? 0u : (uint32_t)(left < NCOL ? left : NCOL);
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(next_B, (uint64_t)ncols * row_bytes);
        const __amdgpu_buffer_rsrc_t rS = make_rsrc(next_S, ncols ? (ms + (uint64_t)ncols * nb * 2 + 3) & ~3ull : 0);
        const __amdgpu_buffer_rsrc_t rZ = make_rsrc(next_Z, p.zp && ncols ? (mz + (uint64_t)ncols * zb + 3) & ~3ull : 0);
#pragma unroll
        for (int n = 0; n < NC; ++n)
#pragma unroll
            for (int j = 0; j < BPL; ++j)
                t.w[n][j] = __builtin_amdgcn_raw_buffer_load_b128(rB, ow[n][j], 0, kNontemporal);
#pragma unroll
        for (int k = 0; k < SD; ++k) t.sd[k] = __builtin_amdgcn_raw_buffer_load_b32(rS, osd[k], 0, kNontemporal);
#pragma unroll
        for (int k = 0; k < ZD; ++k) t.zd[k] = __builtin_amdgcn_raw_buffer_load_b32(rZ, ozd[k], 0, kNontemporal);
        if (left > 0) {   // uniform; past the end the bases stay put
            next_B += NCOL * (int64_t)row_bytes;
            next_S += NCOL * (int64_t)nb * 2;
            if (p.zp) next_Z += NCOL * (int64_t)zb;
        }
        left -= NCOL;
    };

    Tile ring[2];
    issue(ring[0]);
    issue(ring[1]);

    // fp16 (bf16 rounded to nearest even), in the order in which the unpack
    // yields the weights: pairs (a_e, a_e+4) per 8 k, or (a_2e, a_2e+1) for
    // even/odd weights.
    // With XP each (row quad, block group) passes through the wave's LDS
    // buffer (four rows of 64 pieces, rows 65 pieces apart so that eight
    // lanes read 32 distinct banks): lane (g, qi) reads back the four pieces
    // of row 4 rq + qi, block B0 + 16 j + g.  The fences keep the compiler
    // from moving the reads above the writes of other lanes, or the next
    // writes above the reads (one wave's LDS operations run in order, so no
    // wait is emitted).
    uint32_t act[RQ][BPL][16];
#pragma unroll
    for (int rq = 0; rq < RQ; ++rq)
#pragma unroll
        for (int j = 0; j < BPL; ++j) {
            if constexpr (XP) {
                u32x4* const xw = xpose_lds + wv * kXposePieces;
#pragma unroll
                for (int i = 0; i < 4; ++i) xw[65 * i + lane] = raw[rq][j][i];
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                u32x4 mine[4];
#pragma unroll
                for (int pc = 0; pc < 4; ++pc) mine[pc] = xw[65 * qi + 4 * g + pc];
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                activation_pairs(mine, p.a_bf16, p.eo_pairs, act[rq][j]);
            } else {
                activation_pairs(raw[rq][j], p.a_bf16, p.eo_pairs, act[rq][j]);
            }
        }

    // Per block: the exact products of each row quad in one 4x4 result
    // (eight chained MFMAs over the block's 32 k), then acc += D * s.
    auto compute = [&](const Tile& t, float4_t (&acc)[NC][RQ]) {
        // The tile's scale and zero-point dwords into the wave's stage, then
        // each lane's own (the wave's DS operations run in order).
#pragma unroll
        for (int k = 0; k < SD; ++k) st[64 * k + lane] = t.sd[k];
#pragma unroll
        for (int k = 0; k < ZD; ++k) st[64 * (SD + k) + lane] = t.zd[k];
        // Lanes read bytes that other lanes of the wave wrote: the fence keeps
        // the compiler from moving those reads above the writes (the hardware
        // runs one wave's LDS operations in order, so no wait is emitted).
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const uint8_t* sb = reinterpret_cast<const uint8_t*>(st);
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            ZeroPoint zp[BPL];
            float sf[BPL];
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                const uint32_t zq = sb[zread[n] + 8 * j];
                zp[j] = zero_point_pairs(__builtin_amdgcn_ubfe(zq, zshift, 4), zbase);   // + zdef
                const uint16_t sbits = *reinterpret_cast<const uint16_t*>(sb + sread[n] + 32 * j);
                sf[j] = (float)__builtin_bit_cast(_Float16, in_k[j] ? sbits : (uint16_t)0);
            }
            float4_t dsum[BPL][RQ];
#pragma unroll
            for (int j = 0; j < BPL; ++j)
#pragma unroll
                for (int rq = 0; rq < RQ; ++rq) dsum[j][rq] = float4_t{0.f, 0.f, 0.f, 0.f};
            // Dword d of every block, then one MFMA per (block, row quad):
            // consecutive MFMAs are independent, each block's chain keeps its
            // order over k.
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t pr[BPL][4];
#pragma unroll
                for (int j = 0; j < BPL; ++j) unpack_dword(t.w[n][j][d], zp[j], magic, pr[j]);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < BPL; ++j)
#pragma unroll
                        for (int rq = 0; rq < RQ; ++rq)
                            dsum[j][rq] = __builtin_amdgcn_mfma_f32_4x4x4f16(
                                as_half4(act[rq][j][4 * d + 2 * h], act[rq][j][4 * d + 2 * h + 1]),
                                as_half4(pr[j][2 * h], pr[j][2 * h + 1]), dsum[j][rq], 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < BPL; ++j)
#pragma unroll
                for (int rq = 0; rq < RQ; ++rq)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[n][rq][r] = fmaf(dsum[j][rq][r], sf[j], acc[n][rq][r]);
        }
    };

    // Totals of a tile: the column sums inside the wave go to LDS slot k (the
    // tile's place in its pass); after the pass, the sums over the waves in
    // wave order are stored.
    auto store = [&](int64_t qs, int idx, float v) {
        const int64_t col = 4 * qs + idx / (4 * RQ);
        const int row = idx % (4 * RQ);
        if (row < p.m && col < c_stop) {
            const _Float16 h = (_Float16)v;               // fp32 -> fp16, RNE
            uint16_t bits = __builtin_bit_cast(uint16_t, h);
            if (p.out_bf16) bits = f16_to_bf16(bits);     // fp16 -> bf16, RNE
            p.out[(int64_t)row * p.N + col] = bits;
        }
    };
    auto finish = [&](float4_t (&acc)[NC][RQ], int k) {
        const int row = quad_total_row(lane >> 4);
#pragma unroll
        for (int n = 0; n < NC; ++n)
#pragma unroll
            for (int rq = 0; rq < RQ; ++rq) {
                const float t = quad_totals(acc[n][rq][0], acc[n][rq][1], acc[n][rq][2], acc[n][rq][3]);
                if ((lane & 12) == 0) part[(k * 8 + wv) * NV + ((4 * n + qi) * RQ + rq) * 4 + row] = t;
            }
    };

    // Two tiles per pass; an odd last tile is followed by one past the
    // workgroup's columns (zeros, never stored).  The tile's scaled sums are
    // pinned (an empty asm operand) and the scheduler fenced before its
    // reloads, so the last uses of the tile's registers precede the loads
    // that refill them: no copies, and no waits on those loads, at the loop
    // edge.  The pass ends with the sums over waves of its two tiles.
    for (int64_t qs = q_first; qs < q_stop; qs += 2 * NC) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float4_t acc[NC][RQ] = {};
            compute(ring[u], acc);
#pragma unroll
            for (int n = 0; n < NC; ++n)
#pragma unroll
                for (int rq = 0; rq < RQ; ++rq) asm volatile("" : "+v"(acc[n][rq]));
            __builtin_amdgcn_sched_barrier(0);
            issue(ring[u]);   // the tile two ahead: qs + (2 + u) NC
            finish(acc, u);
        }
        __syncthreads();
        for (int e = tid; e < 2 * NV; e += (int)blockDim.x) {   // 2 NV can exceed one wave
            const int t = e / NV, idx = e - t * NV;
            float v = part[t * 8 * NV + idx];
            for (int w = 1; w < W; ++w) v += part[(t * 8 + w) * NV + idx];
            store(qs + (int64_t)t * NC, idx, v);
        }
        __syncthreads();   // the slots are refilled by the next pass
    }
}

// W waves cover K in one pass.  With four blocks per lane group the fewest
// waves that need four take four (waves_hi of them) and the rest three, so
// that a K whose blocks do not fill W waves of four still spreads evenly
// over the SIMDs (K = 14336 on eight waves: four of 64 blocks and four of 48,
// two waves of 3.5 blocks' work per SIMD, where seven waves of 64 put two on
// three SIMDs and one on the fourth).  With every wave at four (waves_hi = W)
// this is the plain split, compiled without the second body (MIX false).
template <int RQ, int BPL, int NC, bool XP, bool MIX>
__global__ __launch_bounds__(512) void mnb_gemv_mfma4_kernel(Mfma4Params p)
{
    constexpr int NV = 16 * NC * RQ;
    constexpr int ST = stage_dwords<BPL, NC>();
    __shared__ float part[2 * 8 * NV];      // per-wave totals of a pass's two tiles
    __shared__ uint32_t stage[8 * ST];      // each wave's scales and zero points of one tile
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (MIX) {
        if (wv >= p.waves_hi) {
            mfma4_wave<RQ, 3, NC, XP>(p, (uint32_t)(64 * p.waves_hi + 48 * (wv - p.waves_hi)), part, stage + wv * ST);
            return;
        }
    }
    mfma4_wave<RQ, BPL, NC, XP>(p, (uint32_t)(16 * BPL * wv), part, stage + wv * ST);
}

typedef void (*Mfma4Fn)(Mfma4Params);

template <int RQ, int BPL, bool XP, bool MIX>
Mfma4Fn by_nc(int nc)
{
    switch (nc) {
    case 1: return mnb_gemv_mfma4_kernel<RQ, BPL, 1, XP, MIX>;
    case 2: return mnb_gemv_mfma4_kernel<RQ, BPL, 2, XP, MIX>;
    }
    return nullptr;
}

template <int RQ, bool XP>
Mfma4Fn by_bpl(int bpl, int nc, bool mix)
{
    switch (bpl) {
    case 1: return by_nc<RQ, 1, XP, false>(nc);
    case 2: return by_nc<RQ, 2, XP, false>(nc);
    case 4: return mix ? by_nc<RQ, 4, XP, true>(nc) : by_nc<RQ, 4, XP, false>(nc);
    }
    return nullptr;
}

// Waves with four blocks per lane group (plan.blocks_per_lane = 4): the
// fewest that, with three for the rest, cover K's nb blocks; all of them
// otherwise.
int mfma4_waves_hi(int64_t K, const mnb_plan& plan)
{
    const int64_t w = plan.threads_per_wg / 64;
    if (plan.blocks_per_lane != 4) return (int)w;
    int64_t hi = (K / 32 - 48 * w + 15) / 16;
    return (int)(hi < 0 ? 0 : (hi > w ? w : hi));
}


size_t mfma4_dynamic_lds(const mnb_plan& plan)
{
    return plan.a_via_lds ? (size_t)(plan.threads_per_wg / 64) * kXposeBytesPerWave : 0;
}

Mfma4Fn lookup_mfma4(int64_t m, int64_t K, const mnb_plan& plan)
{
    const int nc = plan.cols_per_tile / 4;
    const bool xp = plan.a_via_lds != 0;
    const bool mix = mfma4_waves_hi(K, plan) < plan.threads_per_wg / 64;
    const int bpl = plan.blocks_per_lane;
    if (m >= 1 && m <= 4) return xp ? by_bpl<1, true>(bpl, nc, mix) : by_bpl<1, false>(bpl, nc, mix);
    if (m >= 5 && m <= 8) return xp ? by_bpl<2, true>(bpl, nc, mix) : by_bpl<2, false>(bpl, nc, mix);
    return nullptr;
}

}  // namespace

int launch_mfma4(const GemvArgs& a, const mnb_plan& plan, void* stream)
{
    Mfma4Fn fn = lookup_mfma4(a.m, a.K, plan);
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    Mfma4Params p;
    p.A = static_cast<const uint16_t*>(a.A);
    p.B = a.B;
    p.scales = a.scales;
    p.zp = a.zp;
    p.out = static_cast<uint16_t*>(a.out);
    p.N = a.N;
    p.m = (int32_t)a.m;
    p.K = (int32_t)a.K;
    p.nb = (int32_t)(a.K / 32);
    p.zb = (p.nb + 1) / 2;
    p.zero = 0;
    p.a_bf16 = a.a_bf16;
    p.out_bf16 = a.out_bf16;
    p.eo_pairs = plan.b_layout == MNB_LAYOUT_EVEN_ODD;
    p.waves_hi = mfma4_waves_hi(a.K, plan);
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)plan.workgroups),
                                   dim3((unsigned)plan.threads_per_wg), args, mfma4_dynamic_lds(plan),
                                   static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
    return (int)e;
}

int mfma4_workgroups_per_cu(int64_t m, int64_t K, const mnb_plan& plan)
{
    Mfma4Fn fn = lookup_mfma4(m, K, plan);
    if (!fn) return 0;
    return occupancy(reinterpret_cast<const void*>(fn), plan.threads_per_wg, mfma4_dynamic_lds(plan));
}

int mfma4_kernel_info(int64_t m, int64_t K, const mnb_plan& plan, mnb_kernel_info* info)
{
    Mfma4Fn fn = lookup_mfma4(m, K, plan);
    if (!fn) return -1;
    hipFuncAttributes attr;
    hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(fn));
    if (e != hipSuccess) return (int)e;
    info->vgprs = attr.numRegs;
    info->sgprs = 0;
    info->lds_bytes = (int32_t)(attr.sharedSizeBytes + mfma4_dynamic_lds(plan));
    info->max_threads = attr.maxThreadsPerBlock;
    info->wgs_per_cu = mfma4_workgroups_per_cu(m, K, plan);
    return 0;
}

}  // namespace mnb
