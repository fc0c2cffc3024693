// Block-wise INT4 MatMulNBits decode GEMV, hand-written for gfx950 (CDNA4).
//
//   y[r][n] = sum_k a[r][k] * (q[n][k] - z[n][k/32]) * s[n][k/32]
//
// (onnx-genai pull request "perf(cuda): let the split-K decode GEMV store
// bf16 directly", opening paragraphs: block-32 INT4 weights, split-K GEMV,
// fp32 accumulator rounded to fp16 in the epilogue, bf16 narrowed from that
// fp16; pull request "PORT-1 (offline bias+interleave)", "Why the premise
// fails here", item 1: asymmetric per-block zero points, +8 when symmetric.)
//
// Work decomposition.  The K range of a column is cut into 32-weight blocks.
// A "lane group" of lanes_per_col lanes shares one column at a time; lane l
// of the group owns blocks l, l + lpc, l + 2*lpc, ... (blocks_per_lane of
// them per K chunk).  Because that set is fixed for the life of the wave,
// the lane's activations are loaded once, converted to fp16, permuted into
// the pair order of the nibble unpack below and kept in VGPRs while the group
// walks its contiguous range of columns, cols_per_tile at a time.  A group is
// 16, 32 or 64 lanes of one wave (no barriers), or 2..8 whole waves that
// combine their partial sums through LDS.
//
// Per 16-byte weight load (one block of one column) a lane does, for each of
// its 4 dwords x (8 nibbles, k = 8d .. 8d+7), with one v_and_or_b32 each:
//   (x & 0x000F000F)        | 0x64006400 -> fp16 pair (1024+q0, 1024+q4)
//   (x & 0x00F000F0)        | 0x64006400 -> (1024+16q1, 1024+16q5)
//   ((x >> 8) & 0x000F000F) | 0x64006400 -> (1024+q2, 1024+q6)
//   ((x >> 8) & 0x00F000F0) | 0x64006400 -> (1024+16q3, 1024+16q7)
// then per pair one packed fp16 operation that leaves the exact integers
// q - z: an add of -(1024+z) for the (1024+q) pairs, and an fma by 1/16
// with the addend -(64+z) for the (1024+16q) pairs ((1024+16q)/16 = 64+q is
// exact).  One v_dot2_f32_f16 per pair against the matching activation pair
// then adds into the block's single fp32 chain.  Every product a*(q-z) is
// exact in fp32, so the rounding error of the sum is relative to
// sum |a*(q-z)|.  The block's fp16 scale is applied by one fp32 FMA:
//   acc = fma(block_sum, s, acc).
//
// Reduction: a fixed DPP tree across the group's lanes inside a wave, then
// (multi-wave groups) a fixed-order sum over waves through LDS.  No atomics:
// equal inputs give equal bits.
//
// Epilogue (first page, paragraph on matmul_nbits_store_narrowed): one lane
// per (row, column) rounds fp32 -> fp16 (RNE); when the launch-uniform
// out_bf16 flag is set it narrows that fp16 to bf16 (RNE) and stores bf16
// directly.  Each launch writes all m*N outputs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <thread>
#include <type_traits>

#include "mnb.h"
#include "mnb_device.h"
#include "mnb_internal.h"

namespace mnb {
namespace {

struct Params {
    const uint16_t* A;       // [m][K]
    const uint8_t* B;        // [N][K/2]
    const uint16_t* scales;  // [N][nb]
    const uint8_t* zp;       // [N][zb] or null
    uint16_t* out;           // [m][N]
    int64_t N;
    int32_t K, nb, zb;
    int32_t lpc;             // lanes per column group
    int32_t chunks;          // K chunks of lpc*BPL blocks
    int32_t a_bf16, out_bf16;
    int32_t interleave;      // tiles dealt round-robin to groups (else ranges)
    uint32_t zero;           // always 0 (see vgpr_constant)
    int32_t tcap;            // multi-wave groups: LDS slots for deferred sums
                             // (0: reduce across waves after every tile)
    int32_t eo_pairs;        // weights in the even/odd nibble layout: the
                             // unpack yields (k, k+1) pairs, no reorder
};

// v + (v of another lane) through a DPP lane permutation; lanes outside
// ROW_MASK add 0 (they keep `old`).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_add(float v)
{
    const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
    return v + __int_as_float(t);
}

// Fixed-order sum over groups of SPAN (16, 32, 64) lanes.  Inside a 16-lane
// row: swap pairs, swap pairs of pairs, half-row mirror, row mirror -- every
// lane of the row then holds the (bitwise identical) row sum.  Rows are then
// combined with row broadcasts; the group total ends up in every lane of the
// group's last row (lanes SPAN-16 .. SPAN-1 of the group).
template <int SPAN>
__device__ __forceinline__ float group_sum(float v)
{
    v = dpp_add<0xB1>(v);    // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);    // quad_perm [2,3,0,1]
    v = dpp_add<0x141>(v);   // row_half_mirror
    v = dpp_add<0x140>(v);   // row_mirror
    if constexpr (SPAN >= 32) v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
    if constexpr (SPAN >= 64) v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
    return v;
}

// Totals over all 64 lanes of two values in one register: v_permlane32_swap
// plus one add sums each value over the two 32-lane halves (a into lanes
// 0-31, b into 32-63), the row-local DPP steps of group_sum sum each 16-lane
// row, and v_permlane16_swap plus one add joins rows 0 and 1 (a) and rows 2
// and 3 (b).  Eight VALU operations for two values (group_sum<64> takes six
// per value); both values get the same association whatever the other one
// holds.
__device__ __forceinline__ float pair_total64(float a, float b)
{
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    float x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    x = dpp_add<0xB1>(x);    // quad_perm [1,0,3,2]
    x = dpp_add<0x4E>(x);    // quad_perm [2,3,0,1]
    x = dpp_add<0x141>(x);   // row_half_mirror
    x = dpp_add<0x140>(x);   // row_mirror
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ __forceinline__ int64_t uniform64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Kernel modes.  LANES: groups of 16 or 32 lanes inside a wave.  WAVES:
// one whole wave per group, so a group's column range is wave-uniform and
// tile addresses live in SGPRs.  EXACT: WAVES with the K range covered
// exactly once by lanes_per_col * BPL blocks (no ragged blocks, no K
// chunks), which drops every per-lane bounds test.  WAVES_X, EXACT_X: the
// same with a group of 2..8 waves (one workgroup) per column tile, whose
// partial sums meet in LDS.
enum Mode { LANES = 0, WAVES = 1, EXACT = 2, WAVES_X = 3, EXACT_X = 4 };

constexpr bool uniform_mode(int mode) { return mode != LANES; }
constexpr bool multiwave_mode(int mode) { return mode == WAVES_X || mode == EXACT_X; }

// Next-tile prefetch (two register buffers) pays where a tile is small;
// larger tiles already keep enough bytes in flight per wave.  Only for
// wave-uniform column ranges (scalar addressing keeps the second buffer
// cheap).  Multi-wave groups (few waves per CU, long K) prefetch whenever
// the second buffer fits a moderate register budget.
#ifndef MNB_PREFETCH_TILE
#define MNB_PREFETCH_TILE 2   // largest NC*BPL of a one-wave group with two tile buffers
#endif
#ifndef MNB_PREFETCH_X_VGPRS
#define MNB_PREFETCH_X_VGPRS 160
#endif
template <int M, int BPL, int NC, int MODE>
constexpr bool kPrefetch =
    uniform_mode(MODE) &&
    (multiwave_mode(MODE) ? 16 * M * BPL + 2 * 6 * NC * BPL <= MNB_PREFETCH_X_VGPRS
                          : NC * BPL <= MNB_PREFETCH_TILE && M <= 2);

// Rough VGPR need of a variant, to ask the compiler for an occupancy it can
// meet without spilling: activations 16*M*BPL, weights/scales/zero points
// 6*NC*BPL per tile buffer, sums NC*M (counted thrice: live through
// reduction and selection), block temporaries 2*M, 64-bit per-lane
// addresses when the column range is not wave-uniform, constants.
template <int M, int BPL, int NC, int MODE>
constexpr int kWavesPerEu()
{
    constexpr bool uni = uniform_mode(MODE);
    constexpr int bufs = kPrefetch<M, BPL, NC, MODE> ? 2 : 1;
    constexpr int est = 16 * M * BPL + bufs * (8 + (uni ? 0 : 2)) * NC * BPL +
                        3 * NC * M + 2 * M + 28 + 16;
    constexpr int w = 512 / ((est + 7) / 8 * 8);
#ifdef MNB_WPE_M1
    if constexpr (M == 1 && uni) return MNB_WPE_M1;
#endif
    return w > 8 ? 8 : (w < 1 ? 1 : w);
}

template <int M, int BPL, int NC, int MODE>
__global__ __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(kWavesPerEu<M, BPL, NC, MODE>())))
void mnb_gemv_kernel(Params p)
{
    constexpr bool UNI = uniform_mode(MODE);
    constexpr bool xwave = multiwave_mode(MODE);
    constexpr bool EXACT_K = MODE == EXACT || MODE == EXACT_X;
    constexpr int NV = NC * M;                  // partial sums per lane
    // Multi-wave groups: per-wave partial sums, [tile][wave][NV] when
    // deferred to the end of the kernel (tcap slots), else [2][wave][NV].
    extern __shared__ float part[];

    const int tid = threadIdx.x;
    const int lpc = p.lpc;
    const int lane = xwave ? tid : (tid & (lpc - 1));
    const int grp = xwave ? 0 : (tid / lpc);
    const int gpw = xwave ? 1 : (int)(blockDim.x / lpc);
    const int64_t gg = (int64_t)blockIdx.x * gpw + grp;
    const int64_t TG = (int64_t)gridDim.x * gpw;
    // Column tiles of this group: a contiguous range of columns, or every
    // TG-th tile (all groups then sweep the weights as one moving front).
    int64_t c_first, c_step, c_stop;
    if (p.interleave) {
        c_first = gg * NC;
        c_step = TG * NC;
        c_stop = p.N;
    } else {
        c_first = p.N * gg / TG;
        c_step = NC;
        c_stop = p.N * (gg + 1) / TG;
    }
    if constexpr (UNI) {
        c_first = uniform64(c_first);
        c_step = uniform64(c_step);
        c_stop = uniform64(c_stop);
    }
    const uint32_t row_bytes = (uint32_t)p.K / 2;
    const uint32_t nb = (uint32_t)p.nb, zb = (uint32_t)p.zb;
    const int zshift = (lane & 1) * 4;          // block parity == lane parity (lpc even)
    const uint32_t zdef = p.zp ? 0u : 8u;       // zero point 8 when none are given
    const ZeroPoint zbase = zero_point_pairs(zdef);
    const uint32_t magic = vgpr_constant(0x64006400u, p.zero);   // fp16 pair (1024, 1024)

    uint32_t act[M][BPL][16];                   // permuted fp16 pairs
    typedef uint4 RawActs[M][BPL][4];           // activations as loaded

    // This lane's activation blocks of K chunk ch (zeros past K).
    auto fetch_acts = [&](int ch, RawActs& raw) {
#pragma unroll
        for (int j = 0; j < BPL; ++j) {
            const uint32_t b = (uint32_t)((ch * BPL + j) * lpc + lane);
            const bool ok = EXACT_K || b < nb;
#pragma unroll
            for (int r = 0; r < M; ++r) {
                if (ok) {
                    const uint4* src = reinterpret_cast<const uint4*>(
                        p.A + (int64_t)r * p.K + 32 * (int64_t)b);
#pragma unroll
                    for (int i = 0; i < 4; ++i) raw[r][j][i] = src[i];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) raw[r][j][i] = make_uint4(0, 0, 0, 0);
                }
            }
        }
    };

    // Eight activations (one uint4) to fp16 (bf16 rounded to nearest even),
    // permuted into the unpack's pair order.
    auto to_pairs = [&](uint4 v) {
        const u32x4 o = f16_pairs(u32x4{v.x, v.y, v.z, v.w}, p.a_bf16, p.eo_pairs);
        return make_uint4(o[0], o[1], o[2], o[3]);
    };

    auto place_acts = [&](const RawActs& raw) {
#pragma unroll
        for (int j = 0; j < BPL; ++j)
#pragma unroll
            for (int r = 0; r < M; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 o = to_pairs(raw[r][j][i]);
                    act[r][j][4 * i + 0] = o.x;
                    act[r][j][4 * i + 1] = o.y;
                    act[r][j][4 * i + 2] = o.z;
                    act[r][j][4 * i + 3] = o.w;
                }
    };

    // One-wave groups: the four waves of a workgroup own the same blocks of
    // K lane by lane, so the workgroup fetches and converts the activations
    // once and each wave copies its lanes' share out of LDS (a quarter of
    // the L2 reads and conversions of per-wave fetching).  Thread t fetches
    // 16-byte piece i = t / 64 of lane t % 64's blocks, for every row and
    // block of the lane; LDS holds [row][block][piece][lane].
    constexpr bool kShareActs = UNI && !xwave;
    constexpr int kShare = kShareActs ? M * BPL : 1;
    uint4* const act_lds = reinterpret_cast<uint4*>(part);
    auto fetch_shared = [&](uint4 (&sv)[kShare]) {
        const int piece = tid >> 6, ln = tid & 63;
#pragma unroll
        for (int s = 0; s < kShare; ++s) {
            const int r = s / BPL, j = s - r * BPL;
            const uint32_t b = (uint32_t)(j * 64 + ln);
            sv[s] = make_uint4(0, 0, 0, 0);
            if (EXACT_K || b < nb)
                sv[s] = *reinterpret_cast<const uint4*>(p.A + (int64_t)r * p.K + 32 * (int64_t)b + 8 * piece);
        }
    };
    auto place_shared = [&](const uint4 (&sv)[kShare]) {
#pragma unroll
        for (int s = 0; s < kShare; ++s) act_lds[s * 256 + tid] = to_pairs(sv[s]);
        __syncthreads();
        const int ln = tid & 63;
#pragma unroll
        for (int r = 0; r < M; ++r)
#pragma unroll
            for (int j = 0; j < BPL; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 o = act_lds[((r * BPL + j) * 4 + i) * 64 + ln];
                    act[r][j][4 * i + 0] = o.x;
                    act[r][j][4 * i + 1] = o.y;
                    act[r][j][4 * i + 2] = o.z;
                    act[r][j][4 * i + 3] = o.w;
                }
    };

    auto load_acts = [&](int ch) {
        RawActs raw;
        fetch_acts(ch, raw);
        place_acts(raw);
    };

    // Registers of one tile: NC columns x BPL blocks of this lane.
    // Scales stay 16-bit: the fp16 -> fp32 conversion reads the low half,
    // so no zero extension (and no wait on the load) is needed at issue.
    struct Tile {
        u32x4 w[NC][BPL];
        uint16_t sc[NC][BPL];
        uint32_t zq[NC][BPL];
    };

    // Queue the loads of columns c0 .. c0+NC-1, K chunk ch.  Tile bases are
    // scalar when the column range is wave-uniform; per-lane offsets are 32-bit.
    auto issue = [&](Tile& t, int64_t c0, int ch) {
        if constexpr (UNI) {
            // One buffer resource per column and array (scalar), covering
            // exactly that column's row, so the per-lane offsets are the same
            // for every column and every tile (BPL registers per array).
            // Offsets past a resource's end (ragged blocks, columns past N,
            // absent zero points) load zeros without touching memory, so
            // every load is issued unconditionally and the compiler's wait
            // counts stay exact across the prefetch loop.
            uint32_t ow[BPL], os[BPL], oz[BPL];
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                const uint32_t b = (uint32_t)((ch * BPL + j) * lpc + lane);
                const bool ok = EXACT_K || b < nb;
                ow[j] = ok ? 16 * b : kOutOfRange;
                os[j] = ok ? 2 * b : kOutOfRange;
                oz[j] = ok ? (b >> 1) : kOutOfRange;
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int64_t col = c0 + c;
                const bool in = col < p.N;
                const int64_t cc = in ? col : 0;
                // K <= MNB_MAX_K keeps every size far below kOutOfRange.
                const __amdgpu_buffer_rsrc_t rB = make_rsrc_small(p.B + cc * row_bytes, in ? row_bytes : 0);
                const __amdgpu_buffer_rsrc_t rS = make_rsrc_small(p.scales + cc * nb, in ? 2 * nb : 0);
                const __amdgpu_buffer_rsrc_t rZ =
                    make_rsrc_small(p.zp ? p.zp + cc * zb : p.B, in && p.zp ? zb : 0);
#pragma unroll
                for (int j = 0; j < BPL; ++j) {
                    t.w[c][j] = __builtin_amdgcn_raw_buffer_load_b128(rB, ow[j], 0, kNontemporal);
                    t.sc[c][j] = __builtin_amdgcn_raw_buffer_load_b16(rS, os[j], 0, kNontemporal);
                    t.zq[c][j] = __builtin_amdgcn_raw_buffer_load_b8(rZ, oz[j], 0, kNontemporal);
                }
            }
        } else {
            const uint8_t* Bt = p.B + c0 * row_bytes;
            const uint16_t* St = p.scales + c0 * nb;
            const uint8_t* Zt = p.zp ? p.zp + c0 * zb : nullptr;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bool col_ok = c0 + c < c_stop;
#pragma unroll
                for (int j = 0; j < BPL; ++j) {
                    const uint32_t b = (uint32_t)((ch * BPL + j) * lpc + lane);
                    t.w[c][j] = u32x4{0, 0, 0, 0};
                    t.sc[c][j] = 0;
                    t.zq[c][j] = 0;
                    if (col_ok && b < nb) {
                        t.w[c][j] = stream_load(reinterpret_cast<const u32x4*>(Bt + (c * row_bytes + 16 * b)));
                        t.sc[c][j] = stream_load(St + (c * nb + b));
                        if (Zt) t.zq[c][j] = stream_load(Zt + (c * zb + (b >> 1)));
                    }
                }
            }
        }
    };

    // Unpack, subtract zero points, dot with the resident activations, scale.
    // Every pair is an exact q - z, so one fp32 chain per block and row.
    auto compute = [&](const Tile& t, float (&acc)[NC][M]) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                // With no zero points the loads return 0 and zdef = 8 is the
                // zero point; otherwise zdef = 0.
                const ZeroPoint zp = zero_point_pairs(__builtin_amdgcn_ubfe(t.zq[c][j], zshift, 4), zbase);
                float s[M];
#pragma unroll
                for (int r = 0; r < M; ++r) s[r] = 0.f;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint32_t pr[4];
                    unpack_dword(t.w[c][j][d], zp, magic, pr);
#pragma unroll
                    for (int r = 0; r < M; ++r) {
                        s[r] = dot2(act[r][j][4 * d + 0], pr[0], s[r]);
                        s[r] = dot2(act[r][j][4 * d + 1], pr[1], s[r]);
                        s[r] = dot2(act[r][j][4 * d + 2], pr[2], s[r]);
                        s[r] = dot2(act[r][j][4 * d + 3], pr[3], s[r]);
                    }
                }
                const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)t.sc[c][j]);
#pragma unroll
                for (int r = 0; r < M; ++r) acc[c][r] = fmaf(s[r], sf, acc[c][r]);
            }
        }
    };

    // fp32 -> fp16 (RNE), optionally -> bf16 (RNE), store value idx (row
    // idx / NC, column idx % NC) of the tile at c0.
    auto store = [&](int64_t c0, int idx, float v) {
        const int c = idx % NC, r = idx / NC;
        const int64_t col = c0 + c;
        if (col < c_stop) {
            const _Float16 h = (_Float16)v;               // fp32 -> fp16, RNE
            uint16_t bits = __builtin_bit_cast(uint16_t, h);
            if (p.out_bf16) bits = f16_to_bf16(bits);     // fp16 -> bf16, RNE
            p.out[(int64_t)r * p.N + col] = bits;
        }
    };

    const int nw = (int)(blockDim.x >> 6);      // waves of a multi-wave group
    const int wv = tid >> 6;
    int buf = 0;
    // Split-K reduction of tile k (at c0).  One-wave and in-wave groups: DPP
    // tree, then store.  Multi-wave groups: each wave's DPP total goes to its
    // LDS slot; with tcap > 0 the sums over waves wait for the end of the
    // kernel (no barrier per tile), else they happen after every tile.
    auto finish = [&](int k, int64_t c0, float (&acc)[NC][M]) {
        const int span = xwave ? 64 : lpc;
        // Value `idx` (row idx / NC, column idx % NC) out of the registers.
        auto pick = [&](int idx) {
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (idx == i) v = acc[i % NC][i / NC];
            return v;
        };
        const int wl = xwave ? (tid & 63) : lane;
        // emit(idx, v) for the values whose total this lane holds.
        auto totals = [&](auto emit) {
            if constexpr (NC % 2 == 0) {
                if (UNI || span == 64) {
                    // Columns 2i and 2i + 1 of a row share one register
                    // (value 2i in lanes 0-31, 2i + 1 in lanes 32-63), so a
                    // row pairs the same values whatever the launch's rows;
                    // lane j and lane 32 + j emit the pairs j, j + 16, ...
                    constexpr int NP = NV / 2;
                    float t[NP];
#pragma unroll
                    for (int i = 0; i < NP; ++i)
                        t[i] = pair_total64(acc[(2 * i) % NC][(2 * i) / NC], acc[(2 * i + 1) % NC][(2 * i + 1) / NC]);
                    if ((wl & 31) < 16) {
                        const int half = wl >> 5;
#pragma unroll
                        for (int i = 0; i < NP; ++i)
                            if (i % 16 == (wl & 15)) emit(2 * i + half, t[i]);
                    }
                    return;
                }
            }
            // One value at a time: the totals sit in the last 16-lane row of
            // each group.
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int r = 0; r < M; ++r) {
                    if (UNI || span == 64) acc[c][r] = group_sum<64>(acc[c][r]);
                    else if (span == 32) acc[c][r] = group_sum<32>(acc[c][r]);
                    else acc[c][r] = group_sum<16>(acc[c][r]);
                }
            const int first = span - 16;
            if (wl >= first)
                for (int idx = wl - first; idx < NV; idx += 16) emit(idx, pick(idx));
        };

        if constexpr (!xwave) {
            totals([&](int idx, float v) { store(c0, idx, v); });
        } else if (p.tcap > 0) {
            if (k < p.tcap) totals([&](int idx, float v) { part[(k * nw + wv) * NV + idx] = v; });
        } else {
            totals([&](int idx, float v) { part[(buf * nw + wv) * NV + idx] = v; });
            __syncthreads();
            if (tid < NV) {
                float v = part[(buf * nw) * NV + tid];
                for (int i = 1; i < nw; ++i) v += part[(buf * nw + i) * NV + tid];
                store(c0, tid, v);
            }
            buf ^= 1;
        }
    };

    if (EXACT_K || (UNI && p.chunks == 1)) {
        // Activations stay resident.  The first tiles' weight loads go out
        // right behind the activation loads, before the activations are
        // converted, so the conversion and the activations' own latency
        // overlap the weights' HBM latency.  With kPrefetch the next tile's
        // loads are in flight while the current tile is computed (two
        // register buffers).
        Tile ta, tb;
        int64_t c0 = c_first;
        int k = 0;
        RawActs raw;
        uint4 sv[kShare];
        if constexpr (kShareActs) fetch_shared(sv);
        else fetch_acts(0, raw);
        issue(ta, c0, 0);
        auto place = [&]() {
            if constexpr (kShareActs) place_shared(sv);
            else place_acts(raw);
        };
        if constexpr (!kPrefetch<M, BPL, NC, MODE>) {
            place();
            while (c0 < c_stop) {
                float acc[NC][M] = {};
                compute(ta, acc);
                finish(k++, c0, acc);
                c0 += c_step;
                issue(ta, c0, 0);
            }
        } else {
            issue(tb, c0 + c_step, 0);
            place();
            while (c0 < c_stop) {
                float acc[NC][M] = {};
                compute(ta, acc);
                finish(k++, c0, acc);
                c0 += c_step;
                if (c0 >= c_stop) break;
                issue(ta, c0 + c_step, 0);
                float acc2[NC][M] = {};
                compute(tb, acc2);
                finish(k++, c0, acc2);
                c0 += c_step;
                issue(tb, c0 + c_step, 0);
            }
        }
    } else if constexpr (!EXACT_K) {
        // Lane groups inside a wave, or K longer than one pass of the group
        // (activations then reloaded per chunk): one tile at a time.
        if (p.chunks == 1) load_acts(0);
        int k = 0;
        for (int64_t c0 = c_first; c0 < c_stop; c0 += c_step) {
            float acc[NC][M] = {};
            for (int ch = 0; ch < p.chunks; ++ch) {
                if (p.chunks > 1) load_acts(ch);
                Tile t;
                issue(t, c0, ch);
                compute(t, acc);
            }
            finish(k++, c0, acc);
        }
    }

    if constexpr (xwave) {
        // Deferred sums over the waves of the group, in wave order, for
        // every tile of the group.
        if (p.tcap > 0) {
            __syncthreads();
            const int64_t tiles = c_first < c_stop ? (c_stop - c_first + c_step - 1) / c_step : 0;
            const int n = (int)(tiles < p.tcap ? tiles : p.tcap) * NV;
            for (int e = tid; e < n; e += (int)blockDim.x) {
                const int k = e / NV, idx = e - k * NV;
                float v = part[(k * nw) * NV + idx];
                for (int i = 1; i < nw; ++i) v += part[(k * nw + i) * NV + idx];
                store(c_first + k * c_step, idx, v);
            }
        }
    }
}

typedef void (*KernelFn)(Params);

template <int M, int BPL, int NC>
constexpr bool kValid = (M * BPL <= 8) && (NC * BPL <= 8) && (NC * M <= 32);

template <int M, int BPL, int NC>
KernelFn variant_if_valid(int mode)
{
    if constexpr (kValid<M, BPL, NC>) {
        switch (mode) {
        case LANES: return mnb_gemv_kernel<M, BPL, NC, LANES>;
        case WAVES: return mnb_gemv_kernel<M, BPL, NC, WAVES>;
        case EXACT: return mnb_gemv_kernel<M, BPL, NC, EXACT>;
        case WAVES_X: return mnb_gemv_kernel<M, BPL, NC, WAVES_X>;
        case EXACT_X: return mnb_gemv_kernel<M, BPL, NC, EXACT_X>;
        }
    }
    return nullptr;
}

template <int M, int BPL>
KernelFn by_nc(int nc, int mode)
{
    switch (nc) {
    case 1: return variant_if_valid<M, BPL, 1>(mode);
    case 2: return variant_if_valid<M, BPL, 2>(mode);
    case 4: return variant_if_valid<M, BPL, 4>(mode);
    case 8: return variant_if_valid<M, BPL, 8>(mode);
    }
    return nullptr;
}

template <int M>
KernelFn by_bpl(int bpl, int nc, int mode)
{
    switch (bpl) {
    case 1: return by_nc<M, 1>(nc, mode);
    case 2: return by_nc<M, 2>(nc, mode);
    case 4: return by_nc<M, 4>(nc, mode);
    case 8: return by_nc<M, 8>(nc, mode);
    }
    return nullptr;
}

// Mode for a plan: EXACT when lanes_per_col * blocks_per_lane == K/32,
// multi-wave when a group spans more than one wave.
int mode_of(int64_t K, const mnb_plan& plan)
{
    if (plan.lanes_per_col < 64) return LANES;
    const bool exact = (int64_t)plan.lanes_per_col * plan.blocks_per_lane == K / 32;
    if (plan.lanes_per_col > 64) return exact ? EXACT_X : WAVES_X;
    return exact ? EXACT : WAVES;
}

KernelFn lookup(int64_t m, int64_t K, const mnb_plan& plan)
{
    const int bpl = plan.blocks_per_lane, nc = plan.cols_per_tile;
    const int mode = mode_of(K, plan);
    switch (m) {
    case 1: return by_bpl<1>(bpl, nc, mode);
    case 2: return by_bpl<2>(bpl, nc, mode);
    case 3: return by_bpl<3>(bpl, nc, mode);
    case 4: return by_bpl<4>(bpl, nc, mode);
    case 5: return by_bpl<5>(bpl, nc, mode);
    case 6: return by_bpl<6>(bpl, nc, mode);
    case 7: return by_bpl<7>(bpl, nc, mode);
    case 8: return by_bpl<8>(bpl, nc, mode);
    }
    return nullptr;
}

}  // namespace

int launch_gemv(const GemvArgs& a, const mnb_plan& plan, void* stream)
{
    if (plan.engine == 2) return launch_gemm(a, plan, stream);
    if (plan.engine == 3) return launch_mfma4(a, plan, stream);
    KernelFn fn = lookup(a.m, a.K, plan);
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    Params p;
    p.A = static_cast<const uint16_t*>(a.A);
    p.B = a.B;
    p.scales = a.scales;
    p.zp = a.zp;
    p.out = static_cast<uint16_t*>(a.out);
    p.N = a.N;
    p.K = (int32_t)a.K;
    p.nb = (int32_t)(a.K / 32);
    p.zb = (p.nb + 1) / 2;
    p.lpc = plan.lanes_per_col;
    p.chunks = plan.k_chunks;
    p.a_bf16 = a.a_bf16;
    p.out_bf16 = a.out_bf16;
    p.interleave = plan.interleave;
    p.zero = 0;
    p.eo_pairs = plan.b_layout == MNB_LAYOUT_EVEN_ODD;
    const int64_t lds = gemv_lds_bytes(a.m, a.N, plan, &p.tcap);
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn),
                                   dim3((unsigned)plan.workgroups),
                                   dim3((unsigned)plan.threads_per_wg), args, (size_t)lds,
                                   static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
    return (int)e;
}

int current_device_cus(int* num_cus)
{
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    std::lock_guard<std::mutex> g(mu);
    if (dev >= 0 && dev < 64 && cache[dev] > 0) {
        *num_cus = cache[dev];
        return 0;
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    if (dev >= 0 && dev < 64) cache[dev] = n;
    *num_cus = n;
    return 0;
}

namespace {

// Workspace buffers, one per (device, stream) and, for the per-thread
// default stream, per host thread: work on one stream runs in order, so a
// stream's buffer is free again for the stream's next call.  A buffer grows
// (after its stream has drained) when a call needs more; the oldest entry
// is given up (after the device has drained) when the table is full.  One
// mutex, held from acquire to release, keeps two host threads from
// interleaving their launches on the same buffer.
struct WsEntry {
    int dev;
    hipStream_t stream;
    std::thread::id thread;
    void* ptr;
    size_t bytes;
    uint64_t last_use;
};
constexpr int kWsEntries = 32;
std::mutex g_ws_mu;
WsEntry g_ws[kWsEntries];
int g_ws_used = 0;
uint64_t g_ws_clock = 0;

int acquire_locked(size_t bytes, hipStream_t stream, void** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    const std::thread::id tid = stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id();
    WsEntry* hit = nullptr;
    for (int i = 0; i < g_ws_used; ++i)
        if (g_ws[i].dev == dev && g_ws[i].stream == stream && g_ws[i].thread == tid) hit = &g_ws[i];
    if (!hit) {
        if (g_ws_used < kWsEntries) {
            hit = &g_ws[g_ws_used++];
        } else {
            hit = &g_ws[0];
            for (int i = 1; i < kWsEntries; ++i)
                if (g_ws[i].last_use < hit->last_use) hit = &g_ws[i];
            // Its stream may be gone; drain its device before freeing.
            int cur = dev;
            if (hit->dev != cur) (void)hipSetDevice(hit->dev);
            e = hipDeviceSynchronize();
            if (e == hipSuccess) e = hipFree(hit->ptr);
            if (hit->dev != cur) (void)hipSetDevice(cur);
            if (e != hipSuccess) return (int)e;
        }
        *hit = WsEntry{dev, stream, tid, nullptr, 0, 0};
    }
    if (hit->bytes < bytes) {
        if (hit->ptr) {
            e = hipStreamSynchronize(stream);   // the stream's earlier calls may still read it
            if (e == hipSuccess) e = hipFree(hit->ptr);
            hit->ptr = nullptr;
            hit->bytes = 0;
            if (e != hipSuccess) return (int)e;
        }
        e = hipMalloc(&hit->ptr, bytes);
        if (e != hipSuccess) {
            hit->ptr = nullptr;
            return (int)e;
        }
        hit->bytes = bytes;
    }
    hit->last_use = ++g_ws_clock;
    *ptr = hit->ptr;
    return 0;
}

}  // namespace

int workspace_acquire(size_t bytes, void* stream, void** ptr)
{
    g_ws_mu.lock();
    const int e = acquire_locked(bytes, static_cast<hipStream_t>(stream), ptr);
    if (e != 0) g_ws_mu.unlock();
    return e;
}

void workspace_release() { g_ws_mu.unlock(); }

namespace {

// matmul_nbits_noalloc's workspace.  In host code `scratch` names a host-side
// stand-in, not device memory: kernels get the address hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

}  // namespace

int scratch_address(void** ptr)
{
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return 0;
}

namespace {

// Occupancy queries cost microseconds; they depend only on the device and the
// (kernel, block size, dynamic LDS) triple, so cache them.
struct OccKey {
    int dev;
    const void* fn;
    int threads;
    size_t lds;
};

int cached_occupancy(const void* fn, int threads, size_t lds)
{
    static std::mutex mu;
    static OccKey keys[256];
    static int vals[256];
    static int used = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < used; ++i)
        if (keys[i].dev == dev && keys[i].fn == fn && keys[i].threads == threads &&
            keys[i].lds == lds)
            return vals[i];
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, lds) != hipSuccess) return 0;
    if (used < 256) {
        keys[used] = OccKey{dev, fn, threads, lds};
        vals[used++] = n;
    }
    return n;
}

}  // namespace

int occupancy(const void* fn, int threads, size_t lds) { return cached_occupancy(fn, threads, lds); }

int workgroups_per_cu(int64_t m, int64_t K, int64_t N, const mnb_plan& plan)
{
    if (plan.engine == 2) return gemm_workgroups_per_cu(plan);
    if (plan.engine == 3) return mfma4_workgroups_per_cu(m, K, plan);
    KernelFn fn = lookup(m, K, plan);
    if (!fn) return 0;
    int32_t tcap = 0;
    const int64_t lds = gemv_lds_bytes(m, N, plan, &tcap);
    return cached_occupancy(reinterpret_cast<const void*>(fn), plan.threads_per_wg, (size_t)lds);
}

int kernel_info(int64_t m, int64_t K, const mnb_plan& plan, mnb_kernel_info* info)
{
    if (plan.engine == 2) return gemm_kernel_info(plan, info);
    if (plan.engine == 3) return mfma4_kernel_info(m, K, plan, info);
    KernelFn fn = lookup(m, K, plan);
    if (!fn) return -1;
    hipFuncAttributes attr;
    hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(fn));
    if (e != hipSuccess) return (int)e;
    info->vgprs = attr.numRegs;
    info->sgprs = 0;
    int32_t tcap = 0;
    info->lds_bytes = (int32_t)(attr.sharedSizeBytes + gemv_lds_bytes(m, 1, plan, &tcap));
    info->max_threads = attr.maxThreadsPerBlock;
    info->wgs_per_cu = workgroups_per_cu(m, K, 1, plan);
    return 0;
}

}  // namespace mnb
