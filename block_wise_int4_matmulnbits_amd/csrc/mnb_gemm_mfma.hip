// Prefill INT4 MatMulNBits (m > 8 rows) on the matrix cores of gfx950.
//
//   y[r][n] = sum_k a[r][k] * w[n][k],   w[n][k] = (q[n][k] - z[n][k/32]) * s[n][k/32]
//
// The operation and epilogue of the decode kernels (onnx-genai pull request
// "perf(cuda): let the split-K decode GEMV store bf16 directly", opening
// paragraphs and the paragraph on matmul_nbits_store_narrowed; pull request
// "PORT-1 (offline bias+interleave)", "Why the premise fails here", item 1):
// fp16 (or bf16 rounded to fp16) activations, fp32 accumulation, one fp16
// rounding of the sum and, for bf16 output, the narrowing to bf16 in the
// same kernel.  The first page names a row-batched path without the
// narrowing store as the next step; this is that path with the store.
//
// Weights.  Each weight is dequantized to fp16 the way the second page's
// GEMV holds it (a packed-half scale and zero-point subtrahend per block,
// "Why the premise fails here", item 3): the nibble becomes the exact fp16
// integer q - z, and one packed fp16 multiply by the block's scale rounds
// (q - z) * s to fp16 (RNE, gradual underflow).  The matrix core then
// multiplies exact fp16 products into fp32 accumulators that run over all of
// K, so there is no per-block fp32 result to scale.  Against the exact
// weights the rounding adds at most 2^-11 |a w| per product (normal fp16
// range), inside the decode path's tolerance.
//
// Work decomposition.  A workgroup of four waves owns an output tile of
// 32*RT rows by 128*CT columns; wave w owns columns 32*CT*w .. 32*CT*(w+1)-1
// of it and all RT row tiles, so each weight it unpacks feeds RT matrix
// products and each activation operand it reads from LDS feeds CT.  The
// products are v_mfma_f32_32x32x16_f16 (on gfx950 twice the rate of the
// 16x16x32 shape), two per 32-weight block.  K is walked one quad (4 blocks,
// 128 k) at a time:
//   - activations of the quad (32*RT rows x 128 k) are loaded by all 256
//     threads, converted to fp16 (bf16 rounded to nearest even) in the
//     unpack's pair order and written to one of two LDS buffers;
//   - for each of its CT column tiles, lane (j, h) loads blocks 4t+h and
//     4t+2+h of column j (16 bytes each) with the quad's 4 scales and zero
//     points; v_permlane32_swap leaves dwords 2h, 2h+1 of every block of the
//     quad in lane half h (the B operand layout: half h supplies k = 16h+8s
//     .. 16h+8s+7 to product s of the block);
//   - per block: unpack and scale the CT column tiles, then per row tile and
//     product one LDS read and CT MFMAs into the accumulators.
// Weight loads run four quads ahead of use (two for unaligned scale rows),
// activation loads one; the loop walks the quads in groups of that many,
// and the quads past K in the last group load zeros and add +0.  The
// summation order of an output depends only on K: equal inputs give equal
// bits for any M, N, tiling and grid.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb.h"
#include "mnb_device.h"
#include "mnb_internal.h"

namespace mnb {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cache policy of the weight, scale and zero-point loads: the default one.
// The tiles read each 128-byte line of a column over two or four K steps
// (64 or 32 bytes at a time), and a nontemporal hint sends the later parts
// back to HBM: with it the gate_up m = 16 launch fetched twice the weight
// bytes.  Default against nontemporal, us: gate_up m = 16 44.6 -> 33.2,
// m = 512 170.3 -> 143.9, m = 2048 718.9 -> 549.0; lm_head m = 32 227.7 ->
// 135.0; down m = 64 48.7 -> 38.7, m = 512 156.6 -> 106.5.
constexpr int kPrefillLoadPolicy = 0;

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
    int32_t splits;          // K slices over workgroups (1: none)
    float* ws;               // splits > 1: [splits][M][N] fp32 partial sums
};

// Weight quads in flight per column tile (the per-block loads of the
// unaligned variant take more registers).
template <bool VEC>
constexpr int kGemmRing = VEC ? 4 : 2;

struct WQuad {
    u32x4 w[2];       // load u: 16 bytes of block 4t+2u+h of this lane's column
    uint32_t s[4];    // fp16 scales of blocks 4t..4t+3 (VEC: two words)
    uint32_t z[2];    // zero-point bytes 2t, 2t+1 (VEC: one 16-bit word)
};

// Packed fp16 product (one rounding, RNE).
__device__ __forceinline__ uint32_t hmul2(uint32_t a, uint32_t b)
{
    const half2_t r = __builtin_bit_cast(half2_t, a) * __builtin_bit_cast(half2_t, b);
    return __builtin_bit_cast(uint32_t, r);
}

// Two fp16 halves (lo from x, lo or hi per `hi`, and likewise from y) into
// one dword: the pair (x_e, y_e) of the unpack's order.
__device__ __forceinline__ uint32_t pair16(uint32_t x, uint32_t y, bool hi)
{
    return __builtin_amdgcn_perm(y, x, hi ? 0x07060302u : 0x05040100u);
}

// Two bf16 (the low or high halves of x and y) -> fp16 pair, RNE.
__device__ __forceinline__ uint32_t pair_bf16(uint32_t x, uint32_t y, bool hi)
{
    const float2_t f = hi ? float2_t{__uint_as_float(x & 0xFFFF0000u), __uint_as_float(y & 0xFFFF0000u)}
                          : float2_t{__uint_as_float(x << 16), __uint_as_float(y << 16)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, half2_t));
}

// LDS slot of 16-byte piece d (k = 8d .. 8d+7) of row r (rows are 64
// bytes, four slots).  An MFMA operand read has lane (j, h) take piece 2h+v
// of row j; XOR-ing the slot with bits 2..3 of the row spreads those reads
// over all banks.  Measured with eight waves sharing a CU's LDS, cycles per
// 16-byte read per wave: 32.0 with this swizzle, the same as consecutive
// lanes reading consecutive 16 bytes; 56.1 with the XOR of bits 1..2 and
// 3..4 used before; 106.7 with none.
__device__ __forceinline__ int a_slot(int d, int r)
{
    return d ^ ((r >> 2) & 3);
}

// KS > 1 splits K over the waves: KS slices of W / KS waves, slice s
// walking quads s, s + KS, s + 2 KS, ... of the same columns; at the end the
// slices' accumulators meet in LDS and slice 0 adds them in slice order and
// stores.  More waves then walk a tile's K at once where the tiles are too
// few to fill the chip (the down projection's 4096 columns).  CW = 16 (with
// one 32-column MFMA tile per wave) gives a wave 16 real columns: lanes
// j >= 16 load zeros and store nothing, which doubles the tiles where the
// 32-column ones leave CUs idle.  SPLIT: K is also split over workgroups
// (p.splits slices of 128-wide steps), each tile's slice leaving its fp32
// sums in the workspace for mnb_split_reduce_kernel; a separate variant, so
// that the tiles without it keep their registers and code.
template <int RT, int CT, int W, bool VEC, bool ABF16, int KS, int CW = 32, bool SPLIT = false>
__global__ __launch_bounds__(64 * W) void mnb_gemm_mfma_kernel(GemmParams p)
{
    constexpr int THREADS = 64 * W;
    constexpr int WC = W / KS;               // waves per K slice
    static_assert(WC * KS == W, "whole slices");
    static_assert(CW == 32 || (CW == 16 && CT == 1), "16 columns: one MFMA tile per wave");
    constexpr int MT = 32 * RT;              // rows per workgroup tile
    constexpr int NT = CW * CT * WC;         // columns per workgroup tile
    constexpr int QAQ = 16 * MT;             // 16-byte pieces of activations per quad
    constexpr int QA = KS * QAQ;             // per step: one quad per slice
    constexpr int SPT = QA / THREADS;        // pieces per thread
    static_assert(KS == 1 || (KS - 1) * WC * RT * CT * 16 * 64 * 4 <= 2 * QA * 16,
                  "the partial sums fit the activation stages");
    static_assert(QA % THREADS == 0, "whole pieces per thread");
    constexpr int P = kGemmRing<VEC>;
    extern __shared__ uint4 a_lds[];         // [2][4 blocks][MT rows][4 slots]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int slice = wv / WC, wcol = wv - slice * WC;
    const int j = lane & 31, h = lane >> 5;
    const int nb = p.nb;
    const int nq = (nb + 3) / 4;
    const uint32_t row_bytes = (uint32_t)p.K / 2;
    const uint32_t zdef = p.zp ? 0u : 8u;    // zero point 8 when none are given
    const uint32_t magic = vgpr_constant(0x64006400u, p.zero);
    const int64_t tiles_m = (p.M + MT - 1) / MT;
    const int64_t tiles_n = (p.N + NT - 1) / NT;

    // Piece e0 = tid + THREADS * s of a step's activations: quad e0 / QAQ
    // of the step, and within it (e = e0 % QAQ) block e / (4 MT), row
    // (e / 4) % MT, piece e % 4; its LDS index, block and byte offset in the
    // row block are fixed per thread.
    int pc_blk[SPT], pc_lds[SPT];
    uint32_t pc_off[SPT];
#pragma unroll
    for (int s = 0; s < SPT; ++s) {
        const int e0 = tid + THREADS * s;
        const int qo = e0 / QAQ, e = e0 - qo * QAQ;
        const int br = e >> 2, d = e & 3;
        const int blk = br / MT, row = br - blk * MT;
        pc_blk[s] = 4 * qo + blk;
        pc_lds[s] = qo * QAQ + (blk * MT + row) * 4 + a_slot(d, row);
        pc_off[s] = (uint32_t)row * (uint32_t)p.K * 2 + 256 * qo + 64 * blk + 16 * d;
    }

    const int64_t tiles_mn = tiles_m * tiles_n;
    const int64_t tiles_all = SPLIT ? tiles_mn * p.splits : tiles_mn;
    for (int64_t tile = blockIdx.x; tile < tiles_all; tile += gridDim.x) {
        // Consecutive workgroups share a row block (its activations stay in
        // L2) and walk the column blocks; with K split over workgroups, K
        // slice ks of every tile comes after slice ks - 1 of all of them.
        // (With a split the host keeps tiles_mn * splits below 2^31 and the
        // slice arithmetic in 32 bits; nq * splits < 2^24.)
        uint32_t ks = 0;
        int64_t tmn = tile;
        int qa = 0, qb = nq;
        if constexpr (SPLIT) {
            ks = (uint32_t)tile / (uint32_t)tiles_mn;
            tmn = (int64_t)((uint32_t)tile - ks * (uint32_t)tiles_mn);
            qa = (int)((uint32_t)nq * ks / (uint32_t)p.splits);
            qb = (int)((uint32_t)nq * (ks + 1) / (uint32_t)p.splits);
        }
        const int64_t tm = tmn / tiles_n, tn = tmn - tm * tiles_n;
        const int64_t r0 = tm * MT;
        // Quads [qa, qb) of K: the workgroup's slice (all of K when
        // splits = 1); blocks from bend on load zeros.
        const uint32_t bend = SPLIT ? (uint32_t)(4 * qb < nb ? 4 * qb : nb) : (uint32_t)nb;
        const int nsteps = (qb - qa + KS - 1) / KS;   // steps of KS quads
        const int64_t col0 = tn * NT + CW * CT * wcol;   // this wave's CW*CT columns
        const int64_t left = p.N - col0;
        const uint32_t ncols = left <= 0 ? 0u : (uint32_t)(left < CW * CT ? left : CW * CT);
        const int64_t cb = left <= 0 ? 0 : col0;
        // Buffer resources over the wave's column rows and the tile's
        // activation rows; loads past their end (columns past N, rows past
        // M, blocks past K, absent zero points) return zeros without
        // touching memory.  The host keeps 32 * RT * K * 2 below 2^32.
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B + cb * row_bytes, (uint64_t)ncols * row_bytes);
        const __amdgpu_buffer_rsrc_t rS = make_rsrc(p.scales + cb * nb, (uint64_t)ncols * nb * 2);
        const __amdgpu_buffer_rsrc_t rZ =
            make_rsrc(p.zp ? p.zp + cb * p.zb : p.B, p.zp ? (uint64_t)ncols * p.zb : 0);
        const int64_t mrows = p.M - r0 < MT ? p.M - r0 : MT;
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + r0 * p.K, (uint64_t)mrows * (uint64_t)p.K * 2);

        // Column tile c of the wave: columns col0 + 32c + j; step t of
        // the slice is quad KS t + slice.
        auto issue = [&](WQuad (&qs)[CT], int t) {
            const uint32_t b = 4 * (uint32_t)(qa + KS * t + slice);
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                WQuad& q = qs[c];
                const uint32_t jc = (uint32_t)(32 * c + j);
                const uint32_t wbase = jc * row_bytes + 16 * (uint32_t)h;
                const uint32_t sbase = jc * (uint32_t)nb * 2;
                const uint32_t zbase = jc * (uint32_t)p.zb;
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    q.w[u] = __builtin_amdgcn_raw_buffer_load_b128(
                        rB, b + 2 * u + h < bend ? wbase + 16 * (b + 2 * u) : kOutOfRange, 0,
                        kPrefillLoadPolicy);
                if constexpr (VEC) {
                    const u32x2 sv = __builtin_amdgcn_raw_buffer_load_b64(
                        rS, b < bend ? sbase + 2 * b : kOutOfRange, 0, kPrefillLoadPolicy);
                    q.s[0] = sv[0];
                    q.s[1] = sv[1];
                    q.z[0] = __builtin_amdgcn_raw_buffer_load_b16(
                        rZ, b < bend ? zbase + b / 2 : kOutOfRange, 0, kPrefillLoadPolicy);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        q.s[i] = __builtin_amdgcn_raw_buffer_load_b16(
                            rS, b + i < bend ? sbase + 2 * (b + i) : kOutOfRange, 0, kPrefillLoadPolicy);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        q.z[i] = __builtin_amdgcn_raw_buffer_load_b8(
                            rZ, b + 2 * i < bend ? zbase + b / 2 + i : kOutOfRange, 0, kPrefillLoadPolicy);
                }
            }
        };

        // Activations of step t: quads qa + KS t .. qa + KS t + KS - 1
        // (zeros past M and past the slice).
        auto fetch_a = [&](uint4 (&v)[SPT], int t) {
            const uint32_t q0 = (uint32_t)(qa + KS * t);
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
                const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
                    rA, 4 * q0 + pc_blk[s] < bend ? pc_off[s] + 256 * q0 : kOutOfRange, 0, 0);
                v[s] = make_uint4(x[0], x[1], x[2], x[3]);
            }
        };
        // Eight activations to fp16 in the unpack's pair order
        // (a0,a4) (a1,a5) (a2,a6) (a3,a7), into LDS.
        auto store_a = [&](const uint4 (&v)[SPT], int buf) {
#pragma unroll
            for (int s = 0; s < SPT; ++s) {
                const uint4 x = v[s];
                uint4 o;
                if constexpr (ABF16) {
                    o.x = pair_bf16(x.x, x.z, false);
                    o.y = pair_bf16(x.x, x.z, true);
                    o.z = pair_bf16(x.y, x.w, false);
                    o.w = pair_bf16(x.y, x.w, true);
                } else {
                    o.x = pair16(x.x, x.z, false);
                    o.y = pair16(x.x, x.z, true);
                    o.z = pair16(x.y, x.w, false);
                    o.w = pair16(x.y, x.w, true);
                }
                a_lds[buf * QA + pc_lds[s]] = o;
            }
        };

        float16_t acc[RT][CT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[rt][c][q] = 0.f;

        // The A operands of block i: row tile rt, product v (k = 16h + 8v ..).
        auto read_a = [&](half8_t (&f)[RT][2], int buf, int i) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const int row = rt * 32 + j;
                    const uint4 av = a_lds[buf * QA + slice * QAQ + (i * MT + row) * 4 + a_slot(2 * h + v, row)];
                    f[rt][v] = __builtin_bit_cast(half8_t, u32x4{av.x, av.y, av.z, av.w});
                }
        };

        // Unpack and scale the quad's four blocks of every column tile; two
        // MFMAs per block, row tile and column tile.  The A operands of the
        // next block are read from LDS while the current block multiplies.
        auto compute = [&](const WQuad (&qs)[CT], int buf) {
            // blk[c][i][v]: dword 2h+v of block 4t+i of column tile c.
            uint32_t blk[CT][4][2];
            uint32_t zw[CT];
#pragma unroll
            for (int c = 0; c < CT; ++c) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    // Lane half h holds block 4t+2u+h; swap so that half h
                    // holds dwords 2h, 2h+1 of blocks 4t+2u and 4t+2u+1.
                    const auto s0 = __builtin_amdgcn_permlane32_swap(qs[c].w[u][0], qs[c].w[u][2], false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(qs[c].w[u][1], qs[c].w[u][3], false, false);
                    blk[c][2 * u][0] = s0[0];
                    blk[c][2 * u][1] = s1[0];
                    blk[c][2 * u + 1][0] = s0[1];
                    blk[c][2 * u + 1][1] = s1[1];
                }
                zw[c] = VEC ? qs[c].z[0] : ((qs[c].z[0] & 0xFFu) | ((qs[c].z[1] & 0xFFu) << 8));
            }
            auto unpack = [&](half8_t (&bv)[CT][2], int i) {
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    const ZeroPoint zp = zero_point_pairs(((zw[c] >> (4 * i)) & 0xFu) | zdef);
                    const uint32_t sw = VEC ? (i < 2 ? qs[c].s[0] : qs[c].s[1]) : qs[c].s[i];
                    const uint32_t s2 = __builtin_amdgcn_perm(sw, sw, (VEC && (i & 1)) ? 0x03020302u : 0x01000100u);
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        uint32_t bq[4];
                        unpack_dword(blk[c][i][v], zp, magic, bq);
                        const u32x4 wq = {hmul2(bq[0], s2), hmul2(bq[1], s2), hmul2(bq[2], s2), hmul2(bq[3], s2)};
                        bv[c][v] = __builtin_bit_cast(half8_t, wq);
                    }
                }
            };
            half8_t fa[2][RT][2];
            half8_t bv[2][CT][2];
            read_a(fa[0], buf, 0);
            unpack(bv[0], 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int cur = i & 1, nxt = cur ^ 1;
                if (i < 3) read_a(fa[nxt], buf, i + 1);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int v = 0; v < 2; ++v)
#pragma unroll
                        for (int c = 0; c < CT; ++c)
                            acc[rt][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[cur][rt][v], bv[cur][c][v],
                                                                                acc[rt][c], 0, 0, 0);
                if (i < 3) unpack(bv[nxt], i + 1);
            }
        };

        // The loop body has no branches: quads past K (those that round the
        // last group up to P, and the prefetches past the end) load zeros
        // and add +0.
        WQuad ring[P][CT];
#pragma unroll
        for (int s = 0; s < P; ++s) issue(ring[s], s);
        uint4 av[SPT];
        fetch_a(av, 0);
        __syncthreads();                  // the previous tile's readers are done
        store_a(av, 0);
        fetch_a(av, 1);
        for (int t0 = 0; t0 < nsteps; t0 += P) {
#pragma unroll
            for (int s = 0; s < P; ++s) {
                const int t = t0 + s;
                // Buffer t&1 is complete, and every wave is done with buffer
                // (t+1)&1 (it held quad t-1).  Quad t+1's activations go in
                // after quad t's products, so their loads (issued at the end
                // of the previous step) have a step of work to arrive in
                // (gate_up m = 64: 59.0 -> 52.2 us, down m = 512: 163.8 ->
                // 156.8).
                __syncthreads();
                compute(ring[s], t & 1);
                store_a(av, (t + 1) & 1);
                fetch_a(av, t + 2);
                issue(ring[s], t + P);
            }
        }

        if constexpr (KS > 1) {
            // Slices 1 .. KS-1 leave their sums in the (now idle) stages,
            // lane-contiguous; slice 0 adds them in slice order.
            float* const part = reinterpret_cast<float*>(a_lds);
            auto at = [&](int k, int rt, int c, int q) {
                return ((((k - 1) * WC + wcol) * RT + rt) * CT * 16 + c * 16 + q) * 64 + lane;
            };
            __syncthreads();              // every slice is done with the stages
            if (slice > 0) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int c = 0; c < CT; ++c)
#pragma unroll
                        for (int q = 0; q < 16; ++q) part[at(slice, rt, c, q)] = acc[rt][c][q];
            }
            __syncthreads();
            if (slice > 0) continue;      // wave-uniform; the next tile's barriers are the same
#pragma unroll
            for (int k = 1; k < KS; ++k)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int c = 0; c < CT; ++c)
#pragma unroll
                        for (int q = 0; q < 16; ++q) acc[rt][c][q] += part[at(k, rt, c, q)];
        }
        // Epilogue: fp32 -> fp16 (RNE), optionally -> bf16 (RNE), store; or,
        // with K split over workgroups, the fp32 sums of the slice into its
        // plane of the workspace.  Accumulator element q of lane (j, h) is
        // row (q%4) + 4h + 8(q/4), column j of its 32 x 32 tile.
        float* const plane = p.ws + (int64_t)ks * p.M * p.N;
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const int64_t col = col0 + 32 * c + j;
            if (j < CW && col < p.N) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int64_t row = r0 + rt * 32 + (q & 3) + 4 * h + 8 * (q >> 2);
                        if constexpr (SPLIT) {
                            if (row < p.M) plane[row * p.N + col] = acc[rt][c][q];
                        } else if (row < p.M) {
                            const _Float16 hv = (_Float16)acc[rt][c][q];
                            uint16_t bits = __builtin_bit_cast(uint16_t, hv);
                            if (p.out_bf16) bits = f16_to_bf16(bits);
                            p.out[row * p.N + col] = bits;
                        }
                    }
            }
        }
    }
}

// 256 x 256 tiles with the weights staged through LDS.  Eight waves in a
// 2 x 4 arrangement: wave (wr, wc) owns rows 128 wr .. 128 wr + 127 (four
// row tiles) and columns 64 wc .. 64 wc + 63 (two column tiles) of the
// workgroup tile, 128 accumulators per lane.  K is walked in stages of two
// blocks (64 k).  Per stage every thread converts 4 pieces of activations
// and dequantizes one 32-weight block of one column (thread t: column t/2,
// block t%2 of the stage) into LDS, both in the MFMA operand layout
// ([block][row or column][16-byte slot], XOR-swizzled), so each weight is
// unpacked once per workgroup and feeds 256 rows.  The arithmetic is that
// of the kernel above (fp16 weights (q - z) * s, fp32 accumulation over all
// of K in the matrix core, the same narrowing store).
constexpr int kLdsTileRows = 256, kLdsTileCols = 256, kLdsRing = 2;

template <bool ABF16>
__global__ __launch_bounds__(512) void mnb_gemm_lds_kernel(GemmParams p)
{
    constexpr int THREADS = 512;
    constexpr int RTW = 4, CTW = 2;          // row and column tiles per wave
    constexpr int MT = kLdsTileRows, NT = kLdsTileCols;
    constexpr int SB = 2;                    // blocks per stage
    constexpr int QA = MT * SB * 4;          // 16-byte pieces of activations per stage
    constexpr int QB = NT * SB * 4;          // 16-byte pieces of weights per stage
    constexpr int APT = QA / THREADS;        // pieces per thread
    constexpr int P = kLdsRing;              // weight stages in flight
    static_assert(QA % THREADS == 0 && QB == 4 * THREADS, "one block of one column per thread");
    extern __shared__ uint4 lds[];
    uint4* const a_lds = lds;                // [2][SB][MT][4]
    uint4* const b_lds = lds + 2 * QA;       // [2][SB][NT][4]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wv >> 2, wc = wv & 3;
    const int j = lane & 31, h = lane >> 5;
    const int nb = p.nb;
    const int ns = (nb + SB - 1) / SB;       // stages
    const uint32_t row_bytes = (uint32_t)p.K / 2;
    const uint32_t zdef = p.zp ? 0u : 8u;
    const uint32_t magic = vgpr_constant(0x64006400u, p.zero);
    const int64_t tiles_m = (p.M + MT - 1) / MT;
    const int64_t tiles_n = (p.N + NT - 1) / NT;

    // Activation piece e = tid + THREADS * s of a stage: block e / (4 MT)
    // = s / 2, row (e / 4) % MT = tid / 4 + 128 (s % 2), piece tid % 4.
    // The swizzle does not see the +128, so only the base is per lane.
    static_assert(APT == 4 && 4 * MT == 2 * THREADS, "piece mapping");
    const int a_row = tid >> 2, a_d = tid & 3;
    const int a_lds0 = a_row * 4 + a_slot(a_d, a_row);
    const uint32_t a_off0 = (uint32_t)a_row * (uint32_t)p.K * 2 + 16 * (uint32_t)a_d;
    const uint32_t half_rows = 128u * (uint32_t)p.K * 2;   // bytes of 128 rows
    // This thread's weights: column bc, block bu of each stage.
    const int bc = tid >> 1, bu = tid & 1;

    for (int64_t tile = blockIdx.x; tile < tiles_m * tiles_n; tile += gridDim.x) {
        const int64_t tm = tile / tiles_n, tn = tile - tm * tiles_n;
        const int64_t r0 = tm * MT, c0 = tn * NT;
        const int64_t left = p.N - c0;
        const uint32_t ncols = (uint32_t)(left < NT ? left : NT);
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B + c0 * row_bytes, (uint64_t)ncols * row_bytes);
        const __amdgpu_buffer_rsrc_t rS = make_rsrc(p.scales + c0 * nb, (uint64_t)ncols * nb * 2);
        const __amdgpu_buffer_rsrc_t rZ =
            make_rsrc(p.zp ? p.zp + c0 * p.zb : p.B, p.zp ? (uint64_t)ncols * p.zb : 0);
        const int64_t mrows = p.M - r0 < MT ? p.M - r0 : MT;
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + r0 * p.K, (uint64_t)mrows * (uint64_t)p.K * 2);

        struct WStage {
            u32x4 w;
            uint32_t s, z;
        };
        auto issue = [&](WStage& q, int st) {
            const uint32_t b = (uint32_t)(SB * st + bu);
            const bool ok = b < (uint32_t)nb;
            q.w = __builtin_amdgcn_raw_buffer_load_b128(
                rB, ok ? (uint32_t)bc * row_bytes + 16 * b : kOutOfRange, 0, kPrefillLoadPolicy);
            q.s = __builtin_amdgcn_raw_buffer_load_b16(
                rS, ok ? ((uint32_t)bc * (uint32_t)nb + b) * 2 : kOutOfRange, 0, kPrefillLoadPolicy);
            q.z = __builtin_amdgcn_raw_buffer_load_b8(
                rZ, ok ? (uint32_t)bc * (uint32_t)p.zb + b / 2 : kOutOfRange, 0, kPrefillLoadPolicy);
        };
        auto fetch_a = [&](uint4 (&v)[APT], int st) {
#pragma unroll
            for (int s = 0; s < APT; ++s) {
                const uint32_t off = a_off0 + (s & 1) * half_rows + 64 * (s >> 1) + 128 * (uint32_t)st;
                const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
                    rA, SB * st + (s >> 1) < nb ? off : kOutOfRange, 0, 0);
                v[s] = make_uint4(x[0], x[1], x[2], x[3]);
            }
        };
        // Activations to fp16 in the unpack's pair order; weights dequantized
        // to fp16 (q - z) * s in the same order; both into buffer buf.
        auto store = [&](const uint4 (&v)[APT], const WStage& q, int buf) {
#pragma unroll
            for (int s = 0; s < APT; ++s) {
                const uint4 x = v[s];
                uint4 o;
                if constexpr (ABF16) {
                    o.x = pair_bf16(x.x, x.z, false);
                    o.y = pair_bf16(x.x, x.z, true);
                    o.z = pair_bf16(x.y, x.w, false);
                    o.w = pair_bf16(x.y, x.w, true);
                } else {
                    o.x = pair16(x.x, x.z, false);
                    o.y = pair16(x.x, x.z, true);
                    o.z = pair16(x.y, x.w, false);
                    o.w = pair16(x.y, x.w, true);
                }
                a_lds[buf * QA + a_lds0 + ((s >> 1) * MT + 128 * (s & 1)) * 4] = o;
            }
            // Block SB*st + bu has parity bu (SB is even): its zero point is
            // nibble bu of the byte.
            const uint32_t zn = ((q.z >> (4 * bu)) & 0xFu) | zdef;
            const ZeroPoint zp = zero_point_pairs(zn);
            const uint32_t s2 = __builtin_amdgcn_perm(q.s, q.s, 0x01000100u);
            // Threads 2c and 2c+1 write blocks 0 and 1 of column c, 16 KB
            // apart: the slot also XORs 2 * block, so the two land in
            // different banks (a read takes one block, so it stays spread).
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t bq[4];
                unpack_dword(q.w[d], zp, magic, bq);
                b_lds[buf * QB + (bu * NT + bc) * 4 + (a_slot(d, bc) ^ (2 * bu))] =
                    make_uint4(hmul2(bq[0], s2), hmul2(bq[1], s2), hmul2(bq[2], s2), hmul2(bq[3], s2));
            }
        };

        float16_t acc[RTW][CTW];
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[rt][ct][q] = 0.f;

        auto compute = [&](int buf) {
#pragma unroll
            for (int i = 0; i < SB; ++i)
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    half8_t fa[RTW], fb[CTW];
#pragma unroll
                    for (int rt = 0; rt < RTW; ++rt) {
                        const int row = wr * 128 + rt * 32 + j;
                        const uint4 x = a_lds[buf * QA + (i * MT + row) * 4 + a_slot(2 * h + v, row)];
                        fa[rt] = __builtin_bit_cast(half8_t, u32x4{x.x, x.y, x.z, x.w});
                    }
#pragma unroll
                    for (int ct = 0; ct < CTW; ++ct) {
                        const int col = wc * 64 + ct * 32 + j;
                        const uint4 x = b_lds[buf * QB + (i * NT + col) * 4 + (a_slot(2 * h + v, col) ^ (2 * i))];
                        fb[ct] = __builtin_bit_cast(half8_t, u32x4{x.x, x.y, x.z, x.w});
                    }
#pragma unroll
                    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                        for (int ct = 0; ct < CTW; ++ct)
                            acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[rt], fb[ct], acc[rt][ct],
                                                                                 0, 0, 0);
                }
        };

        // Weight stages P ahead, activations one ahead, both stored into
        // LDS one stage ahead of use; one barrier per stage.  Stages past K
        // load zeros and add +0.
        WStage ring[P];
#pragma unroll
        for (int s = 0; s < P; ++s) issue(ring[s], s);
        uint4 av[APT];
        fetch_a(av, 0);
        __syncthreads();                  // the previous tile's readers are done
        store(av, ring[0], 0);
        issue(ring[0], P);
        fetch_a(av, 1);
        for (int s0 = 0; s0 < ns; s0 += P) {
#pragma unroll
            for (int s = 0; s < P; ++s) {
                const int st = s0 + s;
                __syncthreads();
                // Stage st+1 is converted after stage st's products, so the
                // activations fetched at the end of the previous step have
                // them to arrive in (gate_up m = 512: 180 -> 172.5 us, m =
                // 2048: 748 -> 716).
                compute(st & 1);
                store(av, ring[(s + 1) % P], (st + 1) & 1);
                issue(ring[(s + 1) % P], st + 1 + P);
                fetch_a(av, st + 2);
                // The two waves of a SIMD reach each barrier together, so the
                // conversions of a stage only overlap the matrix core if they
                // sit between its MFMAs: four VALU instructions after each of
                // the stage's 32 (2, 3 and 6 were slower).
#pragma unroll
                for (int g = 0; g < 32; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
                }
            }
        }

        // Epilogue: accumulator element q of lane (j, h) of tile (rt, ct) is
        // row 128 wr + 32 rt + (q%4) + 4h + 8(q/4), column 64 wc + 32 ct + j.
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int64_t col = c0 + wc * 64 + ct * 32 + j;
            if (col < p.N) {
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int64_t row = r0 + wr * 128 + rt * 32 + (q & 3) + 4 * h + 8 * (q >> 2);
                        if (row < p.M) {
                            const _Float16 hv = (_Float16)acc[rt][ct][q];
                            uint16_t bits = __builtin_bit_cast(uint16_t, hv);
                            if (p.out_bf16) bits = f16_to_bf16(bits);
                            p.out[row * p.N + col] = bits;
                        }
                    }
            }
        }
    }
}

// K split over workgroups, second launch: output e of the M x N result is
// the sum of its `splits` partial sums in slice order (fp32, slice 0 first),
// rounded to fp16 (RNE) and, for bf16 output, narrowed to bf16 (RNE): the
// store of the tile kernel.  One thread per output, consecutive threads on
// consecutive outputs.
__global__ __launch_bounds__(256) void mnb_split_reduce_kernel(const float* ws, int32_t splits, int64_t MN,
                                                               uint16_t* out, int32_t out_bf16)
{
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < MN; e += (int64_t)gridDim.x * 256) {
        // Eight slices' loads in flight at a time, added in order (slices
        // past the last are skipped, not added as +0, which would turn a -0
        // sum into +0).
        float v = 0.f;
        for (int k0 = 0; k0 < splits; k0 += 8) {
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = k0 + u < splits ? ws[(int64_t)(k0 + u) * MN + e] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (k0 + u < splits) v = k0 + u == 0 ? x[u] : v + x[u];
        }
        const _Float16 hv = (_Float16)v;
        uint16_t bits = __builtin_bit_cast(uint16_t, hv);
        if (out_bf16) bits = f16_to_bf16(bits);
        out[e] = bits;
    }
}

typedef void (*GemmFn)(GemmParams);

template <int CT, int W, bool VEC, bool ABF16, bool SPLIT>
GemmFn lookup_gemm_ct(int rt)
{
    switch (rt) {
    case 1: return mnb_gemm_mfma_kernel<1, CT, W, VEC, ABF16, 1, 32, SPLIT>;
    case 2: return mnb_gemm_mfma_kernel<2, CT, W, VEC, ABF16, 1, 32, SPLIT>;
    case 4: return mnb_gemm_mfma_kernel<4, CT, W, VEC, ABF16, 1, 32, SPLIT>;
    }
    return nullptr;
}

// Two waves with one 32-column tile each (64 columns), four waves with one
// or two (128 or 256 columns), or eight waves with one (256 columns); or
// one 32-row tile whose K the waves split: 32 columns over four waves, 16
// over four or eight.  (32 columns over eight waves was never faster than
// over four in the planner's sweep.)
template <bool VEC, bool ABF16, bool SPLIT>
GemmFn lookup_gemm_shape(int rt, int cols, int waves)
{
    if (cols == 32 || cols == 16) {
        if (rt != 1) return nullptr;
        if (cols == 32) return waves == 4 ? mnb_gemm_mfma_kernel<1, 1, 4, VEC, ABF16, 4, 32, SPLIT> : nullptr;
        if (waves == 4) return mnb_gemm_mfma_kernel<1, 1, 4, VEC, ABF16, 4, 16, SPLIT>;
        return waves == 8 ? mnb_gemm_mfma_kernel<1, 1, 8, VEC, ABF16, 8, 16, SPLIT> : nullptr;
    }
    if (waves == 2 && cols == 64) return lookup_gemm_ct<1, 2, VEC, ABF16, SPLIT>(rt);
    if (waves == 4 && cols == 128) return lookup_gemm_ct<1, 4, VEC, ABF16, SPLIT>(rt);
    if (waves == 4 && cols == 256) return lookup_gemm_ct<2, 4, VEC, ABF16, SPLIT>(rt);
    if (waves == 8 && cols == 256) return lookup_gemm_ct<1, 8, VEC, ABF16, SPLIT>(rt);
    return nullptr;
}

template <bool SPLIT>
GemmFn lookup_gemm_split(int rt, int cols, int w, bool vec, bool a_bf16)
{
    if (vec)
        return a_bf16 ? lookup_gemm_shape<true, true, SPLIT>(rt, cols, w) : lookup_gemm_shape<true, false, SPLIT>(rt, cols, w);
    return a_bf16 ? lookup_gemm_shape<false, true, SPLIT>(rt, cols, w) : lookup_gemm_shape<false, false, SPLIT>(rt, cols, w);
}

GemmFn lookup_gemm(const mnb_plan& plan, bool vec, bool a_bf16)
{
    const int rt = plan.row_tiles, cols = plan.cols_per_tile, w = plan.waves_per_wg;
    if (rt == 8)   // 256 x 256, weights through LDS (any scale alignment)
        return cols == kLdsTileCols && w == 8 && plan.k_splits <= 1
                   ? (a_bf16 ? mnb_gemm_lds_kernel<true> : mnb_gemm_lds_kernel<false>)
                   : nullptr;
    return plan.k_splits > 1 ? lookup_gemm_split<true>(rt, cols, w, vec, a_bf16)
                             : lookup_gemm_split<false>(rt, cols, w, vec, a_bf16);
}

bool gemm_vec_ok(int64_t K, const void* scales, const void* zp)
{
    return (K / 32) % 4 == 0 && ((uintptr_t)scales & 7) == 0 && ((uintptr_t)zp & 1) == 0;
}

}  // namespace

size_t gemm_lds_bytes(const mnb_plan& plan)
{
    if (plan.row_tiles == 8)   // two stages of activations and weights
        return (size_t)2 * (kLdsTileRows + kLdsTileCols) * 2 * 4 * 16;
    // Two steps of 32*rt rows x 128 k (one quad per K slice, one slice per
    // wave of a 32- or 16-column tile), fp16.
    const size_t slices = plan.cols_per_tile <= 32 ? (size_t)plan.waves_per_wg : 1;
    return (size_t)2 * slices * 4 * 32 * plan.row_tiles * 4 * 16;
}

int launch_gemm(const GemvArgs& a, const mnb_plan& plan, void* stream)
{
    GemmFn fn = lookup_gemm(plan, gemm_vec_ok(a.K, a.scales, a.zp), a.a_bf16 != 0);
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
    p.splits = plan.k_splits > 1 ? plan.k_splits : 1;
    p.ws = static_cast<float*>(a.ws);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn),
                                   dim3((unsigned)plan.workgroups), dim3(64 * plan.waves_per_wg), args,
                                   gemm_lds_bytes(plan), s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return (int)e;
    const int64_t MN = a.m * a.N;
    const int64_t groups = (MN + 255) / 256;
    const unsigned grid = (unsigned)(groups < 4096 ? groups : 4096);
    hipLaunchKernelGGL(mnb_split_reduce_kernel, dim3(grid), dim3(256), 0, s, static_cast<const float*>(p.ws),
                       p.splits, MN, p.out, p.out_bf16);
    return (int)hipGetLastError();
}


int gemm_workgroups_per_cu(const mnb_plan& plan)
{
    GemmFn fn = lookup_gemm(plan, true, true);
    if (!fn) return 0;
    return occupancy(reinterpret_cast<const void*>(fn), 64 * plan.waves_per_wg, gemm_lds_bytes(plan));
}

int gemm_kernel_info(const mnb_plan& plan, mnb_kernel_info* info)
{
    GemmFn fn = lookup_gemm(plan, true, true);
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
