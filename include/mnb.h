/*
 * libmnb -- block-wise INT4 MatMulNBits decode GEMV for AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; every pointer marked "device" is a
 * device address owned by the caller.  No call allocates device memory, and
 * no call synchronises the stream it is given.
 *
 * The operation (onnx-genai pull request "perf(cuda): let the split-K decode
 * GEMV store bf16 directly", first two paragraphs, and pull request "PORT-1
 * (offline bias+interleave) -- measured NO-GO on the multicol asymmetric-zp
 * GEMV", "Why the premise fails here", item 1):
 *
 *   y[r][n] = sum_k a[r][k] * (q[n][k] - z[n][k/32]) * s[n][k/32]
 *
 * for 0 <= r < m, 0 <= n < N, 0 <= k < K.  Weights q are 4-bit, packed two
 * per byte along K in blocks of 32; each (column, block) has an fp16 scale s
 * and a 4-bit zero point z (8 when no zero points are given: the symmetric
 * "+8 bias" case).  Activations are fp16, or bf16 converted to fp16 (round
 * to nearest even) for the dot product.  Products are accumulated in fp32,
 * the sum is rounded once to fp16 (RNE), and for bf16 output that fp16 value
 * is narrowed to bf16 (RNE) in the same kernel -- the fp32 -> fp16 -> bf16
 * double rounding of the staged fp16-GEMV-then-cast route, reproduced bit
 * for bit, with no staging buffer and no second launch.
 */
#ifndef MNB_H
#define MNB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MNB_ABI_VERSION 6

/* Element types of A and of the output. */
typedef enum { MNB_F16 = 0, MNB_BF16 = 1 } mnb_dtype;

/* Status codes.  On any code other than MNB_OK nothing was launched, except
 * MNB_ERR_HIP, which reports that the HIP launch itself failed. */
typedef enum {
    MNB_OK = 0,
    MNB_ERR_NULL = 1,     /* a required pointer is NULL                      */
    MNB_ERR_SHAPE = 2,    /* K < 0, N < 0, K not a multiple of 32, too large  */
    MNB_ERR_BLOCK = 3,    /* block != 32                                     */
    MNB_ERR_DTYPE = 4,    /* a_dtype or out_dtype not MNB_F16 / MNB_BF16      */
    MNB_ERR_ALIGN = 5,    /* A or Bpacked not 16-byte aligned, scales or out
                             not 2-byte aligned                              */
    MNB_ERR_M_RANGE = 6,  /* m < 0 or m > MNB_MAX_ROWS                        */
    MNB_ERR_HIP = 7,      /* the HIP runtime reported an error; see
                             mnb_last_hip_error()                            */
    MNB_ERR_ALIAS = 8,    /* out overlaps an input buffer                    */
    MNB_ERR_PLAN = 9,     /* an explicit plan is not one the library runs   */
    MNB_ERR_LAYOUT = 10,  /* unknown weight layout                            */
    MNB_ERR_WORKSPACE = 11 /* matmul_nbits_noalloc: the plan needs more than its
                              fixed workspace (MNB_MAX_SPLIT_WORKSPACE)       */
} mnb_status;

/*
 * Stored layouts of Bpacked (versioned; see mnb_repack_weights).
 *
 * MNB_LAYOUT_NATURAL   byte k/2 of row n holds weight k, even k in the low
 *                      nibble (the layout every entry point takes by default).
 * MNB_LAYOUT_EVEN_ODD  the offline odd/even nibble interleave of the second
 *                      page (pull request "PORT-1 (offline bias+interleave)",
 *                      opening paragraph and "Method"): within every 32-bit
 *                      word of a row (8 consecutive weights k0..k7, little
 *                      endian), nibble p holds k_{2(p mod 4) + p/4}, i.e.
 *                      k0 k2 k4 k6 in the low half-word and k1 k3 k5 k7 in
 *                      the high one, so the dequant yields (k, k+1) pairs and
 *                      the activations need no reorder.  Engines 0 and 3 read it.
 */
#define MNB_LAYOUT_NATURAL 0
#define MNB_LAYOUT_EVEN_ODD 1

/* Row-batched decode bound: one decode launch serves 1 <= m <= 8 rows (the
 * small-batch row loop of the first page, paragraph "What broke in #1549").
 * Beyond it (prefill, m up to MNB_MAX_ROWS) the same call runs a tiled
 * matrix-core kernel with the same narrowing store (the row-batched path the
 * first page leaves without one).  The prefill kernel multiplies fp16
 * weights: each (q - z) * s is rounded to fp16 (RNE) before the product, as
 * the second page's packed-half dequant holds it ("Why the premise fails
 * here", item 3); the decode kernels use the exact q - z and scale each
 * block's fp32 sum. */
#define MNB_MAX_M 8
#define MNB_MAX_ROWS (1 << 20)
/* Largest K accepted (blocks are indexed with 32-bit integers). */
#define MNB_MAX_K (1 << 24)
/* Largest device workspace (bytes) a default plan takes: the planner splits K
 * over workgroups (fp32 partial sums, k_splits * m * N * 4 bytes) only
 * within it. */
#define MNB_MAX_SPLIT_WORKSPACE ((size_t)32 << 20)

/*
 * matmul_nbits -- y = A * dequant(B)^T, kernel launches on `stream`: one;
 * two for a prefill plan that splits K over workgroups (the tiles, then the
 * sum of their slices); or for a decode plan with m > 8 one per 8 rows.
 *
 *   A            device, [m][K] row-major, fp16 or bf16 per a_dtype; 16-byte
 *                aligned.  Must hold finite values that are finite in fp16.
 *   a_dtype      MNB_F16 or MNB_BF16.
 *   m            rows, 0 <= m <= MNB_MAX_ROWS (m <= 8: decode kernels,
 *                except that two or more rows whose K the decode lane split
 *                would walk in several passes -- K > 65536 at two rows,
 *                > 32768 at three or four, > 16384 at five to eight -- run
 *                the prefill kernel; m > 8: prefill kernel, or, for up to
 *                16 rows where the planner's cost model prices them lower,
 *                the decode kernels in launches of 8 rows).  m == 0 or
 *                N == 0: nothing to do, MNB_OK.
 *   K            reduction length, a multiple of 32 (K == 0 gives y = +0).
 *   N            output columns.
 *   Bpacked      device, [N][K/2] bytes; byte k/2 of row n holds weight k,
 *                even k in the low nibble.  16-byte aligned.
 *   scales       device, [N][K/32] fp16 bit patterns; 2-byte aligned.
 *   zero_points  device, [N][ceil(K/64)] bytes, block b of row n in byte
 *                b/2 (even b in the low nibble), or NULL for zero point 8.
 *   block        must be 32.
 *   out          device, [m][N] row-major, fp16 or bf16 per out_dtype;
 *                2-byte aligned; must not overlap any input.  Every one of
 *                the m*N elements is overwritten (no accumulation) by this
 *                call's launches, each of which writes all of its rows.
 *   out_dtype    MNB_F16 (fp32 -> fp16 RNE) or MNB_BF16 (fp32 -> fp16 RNE
 *                -> bf16 RNE).
 *   stream       hipStream_t, or NULL for the default stream.
 *
 * Asynchronous: returns after the launch is queued.  Inputs must stay valid
 * and unmodified until the stream reaches this work.
 * Device memory: a plan that splits K over workgroups (prefill, few
 * columns; at most MNB_MAX_SPLIT_WORKSPACE bytes for a default plan) keeps
 * its fp32 partial sums in a workspace the library holds per device and
 * stream (per host thread on hipStreamPerThread) for the life of the
 * process.  The first such call on a stream, and a call that needs more
 * than the stream's workspace holds, allocate it with hipMalloc (a larger
 * one after the stream has drained); other calls allocate nothing.  Calls
 * that must not allocate use matmul_nbits_noalloc.
 * The fp32 summation order is fixed by (m, K) where the decode kernels run
 * at m <= 8 (never by N or the device), and by (m, K, N) and the device's
 * compute-unit count where the prefill kernel runs (which tiling runs, and
 * whether it splits K, depends on how the tiles fill the device).  So equal
 * inputs give bitwise equal outputs on the same device, column shards of
 * one matrix give the bits of the whole at m <= 8 wherever the decode
 * kernels run, and the bf16 output equals the fp16 output of the same call
 * narrowed to bf16.
 * Thread safety: may be called from several host threads at once (calls
 * that split K queue their two launches under one library lock).
 */
int matmul_nbits(const void* A, int a_dtype, int64_t m, int64_t K, int64_t N,
                 const uint8_t* Bpacked, const uint16_t* scales,
                 const uint8_t* zero_points, int block,
                 void* out, int out_dtype, void* stream);

/*
 * matmul_nbits_noalloc -- matmul_nbits for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses
 * that forbid hipMalloc): same arguments, same plan, same bits.  Where the
 * plan splits K over workgroups, the partial sums go to a fixed workspace
 * of MNB_MAX_SPLIT_WORKSPACE bytes that the library's code object holds on
 * every device it is loaded on, until the process ends, instead of the
 * per-stream workspace; no call allocates or frees anything.  Every call on
 * a device shares that device's workspace: calls whose work overlaps on
 * one device (other streams, other host threads) race and must be ordered
 * by the caller.  The workspace needs no clearing (each call writes every
 * partial sum it reads).  A plan needing more than the fixed workspace
 * returns MNB_ERR_WORKSPACE without launching; default plans never do.
 */
int matmul_nbits_noalloc(const void* A, int a_dtype, int64_t m, int64_t K, int64_t N,
                         const uint8_t* Bpacked, const uint16_t* scales,
                         const uint8_t* zero_points, int block,
                         void* out, int out_dtype, void* stream);

/*
 * Launch plan.  Every plan that mnb_plan_check() accepts computes the same
 * function; plans differ only in fp32 summation order and speed.
 *
 * engine 0 (lane-split dot2 kernel): a group of lanes_per_col lanes shares a
 * column; each lane owns blocks_per_lane 32-weight blocks of K per chunk and
 * keeps their activations in VGPRs; columns are walked cols_per_tile at a
 * time.  Dot products on v_dot2_f32_f16.
 * engine 2 (prefill kernel, m > 8): a workgroup owns a tile of
 * 32 * row_tiles rows by cols_per_tile columns, split by columns over its
 * waves: waves_per_wg = 2 with 64 columns, 4 with 128 or 256, or 8 with
 * 256; K is walked 128 at a time, activations through LDS; weights
 * dequantized to fp16 and v_mfma_f32_32x32x16_f16 accumulating over all of
 * K.  With 32 columns (row_tiles 1, waves_per_wg 4) the four waves split K
 * instead (wave s takes the 128-wide steps s, s + 4, ...) and their fp32
 * sums are added in wave order at the end.  With k_splits > 1 the tiles
 * also split K over workgroups: slice s of k_splits takes the 128-wide
 * steps [S*s/k_splits, S*(s+1)/k_splits) of the S steps, its fp32 sums go
 * to a workspace, and a second launch adds the slices in order and
 * narrows.  Also accepted for any m >= 1 as an explicit plan.
 * engine 3 (4x4x4 MFMA kernel, m <= 8): a workgroup of waves_per_wg waves
 * walks its columns cols_per_tile (4 or 8) at a time; lane i of each group
 * of four lanes holds column i of a quad and rows i and 4 + i of the
 * activations (in VGPRs); the 16 * waves_per_wg lane groups own
 * blocks_per_lane blocks each and together cover K in one pass (with four
 * blocks per lane group, the fewest waves that need four take four and the
 * others three, so that the waves' work is even); per block
 * the exact products come from v_mfma_f32_4x4x4_16b_f16 and the block scale
 * is applied in fp32, as in engine 0.  Needs 16 * waves_per_wg *
 * blocks_per_lane >= K/32 (so K <= 16384).  With a_via_lds each load of
 * activations reads one row's 1 KB run of a wave's 16 blocks and the pieces
 * reach their lanes through LDS (4160 bytes per wave); otherwise each lane
 * loads its own rows and blocks (16 bytes of four rows, 64 bytes apart).
 * Both give the same bits.
 */
typedef struct {
    int32_t engine;          /* 0: lane-split dot2 kernel; 2: prefill kernel;
                                3: 4x4x4 MFMA kernel                            */
    int32_t lanes_per_col;   /* engine 0: 16, 32, 64 (one wave) or 64*W, W=2..8 */
    int32_t blocks_per_lane; /* engine 0: 1, 2, 4 or 8; engine 3: 1, 2 or 4     */
    int32_t cols_per_tile;   /* engine 0: 1, 2, 4 or 8; engine 2: 32, 64, 128 or
                                256; engine 3: 4 or 8 (4 with blocks_per_lane 4
                                when m > 4)                                     */
    int32_t waves_per_wg;    /* engine 2: 2, 4, 8; engine 3: 1..8               */
    int32_t workgroups;      /* grid size, >= 1                                  */
    int32_t interleave;      /* engine 0: 0 = each lane group takes one contiguous
                                range of columns, 1 = column tiles dealt to the
                                groups round-robin                               */
    int32_t threads_per_wg;  /* derived by mnb_plan_check                        */
    int32_t k_chunks;        /* derived: passes over K                           */
    int32_t row_tiles;       /* engine 2: 32-row tiles per workgroup, 1, 2 or 4  */
    int32_t b_layout;        /* MNB_LAYOUT_* of Bpacked; engine 2 takes
                                MNB_LAYOUT_NATURAL only                         */
    int32_t k_splits;        /* engine 2 with row_tiles 1, 2 or 4: K split into
                                this many slices over the workgroups, whose fp32
                                partial sums a second launch adds in slice order
                                (workspace: k_splits * m * N * 4 bytes, the
                                buffer the library keeps per device and
                                stream); 0 or 1: no split.  Must be 0 or 1 for
                                the other engines.                             */
    int32_t a_via_lds;       /* engine 3: 1 = activations loaded a row at a time
                                and passed to their lanes through LDS, 0 = each
                                lane loads its own; must be 0 for the other
                                engines                                         */
} mnb_plan;

/* The plan matmul_nbits uses for (m, K, N) on a device with `num_cus`
 * compute units where the selected kernel variant keeps `wgs_per_cu`
 * workgroups resident per CU (0: a nominal estimate).  The lane split
 * (engine 0: lanes_per_col, blocks_per_lane, k_chunks; engine 3:
 * waves_per_wg, blocks_per_lane) depends on (m, K) only.
 * Host-only; touches no device.  Returns a status code. */
int mnb_plan_default(int64_t m, int64_t K, int64_t N, int num_cus, int wgs_per_cu,
                     mnb_plan* plan);

/* Validate a plan for (m, K, N) and fill its derived fields
 * (threads_per_wg, k_chunks).  A decode plan (engines 0 and 3) must fit 8
 * rows; with m > 8 the call runs it once per 8 rows (the last launch
 * fewer).
 * Host-only.  Returns MNB_OK or MNB_ERR_PLAN. */
int mnb_plan_check(int64_t m, int64_t K, int64_t N, mnb_plan* plan);

/* matmul_nbits with an explicit plan (after mnb_plan_check); same arguments,
 * same contract.  Used by tests that cover every kernel variant and by
 * tuning sweeps. */
int matmul_nbits_planned(const void* A, int a_dtype, int64_t m, int64_t K,
                         int64_t N, const uint8_t* Bpacked,
                         const uint16_t* scales, const uint8_t* zero_points,
                         int block, void* out, int out_dtype, void* stream,
                         const mnb_plan* plan);

/*
 * mnb_repack_weights -- convert packed weights between stored layouts, one
 * kernel launch on `stream` (the loader of the versioned layout).
 *
 *   src, dst     device, [N][K/2] bytes each, 16-byte aligned; dst == src
 *                converts in place, any other overlap is rejected.
 *   src_layout, dst_layout   MNB_LAYOUT_NATURAL or MNB_LAYOUT_EVEN_ODD.
 *   N, K         as for matmul_nbits (K a multiple of 32).
 *
 * Scales and zero points are not affected.  Asynchronous; allocates
 * nothing.  Returns MNB_OK, MNB_ERR_NULL, MNB_ERR_SHAPE, MNB_ERR_ALIGN,
 * MNB_ERR_ALIAS, MNB_ERR_LAYOUT or MNB_ERR_HIP; on error nothing is launched
 * (MNB_ERR_HIP: the launch itself failed).
 */
int mnb_repack_weights(const uint8_t* src, int src_layout, uint8_t* dst, int dst_layout,
                       int64_t N, int64_t K, void* stream);

/*
 * Environment: MNB_LOG set to anything but "0" (read once per process)
 * prints one line per call to stderr, once its plan is fixed and before
 * its launches: the shape, the types, whether the plan was explicit or the
 * default, every plan field, and the number of launches.
 */

/*
 * Counters, updated atomically on the host for every launch that was queued
 * successfully, from the launch's arguments (rows, columns, output type):
 * they record the route each call took, not what a kernel did, so tests
 * pair them with the output bits (the bf16 outputs must equal the fp16
 * outputs narrowed, which a kernel ignoring the flag would fail).  Tests
 * assert them so that a silent change of route fails instead of passing
 * (first page, "Tests" paragraph: the direct-store counter).
 */
typedef struct {
    uint64_t calls;                /* matmul_nbits* calls that returned MNB_OK */
    uint64_t launches;             /* kernel launches                          */
    uint64_t elements_f16;         /* outputs stored as fp16                   */
    uint64_t elements_bf16_direct; /* outputs narrowed and stored as bf16 by the
                                      GEMV epilogue itself                     */
    uint64_t row_batched_launches; /* launches that served m > 1 rows at once  */
} mnb_counters;

void mnb_counters_get(mnb_counters* out);
void mnb_counters_reset(void);

/* Registers and LDS of the kernel variant that (m, K, plan) selects, read
 * from the loaded code object (needs a device).  Returns a status code. */
typedef struct {
    int32_t vgprs;        /* architected VGPRs per lane   */
    int32_t sgprs;
    int32_t lds_bytes;    /* static LDS per workgroup     */
    int32_t max_threads;  /* launch bound of the variant  */
    int32_t wgs_per_cu;   /* occupancy: workgroups per CU at threads_per_wg */
} mnb_kernel_info;

int mnb_get_kernel_info(int64_t m, int64_t K, const mnb_plan* plan,
                        mnb_kernel_info* info);

/* Human-readable text of a status code (static storage). */
const char* mnb_status_string(int status);

/* The hipError_t of the last MNB_ERR_HIP returned on this host thread. */
int mnb_last_hip_error(void);

/* MNB_ABI_VERSION of the loaded library. */
int mnb_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MNB_H */
