// Host front end of libmnb: argument validation, launch planning, counters
// and status strings.  Plain C++ (no HIP headers): everything here runs, and
// is tested, without a GPU.  The kernels and their launch live in
// mnb_gemv.hip.
#include <algorithm>
#include <cmath>
#include <atomic>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "mnb.h"
#include "mnb_internal.h"

namespace {

std::atomic<uint64_t> g_calls{0}, g_launches{0}, g_f16{0}, g_bf16{0}, g_rows{0};
thread_local int t_last_hip_error = 0;

// Register budget: M rows x blocks_per_lane blocks of activations stay in
// VGPRs (16 per block and row), at most 8 such blocks per lane.
int max_blocks_per_lane(int64_t m) { return m == 1 ? 8 : m == 2 ? 4 : m <= 4 ? 2 : 1; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t pow2_ceil(int64_t x)
{
    int64_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

bool is_pow2_in(int64_t x, int64_t lo, int64_t hi)
{
    return x >= lo && x <= hi && (x & (x - 1)) == 0;
}

bool overlaps(const void* a, int64_t an, const void* b, int64_t bn)
{
    if (!a || !b || an <= 0 || bn <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bn && b0 < a0 + (uintptr_t)an;
}

// Nominal resident waves per CU, used to size the grid when the occupancy of
// the chosen kernel variant is not known (host-only planning).
constexpr int kTargetWavesPerCu = 16;
constexpr int kMaxKSplits = 64;   // K slices over workgroups (engine 2)
// Largest workspace a default plan uses (K split over workgroups).
constexpr size_t kMaxSplitWorkspaceBytes = MNB_MAX_SPLIT_WORKSPACE;

int validate(const void* A, int a_dtype, int64_t m, int64_t K, int64_t N,
             const uint8_t* Bpacked, const uint16_t* scales,
             const uint8_t* zero_points, int block, void* out, int out_dtype)
{
    if (m < 0 || m > MNB_MAX_ROWS) return MNB_ERR_M_RANGE;
    if (K < 0 || N < 0 || K > MNB_MAX_K || N > INT32_MAX) return MNB_ERR_SHAPE;
    if (block != 32) return MNB_ERR_BLOCK;
    if (K % 32 != 0) return MNB_ERR_SHAPE;
    if ((a_dtype != MNB_F16 && a_dtype != MNB_BF16) ||
        (out_dtype != MNB_F16 && out_dtype != MNB_BF16))
        return MNB_ERR_DTYPE;
    if (m == 0 || N == 0) return MNB_OK;
    if (!out) return MNB_ERR_NULL;
    if (K > 0 && (!A || !Bpacked || !scales)) return MNB_ERR_NULL;
    if (((uintptr_t)A & 15) || ((uintptr_t)Bpacked & 15) ||
        ((uintptr_t)scales & 1) || ((uintptr_t)out & 1))
        return MNB_ERR_ALIGN;
    const int64_t nb = K / 32;
    const int64_t out_bytes = m * N * 2;
    if (overlaps(out, out_bytes, A, m * K * 2) ||
        overlaps(out, out_bytes, Bpacked, N * (K / 2)) ||
        overlaps(out, out_bytes, scales, N * nb * 2) ||
        overlaps(out, out_bytes, zero_points, N * ((nb + 1) / 2)))
        return MNB_ERR_ALIAS;
    return MNB_OK;
}

// MNB_LOG set to anything but "0" in the environment (read once): each call
// that reaches its launches prints its shape and plan to stderr, one line.
bool log_enabled()
{
    static const bool on = [] {
        const char* v = getenv("MNB_LOG");
        return v && *v && !(v[0] == '0' && v[1] == 0);
    }();
    return on;
}

void log_plan(int64_t m, int64_t K, int64_t N, int a_dtype, int out_dtype, const mnb_plan& p, bool explicit_plan,
              bool fixed_scratch)
{
    const int64_t step = p.engine == 2 ? m : MNB_MAX_M;
    const int64_t launches = (m + step - 1) / step * (p.k_splits > 1 ? 2 : 1);
    fprintf(stderr,
            "mnb: m=%lld K=%lld N=%lld a=%s out=%s %s plan: engine=%d lanes_per_col=%d blocks_per_lane=%d "
            "cols_per_tile=%d waves_per_wg=%d row_tiles=%d k_splits=%d a_via_lds=%d b_layout=%d interleave=%d "
            "workgroups=%d threads_per_wg=%d k_chunks=%d launches=%lld%s\n",
            (long long)m, (long long)K, (long long)N, a_dtype == MNB_BF16 ? "bf16" : "f16",
            out_dtype == MNB_BF16 ? "bf16" : "f16", explicit_plan ? "explicit" : "default", p.engine,
            p.lanes_per_col, p.blocks_per_lane, p.cols_per_tile, p.waves_per_wg, p.row_tiles, p.k_splits,
            p.a_via_lds, p.b_layout, p.interleave, p.workgroups, p.threads_per_wg, p.k_chunks,
            (long long)launches, fixed_scratch ? " fixed-scratch" : "");
}

int run(const void* A, int a_dtype, int64_t m, int64_t K, int64_t N,
        const uint8_t* Bpacked, const uint16_t* scales, const uint8_t* zero_points,
        int block, void* out, int out_dtype, void* stream, const mnb_plan* explicit_plan,
        bool fixed_scratch = false)
{
    int st = validate(A, a_dtype, m, K, N, Bpacked, scales, zero_points, block, out,
                      out_dtype);
    if (st != MNB_OK) return st;
    if (m == 0 || N == 0) {
        g_calls.fetch_add(1, std::memory_order_relaxed);
        return MNB_OK;
    }
    mnb_plan plan;
    if (explicit_plan) {
        plan = *explicit_plan;
        if (mnb_plan_check(m, K, N, &plan) != MNB_OK) return MNB_ERR_PLAN;
    } else {
        int cus = 0;
        int e = mnb::current_device_cus(&cus);
        if (e != 0) {
            t_last_hip_error = e;
            return MNB_ERR_HIP;
        }
        // Plan once with a nominal occupancy to pick the kernel variant, then
        // again with that variant's measured occupancy for the grid.
        st = mnb_plan_default(m, K, N, cus, 0, &plan);
        if (st != MNB_OK) return st;
        const int per_cu = mnb::workgroups_per_cu(plan.engine == 2 ? m : std::min<int64_t>(m, MNB_MAX_M), K, N, plan);
        if (per_cu > 0) {
            st = mnb_plan_default(m, K, N, cus, per_cu, &plan);
            if (st != MNB_OK) return st;
        }
    }
    if (log_enabled()) log_plan(m, K, N, a_dtype, out_dtype, plan, explicit_plan != nullptr, fixed_scratch);
    // One launch (two with K split over workgroups: the tiles, then the sum
    // of their slices), or for a decode plan with more than MNB_MAX_M rows
    // one launch per MNB_MAX_M rows (rows are independent in those kernels).
    const int64_t step = plan.engine == 2 ? m : MNB_MAX_M;
    const size_t a_row = (size_t)K * 2, out_row = (size_t)N * 2;
    const int per_launch = plan.k_splits > 1 ? 2 : 1;
    void* ws = nullptr;
    bool held = false;   // the per-stream workspace is held until the launches are queued
    const size_t ws_bytes = mnb::workspace_bytes(m, N, plan);
    if (ws_bytes && fixed_scratch) {
        if (ws_bytes > mnb::kScratchBytes) return MNB_ERR_WORKSPACE;
        int e = mnb::scratch_address(&ws);
        if (e != 0) {
            t_last_hip_error = e;
            return MNB_ERR_HIP;
        }
    } else if (ws_bytes) {
        int e = mnb::workspace_acquire(ws_bytes, stream, &ws);
        if (e != 0) {
            t_last_hip_error = e;
            return MNB_ERR_HIP;
        }
        held = true;
    }
    int64_t launched = 0, batched = 0;
    for (int64_t r0 = 0; r0 < m; r0 += step) {
        const int64_t mc = std::min<int64_t>(step, m - r0);
        mnb::GemvArgs args{static_cast<const uint8_t*>(A) + r0 * a_row, Bpacked, scales, zero_points,
                           static_cast<uint8_t*>(out) + r0 * out_row, mc, K, N,
                           a_dtype == MNB_BF16, out_dtype == MNB_BF16, ws};
        int e = mnb::launch_gemv(args, plan, stream);
        if (e != 0) {
            t_last_hip_error = e;
            g_launches.fetch_add((uint64_t)launched, std::memory_order_relaxed);
            if (held) mnb::workspace_release();
            return MNB_ERR_HIP;
        }
        launched += per_launch;
        if (mc > 1) ++batched;
    }
    if (held) mnb::workspace_release();
    g_calls.fetch_add(1, std::memory_order_relaxed);
    g_launches.fetch_add((uint64_t)launched, std::memory_order_relaxed);
    if (out_dtype == MNB_BF16) g_bf16.fetch_add((uint64_t)(m * N), std::memory_order_relaxed);
    else g_f16.fetch_add((uint64_t)(m * N), std::memory_order_relaxed);
    g_rows.fetch_add((uint64_t)batched, std::memory_order_relaxed);
    return MNB_OK;
}

}  // namespace

namespace mnb {

size_t workspace_bytes(int64_t m, int64_t N, const mnb_plan& plan)
{
    return plan.engine == 2 && plan.k_splits > 1 ? (size_t)plan.k_splits * (size_t)m * (size_t)N * 4 : 0;
}

int64_t gemv_lds_bytes(int64_t m, int64_t N, const mnb_plan& plan, int32_t* tcap)
{
    *tcap = 0;
    if (plan.engine != 0 || plan.lanes_per_col < 64) return 0;
    if (plan.lanes_per_col == 64)   // activations shared by the workgroup's waves
        return plan.k_chunks == 1 ? m * plan.blocks_per_lane * 256 * 16 : 0;
    const int64_t nw = plan.lanes_per_col / 64;
    const int64_t nv = (int64_t)plan.cols_per_tile * m;
    const int64_t g = plan.workgroups < 1 ? 1 : plan.workgroups;
    // Most tiles any group gets: dealt round-robin, or a contiguous range of
    // at most ceil(N / g) columns.
    const int64_t tiles = plan.interleave ? ceil_div(N, plan.cols_per_tile * g)
                                          : ceil_div(ceil_div(N, g), plan.cols_per_tile);
    const int64_t t = tiles < 1 ? 1 : tiles;
    if (t * nw * nv * 4 <= kDeferLdsBytes) {
        *tcap = (int32_t)t;
        return t * nw * nv * 4;
    }
    return 2 * nw * nv * 4;
}

}  // namespace mnb

namespace {

// Prefill tilings of engine 2 (row tiles, columns, waves, K splits over
// workgroups) and their fitted cost in microseconds on gfx950:
//   t0 + a*k*(R-1) + g*(R-1) + d*k + h*W + u*U
// with k the thousands of K per workgroup (K / splits), R = ceil(tiles /
// CUs) rounds of tiles over the compute units (a split multiplies the
// tiles), W the MB of weights (with scales and zero points) per CU and U the
// MB of fp32 partial sums per CU that a split writes and its second launch
// reads.  a and g price the rounds after the first, d and t0 the first (a CU
// with one tile runs it faster than two that share it), h the weights that
// stream from HBM when few row tiles share them, u the partial sums.
struct Tiling {
    int32_t rt, cols, waves, splits;
    double t0, a, g, d, h, u;
};
constexpr Tiling kTilings[] = {
    {1, 16, 4, 1, 3.8610, 1.3850, 1.9342, 1.8901, 0.0000, 0.0000},   // 16 columns on a 32-column tile, K split over the waves
    {1, 16, 8, 1, 5.8870, 2.0036, 1.9578, 1.7275, 0.0000, 0.0000},
    {1, 32, 4, 1, 4.9887, 1.4723, 2.3993, 1.9066, 3.2569, 0.0000},   // K split over the four waves
    {1, 64, 2, 1, 1.0704, 2.2076, 1.7534, 5.4974, 10.5770, 0.0000},
    {1, 128, 4, 1, 1.3403, 4.3963, 2.3819, 5.5898, 13.0526, 0.0000},
    {2, 128, 4, 1, 3.5663, 5.8118, 2.3400, 6.0021, 6.7267, 0.0000},
    {4, 128, 4, 1, 4.8855, 12.3022, 3.1521, 11.2704, 0.0000, 0.0000},
    {1, 256, 8, 1, 0.0000, 9.4388, 3.2051, 8.9528, 34.2933, 0.0000},
    {2, 256, 8, 1, 1.2841, 12.2381, 4.1168, 10.2565, 24.1162, 0.0000},
    {4, 256, 8, 1, 3.7579, 17.8627, 7.8076, 14.5888, 8.0399, 0.0000},
    {8, 256, 8, 1, 7.1312, 33.1356, 0.0000, 24.0315, 10.5656, 0.0000},   // 256 x 256, weights through LDS
    {1, 128, 4, 2, 5.6571, 3.8579, 0.0000, 4.8528, 7.4596, 198.7183},   // K split over 2..16 workgroups, a second launch adds the slices
    {1, 128, 4, 4, 6.4293, 3.9396, 0.0000, 4.4597, 10.4470, 161.6987},
    {1, 128, 4, 8, 5.9191, 3.4284, 1.3289, 5.3852, 9.2180, 115.3103},
    {1, 128, 4, 16, 6.7797, 1.6008, 1.9160, 4.2164, 17.8949, 115.9995},
    {2, 128, 4, 2, 6.1070, 4.2767, 0.0000, 5.9467, 2.2971, 197.8420},
    {2, 128, 4, 4, 7.1911, 5.1908, 0.0000, 5.7611, 3.9607, 124.0901},
    {2, 128, 4, 8, 7.1840, 4.8146, 0.7588, 6.3397, 3.3817, 110.2482},
    {2, 128, 4, 16, 7.5359, 2.1214, 2.8233, 6.5482, 0.0000, 122.8116},
    {4, 128, 4, 2, 6.8219, 11.1767, 0.0000, 11.0433, 3.0875, 190.7041},
    {4, 128, 4, 4, 8.1219, 11.8653, 0.1360, 10.4706, 12.1705, 145.6724},
    {4, 128, 4, 8, 7.4293, 10.2051, 5.1548, 12.0446, 8.9930, 111.4425},
    {4, 128, 4, 16, 9.2655, 7.5497, 8.0509, 11.1810, 0.0000, 104.2306},
    {1, 256, 8, 2, 3.7288, 7.2387, 0.0000, 8.5014, 23.7040, 193.0096},
    {1, 256, 8, 4, 5.5982, 7.9531, 0.0000, 8.4352, 15.2034, 128.6234},
    {1, 256, 8, 8, 6.1386, 9.1381, 0.0000, 8.8607, 17.0575, 79.5319},
    {1, 256, 8, 16, 7.3761, 7.1060, 2.1161, 7.8029, 18.2416, 59.4031},
    {2, 256, 8, 2, 4.8553, 11.6227, 0.0000, 10.3156, 13.5775, 182.9153},
    {2, 256, 8, 4, 6.4314, 11.4627, 0.0000, 10.2646, 8.3824, 133.9338},
    {2, 256, 8, 8, 6.2573, 12.3964, 0.3921, 10.7960, 14.1889, 108.8004},
    {2, 256, 8, 16, 7.6852, 8.0358, 5.4080, 9.0132, 20.0183, 85.1982},
};
// The decode plan per launch of r <= 8 rows: a part that grows with K (the
// activation staging and the per-wave work of each workgroup) and a part
// linear in the weight MB (with scales and zero points) at a rate per row,
//   exp(c0) * (K / 4096)^c1 + MB * (c2 + c3 * r / 8),
// and no less than 3 us, about what one launch takes however small.  (A
// power law in N, as first fitted, ran 15-20% below the launches on 151936
// columns, where the time is linear in the weights.)
constexpr double kDecode[4] = {1.6501, 0.1652, 0.1290, 0.0767};
constexpr double kBytesPerWeight = 0.578;   // 4 bits, and a 2-byte scale and a 4-bit zero point per 32
constexpr double kDecodeLaunchUs = 3.0;

int64_t prefill_tiles(const Tiling& t, int64_t m, int64_t N)
{
    const int64_t rows = t.rt == 8 ? 256 : 32 * (int64_t)t.rt;
    return ceil_div(m, rows) * ceil_div(N, t.cols) * t.splits;
}

double tiling_cost(const Tiling& t, int64_t m, int64_t K, int64_t N, int num_cus)
{
    const double R = (double)ceil_div(prefill_tiles(t, m, N), num_cus);
    const double k = (double)K / t.splits / 1e3;
    const double w = (double)N * (double)K * kBytesPerWeight / num_cus / 1e6;
    const double ws = t.splits > 1 ? (double)t.splits * (double)m * (double)N * 4 / num_cus / 1e6 : 0.0;
    return t.t0 + t.a * k * (R - 1) + t.g * (R - 1) + t.d * k + t.h * w + t.u * ws;
}

double decode_cost(int64_t m, int64_t K, int64_t N)
{
    const double mb = (double)N * (double)K * kBytesPerWeight / 1e6;
    auto one = [&](int64_t r) {
        const double t = std::exp(kDecode[0]) * std::pow((double)K / 4096, kDecode[1]) +
                         mb * (kDecode[2] + kDecode[3] * (double)r / 8);
        return t > kDecodeLaunchUs ? t : kDecodeLaunchUs;
    };
    const int64_t full = m / MNB_MAX_M, rem = m % MNB_MAX_M;
    return (double)full * one(MNB_MAX_M) + (rem ? one(rem) : 0.0);
}

struct PrefillChoice {
    Tiling t;
    bool decode;
};

// The cheapest plan by the model among the tilings the plan check accepts
// for (m, K, N) and, with `decode`, the decode plan; ties go to the earlier
// tiling.
PrefillChoice cheapest_prefill(int64_t m, int64_t K, int64_t N, int num_cus, bool decode = true)
{
    PrefillChoice best{kTilings[0], decode};
    double best_cost = decode ? decode_cost(m, K, N) : HUGE_VAL;
    for (const Tiling& t : kTilings) {
        mnb_plan q{};
        q.engine = 2;
        q.row_tiles = t.rt;
        q.cols_per_tile = t.cols;
        q.waves_per_wg = t.waves;
        q.k_splits = t.splits;
        q.workgroups = 1;
        if (mnb_plan_check(m, K, N, &q) != MNB_OK) continue;
        // A K split is there to fill the device: only while its tiles fit
        // in less than four rounds over the CUs, within the workspace bound.
        if (t.splits > 1 && (prefill_tiles(t, m, N) >= 4 * (int64_t)num_cus ||
                             mnb::workspace_bytes(m, N, q) > kMaxSplitWorkspaceBytes))
            continue;
        const double c = tiling_cost(t, m, K, N, num_cus);
        if (c < best_cost) {
            best_cost = c;
            best = PrefillChoice{t, false};
        }
    }
    return best;
}

// The prefill plan of tiling t: one resident generation of workgroups, at
// most one per tile.
int prefill_plan(const Tiling& t, int64_t m, int64_t K, int64_t N, int num_cus, int wgs_per_cu, mnb_plan* plan)
{
    const int64_t per_cu = wgs_per_cu > 0 ? wgs_per_cu : 1;
    const int64_t tiles = prefill_tiles(t, m, N);
    int64_t wgs = per_cu * num_cus;
    if (wgs > tiles) wgs = tiles;
    plan->engine = 2;
    plan->row_tiles = t.rt;
    plan->cols_per_tile = t.cols;
    plan->waves_per_wg = t.waves;
    plan->k_splits = t.splits;
    plan->workgroups = (int32_t)(wgs < 1 ? 1 : wgs);
    return mnb_plan_check(m, K, N, plan) == MNB_OK ? MNB_OK : MNB_ERR_PLAN;
}

}  // namespace

extern "C" {

int mnb_plan_check(int64_t m, int64_t K, int64_t N, mnb_plan* plan)
{
    if (!plan || m < 1 || m > MNB_MAX_ROWS || K < 0 || K % 32 || N < 0) return MNB_ERR_PLAN;
    if (plan->workgroups < 1) return MNB_ERR_PLAN;
    if (plan->b_layout != MNB_LAYOUT_NATURAL &&
        !(plan->b_layout == MNB_LAYOUT_EVEN_ODD && (plan->engine == 0 || plan->engine == 3)))
        return MNB_ERR_PLAN;
    if (plan->a_via_lds != 0 && (plan->a_via_lds != 1 || plan->engine != 3)) return MNB_ERR_PLAN;
    const int64_t nb = K / 32;
    if (plan->engine == 2) {
        const bool shape_ok =
            plan->row_tiles == 8 ? (plan->waves_per_wg == 8 && plan->cols_per_tile == 256)
                                 : ((plan->row_tiles == 1 && ((plan->cols_per_tile == 32 && plan->waves_per_wg == 4) ||
                                                              (plan->cols_per_tile == 16 &&
                                                               (plan->waves_per_wg == 4 || plan->waves_per_wg == 8)))) ||
                                    (plan->waves_per_wg == 2 && plan->cols_per_tile == 64) ||
                                    (plan->waves_per_wg == 4 && is_pow2_in(plan->cols_per_tile, 128, 256)) ||
                                    (plan->waves_per_wg == 8 && plan->cols_per_tile == 256));
        if (!is_pow2_in(plan->row_tiles, 1, 8) || !shape_ok ||
            (uint64_t)64 * plan->row_tiles * (uint64_t)K > mnb::kPrefillRowBlockBytes)
            return MNB_ERR_PLAN;
        // K split over workgroups: at least one 128-wide step per slice, not
        // for the LDS-staged 256 x 256 tiles, a workspace below 2^31 floats
        // per slice plane, and fewer than 2^31 tiles (the kernel's slice
        // arithmetic is 32-bit).
        if (plan->k_splits < 0 || plan->k_splits > kMaxKSplits) return MNB_ERR_PLAN;
        if (plan->k_splits > 1 &&
            (plan->row_tiles == 8 || plan->k_splits > ceil_div(nb, 4) || m * N > (int64_t)INT32_MAX ||
             ceil_div(m, 32 * (int64_t)plan->row_tiles) * ceil_div(N, (int64_t)plan->cols_per_tile) *
                     plan->k_splits > (int64_t)INT32_MAX))
            return MNB_ERR_PLAN;
        plan->threads_per_wg = 64 * plan->waves_per_wg;
        plan->k_chunks = (int32_t)ceil_div(nb, 4);   // 128-wide steps of K
        return MNB_OK;
    }
    if (plan->k_splits > 1) return MNB_ERR_PLAN;
    // Decode engines: a launch serves at most MNB_MAX_M rows; more rows run
    // as launches of MNB_MAX_M rows (the last one fewer) under this plan, so
    // the plan must fit MNB_MAX_M rows.
    if (m > MNB_MAX_M) m = MNB_MAX_M;
    if (plan->engine == 3) {
        // 4x4x4 MFMA kernel: the workgroup's 16 * waves lane groups cover K
        // in one pass, blocks_per_lane blocks each; 4 or 8 columns per tile.
        const int64_t w = plan->waves_per_wg, bpl = plan->blocks_per_lane;
        if (w < 1 || w > 8 || !is_pow2_in(bpl, 1, 4) ||
            (plan->cols_per_tile != 4 && plan->cols_per_tile != 8))
            return MNB_ERR_PLAN;
        if (16 * w * bpl < nb) return MNB_ERR_PLAN;
        if (m > 4 && bpl * (plan->cols_per_tile / 4) > 4) return MNB_ERR_PLAN;   // registers
        plan->threads_per_wg = (int32_t)(64 * w);
        plan->k_chunks = 1;
        return MNB_OK;
    }
    if (plan->engine != 0) return MNB_ERR_PLAN;
    const int64_t lpc = plan->lanes_per_col;
    const int64_t bpl = plan->blocks_per_lane;
    const int64_t nc = plan->cols_per_tile;
    const bool inwave = is_pow2_in(lpc, 16, 64);
    const bool xwave = lpc % 64 == 0 && lpc >= 128 && lpc <= 512;
    if (!inwave && !xwave) return MNB_ERR_PLAN;
    if (!is_pow2_in(bpl, 1, 8) || m * bpl > 8) return MNB_ERR_PLAN;
    if (!is_pow2_in(nc, 1, 8) || nc * bpl > 8 || nc * m > 32) return MNB_ERR_PLAN;
    if (plan->interleave != 0 && plan->interleave != 1) return MNB_ERR_PLAN;
    plan->threads_per_wg = inwave ? 256 : (int32_t)lpc;
    const int64_t chunks = nb == 0 ? 1 : ceil_div(nb, lpc * bpl);
    if (chunks > INT32_MAX) return MNB_ERR_PLAN;
    plan->k_chunks = (int32_t)chunks;
    return MNB_OK;
}

int mnb_plan_default(int64_t m, int64_t K, int64_t N, int num_cus, int wgs_per_cu,
                     mnb_plan* plan)
{
    if (!plan) return MNB_ERR_NULL;
    if (m < 1 || m > MNB_MAX_ROWS) return MNB_ERR_M_RANGE;
    if (K < 0 || K % 32 || K > MNB_MAX_K || N < 1 || N > INT32_MAX) return MNB_ERR_SHAPE;
    if (num_cus < 1) num_cus = 1;
    *plan = mnb_plan{};

    if (m > MNB_MAX_M) {
        // Prefill: every tiling of the prefill kernel that the plan check
        // accepts (with K split over workgroups where that fills the
        // device), and the 8-row decode plan run once per 8 rows, priced by
        // a cost model fitted to timings on gfx950 (256 CUs, bf16 in and
        // out, 64 shapes from 9 x 2048 x 8192 to 4096 x 4096 x 28672 and
        // 640 x 4096 x 151936; plan_tune.py measures and fits it).  On
        // those shapes the cheapest modelled plan runs 0.37% slower than
        // the fastest measured one on average (6.9% at most, where a split
        // the model ranks second would have won), and 11.9% faster on
        // average than the fastest plan without a K split (never more than
        // 2.7% slower: a choice between unsplit tilings).
        const PrefillChoice c = cheapest_prefill(m, K, N, num_cus);
        if (c.decode) return mnb_plan_default(MNB_MAX_M, K, N, num_cus, wgs_per_cu, plan);
        return prefill_plan(c.t, m, K, N, num_cus, wgs_per_cu, plan);
    }
    const int64_t nb = K / 32;
    const int64_t bmax = max_blocks_per_lane(m);

    // Two or more rows with K within one pass of a workgroup (8 waves x 16
    // lane groups x 4 blocks): the 4x4x4 MFMA kernel, whose dot products do
    // not grow the VALU work with m (against the lane split below, bf16:
    // lm_head m = 2 82.9 -> 69.7 us, m = 8 104 -> 90.6; gate_up m = 8 70.4 ->
    // 26.9, m = 3 25.4 -> 20.0; down m = 8 26.1 -> 18.5, m = 3 15.6 -> 12.9;
    // the 6144-column shape gains at m = 8 and loses up to 1 us at m <= 3).
    // Lane split, a function of (m, K) only (the exceptions below): the
    // fewest blocks per lane group that
    // cover K with at most four waves, else eight waves, of which the kernel
    // gives the fewest that need them four blocks per lane group and the
    // rest three (K = 14336: four of each, against seven waves of four,
    // interleaved A/B, us: m = 2 11.0 -> 10.4, m = 4 11.7 -> 11.3, m = 6
    // 14.8 -> 13.8, m = 8 15.2 -> 14.1; 10240 x 4096 m = 4 10.3 -> 9.5,
    // 12288 x 8192 m = 8 19.8 -> 18.2).  Four columns per tile.
    // Grid: whole workgroups per CU, about 12 * K/4096 tiles (column quads)
    // each, within one resident generation and at least two tiles each (the
    // tile loop runs in pairs).  Every workgroup stages all of K's
    // activations, so fewer, longer-lived workgroups win until the CUs run
    // short of waves (at one or two rows, two workgroups per CU at least,
    // below).  On a sweep of 50 shapes (m = 2..8, K = 2048..14336, N =
    // 4096..151936, bf16): 0.30% above the fastest grid on average, 6.1% at
    // most (10 * K/4096, fitted on an earlier sweep, gave 0.63% and 8.2% on
    // this one: 2048 x 28672 at six and eight rows took six workgroups per
    // CU where five are 8% faster; 14 * K/4096 and above put 4096 x 14336
    // at three rows on one workgroup per CU, 22% slower).
    // Activations through LDS from three rows up where K or N exceeds 8192
    // (interleaved A/B, same bits, us: down projection m = 3 12.5 -> 11.5,
    // m = 4 13.6 -> 11.9, m = 7 17.5 -> 15.4, m = 8 18.3 -> 15.7; gate_up
    // m = 4 18.7 -> 17.0, m = 8 24.3 -> 22.3; lm_head m = 3 -2.0%, m = 6
    // -1.7%); at 8192 x 8192, 4096 x 6144 and 4096 x 4096 it was 2-4.5%
    // slower, and at m = 2, where half of the lanes' own loads read nothing,
    // 0-4% slower.
    if (m >= 2 && nb >= 1 && nb <= 512) {
        // Up to four rows, at least two blocks per lane group where that
        // still leaves two waves: K = 2048 runs two waves of two blocks
        // instead of four of one (m = 2: 8.2 -> 7.1 us at N = 14336, 11.9 ->
        // 10.4 at 28672, 40.3 -> 34.8 at 151936, 5.8 -> 5.2 at 8192; m = 4
        // 8-13% faster from N = 14336 up, 3% slower at 8192).  From five
        // rows it lost at N = 8192 (m = 8: 7.3 -> 8.2 us), so there the
        // four waves of one stay.  A function of (m, K), like the rest of
        // the lane split.
        int64_t bpl3 = nb >= 64 && m <= 4 ? 2 : 1;
        while (bpl3 < 4 && ceil_div(nb, 16 * bpl3) > 4) bpl3 *= 2;
        // Three waves of four blocks (4096 < K <= 6144) leave one SIMD of
        // each workgroup idle: five or six waves of two instead (5120 x
        // 4096 m = 4 / 6 / 8 7.4 / 9.4 / 9.9 -> 7.0 / 8.4 / 9.3 us; 6144 x
        // 4096 m = 2 / 8 7.6 / 10.5 -> 7.0 / 9.8, 6144 x 14336 m = 6 / 8
        // 19.4 / 19.8 -> 18.4 / 18.5; at 28672 columns 0.5-2.6% slower).
        if (bpl3 == 4 && ceil_div(nb, 64) == 3) bpl3 = 2;
        int64_t w3 = ceil_div(nb, 16 * bpl3);
        if (w3 > 4 && bpl3 == 4) w3 = 8;   // two waves per SIMD; the kernel gives some three blocks per lane group
        const int64_t tiles3 = ceil_div(N, 4);
        const int64_t per_cu3 = wgs_per_cu > 0 ? wgs_per_cu : (w3 >= 4 ? 2 : 4);
        const double per_wg = 12.0 * (double)K / 4096.0;
        int64_t c3 = (int64_t)std::ceil((double)tiles3 / (double)num_cus / per_wg);
        // Two-wave workgroups of two blocks: whole multiples of four per CU
        // (eight waves), about 16 column quads each (K = 2048: four per CU
        // within 1% of the fastest grid up to N = 28672, eight at 151936,
        // where four are 4.5% slower; three or six per CU ran 10-15% slower
        // than four).
        if (w3 == 2 && bpl3 == 2)
            c3 = 4 * std::max<int64_t>(1, std::llround((double)tiles3 / ((double)num_cus * 64.0)));
        // With twelve or more column quads per CU, at least two workgroups
        // per CU where one would leave the CU fewer than six waves (three
        // waves of four blocks at 5120 and 6144 x 14336, m = 4 / 6 / 8: 16.1
        // / 19.1 / 19.2 -> 14.1 / 17.4 / 17.8 us and 16.8 / 20.2 / 20.3 ->
        // 15.2 / 19.4 / 19.8; four waves at 8192 x 14336 m = 4 18.4 -> 18.2,
        // m = 6 and 8 1% slower; six waves of two at 6144 x 14336 ran 1-7%
        // faster at one per CU).
        if (tiles3 >= 12 * num_cus && c3 < 2 && w3 < 6) c3 = 2;
        // One or two rows stage their activations with the lanes' own loads,
        // half of which read nothing: two workgroups per CU at least (4096 x
        // 4096 m = 2 5.72 -> 5.22 us, 8192 x 8192 12.0 -> 11.1).
        if (m <= 2 && c3 < 2) c3 = 2;
        if (c3 < 1) c3 = 1;
        if (c3 > per_cu3) c3 = per_cu3;
        int64_t wgs3 = c3 * num_cus;
        if (wgs3 > ceil_div(tiles3, 2)) wgs3 = ceil_div(tiles3, 2);
        plan->engine = 3;
        plan->waves_per_wg = (int32_t)w3;
        plan->blocks_per_lane = (int32_t)bpl3;
        plan->cols_per_tile = 4;
        plan->a_via_lds = m >= 3 && (K > 8192 || N > 8192);
        plan->workgroups = (int32_t)(wgs3 < 1 ? 1 : wgs3);
        return mnb_plan_check(m, K, N, plan) == MNB_OK ? MNB_OK : MNB_ERR_PLAN;
    }

    // 1. Lane split -- a function of (m, K) only, so the fp32 summation order
    //    of a column never depends on N or on the device (column shards of
    //    one matrix give the bits of the whole).
    //    m = 1: two blocks per lane, so a 4096-long K is one wave per column.
    //    m > 1: one block per lane (activation VGPRs grow with m), whole waves
    //    per column up to 8, then K chunks.
    const int64_t bpl_pref = m == 1 ? 2 : 1;
    int64_t lpc, bpl;
    if (ceil_div(nb, bpl_pref) <= 64) {
        lpc = pow2_ceil(ceil_div(nb, bpl_pref));
        if (lpc < 16) lpc = 16;
        bpl = pow2_ceil(nb == 0 ? 1 : ceil_div(nb, lpc));
    } else {
        lpc = 64 * ceil_div(ceil_div(nb, bpl_pref), 64);
        if (lpc > 512) lpc = 512;
        bpl = pow2_ceil(ceil_div(nb, lpc));
        if (bpl > bmax) bpl = bmax;
    }

    // Two or more rows whose K the lane split cannot cover in one pass (eight
    // waves of one to four blocks per lane, as registers allow: K > 16384 at
    // five to eight rows, K > 32768 at three or four): the chunked passes
    // take one tile at a time and reload the activations per chunk (K =
    // 28672, N = 4096, m = 8: 178 us against 26 at m = 4), so the prefill
    // tiles run instead, K split over workgroups, priced by the prefill cost
    // model (that shape 31.8 us; 28672 x 8192 m = 8 345 -> 52.4, 20480 x 8192
    // 320 -> 44.4, 65536 x 4096 342 -> 59.2).  Whether this happens depends
    // on (m, K) only; which tiling runs then depends on N and the CUs, as
    // for m > 8.
    if (m >= 2 && nb > 0 && ceil_div(nb, lpc * bpl) > 1)
        return prefill_plan(cheapest_prefill(m, K, N, num_cus, false).t, m, K, N, num_cus, wgs_per_cu, plan);

    // 2. Column tile: two columns per lane group in a wave; one column per
    //    multi-wave group, whose waves then keep the next column's loads in
    //    flight (measured on the down-projection shape).
    int64_t nc = lpc <= 64 ? (bpl >= 4 ? 1 : 2) : 1;
    while (nc > 1 && (nc * bpl > 8 || nc * m > 32)) nc /= 2;

    // 3. Grid.  Tiles are dealt round-robin, so all lane groups sweep the
    //    weights as one front.  In-wave groups: about five tiles per group,
    //    in whole rounds of the CU count, between half and three times one
    //    resident generation of workgroups (measured best on the lm_head
    //    and gate_up shapes).  Multi-wave groups: whole workgroups per CU,
    //    about eight waves per CU (more tiles per workgroup share its
    //    activation fetch).  Measured at m = 1 on 11 shapes with K from 6144
    //    to 28672 against half a resident generation (2.5 four-wave
    //    workgroups per CU, which leaves the CUs uneven): the down projection
    //    10.39 -> 9.57 us, 8192 x 14336 14.52 -> 13.69, 16384 x 16384 29.32
    //    -> 26.28; best or within 1% of the best count on eight of the 11,
    //    4.7% from it on the other three.
    const bool inwave = lpc <= 64;
    const int64_t gpw = inwave ? 256 / lpc : 1;
    const int64_t waves_per_wg = inwave ? 4 : lpc / 64;
    const int64_t per_cu = wgs_per_cu > 0 ? wgs_per_cu
                                          : (kTargetWavesPerCu + waves_per_wg - 1) / waves_per_wg;
    const int64_t resident = per_cu * num_cus;
    // Too few columns to give half a resident generation one tile per lane
    // group: one column per tile doubles the groups at work (the 4096-column
    // shape: 4.56 -> 4.36 us).
    while (inwave && nc > 1 && ceil_div(ceil_div(N, nc), gpw) < resident / 2) nc /= 2;
    const int64_t tiles = ceil_div(N, nc);
    int64_t wgs = resident / 2 > num_cus ? resident / 2 : num_cus;
    if (!inwave) {
        int64_t c = (8 + waves_per_wg / 2) / waves_per_wg;   // ~8 waves per CU
        if (c > per_cu) c = per_cu;
        if (c < 1) c = 1;
        wgs = c * num_cus;
    }
    if (inwave) {
        wgs = num_cus * ceil_div(ceil_div(tiles, 5 * gpw), num_cus);   // whole rounds of CUs
        const int64_t lo = resident / 2 > 0 ? resident / 2 : 1;
        if (wgs < lo) wgs = lo;
        if (wgs > 3 * resident) wgs = 3 * resident;
        // One tile per lane group fits in one resident generation: take it.
        if (ceil_div(tiles, gpw) <= resident) wgs = ceil_div(tiles, gpw);
    }
    if (!inwave) {
        // Multi-wave groups: enough workgroups that every wave's partial sums
        // of all of a group's tiles fit the deferred-sum LDS.
        const int64_t slot = waves_per_wg * nc * m * 4;
        const int64_t tmax = mnb::kDeferLdsBytes / slot;
        const int64_t need = ceil_div(tiles, tmax < 1 ? 1 : tmax);
        if (wgs < need) wgs = need;
    }
    if (wgs > ceil_div(tiles, gpw)) wgs = ceil_div(tiles, gpw);

    plan->engine = 0;
    plan->lanes_per_col = (int32_t)lpc;
    plan->blocks_per_lane = (int32_t)bpl;
    plan->cols_per_tile = (int32_t)nc;
    plan->waves_per_wg = 0;
    plan->workgroups = (int32_t)(wgs < 1 ? 1 : wgs);
    plan->interleave = 1;
    return mnb_plan_check(m, K, N, plan) == MNB_OK ? MNB_OK : MNB_ERR_PLAN;
}

int matmul_nbits(const void* A, int a_dtype, int64_t m, int64_t K, int64_t N,
                 const uint8_t* Bpacked, const uint16_t* scales,
                 const uint8_t* zero_points, int block, void* out, int out_dtype,
                 void* stream)
{
    return run(A, a_dtype, m, K, N, Bpacked, scales, zero_points, block, out, out_dtype,
               stream, nullptr);
}

int matmul_nbits_noalloc(const void* A, int a_dtype, int64_t m, int64_t K, int64_t N,
                         const uint8_t* Bpacked, const uint16_t* scales,
                         const uint8_t* zero_points, int block, void* out, int out_dtype,
                         void* stream)
{
    return run(A, a_dtype, m, K, N, Bpacked, scales, zero_points, block, out, out_dtype,
               stream, nullptr, true);
}

int matmul_nbits_planned(const void* A, int a_dtype, int64_t m, int64_t K, int64_t N,
                         const uint8_t* Bpacked, const uint16_t* scales,
                         const uint8_t* zero_points, int block, void* out, int out_dtype,
                         void* stream, const mnb_plan* plan)
{
    if (!plan) return MNB_ERR_NULL;
    return run(A, a_dtype, m, K, N, Bpacked, scales, zero_points, block, out, out_dtype,
               stream, plan);
}

int mnb_repack_weights(const uint8_t* src, int src_layout, uint8_t* dst, int dst_layout,
                       int64_t N, int64_t K, void* stream)
{
    auto known = [](int l) { return l == MNB_LAYOUT_NATURAL || l == MNB_LAYOUT_EVEN_ODD; };
    if (!known(src_layout) || !known(dst_layout)) return MNB_ERR_LAYOUT;
    if (K < 0 || N < 0 || K % 32 || K > MNB_MAX_K || N > INT32_MAX) return MNB_ERR_SHAPE;
    const int64_t bytes = N * (K / 2);
    if (bytes == 0) return MNB_OK;
    if (!src || !dst) return MNB_ERR_NULL;
    if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return MNB_ERR_ALIGN;
    if (dst != src && overlaps(src, bytes, dst, bytes)) return MNB_ERR_ALIAS;
    const int e = mnb::launch_repack(src, src_layout, dst, dst_layout, bytes / 4, stream);
    if (e != 0) {
        t_last_hip_error = e;
        return MNB_ERR_HIP;
    }
    g_launches.fetch_add(1, std::memory_order_relaxed);
    return MNB_OK;
}

void mnb_counters_get(mnb_counters* out)
{
    if (!out) return;
    out->calls = g_calls.load();
    out->launches = g_launches.load();
    out->elements_f16 = g_f16.load();
    out->elements_bf16_direct = g_bf16.load();
    out->row_batched_launches = g_rows.load();
}

void mnb_counters_reset(void)
{
    g_calls = 0;
    g_launches = 0;
    g_f16 = 0;
    g_bf16 = 0;
    g_rows = 0;
}

int mnb_get_kernel_info(int64_t m, int64_t K, const mnb_plan* plan, mnb_kernel_info* info)
{
    if (!plan || !info) return MNB_ERR_NULL;
    mnb_plan p = *plan;
    if (p.workgroups < 1) p.workgroups = 1;
    if (mnb_plan_check(m, K, 1, &p) != MNB_OK) return MNB_ERR_PLAN;
    int e = mnb::kernel_info(p.engine == 2 ? m : std::min<int64_t>(m, MNB_MAX_M), K, p, info);
    if (e == -1) return MNB_ERR_PLAN;
    if (e != 0) {
        t_last_hip_error = e;
        return MNB_ERR_HIP;
    }
    return MNB_OK;
}

const char* mnb_status_string(int status)
{
    switch (status) {
    case MNB_OK: return "ok";
    case MNB_ERR_NULL: return "a required pointer is NULL";
    case MNB_ERR_SHAPE: return "bad shape (K must be a non-negative multiple of 32, N >= 0, within limits)";
    case MNB_ERR_BLOCK: return "block size must be 32";
    case MNB_ERR_DTYPE: return "dtype must be MNB_F16 or MNB_BF16";
    case MNB_ERR_ALIGN: return "A and Bpacked must be 16-byte aligned, scales and out 2-byte aligned";
    case MNB_ERR_M_RANGE: return "m must be in [0, MNB_MAX_ROWS]";
    case MNB_ERR_HIP: return "HIP runtime error (see mnb_last_hip_error)";
    case MNB_ERR_ALIAS: return "out overlaps an input";
    case MNB_ERR_PLAN: return "launch plan not supported";
    case MNB_ERR_LAYOUT: return "unknown weight layout";
    case MNB_ERR_WORKSPACE: return "the plan needs more workspace than matmul_nbits_noalloc's fixed buffer holds";
    }
    return "unknown status";
}

int mnb_last_hip_error(void) { return t_last_hip_error; }

int mnb_abi_version(void) { return MNB_ABI_VERSION; }

}  // extern "C"
