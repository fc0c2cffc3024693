// Internal interface between the host front end (mnb_api.cpp, plain C++)
// and the HIP side (mnb_gemv.hip).  Not installed; not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mnb.h"

namespace mnb {

struct GemvArgs {
    const void* A;
    const uint8_t* B;
    const uint16_t* scales;
    const uint8_t* zp;      // may be null: every zero point is 8
    void* out;
    int64_t m, K, N;
    int a_bf16, out_bf16;
    void* ws;               // device workspace of workspace_bytes(), or null
};

// Queue one GEMV launch.  `plan` has passed mnb_plan_check.  Returns the
// hipError_t of the launch (0 on success).  Dispatches on plan.engine.
int launch_gemv(const GemvArgs& args, const mnb_plan& plan, void* stream);

// The 4x4x4 MFMA kernel (engine 3), mnb_gemv_mfma4.hip: W waves per
// workgroup whose 16 W lane groups cover K in one pass (16 W * blocks_per_lane
// >= K/32), cols_per_tile = 4 or 8.  With plan.a_via_lds, dynamic LDS of 4160
// bytes per wave, through which the activations reach their lanes.
int launch_mfma4(const GemvArgs& args, const mnb_plan& plan, void* stream);
int mfma4_workgroups_per_cu(int64_t m, int64_t K, const mnb_plan& plan);
int mfma4_kernel_info(int64_t m, int64_t K, const mnb_plan& plan, mnb_kernel_info* info);

// The prefill kernel (engine 2), mnb_gemm_mfma.hip: a workgroup of 4 or 8
// waves owns 32 * row_tiles rows by cols_per_tile columns (4 waves: 128 or
// 256 columns, 32 or 64 per wave; 8 waves: 256 columns, 32 per wave).
// A workgroup's activation rows (32 * row_tiles rows of K fp16) are
// addressed with 32-bit buffer offsets: 64 * row_tiles * K must stay within
// this many bytes.
constexpr uint64_t kPrefillRowBlockBytes = 0xFFFFFFF0u;
// With plan.k_splits > 1 the workgroups each take one of k_splits slices of
// K and leave fp32 partial sums in args.ws; a second launch adds them in
// slice order and stores the narrowed result.
int launch_gemm(const GemvArgs& args, const mnb_plan& plan, void* stream);
int gemm_workgroups_per_cu(const mnb_plan& plan);
int gemm_kernel_info(const mnb_plan& plan, mnb_kernel_info* info);
size_t gemm_lds_bytes(const mnb_plan& plan);

// Weight-layout conversion (mnb_layout.hip): `words` 32-bit words of packed
// weights from src_layout to dst_layout.  Returns a hipError_t.
int launch_repack(const uint8_t* src, int src_layout, uint8_t* dst, int dst_layout, int64_t words,
                  void* stream);

// Device workspace a launch under `plan` needs for m x N outputs: the fp32
// partial sums of a K split over workgroups (k_splits x m x N x 4 bytes),
// else 0.  Host-only arithmetic (mnb_api.cpp).
size_t workspace_bytes(int64_t m, int64_t N, const mnb_plan& plan);

// The library's workspace for launches on `stream` (a buffer per device and
// stream, kept for the process and grown with hipMalloc when a call needs
// more): on success (0) the buffer is held until workspace_release(), which
// must follow once the launches that use it are queued; otherwise a
// hipError_t and nothing is held.
int workspace_acquire(size_t bytes, void* stream, void** ptr);
void workspace_release();

// The fixed workspace of matmul_nbits_noalloc: a file-scope device array of
// kScratchBytes in mnb_gemv.hip, one per device for the life of the process.
// Its device address on the current device, looked up (hipGetSymbolAddress)
// on the first call per device.  Returns a hipError_t.
constexpr size_t kScratchBytes = MNB_MAX_SPLIT_WORKSPACE;
int scratch_address(void** ptr);

// Compute units of the current device.  Returns a hipError_t.
int current_device_cus(int* num_cus);

// Occupancy-limited workgroups per CU of kernel `fn` at a block size and
// dynamic LDS size (0 if the query fails).  Cached per (device, kernel,
// threads, LDS).
int occupancy(const void* fn, int threads, size_t lds);

// Occupancy-limited workgroups per CU for the kernel a plan selects, with
// the LDS it needs for N columns (0 if the query fails).
int workgroups_per_cu(int64_t m, int64_t K, int64_t N, const mnb_plan& plan);

// Dynamic LDS of a lane-split launch (engine 0) over N columns.  Multi-wave
// groups keep every wave's partial sums of all their tiles in LDS and sum
// them over waves once, at the end (*tcap = tiles per group), when that
// fits kDeferLdsBytes; otherwise they sum after each tile through two
// slots (*tcap = 0).  One-wave groups with K in one pass stage the
// workgroup's activations (m * blocks_per_lane * 4 KB); groups inside a
// wave need none.  Host-only.
constexpr int64_t kDeferLdsBytes = 48 * 1024;
int64_t gemv_lds_bytes(int64_t m, int64_t N, const mnb_plan& plan, int32_t* tcap);

// Code-object facts of the variant (m, K and the plan select it).  Returns a hipError_t, or -1 when no
// variant matches.
int kernel_info(int64_t m, int64_t K, const mnb_plan& plan, mnb_kernel_info* info);

}  // namespace mnb
