// Host-only stand-ins for the functions the HIP translation units define,
// so that the host front end (mnb_api.cpp: argument validation, launch
// planning, counters, status strings) can be built with the address and
// undefined-behaviour sanitizers and driven by the CPU tests.  Every entry
// that would touch a device reports that no device is present.
#include "mnb_internal.h"

namespace mnb {

namespace {
constexpr int kNoDevice = 100;   // hipErrorNoDevice
}

int launch_gemv(const GemvArgs&, const mnb_plan&, void*) { return kNoDevice; }
int launch_repack(const uint8_t*, int, uint8_t*, int, int64_t, void*) { return kNoDevice; }
int current_device_cus(int* num_cus)
{
    *num_cus = 0;
    return kNoDevice;
}
int workgroups_per_cu(int64_t, int64_t, int64_t, const mnb_plan&) { return 0; }
int kernel_info(int64_t, int64_t, const mnb_plan&, mnb_kernel_info*) { return kNoDevice; }
int workspace_acquire(size_t, void*, void** ptr)
{
    *ptr = nullptr;
    return kNoDevice;
}
void workspace_release() {}
int scratch_address(void** ptr)
{
    *ptr = nullptr;
    return kNoDevice;
}

}  // namespace mnb
