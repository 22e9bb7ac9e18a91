// k_static.hip -- the fixed scratch array of msr_chunkwise_noalloc: device
// memory for the chunkwise form's scratch (operand fragments, GroupNorm
// partials, segment states) for callers that cannot allocate (code under
// HIP graph capture, tight serving loops).  Each GPU the library runs on
// holds its own copy of the array until the process ends; every
// msr_chunkwise_noalloc call on that GPU uses it, so calls that overlap on
// one GPU race.  No kernel reads scratch it has not written in the same
// call, so the array needs no clearing between calls.
#include <mutex>

#include "msr_internal.hpp"

namespace {

__device__ __attribute__((aligned(256))) unsigned char scratch[MSR_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices] = {};
std::once_flag g_once[kMaxDevices];
hipError_t g_status[kMaxDevices] = {};

}  // namespace

// The device address of this GPU's copy of the array, looked up once per
// device with that device current (the array's name is a host-side stand-in,
// not a device address).
hipError_t static_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev] {
        void *p = nullptr;
        g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
    });
    *ptr = g_scratch[dev];
    return g_status[dev];
}
