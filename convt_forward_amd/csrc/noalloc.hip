// convt_forward_scratch: convt_forward with its workspace in a fixed device
// array of this library, for callers that cannot allocate device memory.
//
// The array lives in device memory for as long as the library is loaded
// (one copy on each GPU that the library runs on). In host code its name is
// only a stand-in for the symbol: its device address on the current device is
// fetched once per device with hipGetSymbolAddress and kept, and that address
// is what the kernels receive. The entry point makes no allocation call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "convt.h"
#include "convt_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)CONVT_SCRATCH_MAX_BYTES;

// The workspace of convt_forward_scratch on each device. Every byte a
// forward call reads from it is written earlier in the same call (weight
// reorder, tap table, channel-chunked input copy), so no clearing is needed.
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_ptr[kMaxDevices];  // the array's device address per device, once fetched

// The array's address on the current device (nullptr on failure).
void *scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" {

convt_status convt_forward_scratch(convt_plan_t plan, const void *x, const void *w,
                                   const void *bias, void *y, void *stream) {
    if (!plan) return CONVT_ERR_INVALID_ARGUMENT;
    convt_plan_info info;
    if (convt_plan_query(plan, &info) != CONVT_OK) return CONVT_ERR_INVALID_ARGUMENT;
    if (info.workspace_bytes > (int64_t)kScratchBytes) return CONVT_ERR_UNSUPPORTED;
    void *ws = nullptr;
    if (info.workspace_bytes > 0) {
        ws = scratch_on_current_device();
        if (!ws) return CONVT_ERR_DEVICE;
    }
    return convt_forward(plan, x, w, bias, y, ws, stream);
}

int64_t convt_scratch_max_bytes(void) { return (int64_t)kScratchBytes; }

}  // extern "C"
