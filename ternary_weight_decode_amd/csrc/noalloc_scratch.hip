// The static device workspace behind twd_ternary_linear_bf16_noalloc, for
// callers that cannot allocate: one copy per device, held until the process
// ends, and the per-device lookup of its address.
#include <atomic>
#include <mutex>

#include "twd_internal.h"

// The int8 rows and fp32 scales of the largest supported call (TWD_MAX_M
// token rows of TWD_MAX_K), 128 KiB and 64 bytes.  On the host this name is
// a stand-in, not a device address: host code passes only the address
// hipGetSymbolAddress gives for a device.
static __device__ __align__(256) uint8_t scratch[twd::kNoAllocScratchBytes];

namespace twd {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_addr[kMaxDevices];
std::mutex g_mutex;
}  // namespace

twd_status noalloc_scratch(void *stream, void **out) {
    static_assert(sizeof(scratch) == kNoAllocScratchBytes, "scratch size");
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return set_error(TWD_ERR_HIP, "linear_bf16_noalloc: hipGetDevice: %s",
                         hipGetErrorString(e));
    int dev = cur;
    if (stream) {
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
        if (e != hipSuccess)
            return set_error(TWD_ERR_HIP, "linear_bf16_noalloc: hipStreamGetDevice: %s",
                             hipGetErrorString(e));
    }
    if (dev != cur)
        return set_error(TWD_ERR_INVALID_ARG,
                         "linear_bf16_noalloc: the stream runs on device %d, device %d is current",
                         dev, cur);
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(TWD_ERR_UNSUPPORTED, "linear_bf16_noalloc: device %d beyond the first %d",
                         dev, kMaxDevices);
    void *p = g_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_mutex);
        p = g_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            // With device `dev` current: its own copy of the array.
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return set_error(TWD_ERR_HIP, "linear_bf16_noalloc: hipGetSymbolAddress(scratch): %s",
                                 hipGetErrorString(e));
            if (!p)
                return set_error(TWD_ERR_HIP, "linear_bf16_noalloc: no device address for scratch");
            g_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return TWD_OK;
}

}  // namespace twd
