// The library's static device scratch: the pre-pass workspace of sa3attn_forward_noalloc,
// for callers that cannot allocate device memory (code under graph capture, serving
// loops that must not call the allocator).
//
// `scratch` is a file-scope device array; each device the library runs on holds its
// own copy (loaded with the code object) until the process ends. Host code never
// passes the array's name to a kernel: in host code that name is a stand-in symbol,
// not a device address. The device address is looked up once per device, with that
// device current, and cached.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "sa3attn_internal.hpp"

namespace sa3 {
namespace {

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

int scratch_device_ptr(void **ptr) {
    *ptr = nullptr;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return -1;
    }
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
                (void)hipGetLastError();
                return -1;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return 0;
}

}  // namespace sa3
