// decode_scratch.hip - device scratch for decode callers that cannot allocate.
//
// swa_decode_append_static takes no workspace: the split partials of its long-window decode
// live in this file-scope array instead, 4 MiB, one copy on each GPU the library runs on,
// held until the process ends. In host code the array's name stands for no device address:
// decode_scratch() looks the address up once per device with hipGetSymbolAddress (with that
// device current) and only that address reaches kernels. Every call on a GPU shares that
// GPU's copy, so such calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "swa_kernels.hpp"

constexpr size_t DECODE_SCRATCH_BYTES = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[DECODE_SCRATCH_BYTES];

namespace swa {

size_t decode_scratch_bytes() { return DECODE_SCRATCH_BYTES; }

hipError_t decode_scratch(void **ptr) {
    constexpr int MAX_DEV = 64;
    static std::atomic<void *> addr[MAX_DEV];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace swa
