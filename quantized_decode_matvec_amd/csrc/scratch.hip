// Device-resident scratch memory for the allocation-free fused lm_head +
// argmax entry point (qmatvec_argmax_noalloc). Callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc) get the argmax workspace from this fixed array
// instead of passing one. Each GPU the library runs on holds its own copy of
// the array, at its own address, until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qmv_launch.h"

namespace qmv {

constexpr size_t kScratchBytes = size_t(16) << 20;   // header + y [B][N] fp32 for B * N <= 4,194,272

// Host code never uses this name as an address: it stands for the device
// symbol only, and the device address comes from hipGetSymbolAddress below.
static __device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

size_t scratch_bytes() { return kScratchBytes; }

// Address of this device's copy of `scratch`, looked up once per device (with
// that device current) and cached.
hipError_t scratch_address(void **out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace qmv
