// Library-owned scratch memory for the entry point that allocates nothing
// (svga_sparse_attn_fwd_noalloc): the persistent launch's work counter and
// split-tail region live in one file-scope device array instead of a
// caller-owned workspace.
//
// In host code `scratch` names a host-side stand-in, not device memory; its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever handed to kernels.
#include <atomic>
#include <mutex>

#include "svga_internal.h"

namespace svga {

namespace {

static __device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace svga
