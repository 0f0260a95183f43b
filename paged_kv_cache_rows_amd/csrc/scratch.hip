// The library's own device scratch, for the entry point that allocates nothing
// (paged_attn_decode_put_static): one file-scope array per GPU, which holds the split partials
// of a call in place of a caller's workspace.
//
// In host code the name `scratch` stands for a host-side shadow, not the device array: its
// device address is looked up once per GPU (hipGetSymbolAddress with that GPU current) and only
// that address is ever handed to kernels.
#include <mutex>

#include "../../include/kvpaged.h"
#include "internal.h"

static __device__ __align__(256) unsigned char scratch[KV_STATIC_SCRATCH_BYTES];

namespace kvp {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void **out, size_t *bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    *bytes = sizeof(scratch);
    return hipSuccess;
}

}  // namespace kvp
