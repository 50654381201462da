// The library's own device scratch for mla_decode_noalloc: a file-scope
// array in device memory (one copy per GPU, held until the process ends), so
// that a caller that cannot allocate needs no workspace of its own.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kMaxScratchDevices = 64;

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

}  // namespace

// The scratch array's device address on the current device. The array's name
// is a host-side stand-in in host code; its address on each GPU comes from
// the runtime, once per device, with that device current.
int32_t noalloc_scratch(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return MLA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MLA_OK;
}

}  // namespace mla
