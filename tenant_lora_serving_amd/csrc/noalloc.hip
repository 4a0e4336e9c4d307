// noalloc.hip -- the library's own fixed device buffer, the workspace of
// lora_delta_fused_noalloc for callers that cannot allocate (code under graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The buffer is a file-scope __device__ array: static storage, so it is zero
// when the code object loads, which is the state a fused workspace needs
// before its first call (its control line's last call tag is then 0).  Each
// GPU the library runs on holds its own copy until the process ends.  In
// host code the array's name is not a device address: its address on the
// current device comes from hipGetSymbolAddress, resolved once per device
// (with that device current) and kept here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lora.h"
#include "kernels.h"

namespace tl {

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[LORA_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void *g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(int device, void **ptr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[device] = p;
    }
    *ptr = g_addr[device];
    return hipSuccess;
}

}  // namespace tl
