// kdn_noalloc.hip -- kdn_forward_noalloc: the layer forward with its
// workspace in a static device array instead of a caller-provided buffer, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` is KDN_NOALLOC_SCRATCH_BYTES of device memory that every
// GPU the library runs this entry point on holds until the process ends.  Its
// device address is obtained once per device, with that device current, by
// hipGetSymbolAddress on the first call on the device; host code uses only
// that address (the array's name in host code is a host-side stand-in, not a
// device address).  Every call on a GPU shares that GPU's array: calls that
// overlap on one GPU (two streams, two threads) race on it.  The forward
// ignores the workspace's contents on entry, so nothing is cleared.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kdn.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// the device address of this device's copy of `scratch` (NULL on failure)
void* scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

size_t kdn_noalloc_scratch_bytes(void) { return KDN_NOALLOC_SCRATCH_BYTES; }

kdn_status kdn_forward_noalloc(const kdn_desc* d, const void* q, const void* k, const void* v,
                               const void* a, const void* qnoise, const void* r,
                               const float* lambda0, const float* S0, void* o, float* S_T,
                               float* lambda_T, void* stream) {
    const kdn_status st = kdn_validate(d);
    if (st != KDN_OK) return st;
    if (kdn_forward_workspace_bytes(d) > KDN_NOALLOC_SCRATCH_BYTES) return KDN_ERR_WORKSPACE;
    void* ws = scratch_address();
    if (!ws) return KDN_ERR_HIP;
    return kdn_forward(d, q, k, v, a, qnoise, r, lambda0, S0, o, S_T, lambda_T, ws,
                       KDN_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
