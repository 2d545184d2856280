// attn_bwd_noalloc: attn_bwd with its workspace in a file-scope device array,
// for callers that cannot allocate device memory (code under stream capture,
// tight serving loops, harnesses that forbid hipMalloc).  The array's device
// address is looked up once per device, on the first call there, and every
// call on that device shares the array: calls on one device must not overlap.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/attn_mi355x.h"
#include "api_error.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];                    // the array's device address on each device
std::mutex g_mu;

// The device address of `scratch` on the current device, or nullptr (with
// attn_last_error() set).  In host code `scratch` names a host-side handle,
// not device memory: only the address hipGetSymbolAddress returns is passed
// to kernels.
void* scratch_on_current_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        attn::report(ATTN_ERR_HIP, "attn_bwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        attn::report(ATTN_ERR_UNSUPPORTED, "attn_bwd_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            attn::report(ATTN_ERR_HIP, "attn_bwd_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t attn_bwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* dO,
                             const float* lse, const float* D, void* dq, void* dk, void* dv, int B,
                             int H, int N, int d, int causal, float scale, void* stream) {
    const size_t need = attn_bwd_workspace_bytes_ex(B, H, H, N, d, causal);
    if (need == 0)                               // empty or invalid: attn_bwd's own checks
        return attn_bwd(q, k, v, dO, lse, D, dq, dk, dv, nullptr, 0, B, H, N, d, causal, scale, stream);
    if (need > kScratchBytes)
        return attn::report(ATTN_ERR_WORKSPACE,
                            "attn_bwd_noalloc: B=%d H=%d N=%d d=%d needs %zu bytes of workspace; the static "
                            "scratch holds %zu",
                            B, H, N, d, need, kScratchBytes);
    void* ws = scratch_on_current_device();
    if (!ws) return ATTN_ERR_HIP;
    return attn_bwd(q, k, v, dO, lse, D, dq, dk, dv, ws, kScratchBytes, B, H, N, d, causal, scale, stream);
}

}  // extern "C"
