// The allocation-free forward entry point (fibattn_fwd_noalloc): fibattn_fwd with its workspace in
// a file-scope device array instead of caller-provided memory, for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops that forbid allocation).
//
// The array lives in this code object: each GPU the library runs on holds its own copy, of
// kScratchBytes, until the process ends. Host code never passes the array's name to a kernel (in
// host code the name is a host-side stand-in, not a device address): the device address is taken
// once per device with hipGetSymbolAddress, with that device current, and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fibattn.h"
#include "fibattn_internal.h"

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(32) << 20;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` per device, once resolved

// The device address of this device's copy of `scratch` (resolved on the first call on a device).
hipError_t scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t fibattn_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

fibattn_status_t fibattn_fwd_noalloc(const void* q, const void* k, const void* v, double alpha, int32_t W,
                                     const int32_t* offsets, int32_t K, int32_t B, int32_t L, int32_t Hq,
                                     int32_t Hkv, int32_t D, int32_t dtype, double rope_theta, void* o,
                                     float* lse, void* stream) {
    const size_t need = fibattn_fwd_workspace_bytes(B, L, Hkv, D, dtype);
    if (need > kScratchBytes) {
        // argument errors come first, as fibattn_fwd reports them (with no workspace nothing is
        // queued); a valid call that needs more than the array holds is a workspace error
        const fibattn_status_t st = fibattn_fwd(q, k, v, alpha, W, offsets, K, B, L, Hq, Hkv, D, dtype, rope_theta,
                                                o, lse, nullptr, 0, nullptr);
        if (st != FIBATTN_ERR_WORKSPACE) return st;
        return static_cast<fibattn_status_t>(fibattn::report_error(FIBATTN_ERR_WORKSPACE,
                                     "the allocation-free forward needs %zu bytes of scratch; it holds %zu per GPU "
                                     "(use fibattn_fwd with a workspace of its own)",
                                     need, kScratchBytes));
    }
    void* ws = nullptr;
    const hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess)
        return static_cast<fibattn_status_t>(
            fibattn::report_error(FIBATTN_ERR_HIP, "allocation-free forward scratch: %s", hipGetErrorString(e)));
    return fibattn_fwd(q, k, v, alpha, W, offsets, K, B, L, Hq, Hkv, D, dtype, rope_theta, o, lse, ws, kScratchBytes,
                       stream);
}

}  // extern "C"
