// aqlm_gemv_packed_noalloc: the packed product with its scratch memory in a fixed
// device array of the library, for callers that cannot allocate or pass a workspace
// (code under graph capture that owns no memory pool, tight serving loops, harnesses
// that forbid allocation).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  Its host-side name is only a
// stand-in, so the device address is looked up once per device (with that device
// current) through hipGetSymbolAddress and kept; every kernel receives that address as
// its workspace pointer.  No call here allocates or frees anything.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "aqlm_mi355x.h"
#include "kernels.hpp"

namespace {

constexpr int64_t kScratchBytes = int64_t(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The device address of `scratch` on the current device (looked up on first use).
hipError_t scratch_ptr(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev] {
        void *p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    *out = g_ptr[dev];
    return g_err[dev];
}

}  // namespace

extern "C" {

int64_t aqlm_noalloc_scratch_bytes(void) { return kScratchBytes; }

aqlm_status_t aqlm_gemv_packed_noalloc(const void *packed_codes, const void *packed_codebooks,
                                       const void *x, void *y, int64_t out_features,
                                       int64_t in_features, int K, int B, int batch,
                                       void *stream) {
    const int64_t need = aqlm_workspace_bytes(AQLM_OP_GEMV_PACKED, AQLM_VARIANT_AUTO, packed_codes,
                                              packed_codebooks, x, y, out_features, in_features, K,
                                              B, batch);
    if (need < 0) return AQLM_ERR_INVALID_ARGUMENT;
    if (need > kScratchBytes) {
        char msg[160];
        std::snprintf(msg, sizeof(msg),
                      "aqlm_gemv_packed_noalloc: this call needs %lld bytes of scratch, more "
                      "than the fixed %lld", (long long)need, (long long)kScratchBytes);
        aqlm::set_last_error_message(msg);
        return AQLM_ERR_INVALID_ARGUMENT;
    }
    void *ws = nullptr;
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) {
        char msg[160];
        std::snprintf(msg, sizeof(msg), "aqlm_gemv_packed_noalloc scratch: %s", hipGetErrorString(e));
        aqlm::set_last_error_message(msg);
        return AQLM_ERR_HIP;
    }
    return aqlm_gemv_packed(packed_codes, packed_codebooks, x, y, out_features, in_features, K, B,
                            batch, ws, kScratchBytes, stream);
}

}  // extern "C"
