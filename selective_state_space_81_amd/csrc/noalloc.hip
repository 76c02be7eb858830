// noalloc.hip -- ms_scan_fwd_noalloc: the forward scan for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  The scratch that ms_scan_fwd
// takes as a caller workspace (segment summaries, their decay, the copy of
// h0) comes from a file-scope device array instead; everything else --
// validation, plan, kernels -- is ms_scan_fwd's.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/msscan.h"
#include "msscan_internal.h"

namespace {

// Every GPU the library runs on holds its own copy of this array until the
// process ends.  On the host the name `scratch` is only a stand-in, not a
// device address: host code uses the address hipGetSymbolAddress returns
// for the current device, looked up once per device and kept.
constexpr size_t kScratchBytes = MS_NOALLOC_MAX_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Address of `scratch` on the calling thread's current device.
hipError_t scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = ptr;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

ms_status ms_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                              const void* C, const float* D, const void* z,
                              const float* delta_bias, uint32_t flags, void* y, const float* h0,
                              float* h_last, const ms_dims* dims, void* stream) {
    msscan::clear_error();
    const size_t need = ms_scan_workspace_bytes(dims, flags);
    if (need == (size_t)-1)  // invalid dims or flags: let the checks report which
        return msscan::scan_fwd_checked(u, delta, A, B, C, D, z, delta_bias, flags, y, h0,
                                        h_last, dims, nullptr, 0, stream);
    if (need > kScratchBytes) {
        char text[200];
        snprintf(text, sizeof text,
                 "this scan needs %zu bytes of scratch; ms_scan_fwd_noalloc holds at most %zu "
                 "(call ms_scan_fwd with a workspace instead)",
                 need, kScratchBytes);
        return msscan::report(MS_ERR_UNSUPPORTED, text);
    }
    void* ws = nullptr;
    const hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess) {
        char text[200];
        snprintf(text, sizeof text, "device scratch lookup failed: %s", hipGetErrorString(e));
        return msscan::report(MS_ERR_HIP, text);
    }
    return msscan::scan_fwd_checked(u, delta, A, B, C, D, z, delta_bias, flags, y, h0, h_last,
                                    dims, need ? ws : nullptr, need ? kScratchBytes : 0, stream);
}

}  // extern "C"
