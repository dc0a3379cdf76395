// kla_noalloc.hip -- kla_scan_fwd_noalloc: the forward scan with its
// workspace in a fixed device array of the library, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The look-back workspace of the scan (flags, tile matrices, inclusive
// states; kla_lookback.h) lives in `scratch`, a file-scope device array of
// kScratchBytes.  Each GPU the library runs on holds its own copy from the
// first call on that GPU until the process ends.  Device code reaches it only
// through the address hipGetSymbolAddress returns on that device (the array's
// name in host code is a host-side stand-in, not a device address), taken once
// per device on the device's first call and kept in g_scratch.
//
// The array starts zero-filled (static storage) and the scan's workspace
// protocol leaves it ready for the next call (tags instead of clearing), so
// no call clears or allocates anything.  Every call on a GPU shares that GPU's
// array: calls that overlap in time on one GPU (two streams, two threads)
// race on it and must be serialised by the caller.

#include <mutex>

#include "kla_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// This device's address of `scratch` (resolved on the device's first call).
kla_status scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return kla::fail(KLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxDevices)
        return kla::fail(KLA_ERR_UNSUPPORTED, "device %d is beyond the %d the library tracks", dev,
                         kMaxDevices);
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !ptr)
            return kla::fail(KLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                             hipGetErrorString(err));
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return KLA_OK;
}

}  // namespace

extern "C" {

size_t kla_scan_fwd_noalloc_max_workspace(void) { return kScratchBytes; }

kla_status kla_scan_fwd_noalloc(const void* a, const void* p, const void* phi, const void* b,
                                kla_dtype in_dtype, const float* lam0, const float* eta0,
                                float* lam, float* eta, int64_t B, int64_t H, int64_t T,
                                int64_t D, hipStream_t stream) {
    // Sizes first (no device state is touched for a rejected call); an
    // empty or invalid problem goes straight to kla_scan_fwd's own checks.
    const size_t need = kla_scan_fwd_workspace_size(B, H, T, D, in_dtype);
    if (need > kScratchBytes)
        return kla::fail(KLA_ERR_WORKSPACE,
                         "the problem needs %zu bytes of workspace; kla_scan_fwd_noalloc has %zu "
                         "(use kla_scan_fwd with a caller-owned workspace)",
                         need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        const kla_status st = scratch_of_current_device(&ws);
        if (st != KLA_OK) return st;
    }
    return kla_scan_fwd(a, p, phi, b, in_dtype, lam0, eta0, lam, eta, B, H, T, D, ws,
                        ws ? kScratchBytes : 0, stream);
}

}  // extern "C"
