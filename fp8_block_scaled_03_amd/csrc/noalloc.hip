// noalloc.hip -- the weight-gradient GEMM without any allocation: its
// split-K slices live in a static device array instead of a caller
// workspace, for callers that cannot allocate device memory.
//
// The array below is a device symbol.  In host code its name is only a
// host-side stand-in, not a device address, so it is never passed to a
// kernel or a runtime call: the address is looked up with
// hipGetSymbolAddress once per device (each device holds its own copy) and
// that pointer is used everywhere.
#include <mutex>

#include "internal.h"

namespace fp8bs {

// Split-K slices of fp8_gemm_wgrad_noalloc: 128 MiB per device, held from
// the library's first use on the device until the process ends.
constexpr size_t kNoallocScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mutex;

// Device address of this device's copy of `scratch` (the current device),
// looked up on the first call on each device; nullptr if the lookup fails
// (it is then tried again on the next call).
void* scratch_address(int dev) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

hipError_t launch_wgrad_noalloc(const uint8_t* dytq, const float* dyts, const uint8_t* xtq,
                                const float* xts, float* dw, int64_t M, int64_t N, int64_t K,
                                int num_cus, hipStream_t stream, bool* too_big) {
    *too_big = false;
    const size_t need = gemm_workspace_bytes(kScaleRow, N, K, M, num_cus);
    if (need > kNoallocScratchBytes) {
        *too_big = true;
        return hipSuccess;
    }
    void* ws = nullptr;
    if (need > 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        ws = scratch_address(dev);
        if (!ws) return hipErrorInvalidSymbol;
    }
    // The same plan and kernels as fp8_gemm_wgrad given a workspace of the
    // queried size; every slice element is written before it is read, so
    // nothing in the array needs clearing between calls.
    return launch_gemm(kScaleRow, dytq, dyts, xtq, xts, dw, false, N, K, M, ws, need, num_cus,
                       stream);
}

}  // namespace fp8bs
