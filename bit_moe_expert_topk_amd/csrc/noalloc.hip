// Scratch for the entry point that allocates nothing (moe_layer_mxfp4_noalloc).
//
// Callers that cannot call hipMalloc -- code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation -- get the fused MoE layer
// with its workspace in a file-scope device array instead of a buffer they
// pass in.  Each GPU the library runs on holds its own copy of the array
// (kNoAllocScratchBytes) until the process ends.  In host code the array's
// name is only a stand-in: its device address is looked up once per device
// with hipGetSymbolAddress and that address is what every launch receives.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace moedec {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_slots[kMaxDevices];

// Zero fill by a kernel (no memset node ever lands in a captured graph).
__global__ void zero_fill_kernel(uint4* p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ScratchSlot& slot = g_slots[dev];
    std::call_once(slot.once, [&] {
        void* p = nullptr;
        hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r == hipSuccess && p == nullptr) r = hipErrorInvalidSymbol;
        if (r == hipSuccess) {
            // The array is zero when the code object loads; clear it once more
            // on the caller's stream unless that stream is being captured
            // (a fill node replayed later would still be harmless: all-zero is
            // the state every launch leaves behind).
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            r = hipStreamIsCapturing(s, &cs);
            if (r == hipSuccess && cs == hipStreamCaptureStatusNone) {
                hipLaunchKernelGGL(zero_fill_kernel, dim3(256), dim3(256), 0, s, static_cast<uint4*>(p),
                                   kNoAllocScratchBytes / sizeof(uint4));
                r = hipGetLastError();
            }
        }
        slot.ptr = (r == hipSuccess) ? p : nullptr;
        slot.err = r;
    });
    if (slot.err != hipSuccess) return slot.err;
    *ptr = slot.ptr;
    return hipSuccess;
}

}  // namespace moedec
