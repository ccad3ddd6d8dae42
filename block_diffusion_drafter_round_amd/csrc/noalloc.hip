// Device scratch of the allocation-free ctx_features entry point
// (dflash_ctx_features_noalloc), for callers that cannot allocate device
// memory: code under HIP graph capture, tight serving loops.
//
// The scratch is one file-scope device array.  Its name is a host-side
// stand-in in host code, so the host never passes `scratch` itself to a
// kernel or a copy: once per device, with that device current, the array's
// device address is looked up with hipGetSymbolAddress and kept, and only
// that address is used afterwards.  Every GPU the library runs on holds its
// own copy of the array until the process ends.
#include <mutex>

#include "kernels.h"

namespace dfl {
namespace {

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_ptr[MAX_DEVICES];

__global__ void zero_words(unsigned *p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(void **out, hipStream_t stream) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        // The split-K counters must start at zero; the GEMM's last arriver
        // returns each counter to zero, so clearing them once per device is
        // enough.  A fill kernel on the caller's stream (no memset node), so
        // the first call may itself be under graph capture.
        unsigned *cnt = reinterpret_cast<unsigned *>(static_cast<char *>(p) + NOALLOC_PART_BYTES);
        hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, stream, cnt, GEMM_MAX_COUNTERS);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace dfl
