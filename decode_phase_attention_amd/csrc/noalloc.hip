// The fixed device scratch behind la_decode_noalloc, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array below is a device symbol: in host code its name stands for a
// host-side shadow, not for device memory, so host code never passes it to a
// kernel or a copy. Its device address is looked up once per device with
// hipGetSymbolAddress (each GPU holds its own copy at its own address) and
// only that address is used from then on.

#include <hip/hip_runtime.h>

#include <mutex>

#include "noalloc.h"

namespace {

static __device__ __align__(256) unsigned char scratch[la::kScratchBytes];

std::mutex g_mu;
void* g_base[la::kMaxDevices];

// Zero `n` words: the control block and the flags at set-up.
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

}  // namespace

namespace la {

hipError_t scratch_setup(int dev, hipStream_t stream, void** base) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_base[dev] == nullptr) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        // Static storage starts zeroed; clearing the words that the exchange
        // protocol reads before writing (exit count, epoch, flags) makes the
        // start state explicit. A fill kernel rather than a memset, so that
        // a first call under graph capture records a kernel node.
        uint32_t* words = static_cast<uint32_t*>(p);
        int n = (int)(kScratchPartOff / sizeof(uint32_t));
        void* args[] = {&words, &n};
        e = hipLaunchKernel((const void*)&clear_words_kernel, dim3(1), dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
        g_base[dev] = p;
    }
    *base = g_base[dev];
    return hipSuccess;
}

void* scratch_base(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    return g_base[dev];
}

}  // namespace la
