// Fixed device working memory of ersj_fill_pass_noalloc, the fill pass for
// callers that cannot allocate device memory.
//
// The array lives in the code object: every GPU the library runs on holds
// its own copy, at its own address, from module load until the process
// ends.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in for the symbol); the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current
// and kept here.  All calls on one GPU share the array and find the last
// call's contents in it; calls that overlap on one GPU race.
#include "ersj_internal.h"

#include <mutex>

namespace ersj {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(int dev, void **out)
{
    *out = nullptr;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev) return hipErrorInvalidDevice;  // the caller makes dev current
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace ersj
