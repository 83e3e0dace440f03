// noalloc.hip -- the static device array behind hla_forward_chunked_noalloc
// (hla_api.cpp): the chunked forward with its workspace in this array instead
// of a caller's buffer, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// The array `scratch` below is file-scope device storage: each GPU the
// library runs on holds its own copy, at its own address, from the first
// call until the process ends.  Host code never uses the array's name as a
// device address: at the first call on a device (with that device current)
// hipGetSymbolAddress yields that device's address, which is kept per device
// and is the only form in which the array reaches the kernels.
//
// Contents.  The first kCtrlBytes are the forward's control block (a
// finished-workgroup counter, the launch epoch, segment tickets and counters
// of the one-launch kernels).  It must be zero before the
// first launch; static storage is zero-initialised when the code object is
// loaded, and every launch leaves the block valid for the next, so nothing is
// cleared here (clearing it again would restart the launch epochs, and a
// wait could then take a flag left by an earlier call for a fresh one).  The
// next kNoallocFlagBytes hold the one-launch kernels' flags and nothing
// else, whatever the params of each call, so a flag only ever holds the epoch
// of an earlier launch (never a partial sum that happens to equal the running
// launch's epoch).  The rest holds per-call partial sums that every call
// writes before it reads them.  Calls on one GPU share the array: calls that
// overlap in time on that GPU (two streams, two threads) race and must not be
// made.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices];  // per device: the address of that device's copy of `scratch`

}  // namespace

hla_status noalloc_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(HLA_ERR_DEVICE, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return set_error(HLA_ERR_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return set_error(HLA_ERR_DEVICE, e != hipSuccess ? hipGetErrorString(e) : "no scratch address");
        g_ptr[dev] = ptr;
    }
    *out = g_ptr[dev];
    return HLA_OK;
}

}  // namespace hla
