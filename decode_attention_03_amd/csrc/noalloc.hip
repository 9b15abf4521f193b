// noalloc.hip -- the library-owned scratch buffer behind fd_decode_noalloc,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// One file-scope device array of kScratchBytes; every GPU the library runs on
// holds its own copy until the process ends.  In host code the array's name
// is only a host-side stand-in, so the device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept; the
// kernels only ever see that address, as they see a caller's workspace.
//
// Nothing in the scratch needs clearing between calls: every word a decode
// step reads from its workspace is written earlier in the same step (the
// split stage writes every partial and descriptor the combine reads).  Calls
// that overlap on one GPU (several host threads, or several streams) share
// the one array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fd_internal.h"

static __device__ __align__(256) char scratch[fd::kScratchBytes];

namespace fd {

namespace {
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
}  // namespace

hipError_t scratch_buffer(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace fd
