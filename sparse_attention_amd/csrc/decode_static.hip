// dsa_decode_step_static: the fused decode step with its scratch space in a
// library-owned device array instead of a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It runs exactly the kernels of
// dsa_decode_step on the same arguments; nothing here allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dsa.h"
#include "dsa_internal.h"

// The scratch space: one copy on every GPU the library runs on, held until
// the process ends.  Host code must never pass this name to a kernel or a
// copy (on the host it is only a stand-in for the device symbol); the device
// address comes from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[DSA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's copy of `scratch`, looked up on the first call made
// with that device current and kept for later calls.
hipError_t scratch_address(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" dsa_status_t dsa_decode_step_static(const dsa_decode_args_t* args, hipStream_t stream)
{
    size_t need = 0;
    const dsa_status_t s = dsa::decode_step_check(args, &need);
    if (s != DSA_OK) return s;
    if (need > DSA_STATIC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return DSA_ERR_LAUNCH;
    // The top-k header the step needs zeroed is cleared by the step's first
    // kernel, and every other scratch byte it reads was written earlier in
    // the same step, so what a previous call left behind is never read.
    return dsa_decode_step(args, ws, DSA_STATIC_SCRATCH_BYTES, stream);
}
