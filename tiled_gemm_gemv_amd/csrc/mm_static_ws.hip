// mm_static_ws.hip -- mm_gemm_f32_ws_static: the K split of mm_gemm_f32_ws with the
// library's own device scratch in place of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The scratch is one file-scope device array, `scratch`, of MM_STATIC_SCRATCH_BYTES; each
// GPU the library runs on holds its own copy, at its own address, for the life of the
// process. Host code never passes the array's name to a kernel (in host code it names a
// host-side stand-in): on a device's first call, with that device current, the array's
// device address is looked up once with hipGetSymbolAddress and kept per device; every
// launch takes that address.
#include <mutex>
#include <stdint.h>
#include <stdio.h>

#include "mm.h"
#include "mm_internal.h"

static_assert(MM_STATIC_SCRATCH_BYTES % 16 == 0, "whole 16-byte lanes");
static __device__ __align__(256) float scratch[MM_STATIC_SCRATCH_BYTES / 4];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float *g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` per device, once looked up

thread_local char g_static_error[256] = "";

int fail(int status, const char *what, hipError_t e = hipSuccess)
{
    if (e != hipSuccess)
        snprintf(g_static_error, sizeof g_static_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    else
        snprintf(g_static_error, sizeof g_static_error, "%s", what);
    return status;
}

// The device address of `scratch` on device `dev` (the current device).
int scratch_on(int dev, float **out)
{
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(e == hipErrorNoDevice ? MM_ERR_NO_DEVICE : MM_ERR_LAUNCH,
                        "hipGetSymbolAddress of the static scratch", e);
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_ptr[dev];
    return MM_OK;
}

}  // namespace

namespace mm {

// Called by mm_gemm_f32_ws_static (mm_api.hip) after its argument checks, for shapes whose
// split needs 1 .. MM_STATIC_SCRATCH_BYTES bytes: finds the device, then launches the split
// with the scratch as its workspace. Returns an mm_status; error text via static_ws_error().
int gemm_split_static_launch(const GemmArgs &a, hipStream_t stream)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(e == hipErrorNoDevice ? MM_ERR_NO_DEVICE : MM_ERR_LAUNCH, "hipGetDevice", e);
    if (dev < 0 || dev >= kMaxDevices) return fail(MM_ERR_INVALID_ARG, "device index above 63");
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return fail(MM_ERR_LAUNCH, "hipStreamGetDevice", e);
        if (sdev != dev) return fail(MM_ERR_INVALID_ARG, "stream belongs to another device than the current one");
    }
    float *ws = nullptr;
    const int st = scratch_on(dev, &ws);
    if (st != MM_OK) return st;
    e = gemm_split_launch(a, ws, stream);
    if (e != hipSuccess) return fail(MM_ERR_LAUNCH, "split gemm launch (static scratch)", e);
    return MM_OK;
}

const char *static_ws_error() { return g_static_error; }

}  // namespace mm
