// noalloc.hip -- conv2d_grad_input_noalloc: fp32 grad_input that allocates
// nothing, for callers that cannot call hipMalloc (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The scratch the fp32 plans need (the weight reordered into the order the
// contraction kernel reads it; the RGB-stem plan needs none) lives in one
// file-scope device array per GPU.  Its device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and the looked-up
// pointer -- never the array's host-side name -- is what the kernels receive.
// Every call on a device shares that device's array: calls that can overlap
// on one GPU (different streams without an ordering event) race.  The
// reorder prologue rewrites every element the kernel reads on every call, so
// nothing has to be cleared and nothing is carried between calls.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "api_internal.h"
#include "conv2d_grad_input.h"

namespace {

constexpr size_t kScratchBytes = CONV2D_GI_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
std::map<int, void *> g_ptr;  // device -> device address of `scratch`

// The device address of this device's copy of `scratch`, looked up on the
// first call on that device (the caller's current device).
hipError_t scratch_for(int dev, void **out) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_ptr.find(dev);
    if (it != g_ptr.end()) {
        *out = it->second;
        return hipSuccess;
    }
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = ptr;
    *out = ptr;
    return hipSuccess;
}

}  // namespace

extern "C" {

int conv2d_grad_input_noalloc(const float *grad_out, const float *weight, float *dst,
                              conv2d_gi_params p, hipStream_t stream) {
    const int rc = conv2d_gi_validate(p);
    if (rc != CONV2D_GI_OK) return rc;
    if (!grad_out || !weight || !dst) return CONV2D_GI_EINVAL;
    if (gi::grad_input_f32_scratch_bytes(p) > kScratchBytes) return CONV2D_GI_EUNSUPPORTED;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    void *ptr = nullptr;
    if (e == hipSuccess) e = scratch_for(dev, &ptr);
    if (e != hipSuccess) return gi::record_hip_error(e);
    return gi::grad_input_f32_on_scratch(grad_out, weight, dst, p, stream, ptr, kScratchBytes);
}

}  // extern "C"
