// api_internal.h -- library-internal entry points shared between api.cpp and
// the no-allocation entry point (noalloc.hip).  Not part of the C ABI.
#pragma once

#include <cstddef>

#include <hip/hip_runtime_api.h>

#include "conv2d_grad_input.h"

namespace gi {

// Scratch bytes the fp32 grad_input plan for p needs (0 for an invalid
// shape); host only, no HIP call.
size_t grad_input_f32_scratch_bytes(const conv2d_gi_params &p);

// fp32 grad_input with `scratch` (cap bytes of device memory) in place of the
// per-stream cache: nothing is allocated.  Same status codes as
// conv2d_grad_input; a plan needing more than cap bytes returns
// CONV2D_GI_EUNSUPPORTED before any HIP call.
int grad_input_f32_on_scratch(const float *grad_out, const float *weight, float *dst,
                              const conv2d_gi_params &p, hipStream_t stream, void *scratch,
                              size_t cap);

// Keep e's text for conv2d_gi_last_hip_error (this thread) and return
// CONV2D_GI_EHIP.
int record_hip_error(hipError_t e);

}  // namespace gi
