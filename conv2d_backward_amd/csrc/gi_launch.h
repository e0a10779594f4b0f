// gi_launch.h -- host-side launchers of the kernels (one per kernel family).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_common.h"

namespace gi {

// Weight reorder prologues.
//   fp32: wt[(tap*Co + co)*Ci + ci] = w[((co*Ci + ci)*kH*kW) + tap]   (ci fastest)
//   bf16: wt[(tap*Ci + ci)*Co + co] = w[((co*Ci + ci)*kH*kW) + tap]   (co fastest)
hipError_t launch_weight_tap_co_ci_f32(const float *w, float *wt, int Co, int Ci,
                                       int kHW, hipStream_t s);
hipError_t launch_weight_tap_ci_co_bf16(const uint16_t *w, uint16_t *wt, int Co,
                                        int Ci, int kHW, hipStream_t s);

// Generic phase-split implicit GEMM (any shape).  Tile: 64 input channels x
// 128 pixels of one phase; grid = (sum of pixel tiles of the launch's phases,
// ceil(Ci/64)).
constexpr int kGenericBM = 64;
constexpr int kGenericBN = 128;
hipError_t launch_generic_f32(const GemmArgs &a, int tiles_x, hipStream_t s);
hipError_t launch_generic_bf16(const GemmArgs &a, int tiles_x, hipStream_t s);

}  // namespace gi
