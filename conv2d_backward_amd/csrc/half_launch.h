// half_launch.h -- launchers of the 16-bit-input kernels for fp16 inputs.
// The bf16 kernels (kernels_halo_bf16.hip, kernels_generic.hip) move raw
// 16-bit patterns through the same prologues and LDS layouts; with fp16
// inputs only their MFMA differs (16x16x32 / 32x32x16 f16, fp32 accumulate).
#pragma once

#include <hip/hip_runtime.h>

#include "gi_common.h"
#include "gi_launch.h"

namespace gi {

hipError_t launch_halo_f16(const HaloBf16Args &a, int cfg, int tiles, int ci_tiles, size_t lds,
                           hipStream_t s, const KernelEvents &ev);
hipError_t launch_generic_f16(const GemmArgs &a, int tiles_x, hipStream_t s,
                              const KernelEvents &ev);

}  // namespace gi
