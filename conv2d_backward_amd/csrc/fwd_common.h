// fwd_common.h -- arguments and host-side launchers of the forward
// convolution (kernels_fwd_f32.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_common.h"
#include "gi_launch.h"

namespace gi {

// The forward cross-correlation (the mapping stated in the doppler direct
// kernel's comment: output pixel oh reads input row oh*stride - pad + kh):
//
//   y[n,co,oh,ow] = sum over ci, kh, kw of
//                   x[n,ci,oh*stride-pad_h+kh, ow*stride-pad_w+kw] * w[co,ci,kh,kw]
//
// as an implicit GEMM C[co, pixel] = A[co, k] * B[k, pixel] with k = (block
// of 16 input channels, tap, channel in the block): A from the weight
// reordered to wt[(tap*Ci + ci)*Co + co] (co fastest), B gathered from x per
// tap (0 outside the image); pixels of all images folded into the column
// axis.
struct FwdArgs {
    const float *x;    // [N, Ci, H, W]
    const float *wt;   // [kH*kW][Ci][Co] (prologue output)
    const float *zero; // kFwdZeroTail zeros (prologue output): out-of-range lanes load here
    float *y;          // [N, Co, oH, oW]
    int32_t N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH, oW;
};

constexpr int kFwdBM = 64;    // output channels per work-group
constexpr int kFwdBN = 128;   // pixels per work-group
constexpr int kFwdMaxFlatK = 2048;   // most K = Ci*kH*kW of the flattened K order
constexpr int kFwdZeroTail = 16;     // zeros the weight reorders write after the weight

// Weight reorders: w [Co, Ci, kH, kW] -> wt [kH*kW][Ci][Co] for the generic
// forward kernel (followed by kFwdZeroTail zeros: wt must hold
// Co*Ci*kH*kW + kFwdZeroTail floats); and -> wf [Ci][Co][kH][kW] with the
// taps reversed, the weight of the equivalent stride-1 grad_input problem
// (see api.cpp).
hipError_t launch_fwd_weight_tap_ci_co_f32(const float *w, float *wt, int Co, int Ci, int kHW,
                                           hipStream_t s);
hipError_t launch_fwd_weight_flip_f32(const float *w, float *wf, int Co, int Ci, int kHW,
                                      hipStream_t s);
// w [Co][K] -> wt [K][Co] (the flattened K order's A operand), followed by
// kFwdZeroTail zeros.
hipError_t launch_fwd_weight_k_co_f32(const float *w, float *wt, int Co, int K, hipStream_t s);
// Whether the generic kernel takes K in the caller's (ci, kh, kw) order
// (fewer than 16 input channels; its weight then comes from
// launch_fwd_weight_k_co_f32, else from launch_fwd_weight_tap_ci_co_f32).
bool fwd_flat_k(const FwdArgs &a);
// The generic forward kernel: a 1-D grid of ceil(N*oH*oW / kFwdBN) *
// ceil(Co / kFwdBM) work-groups, output-channel tile fastest.
hipError_t launch_fwd_generic_f32(const FwdArgs &a, hipStream_t s, const KernelEvents &ev);

}  // namespace gi
