// kernels_peak.hip -- matrix-core peak probe (measurement only).
//
// Every wave issues `iters` rounds of KC independent MFMAs (no instruction
// depends on the one before it within a round, so the matrix core is never
// waiting on a result), on operands built from the lane index and a seed so
// the multipliers see varied bit patterns (a matrix core on zeros draws less
// power and can run at a higher clock than on real data).  The accumulators
// are reduced into one float per work-group so nothing is optimised away.
// Timing it with events gives the rate the chip sustains for that
// instruction at the clock it settles to under that load.  The occupancy
// bound keeps the accumulators in VGPRs: accumulating in AGPRs, this loop
// compiles with copies of the accumulators on every iteration.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "conv2d_grad_input_testing.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int KC = 8;   // independent accumulators per wave

__device__ __forceinline__ unsigned mix(unsigned x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// Operand values of magnitude about 1 with varied mantissas.
__device__ __forceinline__ float val(unsigned h) {
    return __uint_as_float(0x3f800000u | (h & 0x007fffffu)) - 1.5f;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void peak_f32(
    int iters, unsigned seed, float *out) {
    const unsigned t = blockIdx.x * 256 + threadIdx.x;
    float a = val(mix(t ^ seed)), b = val(mix(t * 3u + seed));
    v4f acc[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) acc[k] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < KC; ++k)
            acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[k], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < KC; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
    if (s == 12345.678f) out[blockIdx.x] = s;   // never true in practice; keeps the work
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void peak_bf16(
    int iters, unsigned seed, float *out) {
    const unsigned t = blockIdx.x * 256 + threadIdx.x;
    v8bf a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)val(mix(t * 8u + e + seed));
        b[e] = (__bf16)val(mix(t * 8u + e + 2u * seed + 1u));
    }
    v4f acc[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) acc[k] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < KC; ++k)
            acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < KC; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
    if (s == 12345.678f) out[blockIdx.x] = s;
}

}  // namespace

extern "C" {

int conv2d_gi_mfma_peak_probe(int kind, int workgroups, int iters, float *scratch,
                              hipStream_t stream, double *flops) {
    if ((kind != 0 && kind != 1) || workgroups < 1 || iters < 1 || !scratch || !flops)
        return CONV2D_GI_EINVAL;
    // Flops of one MFMA: 2 * 16 * 16 * K (K = 4 for fp32, 32 for bf16).
    const double per = 2.0 * 16 * 16 * (kind == 0 ? 4 : 32);
    *flops = per * KC * (double)iters * workgroups * 4;   // 4 waves per work-group
    if (kind == 0)
        hipLaunchKernelGGL(peak_f32, dim3(workgroups), dim3(256), 0, stream, iters, 0x9e3779b9u,
                           scratch);
    else
        hipLaunchKernelGGL(peak_bf16, dim3(workgroups), dim3(256), 0, stream, iters, 0x9e3779b9u,
                           scratch);
    return hipGetLastError() == hipSuccess ? CONV2D_GI_OK : CONV2D_GI_EHIP;
}

}  // extern "C"
