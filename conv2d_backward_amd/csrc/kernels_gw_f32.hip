// kernels_gw_f32.hip -- fp32 gradient of a 2-D convolution with respect to
// its weight, for gfx950.
//
// The result is the [outChannels, inChannels, kernelH, kernelW] tensor the
// computeGradWeight branch of doppler conv2d_backward.js produces from
// gradOutput and the forward input; its shader is not on the pages, so this
// is the derivative of the forward mapping (an output pixel oh reads input
// row oh*stride - pad + kh):
//
//   dw[co,ci,kh,kw] = sum over n, oh, ow of g[n,co,oh,ow] * x[n,ci,ih,iw],
//   ih = oh*stride - pad_h + kh, iw = ow*stride - pad_w + kw (x = 0 outside).
//
// As a GEMM: M = Co, N = (ci, kh, kw), K = (n, oh, ow) pixels, so K is long
// and the result small.  The pixels are cut into groups (RPC output rows of
// one image) and the groups into slices; work-group (slice, 64 co, 16 ci,
// kernel rows [kh0, kh0+khg)) sums its slice into part[slice], and a second
// kernel adds the slices in a fixed order (the result does not depend on
// scheduling).
//
// Per group, a two-stage LDS pipeline of direct global -> LDS loads holds
//   * grad_out of 64 channels over the group's pixels, laid out
//     [pixel block of 64][co][68] (68 = 64 + 4 floats, so the 16 channel rows
//     of an A fragment fall on different banks), pixel = row*OWP + column
//     with rows padded to OWP = 4*ceil(oW/4) (padding zero);
//   * the input rows the group's taps read for 16 channels, [ci][row][XPM]
//     (CIP floats per channel, CIP = 4 mod 64), column = iw + pad_w.
// V_MFMA_F32_16X16X4_F32 with rows = 16 output channels, columns = 16 input
// channels, k = 4 pixels of one row: lane l = 16g + i supplies
// A[i][g] = grad_out[co_i][pixel 4s + g] and B[g][i] = x[ci_i][that pixel's
// tap position], and receives D[4g + r][i].  Wave w owns output channels
// 16w .. 16w+15 and keeps one accumulator per tap, so a K step reads one A
// fragment and one B fragment per tap; every address is a per-lane constant
// plus a uniform offset.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_common.h"
#include "gi_launch.h"

namespace gi {

typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9)
constexpr int kOOB = 0x7ffffff0;         // byte offset past the end of every buffer
constexpr int kGwPitch = 68;             // LDS floats per channel per 64-pixel block
constexpr int kGwMaxTaps = 16;           // taps per work-group (kernel rows x kW)
constexpr int kGwMaxGM = 4;              // 64-pixel blocks per group

typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (long)bytes, kRsrcWord3);
}

// Direct global -> LDS load: lane i writes 4 bytes at dst + 4i; an
// out-of-range offset writes 0.  dst must be the same for the whole wave.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void *dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 4, voff, 0, 0, 0);
}

// KHG kernel rows per tap group and KW kernel columns at compile time (0:
// read from A, up to kGwMaxTaps taps).
template <int KHG, int KW>
__global__ __launch_bounds__(256) void gi_gw_f32(const GwArgs A) {
    extern __shared__ __attribute__((aligned(16))) float sm[];
    constexpr int TMAX = (KHG > 0 && KW > 0) ? KHG * KW : kGwMaxTaps;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int i = lane & 15, g = lane >> 4;

    // Logical order: tile (co block, ci block, tap group) fastest, then slice:
    // the work-groups of one slice read the same rows.
    const int tiles = A.co_blocks * A.ci_blocks * A.tap_groups;
    const int J = xcd_order(blockIdx.x, gridDim.x);
    const int tile = J % tiles, slice = J / tiles;
    const int tg = tile % A.tap_groups;
    const int cib = (tile / A.tap_groups) % A.ci_blocks;
    const int cob = tile / (A.tap_groups * A.ci_blocks);
    const int co0 = cob * 64, ci0 = cib * 16, kh0 = tg * A.khg;
    const int khg = KHG > 0 ? KHG : A.khg;
    const int kwn = KW > 0 ? KW : A.kW;
    const int T = khg * kwn;
    const int S = A.stride;
    const int oHW = A.oH * A.oW, HW = A.H * A.W;
    const int C4 = (A.oW + 3) / 4;            // K steps per output row
    const int OWP = 4 * C4;                    // padded row length in pixels
    const int gsz = A.GM * 64 * kGwPitch;      // floats of grad_out per stage
    const int stage = gsz + 16 * A.CIP;
    const int g_total = A.N * A.groups_img;
    const int grp0 = slice * A.groups_slice;
    const int ngrp = max(0, min(g_total, grp0 + A.groups_slice) - grp0);
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(A.grad_out, A.g_bytes);
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(A.x, A.x_bytes);

    // grad_out pixel of this lane in each 64-pixel block: padded index
    // 64m + lane -> (row, column); the float offset within the group's first
    // row, or -1 for a padding column.
    int gpix[kGwMaxGM];
#pragma unroll
    for (int m = 0; m < kGwMaxGM; ++m) {
        const int pp = 64 * m + lane;
        const int rr = pp / OWP, c = pp - (pp / OWP) * OWP;
        gpix[m] = (m < A.GM && rr < A.RPC && c < A.oW) ? rr * A.oW + c : -1;
    }
    const int mpr = A.XPM >> 6;   // 64-column blocks per input row

    // Direct loads of group grp into stage buf.  Loads past the slice's last
    // group, outside the image, past the channels or in padding read zeros.
    auto issue = [&](int grp, int buf) {
        float *st = sm + buf * stage;
        const bool live = grp < ngrp;
        const int gg = grp0 + grp;
        const int n = live ? gg / A.groups_img : 0;
        const int oh0 = live ? (gg - n * A.groups_img) * A.RPC : 0;
        const int gbase = (n * A.Co + co0) * oHW + oh0 * A.oW;
        const int rows_left = A.oH - oh0;      // valid rows of this group: RPC at most
        const int nq_g = A.GM * 64;            // one instruction per (block, channel)
        for (int q = wave; q < nq_g; q += 4) {
            const int m = q >> 6, co = q & 63;
            int gp = -1;
#pragma unroll
            for (int mm = 0; mm < kGwMaxGM; ++mm)
                if (mm == m) gp = gpix[mm];
            const bool v = live && gp >= 0 && gp < rows_left * A.oW && co0 + co < A.Co;
            dma4(grs, st + (m * 64 + co) * kGwPitch, v ? (gbase + co * oHW + gp) * 4 : kOOB);
        }
        const int per_ci = A.XR * mpr;
        const int nq_x = 16 * per_ci;          // one instruction per (ci, row, block)
        const int ih0 = oh0 * S - A.pad_h + kh0;
        const int xbase = (n * A.Ci + ci0) * HW;
        float *xs = st + gsz;
        for (int q = wave; q < nq_x; q += 4) {
            const int ci = q / per_ci;
            const int rem = q - ci * per_ci;
            const int xr = rem / mpr, m = rem - (rem / mpr) * mpr;
            const int ih = ih0 + xr, col = 64 * m + lane, iw = col - A.pad_w;
            const bool v = live && ci0 + ci < A.Ci && ih >= 0 && ih < A.H && iw >= 0 &&
                           iw < A.W && col < A.XP;
            dma4(xrs, xs + ci * A.CIP + xr * A.XPM + 64 * m,
                 v ? (xbase + ci * HW + ih * A.W + iw) * 4 : kOOB);
        }
    };

    v4f acc[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    // Per-lane parts of the fragment addresses (floats within a stage).
    const int a_lane = (16 * wave + i) * kGwPitch + g;
    const int b_lane = gsz + i * A.CIP + g * S;
    // Tap offsets within an input channel's rows.
    int toff[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        const int kh = t / kwn, kw = t - (t / kwn) * kwn;
        toff[t] = kh * A.XPM + kw;
    }

    // Two stages: group grp+1 loads while group grp is multiplied.  One
    // stage: the next group loads once every wave is done with this one.
    const bool two = A.stages == 2;
    issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int grp = 0; grp < ngrp; ++grp) {
        const int cur = two ? (grp & 1) : 0;
        if (two) issue(grp + 1, cur ^ 1);
        const float *st = sm + cur * stage;
        for (int rr = 0; rr < A.RPC; ++rr) {
            for (int c4 = 0; c4 < C4; ++c4) {
                const int pp = rr * OWP + 4 * c4;  // uniform: first pixel of the K step
                const float fa = st[a_lane + (pp >> 6) * 64 * kGwPitch + (pp & 63)];
                const float *xb = st + b_lane + rr * S * A.XPM + 4 * c4 * S;
                float fb[TMAX];
#pragma unroll
                for (int t = 0; t < TMAX; ++t)
                    if (t < T) fb[t] = xb[toff[t]];
#pragma unroll
                for (int t = 0; t < TMAX; ++t)
                    if (t < T) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, fb[t], acc[t],
                                                                             0, 0, 0);
            }
        }
        if (!two) {
            __syncthreads();
            issue(grp + 1, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // Partial sums: D[4g + r][i] of tap t -> part[slice][co][ci][kh0 + kh][kw].
    const int kHW = A.kH * A.kW;
    float *pout = A.part + (size_t)slice * A.Co * A.Ci * kHW;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        const int kh = kh0 + t / kwn, kw = t - (t / kwn) * kwn;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int co = co0 + 16 * wave + 4 * g + r, ci = ci0 + i;
            if (t < T && kh < A.kH && co < A.Co && ci < A.Ci)
                pout[((size_t)co * A.Ci + ci) * kHW + kh * A.kW + kw] = acc[t][r];
        }
    }
}

// dw[e] = sum of part[s][e] over the slices, in slice order.
__global__ __launch_bounds__(256) void gw_reduce_f32(const float *__restrict__ part,
                                                     float *__restrict__ dw, int total,
                                                     int slices) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    float s = 0.f;
    for (int k = 0; k < slices; ++k) s += part[(size_t)k * total + e];
    dw[e] = s;
}

}  // namespace

int gw_f32_max_taps() { return kGwMaxTaps; }
int gw_f32_max_blocks() { return kGwMaxGM; }

size_t gw_f32_lds_bytes(const GwArgs &a) {
    return (size_t)a.stages * ((size_t)a.GM * 64 * kGwPitch + 16 * (size_t)a.CIP) *
           sizeof(float);
}

hipError_t launch_gw_f32(const GwArgs &a, hipStream_t s, const KernelEvents &ev) {
    if (a.GM < 1 || a.GM > kGwMaxGM || a.khg * a.kW > kGwMaxTaps || a.CIP % 64 != 4 ||
        a.XPM % 64 != 0 || a.XP > a.XPM || a.CIP < a.XR * a.XPM || a.stages < 1 ||
        a.stages > 2)
        return hipErrorInvalidValue;
    const size_t lds = gw_f32_lds_bytes(a);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const int64_t wgs = (int64_t)a.co_blocks * a.ci_blocks * a.tap_groups * a.slices;
    const dim3 grid((unsigned)wgs), block(256);
    auto go = [&](const void *fn) -> hipError_t {
        if (lds > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    };
    hipError_t e;
    if (a.khg == 3 && a.kW == 3) {
        if ((e = go((const void *)gi_gw_f32<3, 3>)) != hipSuccess) return e;
        hipExtLaunchKernelGGL((gi_gw_f32<3, 3>), grid, block, (uint32_t)lds, s, ev.start,
                              ev.stop, 0, a);
    } else if (a.khg == 1 && a.kW == 7) {
        if ((e = go((const void *)gi_gw_f32<1, 7>)) != hipSuccess) return e;
        hipExtLaunchKernelGGL((gi_gw_f32<1, 7>), grid, block, (uint32_t)lds, s, ev.start,
                              ev.stop, 0, a);
    } else if (a.khg == 2 && a.kW == 7) {
        if ((e = go((const void *)gi_gw_f32<2, 7>)) != hipSuccess) return e;
        hipExtLaunchKernelGGL((gi_gw_f32<2, 7>), grid, block, (uint32_t)lds, s, ev.start,
                              ev.stop, 0, a);
    } else {
        if ((e = go((const void *)gi_gw_f32<0, 0>)) != hipSuccess) return e;
        hipExtLaunchKernelGGL((gi_gw_f32<0, 0>), grid, block, (uint32_t)lds, s, ev.start,
                              ev.stop, 0, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int total = a.Co * a.Ci * a.kH * a.kW;
    hipExtLaunchKernelGGL(gw_reduce_f32, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                          nullptr, nullptr, 0, a.part, a.dw, total, a.slices);
    return hipGetLastError();
}

}  // namespace gi
