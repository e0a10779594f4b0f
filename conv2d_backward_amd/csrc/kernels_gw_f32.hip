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

#include <algorithm>

#include "gw_common.h"

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

// out[e] = sum of part[s][e] over the slices (slice stride `total`); the
// elements e >= n0 go to out1[e - n0] instead of out0[e] (the bias sums that
// follow the weight sums).  A work-group takes 64 elements; its four waves
// sum the slices s = w, w+4, w+8, ... in order (eight loads in flight per
// lane), then wave 0 adds the four sums in wave order: a fixed order, so the
// result does not depend on scheduling.
__global__ __launch_bounds__(256) void gw_reduce_f32(const float *__restrict__ part,
                                                     float *__restrict__ out0,
                                                     float *__restrict__ out1, int n0,
                                                     int total, int slices) {
    __shared__ float red[4][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    float s = 0.f;
    if (e < total) {
        int k = w;
        for (; k + 28 < slices; k += 32) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(k + 4 * u) * total + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; k < slices; k += 4) s += part[(size_t)k * total + e];
    }
    red[w][lane] = s;
    __syncthreads();
    if (w == 0 && e < total) {
        const float v = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
        if (e < n0)
            out0[e] = v;
        else
            out1[e - n0] = v;
    }
}

// Per-channel sums of grad_out [N, Co, oH*oW] over images [b*ipb, (b+1)*ipb)
// of each channel: work-group (co, b) writes part[b][co].  Threads stride
// over the pixels of each image in turn; the 256 sums are then added in a
// fixed tree order.
__global__ __launch_bounds__(256) void gw_channel_sum_f32(const float *__restrict__ g,
                                                          float *__restrict__ part, int N,
                                                          int Co, int plane, int ipb) {
    __shared__ float red[256];
    const int co = blockIdx.x, b = blockIdx.y;
    const int n1 = min(N, (b + 1) * ipb);
    float s = 0.f;
    for (int n = b * ipb; n < n1; ++n) {
        const float *gp = g + ((size_t)n * Co + co) * plane;
        for (int p = threadIdx.x; p < plane; p += 256) s += gp[p];
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[(size_t)b * Co + co] = red[0];
}

// ---------------------------------------------------------------------------
// gi_gwd_f32: the same GEMM with 16-byte direct loads and four pixels per
// lane per fragment read.
//
// V_MFMA_F32_16X16X4_F32 with rows = 16 output channels, columns = 16 GEMM
// columns (ci, kh, kw), k = 4 pixels.  A K block is 16 pixels; lane
// l = 16g + i takes pixels g, g+4, g+8, g+12 of it as the k index g of four
// MFMAs, so one lane reads A[co_i] and B[column_i] at four positions 4 floats
// apart (two ds_read2_b32 each).  Per-channel LDS runs have a length that is
// 4 times an odd number: the 16 channels of a fragment start in 16 different
// groups of 4 banks and the lane group g adds g, so a stride-1 read touches
// 64 different banks.
//
// Direct loads move 16 bytes per lane into 16 consecutive LDS bytes per
// lane: the stage is a run of 1 KB pieces, grad_out's channel runs first
// (16*LA pieces, a multiple of 64), then the input channels' runs; each lane
// computes which 16 source bytes land in its piece (zeros where there are
// none).  That needs the pieces to start on 16-byte boundaries of the
// source: in the row-padded layout rows of W and oW floats (multiples of 4);
// in the flat layout the LDS run starts at the 16-byte boundary at or below
// the first float needed, and each lane adds the run's offset (0..3).
//
// Flat layout: pixel f of a group (its rows back to back, W == oW) reads
// input float f + kh'*W + kw - pad_w of the group's first needed row; a tap
// whose column leaves the row reads the neighbouring row's float there, so
// the grad_out value is replaced by zero for that (pixel, kw), as it is for
// pixels past the group's end.  Rows above or below the image read zeros:
// the pieces outside the channel's plane are not loaded (plane_zero), or no
// tap reaches such a row (one kernel row, no row padding).
constexpr int kGwdThreads = 256;

// floor(s / d) for 0 <= s < 2^14 from the packed (m, k) of GwdArgs::d24_*:
// one full-rate 24-bit multiply and a shift.
__device__ __forceinline__ int div24(int s, uint32_t v) {
    return (int)(__umul24((uint32_t)s, v & 0xffffffu) >> (v >> 24));
}
__device__ __forceinline__ int mul24(int a, int b) { return (int)__umul24((uint32_t)a, (uint32_t)b); }

// Direct global -> LDS load of 16 bytes per lane: lane i writes dst + 16i;
// an out-of-range offset writes zeros.  dst is the same for the whole wave.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, voff, 0, 0, 0);
}

// NB column blocks of 16 per wave; KW kernel columns (tap-major map, 0 for
// the flattened map); S stride (0: read from A); FLAT pixel layout; PLAIN
// (flat only): K blocks that no kernel column's mask touches skip the masks.
template <int NB, int KW, int S, bool FLAT, bool PLAIN = false>
__global__ __launch_bounds__(kGwdThreads) void gi_gwd_f32(const GwdArgs A) {
    extern __shared__ __attribute__((aligned(16))) float sm[];
    static_assert(!FLAT || (KW > 0 && S == 1), "flat layout: tap-major map, stride 1");
    static_assert(!PLAIN || FLAT, "the mask bypass is for the flat layout");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int i = lane & 15, g = lane >> 4;
    const int st = S > 0 ? S : A.stride;
    const int kHW = A.kH * A.kW;

    const int tiles = A.co_blocks * A.col_tiles;
    const int J = xcd_order(blockIdx.x, gridDim.x);
    const int tile = J % tiles, slice = J / tiles;
    const int ct = tile % A.col_tiles, cob = tile / A.col_tiles;
    const int co0 = cob * 64;
    int ci_lo, kh0, c0 = 0;
    if (KW > 0) {   // tap-major
        const int cib = ct / A.tap_groups;
        ci_lo = cib * 16;
        kh0 = (ct - cib * A.tap_groups) * A.khg;
    } else {
        c0 = ct * 16 * NB;
        ci_lo = c0 / kHW;
        kh0 = 0;
    }

    // LDS offset of each block's column within the input tile, for this
    // lane's first pixel (lane group g).
    const int rowp = FLAT ? A.W : A.XW;
    int cb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        int seg, khr, kw;
        if (KW > 0) {
            seg = i;
            khr = b / KW;
            kw = b % KW;
        } else {
            const int col = min(c0 + 16 * b + i, A.Ci * kHW - 1);
            const int ci = col / kHW, t = col - (col / kHW) * kHW;
            seg = ci - ci_lo;
            khr = t / A.kW;
            kw = t - khr * A.kW;
        }
        cb[b] = 64 * A.LA + seg * A.LX + khr * rowp + kw +
                (FLAT ? g : A.XO - A.pad_w + g * st);
    }
    const int abase = (16 * wave + i) * A.LA + g;

    const int oHW = A.oH * A.oW, HW = A.H * A.W;
    const int g_total = A.N * A.groups_img;
    const int grp0 = slice * A.groups_slice;
    const int ngrp = max(0, min(g_total, grp0 + A.groups_slice) - grp0);
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(A.grad_out, A.g_bytes);
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(A.x, A.x_bytes);
    const int LA4 = A.LA >> 2, LX4 = A.LX >> 2, OWP4 = A.OWP >> 2, XW4 = A.XW >> 2;
    const int nins = (A.nslots + 63) >> 6;

    // Direct loads of group grp (< ngrp) into stage buf.
    auto issue = [&](int grp, int buf) {
        float *stp = sm + buf * A.stage_floats;
        const int gg = grp0 + grp;
        const int n = gg / A.groups_img;
        const int oh0 = (gg - n * A.groups_img) * A.R;
        const int rows_v = min(A.R, A.oH - oh0);
        const int gplane0 = (n * A.Co + co0) * oHW;
        const int xplane0 = (n * A.Ci + ci_lo) * HW;
        // Row-padded: first input row; flat: first needed float of a plane.
        const int ih0 = oh0 * st - A.pad_h + kh0;
        const int fbase = (oh0 - A.pad_h + kh0) * A.W - A.pad_w;
        // Branch-free per piece, on 24-bit multiplies (operands below 2^24:
        // channel and row counts, planes of fewer than 2^24 pixels); an
        // invalid piece's offset is computed and then replaced by kOOB.
        const int gfirst = oh0 * A.oW;   // flat: the group's first pixel in a plane
        for (int k = wave; k < nins; k += 4) {
            const int s = 64 * k + lane;
            if (k < LA4) {   // grad_out pieces (16*LA of them: whole instructions)
                const int co = div24(s, A.d24_la4), q = s - mul24(co, LA4);
                const int plane = gplane0 + mul24(co, oHW);
                bool ok = co0 + co < A.Co;
                int off;
                if (FLAT) {
                    off = ((plane + gfirst) & ~3) + 4 * q;
                } else {
                    const int r = div24(q, A.d24_owp4), cc = q - mul24(r, OWP4);
                    ok = ok & (r < rows_v) & (4 * cc < A.oW);
                    off = plane + mul24(oh0 + r, A.oW) + 4 * cc;
                }
                dma16(grs, stp + 256 * k, ok ? off * 4 : kOOB);
            } else {         // input pieces
                const int s2 = s - 16 * A.LA;
                const int seg = div24(s2, A.d24_lx4), q = s2 - mul24(seg, LX4);
                const int plane = xplane0 + mul24(seg, HW);
                bool ok = (s2 < A.XC * LX4) & (ci_lo + seg < A.Ci);
                int off;
                if (FLAT) {
                    off = ((plane + fbase) & ~3) + 4 * q;
                    ok = ok & (off >= 0) & ((A.plane_zero == 0) | ((off >= plane) & (off < plane + HW)));
                } else {
                    const int xr = div24(q, A.d24_xw4), cc = q - mul24(xr, XW4);
                    const int ih = ih0 + xr, iw = 4 * cc - A.XO;
                    ok = ok & (xr < A.XR) & (ih >= 0) & (ih < A.H) & (iw >= 0) & (iw < A.W);
                    off = plane + mul24(ih, A.W) + iw;
                }
                dma16(xrs, stp + 256 * k, ok ? off * 4 : kOOB);
            }
        }
    };

    v4f acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = v4f{0.f, 0.f, 0.f, 0.f};
    // Sum of the grad_out values this lane feeds to the MFMAs (padding and
    // past-the-end pixels as zeros): the bias gradient's partial sum.
    float bsum = 0.f;

    // Fragments of one K block: A at stp + ab + ua, B of block b at
    // stp + cbg[b] + ub.
    struct Frag {
        float a[4];
        float b[NB][4];
    };
    auto load = [&](Frag &F, const float *stp, int ab, const int *cbg, int ua, int ub) {
        const float *sa = stp + ab + ua;
#pragma unroll
        for (int j = 0; j < 4; ++j) F.a[j] = sa[4 * j];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float *sb = stp + cbg[b] + ub;
#pragma unroll
            for (int j = 0; j < 4; ++j) F.b[b][j] = sb[4 * j * st];
        }
    };
    // The block's 4*NB MFMAs.  FLAT: f0 = first pixel of the block, kv =
    // pixels of the group (grad_out is masked per kernel column).
    auto mma = [&](const Frag &F, int f0, int kv) {
        if (FLAT) {
            constexpr int NKW = KW > 0 ? KW : 1;
            float am[NKW][4];
            // Column masks of the K block: a pixel's value is kept for the
            // kernel columns whose input column stays in its row.
            auto masks = [&](bool with_bias) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // Column of the pixel (W >= 2 here), moved out of every
                    // kernel column's range past the group's end.
                    const int f = f0 + g + 4 * j;
                    const int ow = f < kv ? f - (int)__umulhi((uint32_t)f, A.m_w) * A.W : 1 << 24;
#pragma unroll
                    for (int kw = 0; kw < NKW; ++kw)
                        am[kw][j] = (uint32_t)(ow + kw - A.pad_w) < (uint32_t)A.W ? F.a[j] : 0.f;
                    // The centre column (kw == pad_w, as oW == W) masks only
                    // the pixels past the group's end.
                    if (with_bias) bsum += am[(NKW - 1) / 2][j];
                }
            };
            if constexpr (PLAIN) {
                // A block whose 16 pixels lie in one row, at least the
                // kernel's reach from both of its ends, and before the
                // group's end needs no masks (a uniform test: f0 and kv are
                // the same for the wave).
                const int c0 = f0 - (int)__umulhi((uint32_t)f0, A.m_w) * A.W;
                if (f0 + 16 <= kv && c0 >= A.pad_w && c0 + 15 + (NKW - 1 - A.pad_w) < A.W) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int kw = 0; kw < NKW; ++kw) am[kw][j] = F.a[j];
                } else {
                    masks(false);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) bsum += am[(NKW - 1) / 2][j];
            } else {
                masks(true);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[b % NKW][j], F.b[b][j], acc[b],
                                                                  0, 0, 0);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bsum += F.a[j];
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(F.a[j], F.b[b][j], acc[b], 0, 0,
                                                                  0);
            }
        }
    };

    // K blocks of one group, two in flight: the fragments of block kb+1 are
    // read from LDS while block kb's MFMAs run.
    auto compute = [&](int grp, int buf) {
        const float *stp = sm + buf * A.stage_floats;
        const int gg = grp0 + grp;
        const int n = gg / A.groups_img;
        const int oh0 = (gg - n * A.groups_img) * A.R;
        const int rows_v = min(A.R, A.oH - oh0);
        int cbg[NB];
        int ab, nkb, kv = 0;
        if (FLAT) {
            kv = rows_v * A.oW;
            const int aplane = (n * A.Co + co0 + 16 * wave + i) * oHW + oh0 * A.oW;
            const int fbase = (oh0 - A.pad_h + kh0) * A.W - A.pad_w;
            const int xs = ((n * A.Ci + ci_lo + i) * HW + fbase) & 3;
#pragma unroll
            for (int b = 0; b < NB; ++b) cbg[b] = cb[b] + xs;
            ab = abase + (aplane & 3);
            nkb = (kv + 15) >> 4;
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) cbg[b] = cb[b];
            ab = abase;
            nkb = rows_v * (A.OWP >> 4);
        }
        // Offsets of K block kb: flat 16kb for both operands; row-padded
        // (row r, segment c) -> A r*OWP + 16c, B (r*XW + 16c)*stride.
        const int segs = A.OWP >> 4;
        int r = 0, c = 0;   // row-padded position of the next block to load
        auto next = [&](Frag &F, int kb) {
            if (FLAT) {
                load(F, stp, ab, cbg, 16 * kb, 16 * kb);
            } else {
                load(F, stp, ab, cbg, r * A.OWP + 16 * c, (r * A.XW + 16 * c) * st);
                if (++c == segs) {
                    c = 0;
                    ++r;
                }
            }
        };
        Frag F0, F1;
        if (nkb > 0) next(F0, 0);
        for (int kb = 0; kb < nkb; kb += 2) {
            if (kb + 1 < nkb) next(F1, kb + 1);
            mma(F0, 16 * kb, kv);
            if (kb + 1 < nkb) {
                if (kb + 2 < nkb) next(F0, kb + 2);
                mma(F1, 16 * (kb + 1), kv);
            }
        }
    };

    const bool two = A.stages == 2;
    if (ngrp > 0) issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int grp = 0; grp < ngrp; ++grp) {
        const int cur = two ? (grp & 1) : 0;
        if (two && grp + 1 < ngrp) issue(grp + 1, cur ^ 1);
        compute(grp, cur);
        if (!two) {
            __syncthreads();
            if (grp + 1 < ngrp) issue(grp + 1, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // Partial sums: D[4g + r][i] of block b -> part[slice][co][ci][kh][kw];
    // with the bias, the first column tile adds part[slice][Co*Ci*kH*kW + co]
    // (lane groups g = 0..3 summed in that order).
    float *pout = A.part + (size_t)slice * A.part_stride;
    if (A.bias && ct == 0) {
        float t = bsum + __shfl_xor(bsum, 16);
        t = t + __shfl_xor(t, 32);
        const int co = co0 + 16 * wave + i;
        if (g == 0 && co < A.Co) pout[(size_t)A.Co * A.Ci * kHW + co] = t;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        int ci, kh, kw;
        bool ok;
        if (KW > 0) {
            ci = ci_lo + i;
            kh = kh0 + b / KW;
            kw = b % KW;
            ok = ci < A.Ci && kh < A.kH;
        } else {
            const int col = c0 + 16 * b + i;
            ok = col < A.Ci * kHW;
            ci = col / kHW;
            const int t = col - ci * kHW;
            kh = t / A.kW;
            kw = t - kh * A.kW;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int co = co0 + 16 * wave + 4 * g + r;
            if (ok && co < A.Co)
                pout[((size_t)co * A.Ci + ci) * kHW + kh * A.kW + kw] = acc[b][r];
        }
    }
}

}  // namespace

hipError_t launch_gw_reduce(const float *part, float *out0, float *out1, int n0, int total,
                            int slices, hipStream_t s) {
    hipExtLaunchKernelGGL(gw_reduce_f32, dim3((unsigned)((total + 63) / 64)), dim3(256), 0, s,
                          nullptr, nullptr, 0, part, out0, out1, n0, total, slices);
    return hipGetLastError();
}

int channel_sum_blocks(int N, int Co, int plane) {
    // About 16K floats per work-group, at least one block.
    (void)Co;
    const int ipb = std::max(1, 16384 / std::max(1, plane));
    return std::max(1, (N + ipb - 1) / ipb);
}

hipError_t launch_channel_sum(const float *g, float *part, float *db, int N, int Co, int plane,
                              hipStream_t s) {
    const int nblk = channel_sum_blocks(N, Co, plane);
    const int ipb = std::max(1, (N + nblk - 1) / nblk);
    hipExtLaunchKernelGGL(gw_channel_sum_f32, dim3((unsigned)Co, (unsigned)nblk), dim3(256), 0, s,
                          nullptr, nullptr, 0, g, part, N, Co, plane, ipb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_gw_reduce(part, db, nullptr, Co, Co, nblk, s);
}

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
    return launch_gw_reduce(a.part, a.dw, nullptr, total, total, a.slices, s);
}

// Instantiations of gi_gwd_f32: (NB, KW, S, FLAT).
//   0: flat, tap-major, 3 kernel columns x 3 rows
//   1: flat, tap-major, 7 kernel columns x 1 row
//   2: row-padded, tap-major, 3 x 3, stride 1
//   3: row-padded, tap-major, 3 x 3, stride 2
//   4: row-padded, flattened map, 10 blocks, stride 2
//   5: row-padded, flattened map, 8 blocks, any stride
//   6: as 0, with the mask bypass (rows of at least 18 pixels)
int gwd_f32_blocks(int cfg) {
    static const int nb[] = {9, 7, 9, 9, 10, 8, 9};
    return cfg >= 0 && cfg < 7 ? nb[cfg] : 0;
}

// Work-groups per compute unit that the registers allow: one wave of each
// work-group per SIMD, 512 registers per lane per SIMD shared by VGPRs and
// AGPRs; the counts are those of the gfx950 build of each instantiation
// (cfg 0: 180 + 36, cfg 1: 132 + 28, cfg 2: 128 + 36, cfg 3: 128 + 36,
// cfg 4: 164 + 40, cfg 5: 136 + 32, cfg 6: 184 + 36).
int gwd_f32_max_wgs(int cfg) {
    static const int occ[] = {2, 3, 3, 3, 2, 3, 2};
    return cfg >= 0 && cfg < 7 ? occ[cfg] : 1;
}

size_t gwd_f32_lds_bytes(const GwdArgs &a) {
    return (size_t)a.stages * (size_t)a.stage_floats * sizeof(float);
}

hipError_t launch_gwd_f32(const GwdArgs &a, int cfg, hipStream_t s, const KernelEvents &ev) {
    // (Piece indices below 2^14 and planes below 2^24 pixels: the 24-bit
    // divisions and multiplies of the direct loads.)
    if (a.nslots > 16384 - 64 || (int64_t)a.H * a.W >= (1 << 24) ||
        (int64_t)a.oH * a.oW >= (1 << 24))
        return hipErrorInvalidValue;
    if (cfg < 0 || cfg > 6 || a.LA % 8 != 4 || a.LX % 8 != 4 || a.stages < 1 || a.stages > 2 ||
        a.stage_floats % 256 != 0 || a.nslots != 16 * a.LA + a.XC * (a.LX / 4) ||
        4 * a.nslots > a.stage_floats || (!a.flat && (a.OWP % 16 != 0 || a.XW % 4 != 0 ||
                                                        a.XO % 4 != 0)))
        return hipErrorInvalidValue;
    const size_t lds = gwd_f32_lds_bytes(a);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const int64_t wgs = (int64_t)a.co_blocks * a.col_tiles * a.slices;
    const dim3 grid((unsigned)wgs), block(kGwdThreads);
    auto go = [&](auto kern) -> hipError_t {
        if (lds > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute((const void *)kern,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, s, ev.start, ev.stop, 0, a);
        return hipGetLastError();
    };
    hipError_t e;
    switch (cfg) {
        case 0: e = go(gi_gwd_f32<9, 3, 1, true>); break;
        case 1: e = go(gi_gwd_f32<7, 7, 1, true>); break;
        case 2: e = go(gi_gwd_f32<9, 3, 1, false>); break;
        case 3: e = go(gi_gwd_f32<9, 3, 2, false>); break;
        case 4: e = go(gi_gwd_f32<10, 0, 2, false>); break;
        case 5: e = go(gi_gwd_f32<8, 0, 0, false>); break;
        default: e = go(gi_gwd_f32<9, 3, 1, true, true>); break;
    }
    if (e != hipSuccess) return e;
    const int total = a.Co * a.Ci * a.kH * a.kW;
    return launch_gw_reduce(a.part, a.dw, a.db, total, a.part_stride, a.slices, s);
}

}  // namespace gi
