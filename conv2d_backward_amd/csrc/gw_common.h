// gw_common.h -- arguments and host-side launchers of the fp32 grad_weight
// kernels (kernels_gw_f32.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_common.h"
#include "gi_launch.h"

namespace gi {

// Arguments of the fp32 grad_weight kernels (kernels_gw_f32.hip).
//
//   dw[co,ci,kh,kw] = sum over n, oh, ow of g[n,co,oh,ow] * x[n,ci,ih,iw],
//   ih = oh*stride - pad_h + kh, iw = ow*stride - pad_w + kw (x = 0 outside),
//
// an implicit GEMM with M = Co, N = Ci*kH*kW and a long K = N*oH*oW.  Each
// image's output rows are cut into groups of RPC rows; a "slice" is a run of
// consecutive groups.  A work-group owns 64 output channels x 16 input
// channels x the kernel rows [kh0, kh0+khg) of one slice and writes its sums
// to part[slice]; a second kernel adds the slices in order into dw.
struct GwArgs {
    const float *x;          // [N, Ci, H, W] forward input
    const float *grad_out;   // [N, Co, oH, oW]
    float *part;             // [slices][Co][Ci][kH][kW] partial sums
    float *dw;               // [Co][Ci][kH][kW]
    uint32_t x_bytes, g_bytes;
    int32_t N, Ci, H, W, Co, oH, oW, stride, pad_h, pad_w, kH, kW;
    int32_t co_blocks, ci_blocks, tap_groups, khg;  // work-group tiles; kernel rows per tap group
    int32_t RPC;             // output rows per group (one image)
    int32_t groups_img;      // groups per image: ceil(oH / RPC)
    int32_t groups_slice;    // groups per slice
    int32_t slices;
    int32_t GM;              // grad_out LDS blocks of 64 pixels per group: ceil(RPC*oW / 64)
    int32_t XR, XP, XPM;     // input rows and columns per group; XPM: XP rounded up to 64
    int32_t CIP;             // LDS floats per input channel: XR*XPM + 4
    int32_t stages;          // LDS stages: 2 (next group loads during this one's arithmetic) or 1
};

// grad_weight with 16-byte direct loads (kernels_gw_f32.hip, gi_gwd_f32).
// Columns of the GEMM are (ci, kh, kw); a work-group computes 64 output
// channels x 16*NB columns, in one of two column maps:
//   tap-major: 16 input channels ci0.. x the taps of kernel rows
//              [kh0, kh0+khg) (block b = tap b of the group);
//   flattened: columns c0 .. c0+16*NB-1 of the (ci, kh, kw) order.
// Pixels (the reduction) are taken a group of R output rows of one image at
// a time, in one of two layouts:
//   row-padded: each output row padded to OWP pixels (a multiple of 16); the
//               input rows of the group in LDS with zero columns at both
//               sides (needs W and oW multiples of 4);
//   flat:       the group's R*oW pixels back to back, and the input as the
//               flat run of the plane that the group's taps touch (stride 1
//               with oH == H and oW == W only); taps that cross a row edge
//               are masked on the grad_out side.
struct GwdArgs {
    const float *x;          // [N, Ci, H, W] forward input
    const float *grad_out;   // [N, Co, oH, oW]
    float *part;             // [slices][Co][Ci][kH][kW] partial sums
    float *dw;               // [Co][Ci][kH][kW]
    float *db;               // [Co] bias gradient (with `bias`), else unused
    uint32_t x_bytes, g_bytes;
    int32_t N, Ci, H, W, Co, oH, oW, stride, pad_h, pad_w, kH, kW;
    int32_t bias;            // 1: also the bias gradient from the grad_out values read
    int32_t part_stride;     // floats per slice of part: Co*Ci*kH*kW (+ Co with the bias)
    int32_t flat;            // 1: flat pixel layout, 0: row-padded
    int32_t colmap;          // 0: tap-major, 1: flattened
    int32_t co_blocks, col_tiles;
    int32_t khg, tap_groups; // tap-major: kernel rows per tile, tiles over kernel rows
    int32_t R;               // output rows per group
    int32_t groups_img;      // ceil(oH / R)
    int32_t groups_slice;    // groups per slice
    int32_t slices;
    int32_t OWP;             // row-padded: LDS pixels per output row
    int32_t LA;              // LDS floats per output channel (LA/4 odd)
    int32_t XO;              // row-padded: LDS column of iw = 0 (a multiple of 4)
    int32_t XW;              // row-padded: LDS floats per input row
    int32_t XR;              // row-padded: input rows per group
    int32_t LX;              // LDS floats per input channel (LX/4 odd)
    int32_t XC;              // input channels held per work-group
    int32_t plane_zero;      // flat: zero every 16-byte piece outside the channel's plane
    int32_t nslots;          // 16-byte pieces per stage: 16*LA + XC*LX/4
    int32_t stage_floats;    // LDS floats per stage (a multiple of 256)
    int32_t stages;          // 1 or 2
    // Division by W >= 1: q = W == 1 ? s : umulhi(s, m_w) with
    // m_w = floor(2^32 / W) + 1, exact for s * W < 2^32.
    uint32_t m_w;
    // Divisions by LA/4, OWP/4, LX/4 and XW/4 on 24-bit multiplies (full
    // rate): q = (s * m) >> k with m in the low 24 bits and k in the high 8,
    // exact for 0 <= s < 2^14.
    uint32_t d24_la4, d24_owp4, d24_lx4, d24_xw4;
};

// grad_weight fp32 (kernels_gw_f32.hip): most taps per work-group, most
// 64-pixel blocks per row group, the LDS bytes of a plan, and the launch of
// the main kernel (both events bracket it) and then the slice reduction.
int gw_f32_max_taps();
int gw_f32_max_blocks();
size_t gw_f32_lds_bytes(const GwArgs &a);
hipError_t launch_gw_f32(const GwArgs &a, hipStream_t s, const KernelEvents &ev);
// grad_weight fp32 with 16-byte direct loads: column blocks of instantiation
// cfg (0 if none), work-groups per compute unit its registers allow, LDS
// bytes, launch (main kernel, then the slice reduction).
int gwd_f32_blocks(int cfg);
int gwd_f32_max_wgs(int cfg);
size_t gwd_f32_lds_bytes(const GwdArgs &a);
hipError_t launch_gwd_f32(const GwdArgs &a, int cfg, hipStream_t s, const KernelEvents &ev);
// Sum over slices (deterministic order): part [slices][total] -> out0[e] for
// e < n0, out1[e - n0] for the rest.
hipError_t launch_gw_reduce(const float *part, float *out0, float *out1, int n0, int total,
                            int slices, hipStream_t s);
// Bias gradient alone: per-channel sums of grad_out [N, Co, plane] into
// part [channel_sum_blocks(...)][Co] (scratch), then db [Co].
int channel_sum_blocks(int N, int Co, int plane);
hipError_t launch_channel_sum(const float *g, float *part, float *db, int N, int Co, int plane,
                              hipStream_t s);

}  // namespace gi
