// gi_launch.h -- host-side launchers of the kernels (one per kernel family).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_common.h"

namespace gi {

// Events recorded by a main-kernel launch with the dispatch's own start and
// end timestamps (hipExtLaunchKernelGGL); either may be null.
struct KernelEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

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
hipError_t launch_generic_f32(const GemmArgs &a, int tiles_x, hipStream_t s,
                              const KernelEvents &ev);
hipError_t launch_generic_bf16(const GemmArgs &a, int tiles_x, hipStream_t s,
                               const KernelEvents &ev);

// Halo-tile fp32 kernel (kernels_halo_f32.hip).  Instantiations are indexed
// by (NB pixel blocks of 16 per work-group, HG halo groups of 32 positions
// per wave, the set of per-phase tap counts served as a bit mask of
// halo_f32_tbit(T), 0 for a tap count no instantiation serves);
// halo_f32_config returns the first instantiation that covers the request, or
// -1 when none does.
constexpr int kHaloBC = 8;     // output channels per LDS stage (chunk)
constexpr int kHaloCT = 64;    // input channels per work-group
unsigned halo_f32_tbit(int T);
// hp: halo row pitch in positions; jw: the kernel-width tap count shared by
// every phase with taps (0 if they differ); ks: thread groups of 256 that
// split the output channels of a work-group (1 or 2); nph: phases of a fused
// launch (0: phase at a time).
int halo_f32_config(int nb, unsigned tmask, int hg, int hp, int jw, int ks, int nph);
hipError_t launch_halo_f32(const HaloArgs &a, int cfg, int tiles, int ci_tiles, size_t lds,
                           hipStream_t s, const KernelEvents &ev);
// Chunks of 8 output channels per LDS stage of instantiation cfg, and the LDS
// bytes of the halo kernel: most taps of a phase, halo pitch (float2),
// pipeline stages, chunks per stage.
int halo_f32_cps(int cfg);
// Thread groups of 256 per work-group of instantiation cfg, and the phases
// it fuses (0: none).
int halo_f32_ks(int cfg);
int halo_f32_nph(int cfg);
// True when instantiation cfg has its halo pitch fixed at compile time.
bool halo_f32_fixed_pitch(int cfg);
size_t halo_f32_lds_bytes(int maxT, int HPc, int stages, int cps);  // per thread group

// Weight image of the halo kernel (layout in gi_common.h); `total` floats.
hipError_t launch_weight_image_f32(const float *w, float *wk, const HaloArgs &a, int kH, int kW,
                                   int ci_tiles, int64_t total, hipStream_t s);

// bf16 halo kernel (kernels_halo_bf16.hip), stride 1.  Instantiations are
// indexed by (NBW pixel blocks of 16 per wave, kH x kW taps, halo pitch hp):
// some fix the kernel width and pitch at compile time; -1 when none serves.
int halo_bf16_config(int nbw, int kH, int kW, int hp);
hipError_t launch_halo_bf16(const HaloBf16Args &a, int cfg, int tiles, int ci_tiles, size_t lds,
                            hipStream_t s, const KernelEvents &ev);
// Both prologues of the bf16 halo kernel in one launch (layouts in
// gi_common.h): grad_out -> padded channel planes gp, weight -> fragment
// image wk.
hipError_t launch_prologues_bf16(const uint16_t *g, uint16_t *gp, const uint16_t *w, uint16_t *wk,
                                 const HaloBf16Args &a, int oH, int oW, int pad_h, int pad_w,
                                 int ci_tiles, hipStream_t s);

// Whole-image 16-bit kernel (kernels_img16.hip), stride 1: one work-group
// per (image, 128 input channels).  img16_config returns the instantiation
// for (pixel blocks of 16, taps, kernel width, halo pitch, halo rows), -1 if
// none; img16_plane the LDS bytes of one channel plane it is built for,
// img16_lds the dynamic LDS of a launch.
int img16_config(int nb, int kH, int kW, int hp, int hr);
int img16_blocks(int cfg);
int img16_plane(int cfg);
size_t img16_lds(int cfg);
hipError_t launch_img16(const Img16Args &a, int cfg, bool f16, size_t lds, hipStream_t s,
                        const KernelEvents &ev);
// Weight -> fragment image wk (layout of HaloBf16Args.wk) for Co output and
// Ci input channels, kHW taps, nchunks chunks of 32, wtiles ci tiles of 64.
hipError_t launch_weight_frag16(const uint16_t *w, uint16_t *wk, int Co, int Ci, int kHW,
                                int nchunks, int wtiles, hipStream_t s);

// Small-Ci fp32 kernel (kernels_stem_f32.hip): Ci <= 4, any stride whose
// phases have a tap count in the served set (stem_f32_taps_ok).
bool stem_f32_taps_ok(int taps);
// The halo pitch the stem kernel has a compile-time instance for; the halo
// positions per LDS stage of the instance used for a pitch (every set's
// halo must fit); waves per work-group for a number of phase groups; the
// LDS bytes of the kernel for that many positions and waves.
int stem_f32_fixed_pitch();
int stem_f32_halo_positions(int pitch);
int stem_f32_waves(int ngroups);
size_t stem_f32_lds_bytes(int hpmax, int waves);
hipError_t launch_stem_f32(const StemArgs &a, hipStream_t s, const KernelEvents &ev);

// Column kernel (kernels_col2im_f32.hip): fp32, Ci * kH * kW <= 16 *
// kCol2imMaxBlocks columns, kCol2imMinCo < Co <= kCol2imMaxCo, stride <=
// kCol2imMaxStride, kW <= 4 * stride (no two columns of one fold batch meet
// on the same pixel), and tiles whose grad_out rows take at most
// kCol2imBlocksPerRow blocks of 16 positions.
constexpr int kCol2imMaxBlocks = 10;
constexpr int kCol2imMinCo = 48;
constexpr int kCol2imMaxCo = 64;
constexpr int kCol2imMaxStride = 2;
constexpr int kCol2imBlocksPerRow = 2;
// Row pitch and channel plane of the column kernel's LDS tile: the least
// pitch >= min_pitch with pitch = kW (mod 32), and the least plane >=
// LR * pitch with plane = kH * kW (mod 32).  Column (ci, kh, kw), at
// ci * plane + kh * pitch + kw, then sits on LDS bank (its column index) plus
// a per-lane constant, mod 32, which the kernel's assignment of columns to
// blocks and of positions to lanes makes conflict-free.
inline void col2im_f32_layout(int kH, int kW, int LR, int min_pitch, int &pitch, int &plane) {
    pitch = min_pitch + ((kW - min_pitch) % 32 + 32) % 32;
    const int base = LR * pitch;
    plane = base + ((kH * kW - base) % 32 + 32) % 32;
}
// Row stride of the column kernel's staged weight: at least 16 * (column
// blocks), and 8 (stride 2) or 16 (stride 1) mod 32, so that a B-fragment
// read (lane groups one weight row apart) meets 32 distinct banks per half
// wave for the kernel's columns of a block.
inline int col2im_f32_stage_stride(int ncols, int stride) {
    const int need = (ncols + 15) / 16 * 16, want = stride == 2 ? 8 : 16;
    return need + ((want - need) % 32 + 32) % 32;
}
// ceil(2^16 / d): for 0 <= x < 256 and 1 <= d <= 256, (x * m) >> 16 = x / d
// (the error x * (m - 2^16/d) / 2^16 < x / 2^16 stays below 1/d, the least
// distance from x/d up to the next integer, since x * d < 2^16).
inline uint32_t recip16(int d) { return (65536u + (uint32_t)d - 1u) / (uint32_t)d; }
int col2im_f32_weight_offset(const Col2imArgs &a);
size_t col2im_f32_lds_bytes(const Col2imArgs &a);
hipError_t launch_col2im_f32(const Col2imArgs &a, hipStream_t s, const KernelEvents &ev);

}  // namespace gi
