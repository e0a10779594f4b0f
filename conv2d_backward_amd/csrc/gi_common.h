// gi_common.h -- structures shared by the planner (host) and the kernels.
//
// Phase split.  With stride s, input pixel (ih, iw) only meets taps kh with
// ih + pad_h - kh divisible by s (meganeura conv2d_grad_input_gemm.wgsl,
// general-stride branch of the B gather; doppler conv2d_backward_input.wgsl,
// the divisibility guards).  Group input rows by their residue rho = ih mod s:
// writing ih = rho + s*a, the contributing taps are kh = r + s*j with
// r = (rho + pad_h) mod s and j = 0, 1, ..., and the output row they read is
//     oh = (ih + pad_h - kh) / s = a + q - j,   q = (rho + pad_h) div s.
// The same holds along w.  Each residue pair (rho_h, rho_w) is therefore a
// dense stride-1 sub-problem over its own pixels (a, b) and its own taps
// (j, jw), with K = Co * J_h * J_w.  Stride 1 is the single phase rho = r = 0,
// q = pad.  A phase with no taps (J = 0, when the kernel is shorter than the
// stride) still owns its pixels and writes zeros there.
#pragma once

#include <stdint.h>

namespace gi {

// The dispatcher hands work-groups to the chip's 8 XCDs in turn by linear id,
// and each XCD has its own L2.  xcd_order maps linear id L of a 1-D grid of G
// work-groups to a logical index such that XCD x = L mod 8 receives the
// contiguous logical range starting at x*(G/8) + min(x, G mod 8), in order:
// work-groups that read the same grad_out lines (the input-channel tiles or
// phases of one pixel tile, neighbouring tiles) then run on one L2 at about
// the same time.  It is a bijection on [0, G) whatever the dispatch order.
constexpr int kXcds = 8;
__host__ __device__ inline int xcd_order(int L, int G) {
    const int x = L % kXcds, k = L / kXcds;
    const int q = G / kXcds, r = G % kXcds;
    return x * q + (x < r ? x : r) + k;
}

constexpr int kMaxPhasesPerLaunch = 16;

struct Phase {
    int32_t rho_h, rho_w;   // input-pixel residues mod stride
    int32_t q_h, q_w;       // (rho + pad) div stride
    int32_t r_h, r_w;       // first tap of the phase: (rho + pad) mod stride
    int32_t J_h, J_w;       // taps of the phase per dimension
    int32_t Ha, Wb;         // pixels of the phase per image: rows, columns
    int32_t tile_begin;     // first pixel tile of the phase within its launch
    int32_t pad_;           // keeps the struct 48 bytes
};

// Kernel arguments of one launch of a phase-split GEMM kernel.
struct GemmArgs {
    const void *grad_out;   // [N, Co, oH, oW], fp32 or bf16
    const void *wt;         // weight in kernel order (see prologue), fp32 or bf16
    float *dst;             // [N, Ci, H, W] fp32
    int32_t N, Ci, H, W, Co, kH, kW, stride, oH, oW;
    int32_t nphases;
    int32_t ci_tiles;
    Phase ph[kMaxPhasesPerLaunch];
};

}  // namespace gi

namespace gi {

// One residue class of the stride for the halo kernel.
struct HaloPhase {
    int32_t rho_h, rho_w;   // input-pixel residues mod stride
    int32_t q_h, q_w;       // (rho + pad) div stride
    int32_t r_h, r_w;       // first tap of the phase: (rho + pad) mod stride
    int32_t J_h, J_w;       // taps of the phase per dimension
    int32_t Ha, Wb;         // pixels of the phase per image: rows, columns
    int32_t woff;           // first float of the phase's weight blocks in a ci tile
    int32_t tb;             // fused launches: first tap of the phase in a chunk's taps
    int32_t dr, dc;         // fused launches: origin of the phase's halo in the shared one
    int32_t pad_;
};

// Arguments of one launch of the fp32 halo kernel.  A work-group owns a tile
// of TR x TC pixels of the phase grid (the same tile in every phase) and 64
// input channels, and walks the phases one after another.
//
// Weight image (written by the prologue, zero-padded in ci and co):
//   wk[ci_tile][phase][chunk of 8 co][tap][co pair cp][ci of 64][2]
// so one chunk of one phase is a contiguous block of taps * 512 floats; a
// ci tile spans w_ci_stride floats.  Fused launches (fused = 1: every phase
// of a chunk from one shared halo) order it chunk-major instead,
//   wk[ci_tile][chunk][tap of any phase: tb + t][co pair cp][ci of 64][2],
// so one chunk of every phase is one block of Tall * 512 floats.
struct HaloArgs {
    const float *grad_out;  // [N, Co, oH, oW]
    const float *wk;        // weight image (above)
    float *dst;             // [N, Ci, H, W]
    uint32_t g_bytes;       // size of grad_out in bytes (< 2^31)
    uint32_t w_bytes;       // size of the weight image in bytes (< 2^31)
    uint32_t d_bytes;       // size of dst in bytes (< 2^31)
    int32_t N, Ci, H, W, Co, oH, oW, stride;
    int32_t nphases;
    int32_t TR, TC;         // tile rows / columns in phase-grid pixels
    int32_t row_tiles, col_tiles;
    int32_t fold;           // 1: tile rows run across images (every phase has J_h <= 1)
    int32_t nchunks;        // ceil(Co / 8)
    int32_t HP;             // halo row pitch in positions (>= TC + J_w - 1 of every phase)
    int32_t HPc;            // LDS pitch of one co pair's halo, in float2
    int32_t stages;         // LDS stages of the chunk pipeline (2 or 3)
    int32_t maxT;           // most taps of any phase
    int32_t w_ci_stride;    // floats of the weight image per ci tile
    int32_t ci_tiles;       // ceil(Ci / 64); grid = tiles * ci_tiles (1-D, xcd_order)
    int32_t fused;          // 1: all phases per chunk over one halo (see the weight image)
    int32_t Tall;           // fused: taps of all phases
    int32_t org_h, org_w;   // fused: shared halo origin relative to the tile
    int32_t HR, HC;         // fused: shared halo rows / columns
    int8_t gph[2][4];       // fused: phases of each thread group (-1: none)
    HaloPhase ph[kMaxPhasesPerLaunch];
};

}  // namespace gi

namespace gi {

// Arguments of the bf16 halo kernel (stride 1).
//
// gp: grad_out as zero-padded planes of 8 channels, bf16,
//     gp[N][nchunks][4][YP][XP][8] with YP = H + kH - 1, XP = W + kW - 1:
//     plane g of chunk c holds channels 32c + 8g .. +7, and position (y, x)
//     holds grad_out[oh = y - (kH-1-pad_h)][ow = x - (kW-1-pad_w)] (zero
//     outside the image or past Co), so tap (kh, kw) of input pixel (ih, iw)
//     reads position (ih + kH-1-kh, iw + kW-1-kw).
// wk: weights in the lane order of the MFMA A fragments,
//     wk[ci tile][chunk][tap][ci block of 16][lane][8]: lane l holds the 8
//     output channels chunk*32 + 8*(l/16) + e of input channel
//     tile*64 + block*16 + l%16 (zero past Ci or Co).
constexpr int kHaloBf16Loads = 8;   // most 64-position halo loads per plane
struct HaloBf16Args {
    const uint16_t *gp;
    const uint16_t *wk;
    float *dst;             // [N, Ci, H, W] fp32
    uint32_t gp_bytes, wk_bytes, d_bytes;
    int32_t N, Ci, H, W, Co, kH, kW;
    int32_t YP, XP, Cop, nchunks;
    int32_t TR, TC, row_tiles, col_tiles;
    int32_t HR, HC;         // halo rows / columns: TR + kH - 1, TC + kW - 1
    int32_t HP;             // LDS pitch of a halo row in positions: at least HC,
                            // congruent to TC mod 16 (see the kernel)
    int32_t nql;            // 64-position loads per plane: ceil(HR * HP / 64) <= 8
    int32_t PS;             // LDS bytes per plane: nql * 1024
    int32_t ci_tiles;       // ceil(Ci / 64); grid = tiles * ci_tiles (1-D, xcd_order)
};

}  // namespace gi

namespace gi {

// One stride phase of the small-Ci ("stem") kernel.
struct StemPhase {
    int32_t rho_h, rho_w;   // input-pixel residues mod stride
    int32_t q_h, q_w;       // (rho + pad) div stride
    int32_t r_h, r_w;       // first tap of the phase: (rho + pad) mod stride
    int32_t J_h, J_w;       // taps of the phase per dimension
    int32_t Ha, Wb;         // pixels of the phase per image
    int32_t dr, dc;         // origin of the phase's halo inside its work-group's halo
    int32_t tb;             // first tap of the phase in its work-group's weight staging
};

// Work-group shape of the small-Ci kernel: waves per work-group is
// 2 * (phase groups per work-group), each wave owning 8 tile rows of one
// group; the weights of up to kStemTapsPerWave taps per wave are staged.
constexpr int kStemGroupsPerWg = 2;
constexpr int kStemTapsPerWave = 16;

// Arguments of the fp32 small-Ci kernel (Ci <= 4).  Work units are
// (image, tile row, tile column, set of phase groups), the set fastest; a tile
// is 16 x 16 pixels of the phase grid.  The first nfull units are one
// work-group each; with one set per tile, the units after them are split
// into four work-groups of 4 tile rows each.  A phase group is one or two phases
// whose tap counts add up to about the same as the other groups'; a
// work-group runs up to kStemGroupsPerWg groups side by side (two waves per
// group) over one grad_out halo that covers every phase of the set.  The
// kernel reads the weight in the caller's layout [Co][Ci][kH][kW] (no
// reordered copy).
struct StemArgs {
    const float *grad_out;  // [N, Co, oH, oW]
    const float *w;         // [Co, Ci, kH, kW]
    float *dst;             // [N, Ci, H, W]
    uint32_t g_bytes, w_bytes, d_bytes;
    int32_t N, Ci, H, W, Co, oH, oW, stride, kH, kW;
    int32_t nphases, nchunks;
    int32_t tiles_r, tiles_c;
    int32_t HPmax;          // LDS halo positions per stage (a multiple of 16 * waves)
    int32_t pitch;          // halo row pitch in positions (>= every set's halo width)
    int32_t ngroups;        // phase groups
    int32_t nsets;          // sets of phase groups (work-groups per tile)
    int32_t nfull;          // (image, tile, set) units run whole; the rest in quarters
    int8_t group[kMaxPhasesPerLaunch][2];  // phases of each group (second -1 if alone)
    // Per set: halo origin relative to the tile (rows, columns) and its
    // extent (rows, columns).
    int32_t set_org[kMaxPhasesPerLaunch][2];
    int32_t set_ext[kMaxPhasesPerLaunch][2];
    StemPhase ph[kMaxPhasesPerLaunch];
};

}  // namespace gi

namespace gi {

// Arguments of the whole-image 16-bit kernel (kernels_img16.hip, stride 1).
// A work-group owns one image and 128 input channels; grad_out is read from
// the caller's NCHW tensor (no padded copy) and the weight from the fragment
// image wk of the bf16 halo kernel (layout above; its ci tiles are 64 wide,
// so a 128-channel work-group reads two of them).
//
// LDS: two stages, each 4 channel planes of PS bytes; plane g of a stage
// holds output channels chunk*32 + 8g .. +7 as 16-byte positions, halo row
// pitch HP, and position (hr, hc) holds grad_out[hr - oy][hc - ox], zero
// outside the grad_out plane (the transposed padding: oy = kH-1-pad_h,
// ox = kW-1-pad_w).  Input pixel (ih, iw) at tap (kh, kw) reads position
// (ih + kH-1-kh, iw + kW-1-kw).
struct Img16Args {
    const uint16_t *g;      // grad_out [N, Co, oH, oW], bf16 or fp16 bits
    const uint16_t *wk;     // weight fragment image (64-channel ci tiles)
    float *dst;             // [N, Ci, H, W] fp32
    uint32_t g_bytes, wk_bytes, d_bytes;
    int32_t N, Ci, H, W, Co, oH, oW, kH, kW;
    int32_t oy, ox;         // halo position of grad_out pixel (0, 0)
    int32_t HR, HC, HP;     // halo rows (H + kH - 1), columns (W + kW - 1), row pitch
    int32_t PS;             // LDS bytes of one channel plane (multiple of 256)
    int32_t nchunks;        // ceil(Co / 32)
    int32_t ci_tiles;       // ceil(Ci / 128); grid = N * ci_tiles (1-D, xcd_order)
    int32_t nq;             // 4-pixel quads of one grad_out plane: oH * oW / 4
    uint32_t rcp_w, rcp_ow;  // ceil(2^16 / W), ceil(2^16 / oW): pixel index -> row
};

}  // namespace gi

namespace gi {

// Arguments of the column kernel (kernels_col2im_f32.hip: fp32, few input
// channels).  The sum over (co, kh, kw) is taken in two steps: for every
// grad_out position q = (oh, ow) the columns
//   Y[q][c] = sum_co grad_out[co][q] * w[co][c],   c = (ci, kh, kw),
// a GEMM with K = Co on the matrix cores, and then every Y[q][c] is added to
// grad_input[ci][s*oh - pad_h + kh][s*ow - pad_w + kw] (the fold of the
// columns) in an LDS tile.  Each column lands on exactly one input pixel, so
// no tap that the stride rules out is ever multiplied.  A work-group owns a
// TH x TW tile of one image and computes the columns of every grad_out
// position whose footprint meets the tile (those on the tile's border are
// also computed by the neighbouring work-group, each keeping its own part).
struct Col2imArgs {
    const float *grad_out;  // [N, Co, oH, oW]
    const float *w;         // [Co, Ci, kH, kW], i.e. [Co][ncols]
    float *dst;             // [N, Ci, H, W]
    uint32_t g_bytes, w_bytes, d_bytes;
    int32_t N, Ci, H, W, Co, oH, oW, kH, kW, stride, pad_h, pad_w;
    int32_t ncols;          // Ci * kH * kW
    int32_t TH, TW;         // input pixels owned by a work-group
    int32_t tiles_r, tiles_c;  // grid = N * tiles_r * tiles_c (1-D, xcd_order)
    int32_t RW;             // grad_out rows per wave and tile; stride * RW >= kH
    int32_t LR, LP;         // LDS tile rows and row pitch (floats), per input channel
    int32_t plane;          // LDS floats per input channel (>= LR * LP)
    int32_t r0, c0;         // LDS row and column of tile pixel (0, 0)
    int32_t wofs;           // LDS float offset of the staged weight
    int32_t ws;             // staged weight row stride (floats), >= 16 * column blocks
    uint32_t magic_khw, magic_kw;  // ceil(2^16 / (kH * kW)), ceil(2^16 / kW)
};

}  // namespace gi
