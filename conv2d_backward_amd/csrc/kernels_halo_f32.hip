// kernels_halo_f32.hip -- fp32 halo-tile implicit-GEMM kernel for gfx950.
//
// The contraction is the implicit GEMM of meganeura conv2d_grad_input_gemm.wgsl
// (header comment: C[Ci, pixels] = A[Ci, K] x B[K, pixels], A the weight read
// as [Ci, Co*kH*kW], B the im2col of grad_out), restricted to the taps of one
// residue class of the stride at a time (see gi_common.h).  B is never
// gathered per tap: for each chunk of 8 output channels a work-group stages in
// LDS
//   * the grad_out "halo" of its pixel tile, i.e. the (TR + J_h - 1) x
//     (TC + J_w - 1) output rows/columns its TR x TC pixels read, zero outside
//     the image (this zero border is the transposed padding kH-1-pad of the
//     shader's header comment), and
//   * the weights of the chunk for its 64 input channels and every tap of the
//     phase, copied from a weight image laid out by the prologue below,
// and every tap (j, jw) reads its B fragment as the halo shifted by
// (J_h-1-j, J_w-1-jw) positions: one LDS read per fragment, the shift a
// uniform offset.
//
// Matrix cores: V_MFMA_F32_16X16X4_F32, rows = 16 input channels, columns = 16
// pixels, k = 4 output channels of one tap.  Lane l = 16*g + i supplies
// A[i][k=g], B[k=g][i] and receives D[4g + r][i], r = 0..3.  The K axis is
// permuted so that MFMA step s (0, 1) of a tap uses output channel 2g + s for
// lane group g: a lane then reads both of its k values with one 8-byte LDS
// read.  Each of the 4 waves owns 16 input channels and all NB pixel blocks of
// the tile; the next tap's fragments are read from LDS while the current
// tap's 2*NB MFMAs run.  Chunks are double-buffered in LDS and staged with
// direct global -> LDS loads, the next chunk's in flight during the current
// chunk's MFMAs.
//
// Out-of-range elements (halo outside the image, output channels past Co,
// pixels past the tile's edge, input channels past Ci) are handled with raw
// buffer loads and stores whose offset is pushed past the end of the buffer:
// the hardware returns 0 for such loads and drops such stores, so the loops
// carry no branches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "gi_common.h"
#include "lds_barrier.h"
#include "gi_launch.h"

namespace gi {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

namespace {

static_assert(kHaloCT == 64, "four waves of 16 input channels");
static_assert(kHaloBC == 8, "four co pairs per chunk");
constexpr int kHalo64 = 64;              // input channels of a weight-image row

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9)
constexpr int kOOB = 0x7ffffff0;         // byte offset past the end of every buffer

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (long)bytes, kRsrcWord3);
}

// Phase-grid pixel px (row-major in the TR x TC tile at origin (a0, b0)):
// image and coordinates, false outside the phase grid.
__device__ __forceinline__ bool tile_pixel(const HaloArgs &A, const HaloPhase &P, int px,
                                           int a0, int b0, int n_img, int &img, int &a,
                                           int &b) {
    const int r = px / A.TC, c = px - r * A.TC;
    img = 0;
    a = 0;
    b = b0 + c;
    if (px >= A.TR * A.TC || b >= P.Wb) return false;
    if (A.fold) {
        const int R = a0 + r;
        if (R >= A.N * P.Ha) return false;
        img = R / P.Ha;
        a = R - img * P.Ha;
        return true;
    }
    if (a0 + r >= P.Ha) return false;
    img = n_img;
    a = a0 + r;
    return true;
}

// Bit of tap count T in a kernel's TMASK.
constexpr unsigned tbit(int T) { return 1u << T; }

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Direct global -> LDS loads (no registers): lane i of the wave writes its
// `bytes` at LDS address dst + i * bytes; an out-of-range offset writes 0.
// dst must be the same for the whole wave.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void *dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *dst, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, voff, 0, 0, 0);
}
// Wait until at most N direct loads of this wave are outstanding (loads
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_dma() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// All chunks of one phase with T = J_h * J_w taps (compile time) for this
// work-group's tile; accumulates into acc.  Every thread of the work-group
// calls it (it contains barriers).  HG = halo groups of 32 positions staged
// per wave; CPS = chunks of 8 output channels per LDS stage (several for
// phases with few taps, so a barrier covers enough work).
//
// LDS stage (float2 units): weights [CPS][maxT][4 co pairs][64 ci], then
// halos [CPS][4 co pairs][HPc positions]; both written by direct loads:
//   * weights: the stage's chunks are consecutive blocks of the weight image,
//     T * 2 KB each, copied in 1 KB pieces (16 bytes per lane);
//   * halo: for co pair cp and a group of 32 positions, even lanes load
//     output channel 2cp and odd lanes 2cp+1 of position base + lane/2, which
//     lands exactly on the float2 layout.
template <int T, int NB, int HG, int CPS, int PITCH, int JW, int KS>
__device__ __forceinline__ void run_phase(const HaloArgs &A, const HaloPhase &P, v2f *smem2,
                                          const int (&pbase)[NB], v4f (&acc)[NB], int a0,
                                          int b0, int n_img, int ci_tile, int kg,
                                          __amdgpu_buffer_rsrc_t grs,
                                          __amdgpu_buffer_rsrc_t wrs) {
    const int tid = threadIdx.x & 255;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int wreg = CPS * A.maxT * 256;
    const int stage_f2 = wreg + CPS * 4 * A.HPc;
    // Tap grid of the phase (compile time when JW is), halo extent, and the
    // halo row pitch in LDS (compile time when PITCH is): every tap's shift
    // is then an immediate offset of the fragment reads.
    const int J_w = JW > 0 ? JW : P.J_w;
    const int J_h = JW > 0 ? T / JW : P.J_h;
    const int HP = PITCH > 0 ? PITCH : A.HP;
    const int HC = A.TC + J_w - 1;
    const int HR = A.TR + J_h - 1;
    const int hpos = HR * HP;
    const int groups = (hpos + 31) / 32;
    const int oHW = A.oH * A.oW;
    const int nstages = (A.nchunks + CPS - 1) / CPS;
    // This thread group's stages [s0, s1): with KS groups, group kg takes the
    // kg-th of KS near-equal runs; every group iterates h times (past s1 with
    // no arithmetic and loads that read zeros) so the barriers line up.
    const int h = (nstages + KS - 1) / KS;
    const int s0 = kg * h, s1 = min(nstages, s0 + h);

    // Halo shift of every tap (j, jw): (J_h-1-j) rows and (J_w-1-jw) columns.
    int shift[T];
    {
        int j = 0, jw = 0;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            shift[t] = (J_h - 1 - j) * HP + (J_w - 1 - jw);
            if (++jw == J_w) {
                jw = 0;
                ++j;
            }
        }
    }

    // Halo position of this lane in each of its wave's groups: grad_out byte
    // offset of output channel 0 (kOOB outside the image or the halo).
    int hoff[HG];
#pragma unroll
    for (int k = 0; k < HG; ++k) {
        const int pos = (wave + 4 * k) * 32 + (lane >> 1);
        const int hr = pos / HP, hc = pos - (pos / HP) * HP;
        const int ow = b0 + P.q_w - (J_w - 1) + hc;
        bool v = pos < hpos && hc < HC && ow >= 0 && ow < A.oW;
        int img, oh;
        if (A.fold) {
            const int R = a0 + hr;
            img = R / P.Ha;
            oh = (R - img * P.Ha) + P.q_h;
            v = v && R < A.N * P.Ha;
        } else {
            img = n_img;
            oh = a0 + P.q_h - (J_h - 1) + hr;
        }
        v = v && oh >= 0 && oh < A.oH;
        hoff[k] = v ? ((img * A.Co) * oHW + oh * A.oW + ow) * 4 : kOOB;
    }
    const int wbyte0 = (ci_tile * A.w_ci_stride + P.woff) * 4;
    const int co_lane = lane & 1;

    // Every wave issues the same fixed number of direct loads per stage (the
    // surplus ones read past the end of their buffer, i.e. zeros, into a
    // scratch kilobyte of LDS nobody reads), so "this stage's loads are done"
    // is a wait on a compile-time count.
    constexpr int WPW = (2 * T * CPS + 3) / 4;  // 1 KB weight pieces per wave
    constexpr int NDMA = WPW + 4 * HG * CPS;     // direct loads per wave per stage
    static_assert(NDMA <= 63, "vmcnt holds at most 63");
    v2f *const dummy = smem2 + A.stages * stage_f2;
    auto issue = [&](int stg, int buf) {
        v2f *st = smem2 + buf * stage_f2;
        const int wb = wbyte0 + stg * (CPS * T * 2048) + lane * 16;
#pragma unroll
        for (int i = 0; i < WPW; ++i) {
            const int m = wave + 4 * i;
            const bool real =
                stg < s1 && m < 2 * T * CPS && stg * CPS + m / (2 * T) < A.nchunks;
            dma16(wrs, real ? st + m * 128 : dummy, real ? wb + m * 1024 : kOOB);
        }
        v2f *hs = st + wreg;
        // Opaque copies: the offsets below are formed at each issue (a few
        // VALU ops per load) rather than strength-reduced into one register
        // per load held across the whole loop.
        int ho[HG];
#pragma unroll
        for (int k = 0; k < HG; ++k) {
            ho[k] = hoff[k];
            asm volatile("" : "+v"(ho[k]));
        }
#pragma unroll
        for (int o = 0; o < CPS; ++o) {
#pragma unroll
            for (int k = 0; k < HG; ++k) {
                const int g = wave + 4 * k;
                const bool real = g < groups && stg < s1;
#pragma unroll
                for (int cp = 0; cp < 4; ++cp) {
                    const int co = (stg * CPS + o) * kHaloBC + 2 * cp + co_lane;
                    const int off =
                        (real && ho[k] != kOOB && co < A.Co) ? ho[k] + co * oHW * 4 : kOOB;
                    dma4(grs, real ? hs + (o * 4 + cp) * A.HPc + g * 32 : dummy, off);
                }
            }
        }
    };

    // Stage pipeline: with 3 LDS stages, stage s+2 is in flight while stage s
    // is multiplied (with 2, stage s+1).
    const int D = A.stages - 1;
    wait_dma<0>();  // the previous phase's stores count too: drain them first
    issue(s0, 0);
    if (D == 2 && h > 1) {
        issue(s0 + 1, 1);
        wait_dma<NDMA>();
    } else {
        wait_dma<0>();
    }
    lds_barrier();
    for (int i = 0; i < h; ++i) {
        const int stg = s0 + i;
        const int cur = i % A.stages;
        const bool ahead = i + D < h;
        if (ahead) issue(stg + D, (i + D) % A.stages);
#pragma unroll
        for (int o = 0; o < CPS; ++o) {
            if (stg >= s1 || (CPS > 1 && stg * CPS + o >= A.nchunks)) break;
            // Odd co pairs hold their 64 input channels rotated by 16 (weight
            // image layout), so the two co pairs of a half-wave fall on
            // disjoint banks.
            const v2f *as = smem2 + cur * stage_f2 + o * T * 256 + g4 * 64 +
                            ((wave * 16 + l16 + 16 * (g4 & 1)) & 63);
            const v2f *hs = smem2 + cur * stage_f2 + wreg + (o * 4 + g4) * A.HPc;
            // Two fragment slots: tap t+1 is read from LDS while tap t's MFMAs
            // run.
            v2f fa[2], fb[2][NB];
            auto fetch = [&](int t, int slot) {
                fa[slot] = as[t * 4 * 64];
#pragma unroll
                for (int blk = 0; blk < NB; ++blk) fb[slot][blk] = hs[pbase[blk] + shift[t]];
            };
            fetch(0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int slot = t & 1;
                if (t + 1 < T) fetch(t + 1, slot ^ 1);
#pragma unroll
                for (int blk = 0; blk < NB; ++blk)
                    acc[blk] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[slot].x, fb[slot][blk].x,
                                                                    acc[blk], 0, 0, 0);
#pragma unroll
                for (int blk = 0; blk < NB; ++blk)
                    acc[blk] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[slot].y, fb[slot][blk].y,
                                                                    acc[blk], 0, 0, 0);
                // Keep taps in order: nothing moves across a tap boundary.
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // Stage s+1 must have landed: with 3 stages the loads of stage s+2
        // (issued this iteration) may still be in flight.
        if (D == 2 && ahead)
            wait_dma<NDMA>();
        else
            wait_dma<0>();
        lds_barrier();
    }
}

// Fused launches: the taps of one phase (tap grid JH x JW, compile time) over
// one staged chunk.  as: the phase's first tap in the stage's weights (this
// lane's A slot); hs: the shared halo of this lane's co pair, offset to the
// phase's origin in it.
template <int JH, int JW, int NB, int PITCH>
__device__ __forceinline__ void fused_taps(const v2f *as, const v2f *hs, const int (&pbase)[NB],
                                           int HP_rt, v4f (&acc)[NB]) {
    constexpr int T = JH * JW;
    const int HP = PITCH > 0 ? PITCH : HP_rt;
    int shift[T];
    {
        int j = 0, jw = 0;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            shift[t] = (JH - 1 - j) * HP + (JW - 1 - jw);
            if (++jw == JW) {
                jw = 0;
                ++j;
            }
        }
    }
    v2f fa[2], fb[2][NB];
    auto fetch = [&](int t, int slot) {
        fa[slot] = as[t * 4 * 64];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) fb[slot][blk] = hs[pbase[blk] + shift[t]];
    };
    fetch(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int slot = t & 1;
        if (t + 1 < T) fetch(t + 1, slot ^ 1);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
            acc[blk] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[slot].x, fb[slot][blk].x, acc[blk],
                                                            0, 0, 0);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
            acc[blk] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[slot].y, fb[slot][blk].y, acc[blk],
                                                            0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Fused launches: every phase of the tile per chunk of 8 output channels,
// from one LDS stage holding the weights of all the phases' taps (one block
// of the chunk-major weight image) and one grad_out halo covering every
// phase (A.HR x A.HC positions from (A.org_h, A.org_w) relative to the tile,
// pitch HP).  A stride-2 3 x 3 kernel has phases of 1, 2, 2 and 4 taps:
// loading one halo per phase per chunk, as the phase-at-a-time path does,
// gives each halo load a quarter of the matrix work.  Tap grids of 1 or 2 in
// each direction are served (the stride-2 phases of kernels up to 4 x 4).
//
// KS thread groups of 4 waves share every stage; group kg computes the
// phases A.gph[kg][0..MP-1] (-1: none), so each wave holds MP phases'
// accumulators.  All 4*KS waves issue the stage's direct loads.
constexpr int kFusedPieces = 24;  // 1 KB weight pieces per stage: up to 12 taps
template <int NB, int HG, int MP, int KS, int PITCH>
__device__ __forceinline__ void run_fused(const HaloArgs &A, v2f *smem2, const int (&pbase)[NB],
                                          const int (&myph)[MP], v4f (&acc)[MP][NB], int a0,
                                          int b0, int n_img, int ci_tile,
                                          __amdgpu_buffer_rsrc_t grs,
                                          __amdgpu_buffer_rsrc_t wrs) {
    constexpr int NW = 4 * KS;                          // waves issuing loads
    constexpr int WPW = (kFusedPieces + NW - 1) / NW;   // weight pieces per wave
    const int lane = threadIdx.x & 63;
    const int wall = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // 0 .. NW-1
    const int wave = wall & 3;                          // within the thread group
    const int l16 = lane & 15, g4 = lane >> 4;
    const int HP = PITCH > 0 ? PITCH : A.HP;
    const int wreg = A.Tall * 256;
    const int stage_f2 = wreg + 4 * A.HPc;
    const int hpos = A.HR * HP;
    const int groups = (hpos + 31) / 32;
    const int oHW = A.oH * A.oW;

    // Halo position of this lane in each of its wave's groups: grad_out byte
    // offset of output channel 0 (kOOB outside the image or the halo).
    int hoff[HG];
#pragma unroll
    for (int k = 0; k < HG; ++k) {
        const int pos = (wall + NW * k) * 32 + (lane >> 1);
        const int hr = pos / HP, hc = pos - (pos / HP) * HP;
        const int oh = a0 + A.org_h + hr, ow = b0 + A.org_w + hc;
        const bool v = pos < hpos && hc < A.HC && oh >= 0 && oh < A.oH && ow >= 0 && ow < A.oW;
        hoff[k] = v ? ((n_img * A.Co) * oHW + oh * A.oW + ow) * 4 : kOOB;
    }
    const int wbyte0 = ci_tile * A.w_ci_stride * 4;
    const int co_lane = lane & 1;
    constexpr int NDMA = WPW + 4 * HG;  // direct loads per wave per stage
    static_assert(NDMA <= 63, "vmcnt holds at most 63");
    v2f *const dummy = smem2 + A.stages * stage_f2;
    auto issue = [&](int chunk, int buf) {
        v2f *st = smem2 + buf * stage_f2;
        const bool live = chunk < A.nchunks;
        const int wb = wbyte0 + chunk * (A.Tall * 2048) + lane * 16;
#pragma unroll
        for (int i = 0; i < WPW; ++i) {
            const int m = wall + NW * i;
            const bool real = live && m < 2 * A.Tall;
            dma16(wrs, real ? st + m * 128 : dummy, real ? wb + m * 1024 : kOOB);
        }
        v2f *hs = st + wreg;
        int ho[HG];
#pragma unroll
        for (int k = 0; k < HG; ++k) {
            ho[k] = hoff[k];
            asm volatile("" : "+v"(ho[k]));
        }
#pragma unroll
        for (int k = 0; k < HG; ++k) {
            const int g = wall + NW * k;
            const bool real = live && g < groups;
#pragma unroll
            for (int cp = 0; cp < 4; ++cp) {
                const int co = chunk * kHaloBC + 2 * cp + co_lane;
                const int off = (real && ho[k] != kOOB && co < A.Co) ? ho[k] + co * oHW * 4 : kOOB;
                dma4(grs, real ? hs + cp * A.HPc + g * 32 : dummy, off);
            }
        }
    };

    const int D = A.stages - 1;
    issue(0, 0);
    if (D == 2 && A.nchunks > 1) {
        issue(1, 1);
        wait_dma<NDMA>();
    } else {
        wait_dma<0>();
    }
    lds_barrier();
    for (int chunk = 0; chunk < A.nchunks; ++chunk) {
        const int cur = chunk % A.stages;
        const bool ahead = chunk + D < A.nchunks;
        if (ahead) issue(chunk + D, (chunk + D) % A.stages);
        const v2f *st = smem2 + cur * stage_f2;
        const v2f *as0 = st + g4 * 64 + ((wave * 16 + l16 + 16 * (g4 & 1)) & 63);
        const v2f *hs0 = st + wreg + g4 * A.HPc;
#pragma unroll
        for (int k = 0; k < MP; ++k) {
            if (myph[k] < 0) continue;
            const HaloPhase &P = A.ph[myph[k]];
            const v2f *as = as0 + P.tb * 256;
            const v2f *hs = hs0 + P.dr * HP + P.dc;
            switch (P.J_h * 4 + P.J_w) {
                case 5: fused_taps<1, 1, NB, PITCH>(as, hs, pbase, HP, acc[k]); break;
                case 6: fused_taps<1, 2, NB, PITCH>(as, hs, pbase, HP, acc[k]); break;
                case 9: fused_taps<2, 1, NB, PITCH>(as, hs, pbase, HP, acc[k]); break;
                case 10: fused_taps<2, 2, NB, PITCH>(as, hs, pbase, HP, acc[k]); break;
                default: break;  // no taps: the phase's pixels are zero
            }
        }
        if (D == 2 && ahead)
            wait_dma<NDMA>();
        else
            wait_dma<0>();
        lds_barrier();
    }
}

// KS > 1: the work-group is KS groups of 4 waves that split the output
// channels of every phase (each group its own LDS stages, run to the same
// barrier count), and sum their accumulators through LDS before the store:
// for grids too small to put two work-groups on every compute unit, it gives
// each SIMD two waves instead of one.
//
// NPH > 0: a fused launch of NPH phases (run_fused); CPS, TMASK, JW and KS
// are then unused.
template <int NB, int HG, unsigned TMASK, int CPS, int OCC, int PITCH, int JW, int KS, int NPH>
__global__ __launch_bounds__(256 * KS, OCC) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void gi_halo_f32(
    const HaloArgs A) {
    extern __shared__ __attribute__((aligned(16))) v2f smem_all[];

    const int tid = threadIdx.x & 255;
    const int kg = KS > 1 && NPH == 0 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 8) : 0;
    v2f *const smem2 =
        smem_all + kg * (A.stages * CPS * (A.maxT * 4 * 64 + 4 * A.HPc) + 128);
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;

    // Logical order: input-channel tile fastest, then column, row, image.
    const int J = xcd_order(blockIdx.x, gridDim.x);
    const int ci_tile = J % A.ci_tiles;
    int t = J / A.ci_tiles;
    const int ct = t % A.col_tiles;
    t /= A.col_tiles;
    int rt, n_img = 0;
    if (A.fold) {
        rt = t;
    } else {
        rt = t % A.row_tiles;
        n_img = t / A.row_tiles;
    }
    const int ci0 = ci_tile * kHaloCT;
    const int a0 = rt * A.TR, b0 = ct * A.TC;
    const int plane = A.H * A.W;
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(A.grad_out, A.g_bytes);
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(A.wk, A.w_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(A.dst, A.d_bytes);

    if constexpr (NPH > 0) {
        // Fused: thread group kg runs phases A.gph[kg][0 .. MP-1] over the
        // stages both groups share (the LDS is not split).
        constexpr int MP = NPH / KS;
        const int gk = KS > 1 ? (int)(threadIdx.x >> 8) : 0;
        int myph[MP];
#pragma unroll
        for (int k = 0; k < MP; ++k) myph[k] = A.gph[gk][k];
        const int HP = PITCH > 0 ? PITCH : A.HP;
        // Halo position of this lane's pixel in each block (the same tile in
        // every phase).  Lanes past the tile read position l16 when every
        // phase's largest shift keeps that inside the halo plane, else 0.
        int max_shift = 0;
        for (int p = 0; p < A.nphases; ++p) {
            const HaloPhase &P = A.ph[p];
            if (P.J_h * P.J_w > 0)
                max_shift = max(max_shift, (P.dr + P.J_h - 1) * HP + P.dc + P.J_w - 1);
        }
        const int inv = l16 + max_shift < A.HPc ? l16 : 0;
        int pbase[NB];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const int px = blk * 16 + l16;
            pbase[blk] = px < A.TR * A.TC ? (px / A.TC) * HP + (px - (px / A.TC) * A.TC) : inv;
        }
        v4f acc[MP][NB];
#pragma unroll
        for (int k = 0; k < MP; ++k)
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) acc[k][blk] = v4f{0.f, 0.f, 0.f, 0.f};
        run_fused<NB, HG, MP, KS, PITCH>(A, smem_all, pbase, myph, acc,
                                         a0, b0, n_img, ci_tile, grs, wrs);
        // Stride 2, four phases: a phase's pixels are every other float of
        // an input row, so storing each phase by itself writes every cache
        // line in two halves at different moments (twice the output bytes
        // reach HBM).  Instead the four phases' sums meet in LDS, 16 input
        // channels at a time (both groups' wave w), and all threads store
        // whole rows of the 2TR x 2TC input tile, 16 bytes per lane.  (The
        // stages are free: run_fused ends on a barrier after its last reads.)
        const int TT = A.TR * A.TC;
        const size_t lds_bytes = ((size_t)A.stages * (A.Tall * 4 * 64 + 4 * A.HPc) + 128) * 8;
        if (A.stride == 2 && A.nphases == 4 && NPH == 4 && !A.fold && (A.W & 3) == 0 &&
            (A.TC & 1) == 0 && (size_t)256 * TT <= lds_bytes) {
            float *const X = (float *)smem_all;   // [phase][16 channels][TT]
            int pidx[2][2] = {{0, 0}, {0, 0}};
#pragma unroll
            for (int q = 0; q < 4; ++q) pidx[A.ph[q].rho_h & 1][A.ph[q].rho_w & 1] = q;
            const int qpr = A.TC / 2;                 // 16-byte quads per input row of the tile
            const int nquad = 16 * 2 * A.TR * qpr;
            for (int w = 0; w < 4; ++w) {
                if (wave == w) {
#pragma unroll
                    for (int k = 0; k < MP; ++k) {
                        if (myph[k] < 0) continue;
#pragma unroll
                        for (int blk = 0; blk < NB; ++blk) {
                            const int px = blk * 16 + l16;
                            if (px < TT)
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const float v = acc[k][blk][r];
                                    X[(myph[k] * 16 + 4 * g4 + r) * TT + px] = v;
                                }
                        }
                    }
                }
                __syncthreads();
                for (int q = (int)threadIdx.x; q < nquad; q += 256 * KS) {
                    const int cl = q / (2 * A.TR * qpr), rem = q - cl * (2 * A.TR * qpr);
                    const int row = rem / qpr, qc = rem - (rem / qpr) * qpr;
                    const int rh = row & 1, a = row >> 1;
                    const int ih = 2 * a0 + row, iw = 2 * b0 + 4 * qc;
                    const int ci = ci0 + w * 16 + cl;
                    const float *x0 = X + (pidx[rh][0] * 16 + cl) * TT + a * A.TC + 2 * qc;
                    const float *x1 = X + (pidx[rh][1] * 16 + cl) * TT + a * A.TC + 2 * qc;
                    const v4u v = v4u{__float_as_uint(x0[0]), __float_as_uint(x1[0]),
                                      __float_as_uint(x0[1]), __float_as_uint(x1[1])};
                    const int off = (ih < A.H && iw < A.W && ci < A.Ci)
                                        ? (((n_img * A.Ci + ci) * A.H + ih) * A.W + iw) * 4
                                        : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b128(v, drs, off, 0, 0);
                }
                __syncthreads();
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < MP; ++k) {
            if (myph[k] < 0) continue;
            const HaloPhase &P = A.ph[myph[k]];
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                int img, a, b;
                const bool pv = tile_pixel(A, P, blk * 16 + l16, a0, b0, n_img, img, a, b);
                const int pix = (P.rho_h + A.stride * a) * A.W + P.rho_w + A.stride * b;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ci = ci0 + wave * 16 + 4 * g4 + r;
                    const int off =
                        (pv && ci < A.Ci) ? ((img * A.Ci + ci) * plane + pix) * 4 : kOOB;
                    const float v = acc[k][blk][r];
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), drs, off, 0, 0);
                }
            }
        }
        return;
    }

    for (int p = 0; p < A.nphases; ++p) {
        const HaloPhase P = A.ph[p];
        const int T = P.J_h * P.J_w;
        const int HP = PITCH > 0 ? PITCH : A.HP;

        // Halo position of this lane's pixel in each block.  A pixel outside
        // the phase grid reads position l16 (its column is never stored;
        // distinct positions keep the read conflict-free) when every tap's
        // shift keeps that inside the halo plane, else position 0.
        const int max_shift = (P.J_h - 1) * HP + (P.J_w - 1);
        const int inv = l16 + max_shift < A.HPc ? l16 : 0;
        int pbase[NB];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            int img, a, b;
            const int px = blk * 16 + l16;
            pbase[blk] = tile_pixel(A, P, px, a0, b0, n_img, img, a, b)
                             ? (px / A.TC) * HP + (px - (px / A.TC) * A.TC)
                             : inv;
        }

        v4f acc[NB];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) acc[blk] = v4f{0.f, 0.f, 0.f, 0.f};

        // JW < 0: each phase's tap grid is dispatched to a compile-time
        // instance when one exists (else the run-time one below).
        bool done = false;
#define GI_HALO_CASE_JW(TT, JJ)                                                              \
    case TT * 16 + JJ:                                                                       \
        if constexpr ((TMASK & tbit(TT)) != 0) {                                             \
            run_phase<TT, NB, HG, CPS, PITCH, JJ, KS>(A, P, smem2, pbase, acc, a0, b0, n_img,  \
                                                      ci_tile, kg, grs, wrs);                \
            done = true;                                                                     \
        }                                                                                    \
        break;
        if constexpr (JW < 0) {
            switch (T * 16 + P.J_w) {
                GI_HALO_CASE_JW(1, 1)
                GI_HALO_CASE_JW(2, 1)
                GI_HALO_CASE_JW(2, 2)
                GI_HALO_CASE_JW(4, 2)
                default: break;
            }
        }
#undef GI_HALO_CASE_JW
#define GI_HALO_CASE(TT)                                                                     \
    case TT:                                                                                 \
        if constexpr ((TMASK & tbit(TT)) != 0)                                               \
            run_phase<TT, NB, HG, CPS, PITCH, (JW > 0 ? JW : 0), KS>(                          \
                A, P, smem2, pbase, acc, a0, b0, n_img, ci_tile, kg, grs, wrs);              \
        break;
        if (!done) switch (T) {
            GI_HALO_CASE(1)
            GI_HALO_CASE(2)
            GI_HALO_CASE(3)
            GI_HALO_CASE(4)
            GI_HALO_CASE(6)
            GI_HALO_CASE(7)
            GI_HALO_CASE(9)
            default: break;  // T = 0: no taps, the phase's pixels are zero
        }
#undef GI_HALO_CASE

        // Groups past the first hand their sums to the first through LDS
        // (free once every group's last stage is done: run_phase ends on a
        // barrier after its loads have landed), in group order.
        if constexpr (KS > 1) {
            v4f *red = (v4f *)smem_all;
#pragma unroll
            for (int g = 1; g < KS; ++g) {
                if (kg == g)
#pragma unroll
                    for (int blk = 0; blk < NB; ++blk) red[blk * 256 + tid] = acc[blk];
                __syncthreads();
                if (kg == 0)
#pragma unroll
                    for (int blk = 0; blk < NB; ++blk) acc[blk] += red[blk * 256 + tid];
                __syncthreads();
            }
        }
        // Epilogue: D[4*g4 + r][l16] of each block, NCHW.
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            if (KS > 1 && kg != 0) break;
            int img, a, b;
            const bool pv = tile_pixel(A, P, blk * 16 + l16, a0, b0, n_img, img, a, b);
            const int pix = (P.rho_h + A.stride * a) * A.W + P.rho_w + A.stride * b;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ci = ci0 + wave * 16 + 4 * g4 + r;
                const int off = (pv && ci < A.Ci) ? ((img * A.Ci + ci) * plane + pix) * 4 : kOOB;
                // Copy the element to a scalar first: a bit-cast taken directly
                // of a vector element reads element 0 with this compiler.
                const float v = acc[blk][r];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), drs, off, 0, 0);
            }
        }
    }
}

constexpr unsigned kT9 = tbit(9);
constexpr unsigned kT7 = tbit(7);
constexpr unsigned kTs2 = tbit(1) | tbit(2) | tbit(4);
constexpr unsigned kTall = tbit(1) | tbit(2) | tbit(3) | tbit(4) | tbit(6) | tbit(7) | tbit(9);

template <int NB, int HG, unsigned TMASK, int CPS, int OCC, int PITCH, int JW, int KS = 1,
          int NPH = 0>
hipError_t launch_one(const HaloArgs &a, int tiles, int ci_tiles, size_t lds, hipStream_t s,
                      const KernelEvents &ev) {
    // Every group's stages, and the accumulator hand-over of the split.
    const size_t group =
        NPH > 0 ? ((size_t)a.stages * (a.Tall * 4 * 64 + 4 * a.HPc) + 128) * 8
                : ((size_t)a.stages * CPS * (a.maxT * 4 * 64 + 4 * a.HPc) + 128) * 8;
    if (lds < (NPH > 0 ? 1 : KS) * group || (KS > 1 && NPH == 0 && lds < (size_t)NB * 256 * 16))
        return hipErrorInvalidValue;
    if (NPH > 0) {
        // Fused: NPH phases of tap grids up to 2 x 2, the chunk's weights in
        // at most kFusedPieces pieces of 1 KB, the halo in at most 4*KS*HG
        // groups of 32 positions, and every phase in exactly one thread
        // group's list.
        if (a.fused != 1 || a.nphases != NPH || a.Tall * 2 > kFusedPieces ||
            (a.HR * (PITCH > 0 ? PITCH : a.HP) + 31) / 32 > 4 * KS * HG)
            return hipErrorInvalidValue;
        int seen[NPH] = {};
        for (int g = 0; g < KS; ++g)
            for (int k = 0; k < NPH / KS; ++k) {
                const int p = a.gph[g][k];
                if (p >= NPH) return hipErrorInvalidValue;
                if (p >= 0) ++seen[p];
            }
        for (int i = 0; i < NPH; ++i)
            if (a.ph[i].J_h > 2 || a.ph[i].J_w > 2 || seen[i] != 1) return hipErrorInvalidValue;
    } else if (a.fused != 0) {
        return hipErrorInvalidValue;
    }
    if (PITCH > 0 && a.HP != PITCH) return hipErrorInvalidValue;
    // Every phase-at-a-time phase with taps has its tap count in TMASK (a
    // phase the kernel has no case for would be left at zero).
    for (int i = 0; NPH == 0 && i < a.nphases; ++i) {
        const int T = a.ph[i].J_h * a.ph[i].J_w;
        if (T > 0 && (T >= 32 || (TMASK & tbit(T)) == 0)) return hipErrorInvalidValue;
    }
    // JW > 0: every phase with taps has that kernel-width tap count.
    for (int i = 0; JW > 0 && i < a.nphases; ++i)
        if (a.ph[i].J_w != JW && a.ph[i].J_h * a.ph[i].J_w != 0) return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(
            (const void *)gi_halo_f32<NB, HG, TMASK, CPS, OCC, PITCH, JW, KS, NPH>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (a.ci_tiles != ci_tiles) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL((gi_halo_f32<NB, HG, TMASK, CPS, OCC, PITCH, JW, KS, NPH>),
                          dim3(tiles * ci_tiles), dim3(256 * KS), (uint32_t)lds, s, ev.start,
                          ev.stop, 0, a);
    return hipGetLastError();
}

// Instantiations: pixel blocks, halo groups of 32 positions per wave, tap
// counts served, chunks of 8 output channels per LDS stage (the 4-chunk
// kernel holds one work-group per CU by LDS, so it is compiled for one wave
// per SIMD and the whole register file), and the halo pitch and kernel width
// when fixed at compile time (pitch 0: read at run time; jw -1: each phase's
// tap grid dispatched to a compile-time instance).  Served at fixed pitch:
// 3 x 3 stride-1 kernels on 14-wide tiles (conflict-free pitch 30) and
// 28-wide ones (30), 1 x 7 kernels on 17-wide tiles (conflict-free 33, or
// 23), and the four phases of 3 x 3 stride-2 kernels on 14-wide tiles (15).
// ks: thread groups splitting the output channels (two for a 1 x 7 instance:
// a 17 x 17 image batch of 32 gives fewer work-groups than compute units).
// nph > 0: fused launches of that many phases (tap grids up to 2 x 2; the
// 3 x 3 stride-2 ones at pitch 15 on 14-wide tiles, fixed, or any pitch),
// ks then the thread groups sharing each stage, each with nph / ks phases.
struct HaloCfg {
    int nb, hg;
    unsigned tmask;
    int cps, pitch, jw, ks, nph;
};
constexpr HaloCfg kCfg[] = {
    {13, 4, kT9, 1, 30, 3, 1, 0},   {13, 2, kT9, 1, 0, 0, 1, 0},   {13, 2, kTs2, 4, 15, -1, 1, 0},
    {13, 2, kTs2, 4, 0, 0, 1, 0},   {8, 2, kT7, 1, 33, 7, 1, 0},   {8, 2, kT7, 1, 23, 7, 1, 0},
    {8, 2, kT7, 1, 0, 0, 1, 0},     {13, 4, kTall, 1, 0, 0, 1, 0}, {8, 4, kTall, 1, 0, 0, 1, 0},
    {4, 4, kTall, 1, 0, 0, 1, 0},   {8, 2, kT7, 1, 23, 7, 2, 0},   {13, 1, kTs2, 1, 15, 0, 2, 4},
    {8, 1, kTs2, 1, 15, 0, 2, 4},   {13, 2, kTs2, 1, 0, 0, 2, 4},
};

}  // namespace

unsigned halo_f32_tbit(int T) { return T >= 1 && T < 32 ? tbit(T) & kTall : 0u; }

int halo_f32_config(int nb, unsigned tmask, int hg, int hp, int jw, int ks, int nph) {
    for (int i = 0; i < (int)(sizeof(kCfg) / sizeof(kCfg[0])); ++i) {
        const HaloCfg &c = kCfg[i];
        if (c.nb != nb || c.ks != ks || c.nph != nph || c.hg < hg || (c.tmask & tmask) != tmask)
            continue;
        if (nph > 0) {
            if (c.pitch == 0 || c.pitch == hp) return i;
            continue;
        }
        if (c.pitch == 0 || (c.pitch == hp && (c.jw == jw || c.jw < 0))) return i;
    }
    return -1;
}

int halo_f32_cps(int cfg) { return kCfg[cfg].cps; }

int halo_f32_ks(int cfg) { return kCfg[cfg].ks; }

bool halo_f32_fixed_pitch(int cfg) { return kCfg[cfg].pitch > 0; }

int halo_f32_nph(int cfg) { return kCfg[cfg].nph; }

size_t halo_f32_lds_bytes(int maxT, int HPc, int stages, int cps) {
    // stages x (weights + halos of cps chunks), plus the kilobyte the
    // surplus loads write.
    return ((size_t)stages * cps * (maxT * 4 * 64 + 4 * HPc) + 128) * sizeof(v2f);
}

hipError_t launch_halo_f32(const HaloArgs &a, int cfg, int tiles, int ci_tiles, size_t lds,
                           hipStream_t s, const KernelEvents &ev) {
    switch (cfg) {
        case 0: return launch_one<13, 4, kT9, 1, 2, 30, 3>(a, tiles, ci_tiles, lds, s, ev);
        case 1: return launch_one<13, 2, kT9, 1, 2, 0, 0>(a, tiles, ci_tiles, lds, s, ev);
        case 2: return launch_one<13, 2, kTs2, 4, 1, 15, -1>(a, tiles, ci_tiles, lds, s, ev);
        case 3: return launch_one<13, 2, kTs2, 4, 1, 0, 0>(a, tiles, ci_tiles, lds, s, ev);
        case 4: return launch_one<8, 2, kT7, 1, 2, 33, 7>(a, tiles, ci_tiles, lds, s, ev);
        case 5: return launch_one<8, 2, kT7, 1, 2, 23, 7>(a, tiles, ci_tiles, lds, s, ev);
        case 6: return launch_one<8, 2, kT7, 1, 2, 0, 0>(a, tiles, ci_tiles, lds, s, ev);
        case 7: return launch_one<13, 4, kTall, 1, 2, 0, 0>(a, tiles, ci_tiles, lds, s, ev);
        case 8: return launch_one<8, 4, kTall, 1, 2, 0, 0>(a, tiles, ci_tiles, lds, s, ev);
        case 9: return launch_one<4, 4, kTall, 1, 2, 0, 0>(a, tiles, ci_tiles, lds, s, ev);
        case 10: return launch_one<8, 2, kT7, 1, 2, 23, 7, 2>(a, tiles, ci_tiles, lds, s, ev);
        case 11: return launch_one<13, 1, kTs2, 1, 2, 15, 0, 2, 4>(a, tiles, ci_tiles, lds, s, ev);
        case 12: return launch_one<8, 1, kTs2, 1, 2, 15, 0, 2, 4>(a, tiles, ci_tiles, lds, s, ev);
        case 13: return launch_one<13, 2, kTs2, 1, 2, 0, 0, 2, 4>(a, tiles, ci_tiles, lds, s, ev);
        default: return hipErrorInvalidValue;
    }
}

// Weight image [ci_tile][phase][chunk][tap][cp][ci'][2] (fused launches:
// [ci_tile][chunk][tb + tap][cp][ci'][2]), zero where ci >= Ci or co >= Co; ci' = (ci + 16 * (cp & 1)) mod 64, a rotation that puts the
// fragment reads of neighbouring co pairs on disjoint LDS banks.  One thread
// per float4 of the image (input channels 2q, 2q+1 x output channels 2cp,
// 2cp+1 of one tap): four independent loads and one store, so the whole
// image costs about one memory round trip.  Grid: (float4s of the largest
// phase block / 256, phases, ci tiles).
__global__ __launch_bounds__(256) void weight_image_f32(const float *__restrict__ w,
                                                        float *__restrict__ wk, const HaloArgs A,
                                                        int kH, int kW) {
    const int p = blockIdx.y, ct = blockIdx.z;
    const HaloPhase &P = A.ph[p];
    const int T = P.J_h * P.J_w;
    const int e = blockIdx.x * 256 + threadIdx.x;  // float4 within the phase block
    if (e >= A.nchunks * T * 128) return;
    const int qr = e & 31, cp = (e >> 5) & 3;
    const int tap = (e >> 7) % T, chunk = (e >> 7) / T;
    const int q = (qr - 8 * (cp & 1)) & 31;  // undo the rotation
    const int j = tap / P.J_w, jw = tap - (tap / P.J_w) * P.J_w;
    const int t = (P.r_h + A.stride * j) * kW + P.r_w + A.stride * jw;
    const int kHW = kH * kW;
    const int ci0 = ct * kHalo64 + 2 * q, co0 = chunk * kHaloBC + 2 * cp;
    auto ld = [&](int co, int ci) {
        return (co < A.Co && ci < A.Ci) ? w[((int64_t)co * A.Ci + ci) * kHW + t] : 0.f;
    };
    const v4f v = {ld(co0, ci0), ld(co0 + 1, ci0), ld(co0, ci0 + 1), ld(co0 + 1, ci0 + 1)};
    // Fused launches read one chunk of every phase as one block.
    const int64_t at = A.fused ? (int64_t)(chunk * A.Tall + P.tb + tap) * 128 + (e & 127)
                               : (int64_t)P.woff / 4 + e;
    ((v4f *)(wk + (int64_t)ct * A.w_ci_stride))[at] = v;
}

hipError_t launch_weight_image_f32(const float *w, float *wk, const HaloArgs &a, int kH, int kW,
                                   int ci_tiles, int64_t total, hipStream_t s) {
    (void)total;
    int most = 0;
    for (int p = 0; p < a.nphases; ++p)
        most = std::max(most, a.nchunks * a.ph[p].J_h * a.ph[p].J_w * 128);
    if (most == 0) return hipSuccess;
    hipLaunchKernelGGL(weight_image_f32, dim3((most + 255) / 256, a.nphases, ci_tiles),
                       dim3(256), 0, s, w, wk, a, kH, kW);
    return hipGetLastError();
}

}  // namespace gi
