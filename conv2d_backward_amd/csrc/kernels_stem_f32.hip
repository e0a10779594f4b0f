// kernels_stem_f32.hip -- fp32 implicit-GEMM kernel for few input channels
// (Ci <= 4, e.g. an RGB stem) on gfx950.
//
// The contraction is the implicit GEMM of meganeura conv2d_grad_input_gemm.wgsl
// (header comment: C[Ci, pixels] = A[Ci, K] x B[K, pixels], K = Co*kH*kW),
// taken one residue class of the stride at a time (see gi_common.h).  With
// Ci <= 4 the wide matrix-core shapes would be mostly padding, so the kernel
// uses V_MFMA_F32_4X4X1_16B_F32: 16 independent 4x4x1 blocks per instruction.
// Block b of an instruction has rows = the 4 input channels (A, the weights)
// and columns = 4 pixels (B, grad_out); lane l supplies A[b][l%4] and B[b][l%4]
// with b = l/4, and receives D[b][r][l%4] in register r.  So lane l's column
// is pixel l of the wave's 64-pixel block, and after the contraction lane l
// holds input channels 0..3 of its own pixel.
//
// Work-group: up to 4 waves over a 16 x 16 tile of the phase grids.  The
// phases are paired into groups of near-equal total taps (for a 7 x 7
// stride-2 kernel: 4x4 with 3x3, 3x4 with 4x3), and a work-group runs up to
// two groups side by side, waves 2g and 2g+1 on group g, each over 8 tile
// rows as two 4 x 16 pixel blocks.  Output channels are streamed 4 at a time
// through a 3-stage LDS pipeline filled by direct global -> LDS loads: per
// stage one grad_out halo for the 4 channels that covers every phase of the
// work-group (a position's 4 channels are one 16-byte word, so one LDS read
// serves 4 MFMAs), and the chunk's weights of every tap of those phases (a
// 16-byte word per (tap, input channel) holding its 4 output channels; the
// 64 lanes read 4 distinct words, a broadcast).  Loading one halo for all
// the phases rather than one per phase cuts the direct loads per MFMA to
// about a third: their issue, not the memory traffic, was what kept the
// matrix cores waiting.  The weights are gathered by the same direct loads
// from the caller's [Co][Ci][kH][kW] tensor, 4 bytes per lane, so no
// reordered copy (and no prologue launch) is needed; they come through LDS
// rather than from memory per tap, since a 16-byte-per-lane load per tap for
// 4 distinct values would keep the texture units of the CU busy for longer
// than the matrix cores.  When the halo pitch and the tap grid are
// compile-time constants every tap's shift is an immediate offset of the
// fragment reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_common.h"
#include "gi_launch.h"

namespace gi {

typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9)
constexpr int kOOB = 0x7ffffff0;         // byte offset past the end of every buffer
constexpr int kStemTile = 16;            // tile side in phase-grid pixels
constexpr int kStemStages = 3;           // LDS pipeline stages

typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (long)bytes, kRsrcWord3);
}

template <int N>
__device__ __forceinline__ void wait_dma() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Column (0..15) of tile row `row` handled by lane: lane l = 16r + j takes
// column (j - row * pitch) mod 16, so its halo position row * pitch + column
// is j mod 16 plus a constant for every lane of a fragment read.  A 16-byte
// LDS read is served 16 lanes per cycle, and on gfx950 the lanes of a cycle
// are, within each half wave, those whose index bits 2..4 have the same
// parity: rows r and r+1 then contribute complementary column quads, i.e.
// 16 different j, i.e. 16 different bank groups, whatever the pitch.  (With
// column j the rows' positions overlap mod 16 unless the pitch is a multiple
// of 16.)
__device__ __forceinline__ int stem_column(int lane, int row, int pitch) {
    return ((lane & 15) - row * pitch) & 15;
}

// Halo shift of tap t of a phase with taps J_h x J_w: (J_h-1-j) rows and
// (J_w-1-jw) columns.
template <int T>
__device__ __forceinline__ void tap_shifts(int (&shift)[T], int J_h, int J_w, int HP) {
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

// The taps of one phase over one staged chunk of 4 output channels, for NB
// pixel blocks of this wave.  JW > 0 fixes the phase's tap columns and
// PITCH > 0 the halo row pitch at compile time (they must equal the run-time
// values); every tap's shift is then an immediate offset of the fragment
// reads.  hs: the stage's halo; as: the phase's first tap in the stage's
// weights, offset by this lane's input channel; pb: this lane's halo
// position in each block, including the phase's origin in the halo.
//
// Accumulators: two per pixel block (even and odd output channels of the
// chunk), so consecutive MFMAs never depend on each other; the other
// waves of the SIMD cover the rest of the 4x4x1 latency.
template <int T, int JW, int PITCH, int NB>
__device__ __forceinline__ void stem_taps(const v4f *hs, const v4f *as, const int (&pb)[NB],
                                          int J_h_rt, int J_w_rt, int HP_rt,
                                          v4f (&acc)[NB][2]) {
    const int J_w = JW > 0 ? JW : J_w_rt;
    const int J_h = JW > 0 ? T / (JW > 0 ? JW : 1) : J_h_rt;
    const int HP = PITCH > 0 ? PITCH : HP_rt;
    int shift[T];
    tap_shifts<T>(shift, J_h, J_w, HP);
    int pp[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
        pp[blk] = pb[blk];
        asm volatile("" : "+v"(pp[blk]));
    }
    // B fragments two taps ahead (three slots), A one tap ahead.
    v4f fb[3][NB], fa[2];
    auto bfetch = [&](int t, int sl) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) fb[sl][blk] = hs[pp[blk] + shift[t]];
    };
    bfetch(0, 0);
    fa[0] = as[0];
    if (T > 1) bfetch(1, 1);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if (t + 2 < T) bfetch(t + 2, (t + 2) % 3);
        if (t + 1 < T) fa[(t + 1) & 1] = as[(t + 1) * 4];
        const int sl = t % 3;
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
                acc[blk][e & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(
                    fa[t & 1][e], fb[sl][blk][e], acc[blk][e & 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One phase's taps for one chunk, dispatched to a compile-time tap grid.
template <int PITCH, int NB>
__device__ __forceinline__ void stem_phase_chunk(const StemPhase &P, const v4f *hs,
                                                 const v4f *as, const int (&pb)[NB], int HP,
                                                 v4f (&acc)[NB][2]) {
    const int T = P.J_h * P.J_w;
    // Compile-time tap grids of the 7 x 7 stride-2 phases when the pitch is
    // fixed; everything else through the run-time instances.
    if constexpr (PITCH > 0) {
        switch (T * 16 + P.J_w) {
            case 9 * 16 + 3: stem_taps<9, 3, PITCH, NB>(hs, as, pb, P.J_h, P.J_w, HP, acc); return;
            case 12 * 16 + 3: stem_taps<12, 3, PITCH, NB>(hs, as, pb, P.J_h, P.J_w, HP, acc); return;
            case 12 * 16 + 4: stem_taps<12, 4, PITCH, NB>(hs, as, pb, P.J_h, P.J_w, HP, acc); return;
            case 16 * 16 + 4: stem_taps<16, 4, PITCH, NB>(hs, as, pb, P.J_h, P.J_w, HP, acc); return;
            default: break;
        }
    }
#define GI_STEM_CASE(TT)                                                   \
    case TT:                                                               \
        stem_taps<TT, 0, PITCH, NB>(hs, as, pb, P.J_h, P.J_w, HP, acc);    \
        return;
    switch (T) {
        GI_STEM_CASE(1)
        GI_STEM_CASE(2)
        GI_STEM_CASE(3)
        GI_STEM_CASE(4)
        GI_STEM_CASE(6)
        GI_STEM_CASE(8)
        GI_STEM_CASE(9)
        GI_STEM_CASE(12)
        GI_STEM_CASE(16)
        default: return;  // no taps: the phase's pixels are zero
    }
#undef GI_STEM_CASE
}

// The work of one wave over a tile: phases myph (up to two, -1 for none) of
// NB pixel blocks of 4 x 16 starting at tile row row0.  Every wave of the
// work-group runs it (it contains the work-group's barriers and its share of
// the direct loads).  G: halo loads of 16 positions per wave and stage (the
// stage's halo region is NW * G * 16 = A.HPmax positions).
//
// Per chunk of 4 output channels, one 3-stage LDS pipeline stage holds the
// halo that covers every phase of the set (a position's 4 channels are one
// 16-byte word: one LDS read serves 4 MFMAs) and the weights of every tap of
// the set (a 16-byte word per (tap, input channel) holding its 4 output
// channels; the 64 lanes read 4 distinct words, a broadcast).  Both are
// filled by direct loads, 4 bytes per lane, the weights gathered from the
// caller's [Co][Ci][kH][kW] tensor.  Every load writes its own slot of the
// stage it fills, also past the last chunk (that stage is not read again;
// such loads read zeros or unused weights), so the issue carries no
// per-load selects, and every wave issues the same fixed number of loads
// per stage, so "this stage has landed" is a wait on a compile-time count.
template <int PITCH, int G, int NW, int NB>
__device__ __forceinline__ void stem_tile(const StemArgs &A, v4f *sm4, int n, int a0, int b0,
                                          int set, const int (&myph)[2], int row0) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(A.grad_out, A.g_bytes);
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(A.w, A.w_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(A.dst, A.d_bytes);
    const int HP = PITCH > 0 ? PITCH : A.pitch;
    const int oHW = A.oH * A.oW;
    constexpr int kWT = NW * kStemTapsPerWave;  // staged taps
    const int stage = A.HPmax + 4 * kWT;        // v4f per stage
    constexpr int kWP = 4;                      // weight pieces of 64 floats per wave
    constexpr int kDma = G + kWP;               // direct loads per wave and stage
    static_assert(kDma <= 63, "vmcnt holds at most 63");
    static_assert(NW * kWP * 64 == 16 * kWT, "weight pieces cover the staged taps");

    // Halo DMA: group q = wave + NW*k covers positions 16q .. 16q+15 of the
    // set's halo; lane -> (position 16q + lane/4, channel lane%4).
    // Positions past the halo or its columns, or outside the image, get an
    // offset past the buffer.
    const int org_h = A.set_org[set][0], org_w = A.set_org[set][1];
    const int ext_h = A.set_ext[set][0], ext_w = A.set_ext[set][1];
    int goff[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
        const int q = wave + NW * k;
        const int pos = q * 16 + (lane >> 2);
        const int hr = pos / HP, hc = pos - (pos / HP) * HP;
        const int oh = a0 + org_h + hr;
        const int ow = b0 + org_w + hc;
        const bool v = hr < ext_h && hc < ext_w && oh >= 0 && oh < A.oH && ow >= 0 && ow < A.oW;
        goff[k] = v ? ((n * A.Co) * oHW + oh * A.oW + ow) * 4 : kOOB;
    }
    const int co_l = lane & 3;
    // Weights of a chunk in LDS: float (tap * 4 + ci) * 4 + co over the set's
    // taps (each phase from its first tap tb on), i.e. piece k of 64 floats
    // holds taps 4k .. 4k+3; wave w loads pieces w + NW*u.  Lane i of piece
    // k reads weight[chunk*4 + i%4][(i/4)%4][kh][kw] of tap 4k + i/16 (an
    // offset past the buffer, i.e. zero, for ci >= Ci or a tap no phase of
    // the set has; a channel past Co lies past the buffer by itself).
    const int kHW = A.kH * A.kW;
    int wofs[kWP];
#pragma unroll
    for (int u = 0; u < kWP; ++u) {
        const int tap = 4 * (wave + NW * u) + (lane >> 4);
        const int ci = (lane >> 2) & 3;
        int off = (int)A.w_bytes;
        for (int g = 0; g < kStemGroupsPerWg; ++g) {
            const int gg = set * kStemGroupsPerWg + g;
            if (gg >= A.ngroups) break;
            for (int k = 0; k < 2; ++k) {
                const int p = A.group[gg][k];
                if (p < 0) continue;
                const StemPhase &P = A.ph[p];
                const int t = tap - P.tb;
                if (t < 0 || t >= P.J_h * P.J_w || ci >= A.Ci) continue;
                const int j = t / P.J_w, jw = t - (t / P.J_w) * P.J_w;
                const int kh = P.r_h + A.stride * j, kw = P.r_w + A.stride * jw;
                off = ((co_l * A.Ci + ci) * kHW + kh * A.kW + kw) * 4;
            }
        }
        wofs[u] = off;
    }
    const int chunk_w = 4 * A.Ci * kHW * 4;  // bytes of 4 output channels
    auto issue = [&](int chunk, int buf) {
        // Channel part of this lane's offset; the buffer size (an offset past
        // its end) for a channel past Co or a chunk past the last.  Offsets
        // stay below 2^32: goff <= kOOB < 2^31 and this part <= g_bytes < 2^31.
        const int co = chunk * 4 + co_l;
        const int cc = (chunk < A.nchunks && co < A.Co) ? co * oHW * 4 : (int)A.g_bytes;
        v4f *st = sm4 + buf * stage;
#pragma unroll
        for (int k = 0; k < G; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                grs, (lds_ptr_t)(st + (wave + NW * k) * 16), 4, goff[k] + cc, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kWP; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wrs, (lds_ptr_t)(st + A.HPmax + (wave + NW * u) * 16), 4, wofs[u],
                chunk * chunk_w, 0, 0);
    };

    // Halo position of this lane's pixel in each block (column from
    // stem_column), per phase with the phase's origin in the set's halo.
    int pb[2][NB];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int p = myph[k] < 0 ? 0 : myph[k];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const int row = row0 + 4 * blk + (lane >> 4);
            pb[k][blk] = (row + A.ph[p].dr) * HP + A.ph[p].dc + stem_column(lane, row, HP);
        }
    }

    v4f acc[2][NB][2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
            acc[k][blk][0] = acc[k][blk][1] = v4f{0.f, 0.f, 0.f, 0.f};

    issue(0, 0);
    issue(1, 1);
    wait_dma<kDma>();
    __syncthreads();
    static_assert(kStemStages == 3, "stage rotation below");
    int cur = 0;
    for (int chunk = 0; chunk < A.nchunks; ++chunk) {
        const int ahead = cur == 0 ? 2 : cur - 1;  // (chunk + 2) mod 3
        issue(chunk + 2, ahead);
        const v4f *hs = sm4 + cur * stage;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (myph[k] < 0) continue;
            const StemPhase &P = A.ph[myph[k]];
            stem_phase_chunk<PITCH, NB>(P, hs, hs + A.HPmax + P.tb * 4 + co_l, pb[k], HP,
                                        acc[k]);
        }
        // Stage chunk+1 must have landed; the loads of chunk+2 may still be
        // in flight.
        wait_dma<kDma>();
        __syncthreads();
        cur = cur == 2 ? 0 : cur + 1;
    }
    // Nothing may still write LDS when the work-group ends.
    wait_dma<0>();

    // Epilogue: lane l holds input channels 0..3 of its pixel of each block.
    const int plane = A.H * A.W;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (myph[k] < 0) continue;
        const StemPhase &P = A.ph[myph[k]];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const int row = row0 + 4 * blk + (lane >> 4);
            const int a = a0 + row;
            const int b = b0 + stem_column(lane, row, HP);
            const bool pv = a < P.Ha && b < P.Wb;
            const int pix = (P.rho_h + A.stride * a) * A.W + P.rho_w + A.stride * b;
            const v4f sum = acc[k][blk][0] + acc[k][blk][1];
#pragma unroll
            for (int ci = 0; ci < 4; ++ci) {
                const int off = (pv && ci < A.Ci) ? ((n * A.Ci + ci) * plane + pix) * 4 : kOOB;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum[ci]), drs, off, 0, 0);
            }
        }
    }
}

// Work-groups: NW = 2 * (phase groups per set) waves.  The first A.nfull
// work-groups each take a whole (image, tile, set): waves 2g and 2g+1 run
// group g over 8 tile rows each (two pixel blocks).  The remaining ones
// (present only with one set per tile) each take a quarter of one of the
// tiles left over: 4 tile rows, wave w running the w-th phase of the set on
// one pixel block.  Spreading those last tiles as quarters keeps every
// compute unit's share of the grid within a quarter tile of the others'.
template <int PITCH, int G, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4))) void gi_stem_f32(
    const StemArgs A) {
    extern __shared__ __attribute__((aligned(16))) v4f sm4[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool quarter = (int)blockIdx.x >= A.nfull;
    // Logical order within each part: set (or quarter) fastest, then tile
    // column, row, image.
    int bid, set = 0, qr = 0;
    if (!quarter) {
        bid = xcd_order(blockIdx.x, A.nfull);
        set = bid % A.nsets;
        bid /= A.nsets;
    } else {
        bid = xcd_order(blockIdx.x - A.nfull, gridDim.x - A.nfull);
        qr = bid & 3;
        bid = A.nfull + (bid >> 2);
    }
    const int tc = bid % A.tiles_c;
    bid /= A.tiles_c;
    const int tr = bid % A.tiles_r;
    const int n = bid / A.tiles_r;
    const int a0 = tr * kStemTile, b0 = tc * kStemTile;

    if (!quarter) {
        // This wave's group and its phases (-1: none).
        const int grp = set * kStemGroupsPerWg + wave / 2;
        int myph[2] = {-1, -1};
        if (grp < A.ngroups) {
            myph[0] = A.group[grp][0];
            myph[1] = A.group[grp][1];
        }
        stem_tile<PITCH, G, NW, 2>(A, sm4, n, a0, b0, set, myph, 8 * (wave & 1));
    } else {
        // The wave-th phase of the (only) set.
        int myph[2] = {-1, -1};
        int k = 0;
        for (int g = 0; g < kStemGroupsPerWg && g < A.ngroups; ++g)
            for (int e = 0; e < 2; ++e)
                if (A.group[g][e] >= 0 && k++ == wave) myph[0] = A.group[g][e];
        stem_tile<PITCH, G, NW, 1>(A, sm4, n, a0, b0, 0, myph, 4 * qr);
    }
}

}  // namespace

bool stem_f32_taps_ok(int taps) {
    switch (taps) {
        case 0: case 1: case 2: case 3: case 4: case 6: case 8: case 9: case 12: case 16:
            return true;
        default:
            return false;
    }
}

// Halo pitch fixed at compile time: 19 positions holds the halo of every
// phase of a 7 x 7 kernel at stride 2 (tap grids 3 or 4 wide, all with the
// same origin); 20 rows of it fit 24 loads of 16 positions per stage.
// Otherwise 32 such loads (halos of up to 512 positions) and the pitch is
// read at run time.
constexpr int kStemPitch = 19;
constexpr int kStemFixedPositions = 384;
constexpr int kStemPositions = 512;

int stem_f32_fixed_pitch() { return kStemPitch; }

int stem_f32_halo_positions(int pitch) {
    return pitch == kStemPitch ? kStemFixedPositions : kStemPositions;
}

int stem_f32_waves(int ngroups) { return 2 * (ngroups >= kStemGroupsPerWg ? kStemGroupsPerWg : 1); }

size_t stem_f32_lds_bytes(int hpmax, int waves) {
    return (size_t)kStemStages * (hpmax + 4 * waves * kStemTapsPerWave) * sizeof(v4f);
}

hipError_t launch_stem_f32(const StemArgs &a, hipStream_t s, const KernelEvents &ev) {
    if (a.HPmax != stem_f32_halo_positions(a.pitch)) return hipErrorInvalidValue;
    const int nw = stem_f32_waves(a.ngroups);
    if (a.nsets != (a.ngroups + kStemGroupsPerWg - 1) / kStemGroupsPerWg) return hipErrorInvalidValue;
    const size_t lds = stem_f32_lds_bytes(a.HPmax, nw);
    const int64_t units = (int64_t)a.N * a.tiles_r * a.tiles_c * a.nsets;
    if (a.nfull > units || (a.nfull < units && a.nsets != 1)) return hipErrorInvalidValue;
    const int64_t wgs = a.nfull + 4 * (units - a.nfull);
    if (lds > 64 * 1024) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs), block(64 * nw);
    const uint32_t sh = (uint32_t)lds;
    if (a.pitch == kStemPitch && nw == 4)
        hipExtLaunchKernelGGL((gi_stem_f32<kStemPitch, kStemFixedPositions / 64, 4>), grid, block,
                              sh, s, ev.start, ev.stop, 0, a);
    else if (a.pitch == kStemPitch)
        hipExtLaunchKernelGGL((gi_stem_f32<kStemPitch, kStemFixedPositions / 32, 2>), grid, block,
                              sh, s, ev.start, ev.stop, 0, a);
    else if (nw == 4)
        hipExtLaunchKernelGGL((gi_stem_f32<0, kStemPositions / 64, 4>), grid, block, sh, s,
                              ev.start, ev.stop, 0, a);
    else
        hipExtLaunchKernelGGL((gi_stem_f32<0, kStemPositions / 32, 2>), grid, block, sh, s,
                              ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

}  // namespace gi
