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
// Work-group: 128 threads = 2 waves over a 16 x 16 tile of the phase grid,
// for one or two phases in turn (pairs of near-equal total taps, so every
// work-group does about the same work and the grid runs in one round
// without a ragged tail); wave w owns tile rows 8w .. 8w+7 as two 4 x 16
// pixel blocks.  Output
// channels are streamed 4 at a time through a 3-stage LDS pipeline filled by
// direct global -> LDS loads: per stage the tile's grad_out halo for the 4
// channels (a position's 4 channels are one 16-byte word, so one LDS read
// serves 4 MFMAs) and the chunk's weights of every tap (a 16-byte word per
// (tap, input channel) holding its 4 output channels; the 64 lanes read 4
// distinct words, a broadcast).  The weights are gathered by the same direct
// loads from the caller's [Co][Ci][kH][kW] tensor, 4 bytes per lane, so no
// reordered copy (and no prologue launch) is needed; they come through LDS
// rather than from memory per tap, since a 16-byte-per-lane load per tap for
// 4 distinct values would keep the texture units of the CU busy for longer
// than the matrix cores.  When the halo pitch and the tap grid are compile-time constants
// every tap's shift is an immediate offset of the fragment reads.
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
constexpr int kStemA = 64;               // v4f of weights per stage (taps x 4 <= 64)

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

// One phase with T taps (compile time) for this work-group's tile.  JW > 0
// fixes the phase's tap columns and PITCH > 0 the halo row pitch at compile
// time (they must equal P.J_w and A.pitch); 0 reads them at run time.  G:
// halo loads of 16 positions per wave and stage; the stage's halo region is
// 2G x 16 = A.HPmax positions, at least the phase's halo.
//
// Accumulators: one per (output channel of the chunk, pixel block), so the
// 8 MFMAs of a tap are independent and each chain advances once per tap (a
// 4x4x1 MFMA that depends on the one issued just before it stalls).
//
// LDS stage (v4f): halo [HPmax positions], then weights [kStemA].  Every
// load writes its own slot of the stage it fills, also past the last chunk
// (that stage is not read again; such loads read zeros or unused weights),
// so the issue carries no per-load selects.
template <int T, int JW, int PITCH, int G>
__device__ __forceinline__ void stem_phase(const StemArgs &A, const StemPhase &P, v4f *sm4,
                                           v4f (&acc)[4][2], int n, int a0, int b0,
                                           __amdgpu_buffer_rsrc_t grs,
                                           __amdgpu_buffer_rsrc_t wrs) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int J_w = JW > 0 ? JW : P.J_w;
    const int J_h = JW > 0 ? T / (JW > 0 ? JW : 1) : P.J_h;
    const int HP = PITCH > 0 ? PITCH : A.pitch;
    const int HC = kStemTile + J_w - 1;
    const int HR = kStemTile + J_h - 1;
    const int hpos = HR * HP;
    const int oHW = A.oH * A.oW;
    const int stage = A.HPmax + kStemA;  // v4f per stage
    // Direct loads per wave and stage: the halo groups and two weight pieces.
    constexpr int kWP = 2;  // weight pieces of 64 floats per wave: 4 x 64 >= 16 taps x 16
    constexpr int kDma = G + kWP;
    static_assert(kDma <= 63, "vmcnt holds at most 63");

    // Halo DMA: group q = wave + 2k covers positions 16q .. 16q+15; lane ->
    // (position 16q + lane/4, channel lane%4).  Positions past the halo or
    // its columns, or outside the image, get an offset past the buffer.
    int goff[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
        const int q = wave + 2 * k;
        const int pos = q * 16 + (lane >> 2);
        const int hr = pos / HP, hc = pos - (pos / HP) * HP;
        const int oh = a0 + P.q_h - (J_h - 1) + hr;
        const int ow = b0 + P.q_w - (J_w - 1) + hc;
        const bool v = pos < hpos && hc < HC && oh >= 0 && oh < A.oH && ow >= 0 && ow < A.oW;
        goff[k] = v ? ((n * A.Co) * oHW + oh * A.oW + ow) * 4 : kOOB;
    }
    const int co_l = lane & 3;
    // Weights of a chunk in LDS: float (tap * 4 + ci) * 4 + co, i.e. piece k
    // of 64 floats holds taps 4k .. 4k+3; wave w loads pieces w and w + 2.
    // Lane i of piece k reads weight[chunk*4 + i%4][(i/4)%4][kh][kw] of tap
    // 4k + i/16 (an offset past the buffer, i.e. zero, for ci >= Ci or a tap
    // past T; a channel past Co lies past the buffer by itself).
    const int kHW = A.kH * A.kW;
    int wofs[kWP];
#pragma unroll
    for (int u = 0; u < kWP; ++u) {
        const int tap = 4 * (wave + 2 * u) + (lane >> 4);
        const int ci = (lane >> 2) & 3;
        const int j = tap / J_w, jw = tap - (tap / J_w) * J_w;
        const int kh = P.r_h + A.stride * j, kw = P.r_w + A.stride * jw;
        wofs[u] = (tap < T && ci < A.Ci) ? ((co_l * A.Ci + ci) * kHW + kh * A.kW + kw) * 4
                                          : (int)A.w_bytes;
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
                grs, (lds_ptr_t)(st + (wave + 2 * k) * 16), 4, goff[k] + cc, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kWP; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wrs, (lds_ptr_t)(st + A.HPmax + (wave + 2 * u) * 16), 4, wofs[u],
                chunk * chunk_w, 0, 0);
    };

    // Halo position of this lane's pixel in each block (column from
    // stem_column), and tap shifts.
    int pb[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int row = 8 * wave + 4 * blk + (lane >> 4);
        pb[blk] = row * HP + stem_column(lane, row, HP);
    }
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

    wait_dma<0>();  // the previous phase's loads and stores count too: drain them
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
        const v4f *as = hs + A.HPmax + co_l;
        int pp[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            pp[blk] = pb[blk];
            asm volatile("" : "+v"(pp[blk]));
        }
        // B fragments two taps ahead (three slots), A one tap ahead.
        v4f fb[3][2], fa[2];
        auto bfetch = [&](int t, int sl) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) fb[sl][blk] = hs[pp[blk] + shift[t]];
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
                for (int blk = 0; blk < 2; ++blk)
                    acc[e][blk] = __builtin_amdgcn_mfma_f32_4x4x1f32(
                        fa[t & 1][e], fb[sl][blk][e], acc[e][blk], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Stage chunk+1 must have landed; the loads of chunk+2 may still be
        // in flight.
        wait_dma<kDma>();
        __syncthreads();
        cur = cur == 2 ? 0 : cur + 1;
    }
    // Nothing may still write LDS that a later phase or work-group uses.
    wait_dma<0>();
}

template <int PITCH, int G>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(4))) void gi_stem_f32(
    const StemArgs A) {
    extern __shared__ __attribute__((aligned(16))) v4f sm4[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // Logical order: phase group fastest, then tile column, row, image.
    int bid = xcd_order(blockIdx.x, gridDim.x);
    const int grp = bid % A.ngroups;
    bid /= A.ngroups;
    const int tc = bid % A.tiles_c;
    bid /= A.tiles_c;
    const int tr = bid % A.tiles_r;
    const int n = bid / A.tiles_r;
    const int a0 = tr * kStemTile, b0 = tc * kStemTile;
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(A.grad_out, A.g_bytes);
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(A.w, A.w_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(A.dst, A.d_bytes);
    const int plane = A.H * A.W;

    for (int k = 0; k < 2; ++k) {
        const int p = A.group[grp][k];
        if (p < 0) break;
        const StemPhase P = A.ph[p];
        const int T = P.J_h * P.J_w;

        v4f acc[4][2];
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) acc[e][blk] = v4f{0.f, 0.f, 0.f, 0.f};
        // Compile-time tap grids of the 7 x 7 stride-2 phases when the pitch is
        // fixed; everything else through the run-time instances.
        bool done = false;
        if constexpr (PITCH > 0) {
            switch (T * 16 + P.J_w) {
                case 9 * 16 + 3: stem_phase<9, 3, PITCH, G>(A, P, sm4, acc, n, a0, b0, grs, wrs); done = true; break;
                case 12 * 16 + 3: stem_phase<12, 3, PITCH, G>(A, P, sm4, acc, n, a0, b0, grs, wrs); done = true; break;
                case 12 * 16 + 4: stem_phase<12, 4, PITCH, G>(A, P, sm4, acc, n, a0, b0, grs, wrs); done = true; break;
                case 16 * 16 + 4: stem_phase<16, 4, PITCH, G>(A, P, sm4, acc, n, a0, b0, grs, wrs); done = true; break;
                default: break;
            }
        }
#define GI_STEM_CASE(TT)                                                        \
    case TT:                                                                    \
        stem_phase<TT, 0, PITCH, G>(A, P, sm4, acc, n, a0, b0, grs, wrs);       \
        break;
        if (!done) switch (T) {
            GI_STEM_CASE(1)
            GI_STEM_CASE(2)
            GI_STEM_CASE(3)
            GI_STEM_CASE(4)
            GI_STEM_CASE(6)
            GI_STEM_CASE(8)
            GI_STEM_CASE(9)
            GI_STEM_CASE(12)
            GI_STEM_CASE(16)
            default: break;  // no taps: the phase's pixels are zero
        }
#undef GI_STEM_CASE

        // Epilogue: lane l holds input channels 0..3 of its pixel of each block.
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int row = 8 * wave + 4 * blk + (lane >> 4);
            const int a = a0 + row;
            const int b = b0 + stem_column(lane, row, A.pitch);
            const bool pv = a < P.Ha && b < P.Wb;
            const int pix = (P.rho_h + A.stride * a) * A.W + P.rho_w + A.stride * b;
            const v4f sum = (acc[0][blk] + acc[1][blk]) + (acc[2][blk] + acc[3][blk]);
#pragma unroll
            for (int ci = 0; ci < 4; ++ci) {
                const int off = (pv && ci < A.Ci) ? ((n * A.Ci + ci) * plane + pix) * 4 : kOOB;
                const float v = sum[ci];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), drs, off, 0, 0);
            }
        }
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

// Halo pitch fixed at compile time: 19 positions holds every phase of a
// 7 x 7 kernel at stride 2 (tap grids 3 or 4 wide); its halos (at most 20
// rows) fit 12 loads of 16 positions per wave.  Otherwise 16 loads per wave
// (halos of up to 512 positions) and the pitch is read at run time.
constexpr int kStemPitch = 19;
constexpr int kStemFixedG = 12;
constexpr int kStemG = 16;

int stem_f32_fixed_pitch() { return kStemPitch; }

int stem_f32_halo_positions(int pitch) {
    return 2 * 16 * (pitch == kStemPitch ? kStemFixedG : kStemG);
}

size_t stem_f32_lds_bytes(int hpmax) {
    return (size_t)kStemStages * (hpmax + kStemA) * sizeof(v4f);
}

hipError_t launch_stem_f32(const StemArgs &a, hipStream_t s, const KernelEvents &ev) {
    if (a.HPmax != stem_f32_halo_positions(a.pitch)) return hipErrorInvalidValue;
    const size_t lds = stem_f32_lds_bytes(a.HPmax);
    const int64_t wgs = (int64_t)a.N * a.tiles_r * a.tiles_c * a.ngroups;
    if (lds > 64 * 1024) return hipErrorInvalidValue;
    if (a.pitch == kStemPitch)
        hipExtLaunchKernelGGL((gi_stem_f32<kStemPitch, kStemFixedG>), dim3((unsigned)wgs),
                              dim3(128), (uint32_t)lds, s, ev.start, ev.stop, 0, a);
    else
        hipExtLaunchKernelGGL((gi_stem_f32<0, kStemG>), dim3((unsigned)wgs), dim3(128),
                              (uint32_t)lds, s, ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

}  // namespace gi
