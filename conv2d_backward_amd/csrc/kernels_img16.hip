// kernels_img16.hip -- whole-image implicit-GEMM kernel for 16-bit inputs
// (bf16 or fp16) on gfx950, stride 1, fp32 accumulation and output.
//
// The contraction is the implicit GEMM of meganeura conv2d_grad_input_gemm.wgsl
// (header comment: C[Ci, pixels] = A[Ci, K] x B[K, pixels], K = Co*kH*kW),
// with K ordered (chunk of 32 output channels, tap, channel).  The 16-bit
// matrix cores take 8 consecutive k per lane from both operands:
//   * A (the weight read as [Ci, K]) comes from a fragment image that a
//     prologue writes in the exact lane order of the MFMA A fragments;
//   * B (the im2col of grad_out) is read from the caller's NCHW tensor and
//     turned channel-minor on its way into LDS: each wave copies 8 channel
//     planes into a landing area with direct loads, reads them back with
//     gfx950's transposing LDS read (4 channels of one pixel per lane) and
//     writes 16-byte positions of 8 channels.  Positions outside the grad_out
//     plane stay zero: that border is the transposed padding kH-1-pad of the
//     shader's header comment.
//
// Work-group: 256 threads (4 waves) own one image and 128 input channels.
// Wave w owns input-channel blocks 2w, 2w+1 (16 channels each) and all NB
// pixel blocks of 16 of the image, so no A fragment is loaded by two waves,
// and the image's pixels fill the blocks with at most 15 slots to spare (the
// 14 x 14 deep stage: 196 pixels in 208 slots).  Per chunk of 32 output
// channels and tap, a wave issues 2 x NB MFMAs, 2 A-fragment loads (from L2,
// several taps ahead) and NB LDS reads (the next tap's B fragments).  The
// next chunk's grad_out block is loaded into registers while the current
// chunk computes, and transposed into the other LDS stage at its end.
//
// LDS banks: a 16-byte-per-lane LDS read is served 16 lanes per cycle (64
// banks of 4 bytes); within each half of the wave, the lanes whose index bits
// 2, 3 and 4 have even parity form one cycle and the odd ones the other.
// Each channel plane starts at a multiple of 256 bytes and halo rows sit HP
// positions apart with HP = W (mod 16), so the 16 pixels of a block (which
// wrap across image rows) sit at 16 positions that are consecutive mod 16
// whatever the tap shift: every cycle's lanes touch 16 different bank groups.
//
// V_MFMA_F32_16X16X32_BF16 / _F16: lane l = 16*g + i supplies A[i][k = 8g ..
// 8g+7] and B[k = 8g .. 8g+7][i] and receives D[4g + r][i], r = 0..3.  The
// two fragments have the same lane layout, so the kernel computes the
// transpose C^T[pixels, Ci] = B^T x A^T: the grad_out fragment goes in as the
// MFMA's A operand and the weight fragment as its B operand, and each lane
// ends with 4 consecutive pixels of one input channel, stored as 16 bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gi_common.h"
#include "lds_barrier.h"
#include "gi_launch.h"

namespace gi {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void *lds_ptr_t;

namespace {

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9)
constexpr int kOOB = 0x7ffffff0;         // byte offset past the end of every buffer

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (long)bytes, kRsrcWord3);
}

// F16: fp16 inputs (V_MFMA_F32_16X16X32_F16), else bf16.  NB pixel blocks of
// 16 per wave (the image's pixels, H*W <= 16*NB), T taps, KW the kernel
// width, HPT the halo pitch and HRT the most halo rows (all fixed at compile
// time; A.PS must equal the plane size they give).
template <int HRT, int HPT>
constexpr int img16_plane_bytes() { return (HRT * HPT * 16 + 255) / 256 * 256; }

constexpr int kLand = 4096;    // landing area of one wave's direct loads (4 x 1 KB)
constexpr int kStages = 3;     // LDS stages of channel planes

// Three stages of 4 channel planes, the 4 waves' landing areas, then one
// 16-byte slot per lane that takes the staging writes of quads past the
// grad_out plane.
template <int HRT, int HPT>
constexpr int img16_lds_bytes() {
    return kStages * 4 * img16_plane_bytes<HRT, HPT>() + 4 * kLand + 64 * 16;
}

template <bool F16, int NB, int T, int KW, int HPT, int HRT>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void gi_img16(
    const Img16Args A) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int KH = T / KW;
    constexpr int HP = HPT;
    constexpr int PS = img16_plane_bytes<HRT, HPT>();   // bytes of one channel plane
    constexpr int kStage = 4 * PS;                      // bytes of one stage: 4 planes
    // Within a chunk's taps: the next chunk's landed planes are read into
    // registers in tap kReadTap, transposed into its stage during tap
    // kStageTap and made visible by the barrier of tap kBarTap; the last tap
    // reads the next chunk's first B fragments.  The copy of the chunk after
    // next goes out one quarter per tap over the last four taps: a quarter
    // of the chip's copy traffic at a time, and every A prefetch issued
    // after a quarter (whose wait, in issue order, includes it) is waited
    // for eight taps later.
    constexpr int kReadTap = T / 3;
    constexpr int kStageTap = kReadTap + 1;
    constexpr int kBarTap = kStageTap + 2;
    constexpr int kLoadTap = T - 4;
    static_assert(kReadTap >= 1 && kStageTap < kLoadTap && kBarTap < T - 1, "tap schedule");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j16 = lane & 15, g = lane >> 4;

    // Logical order: image fastest, then the 128-channel tile, so the
    // work-groups of one L2 (a contiguous logical range, xcd_order) share the
    // weight fragments of one or two tiles.
    const int J = xcd_order(blockIdx.x, gridDim.x);
    const int ci_tile = J / A.N;
    const int n = J - ci_tile * A.N;

    const __amdgpu_buffer_rsrc_t grs = make_rsrc(A.g, A.g_bytes);
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(A.wk, A.wk_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(A.dst, A.d_bytes);

    // Staging.  Wave w stages channels 8w .. 8w+7 of every chunk: four
    // 16-byte direct loads per lane copy those 8 channel planes of grad_out
    // (contiguous in NCHW) into the wave's own 4 KB landing area a chunk
    // ahead; gfx950's transposing LDS read then turns them channel-minor on
    // the way into registers, and lane l writes pixel 64s + l of the chunk's
    // stage in write s (8 channels, 16 bytes).  A wave transposes only what
    // it loaded itself, so its own load counter is the only wait.  The copy
    // starts at the 16-byte boundary at or below the planes, which then sit
    // `shift` bytes into the landing area (0 or 8: whole 4-pixel quads keep
    // every plane 8-byte aligned).
    const int oHW = A.oH * A.oW;
    const int plane_bytes = oHW * 2;
    const int chunk_bytes = 32 * plane_bytes;
    const int base = (n * A.Co + 8 * wave) * plane_bytes;
    const int shift = base & 15;
    const int loff = base - shift + lane * 16;   // + 1024 * load, + chunk * chunk_bytes
    unsigned char *const land = smem + kStages * kStage + wave * kLand;
    // Every wave issues all four loads per chunk (past the tensor they read
    // zeros, past the chunk's channels data the transposition ignores), so
    // the number of loads in flight is known at compile time.
    auto sload_one = [&](int c, int k) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(grs, (lds_ptr_t)(land + 1024 * k), 16,
                                                 loff + 1024 * k, c * chunk_bytes, 0, 0);
    };
    auto sload = [&](int c) {
#pragma unroll
        for (int k = 0; k < 4; ++k) sload_one(c, k);
    };
    // Filled after the stages are zeroed (below): the LDS byte address, in
    // each stage, of pixel 64s + lane (write s), and this lane's pixel in
    // each block.
    int wdst[kStages][4];
    const int HW = A.H * A.W;
    int bbase[NB];
    // ds_read_b64_tr_b16 (lane layout measured on the GPU): within each 16
    // lanes, lanes 4r .. 4r+3 each load 4 consecutive 16-bit values, which
    // together form row r (16 values); lane i receives element i of rows
    // 0 .. 3.  Read (s, h): row r of the lanes 16g + 4r + j is channel
    // 4h + r, pixels 64s + 16g + 4j .. +3, so lane l = 16g + i receives
    // channels 4h .. 4h+3 of pixel 64s + l, packed two per dword in channel
    // order: reads (s, 0) and (s, 1) are the 16 bytes of write s.  Pixels
    // past the plane (up to 255) stay inside the landing area (8 planes of
    // at most 255 pixels after at most 8 bytes); their writes go to a
    // per-lane slot.  In two parts a tap apart: sread_one takes a piece into
    // registers, swrite_one writes a position, so the writes never wait on
    // the reads' LDS round trip.
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s *lds_v4s_t;
    const int rb = shift + ((lane >> 2) & 3) * plane_bytes + (16 * (lane >> 4) + 4 * (lane & 3)) * 2;
    const int rb4 = rb + 4 * plane_bytes;
    v2u tv[4][2];
    auto sread_one = [&](int i) {   // piece (s, h) = (i / 2, i % 2)
        const int s = i >> 1, h = i & 1;
        tv[s][h] = __builtin_bit_cast(
            v2u, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t)(land + (h ? rb4 : rb) + 128 * s)));
    };
    auto sread = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) sread_one(i);
    };
    auto smask = [&](int c) {
        const int room = A.Co - 32 * c - 8 * wave;   // channels of the wave's 8 that exist
        if (room < 8) {   // (uniform: only the last chunk of a ragged Co)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const int ch = 4 * h + 2 * d;   // channels ch (low half), ch + 1 (high)
                    const unsigned keep = (ch < room ? 0xffffu : 0u) | (ch + 1 < room ? 0xffff0000u : 0u);
#pragma unroll
                    for (int t = 0; t < 4; ++t) tv[t][h][d] &= keep;
                }
        }
    };
    auto swrite_one = [&](int t, int buf) {
        *(v4u *)(smem + wdst[buf][t]) = v4u{tv[t][0].x, tv[t][0].y, tv[t][1].x, tv[t][1].y};
    };
    auto swrite = [&](int c, int buf) {
        smask(c);
#pragma unroll
        for (int t = 0; t < 4; ++t) swrite_one(t, buf);
    };

    // A fragments: wave w's ci blocks 2w, 2w+1 of the 128-channel tile are
    // blocks 2*(w&1) + cb of the image's 64-channel tile 2*ci_tile + (w>>1).
    // Past the last chunk the offset is out of range (zeros); every prefetch
    // is issued unconditionally so the compiler's wait counts stay exact.
    const int t64 = 2 * ci_tile + (wave >> 1);
    const int wlane = ((t64 * A.nchunks * T) * 4 + 2 * (wave & 1)) * 1024 + lane * 16;
    auto aload = [&](int chunk, int tap, int cb) {
        const int soff = chunk < A.nchunks ? ((chunk * T + tap) * 4 + cb) * 1024 : kOOB;
        return __builtin_bit_cast(v8bf, __builtin_amdgcn_raw_buffer_load_b128(wrs, wlane, soff, 0));
    };

    // A ring of T slots indexed by tap: step s = chunk*T + tap uses slot
    // tap, and step s + AD is loaded while step s computes.  Every chunk
    // brings fresh weight lines, which each L2 fetches once for all of its
    // work-groups, so their first use waits for memory beyond the L2: they
    // are fetched nearly a chunk ahead.
    constexpr int AD = T - 1;
    static_assert(AD >= 1, "prefetch distance");
    v8bf fa[T][2];
    v8bf fb[NB];
    // Within a tap: the second A prefetch goes with block kA1Block's MFMAs,
    // a quarter of the copy with the last block's.
    static_assert(NB >= 9, "a tap carries eight landing reads");
    constexpr int kA1Block = NB / 2;
    // Loads issued after the copy's last quarter (the last tap's last block)
    // until the next chunk's landed planes are read: the two A prefetches of
    // each of its taps before kReadTap and the first of tap kReadTap.  In
    // chunk 0 the copy went out in the set-up, after every set-up fragment:
    // the same count.
    constexpr int kAfterLanding = 2 * kReadTap + 1;

    // Chunk 0's copy goes out first, then the first A fragments interleaved
    // with the zeroing of the stages (the landing areas lie past the stages),
    // so the load queue and the LDS work side by side; the address tables
    // are computed while the loads are in flight.  Positions the staging
    // never writes (the border) stay zero for the whole kernel.
    sload(0);
    constexpr int kZeroIters = (kStages * kStage / 16 + 255) / 256;
#pragma unroll
    for (int it = 0; it < kZeroIters; ++it) {
        const int i = tid + 256 * it;
        if (i < kStages * kStage / 16) ((v4u *)smem)[i] = v4u{0u, 0u, 0u, 0u};
        if (it < AD) {
            fa[it][0] = aload(0, it, 0);
            fa[it][1] = aload(0, it, 1);
        }
    }
    static_assert(kZeroIters >= AD, "every set-up fragment issued");
    __builtin_amdgcn_sched_barrier(0);
    // LDS byte address, in each stage, of pixel 64s + lane; pixels outside
    // the halo (only with padding beyond kH-1) or past the plane go to the
    // lane's own slot past the landing areas, so the staging writes every
    // position without a branch.  (Pixel index p < 256 and oW <= 256: the
    // reciprocal multiply is the exact row.)
    const int dummy = kStages * kStage + 4 * kLand + lane * 16;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int p = 64 * t + lane;
        const int oh = (int)(((uint32_t)p * A.rcp_ow) >> 16), ow = p - oh * A.oW;
        const int hr = oh + A.oy, hc = ow + A.ox;
        const bool v = p < oHW && hr >= 0 && hr < A.HR && hc >= 0 && hc < A.HC;
#pragma unroll
        for (int st = 0; st < kStages; ++st)
            wdst[st][t] = v ? st * kStage + wave * PS + (hr * HP + hc) * 16 : dummy;
    }
    // This lane's pixel in each block: LDS byte offset of its halo position
    // in plane g of a stage.  Slots past the image read position j16 (their
    // column is never stored; distinct positions keep the read conflict-free).
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int p = b * 16 + j16;   // < 256, and W <= 256: exact row by reciprocal
        const int ih = (int)(((uint32_t)p * A.rcp_w) >> 16), iw = p - ih * A.W;
        bbase[b] = g * PS + (p < HW ? ih * HP + iw : j16) * 16;
    }

    v4f acc[2][NB];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[cb][b] = v4f{0.f, 0.f, 0.f, 0.f};

    // Byte offset of tap tp in stage `st`: the stage plus a shift of
    // (kH-1-kh) rows and (kW-1-kw) columns; a compile-time immediate.
    auto tap_offset = [&](int st, int tp) {
        const int kh = tp / KW, kw = tp - (tp / KW) * KW;
        return st * kStage + ((KH - 1 - kh) * HP + (KW - 1 - kw)) * 16;
    };

    // Set-up: chunk 0 staged into stage 0, chunk 1's copy in flight, the
    // first A fragments in flight, chunk 0's first B fragments read.
    lds_barrier();   // the zeroing is done before any position is staged
    // (Chunk 0's copy and the first A fragments went out before the zeroing,
    // into the landing areas and registers, so their latencies overlap it
    // and each other; the copy is complete once at most the 2 AD fragment
    // loads issued after it are outstanding.)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * AD) : "memory");
    sread();
    swrite(0, 0);
    sload(1);
    lds_barrier();
#pragma unroll
    for (int b = 0; b < NB; ++b) fb[b] = *(const v8bf *)(smem + bbase[b] + tap_offset(0, 0));

    // One chunk of 32 output channels on stage ST (a compile-time index, so
    // every LDS address is a base register plus an immediate).  The B
    // fragments are single-buffered: block b's fragment for the next tap is
    // read after block b + 1's MFMAs of this tap are issued, so the read
    // never waits for the MFMAs that still read the register (in the last
    // tap: the next chunk's first tap, from its stage, staged and made
    // visible earlier in this chunk).  With one wave per SIMD, every other
    // instruction has to issue in the shadow of the MFMAs: each block's pair
    // of MFMAs carries at most one piece of the remaining work (an A
    // prefetch, a landing read, a quad write, a direct load).
    auto run_chunk = [&](const int chunk, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        constexpr int NX = (ST + 1) % kStages;   // stage of the next chunk
        const bool more = chunk + 1 < A.nchunks;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tp = 0; tp < T; ++tp) {
            // Block b's B fragment for the step after tap tp.
            auto next_b = [&](int b) {
                if (tp + 1 < T)
                    fb[b] = *(const v8bf *)(smem + bbase[b] + tap_offset(ST, tp + 1));
                else if (more)
                    fb[b] = *(const v8bf *)(smem + bbase[b] + tap_offset(NX, 0));
            };
            const int t2 = tp + AD;
            const int c2 = t2 < T ? chunk : chunk + 1;
            const int t2m = t2 < T ? t2 : t2 - T;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b == 0) fa[t2m][0] = aload(c2, t2m, 0);
                if (b == kA1Block) fa[t2m][1] = aload(c2, t2m, 1);
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    if constexpr (F16)
                        acc[cb][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(v8h, fb[b]), __builtin_bit_cast(v8h, fa[tp][cb]),
                            acc[cb][b], 0, 0, 0);
                    else
                        acc[cb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            fb[b], fa[tp][cb], acc[cb][b], 0, 0, 0);
                if (b >= 1) next_b(b - 1);
                if (tp == kReadTap && more) {
                    if (b == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kAfterLanding) : "memory");
                    if (b < 8) sread_one(b);
                }
                if (tp == kStageTap && more) {
                    // The stage was last read two chunks ago, before the
                    // last barrier.
                    if (b == 0) smask(chunk + 1);
                    if (b >= 1 && b <= 4) swrite_one(b - 1, NX);
                }
                // The landing area is refilled only after every landed value
                // is in registers (the stage writes used them).
                if (tp >= kLoadTap && b == NB - 1 && more) sload_one(chunk + 2, tp - kLoadTap);
                __builtin_amdgcn_sched_barrier(0);
            }
            next_b(NB - 1);
            if (tp == kBarTap) lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Output stores.  grad_out is the MFMA's A operand and the weight its B
    // operand, so lane (j16, g) holds D[4g + r][j16] of each block: pixels
    // 16b + 4g .. 16b + 4g + 3 (consecutive in the NCHW plane, and 16-byte
    // aligned as H*W is a multiple of 4, checked at launch) of input channel
    // j16 of the wave's channel block cb.  One 16-byte store each, every
    // 4 lanes of a channel a full 64-byte run; slots past the image are not
    // stored.
    auto store_block = [&](int b) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int ci = ci_tile * 128 + wave * 32 + cb * 16 + j16;
            const int p = 16 * b + 4 * g;
            const int off = (p < HW && ci < A.Ci) ? ((n * A.Ci + ci) * HW + p) * 4 : kOOB;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc[cb][b]), drs, off,
                                                   0, 0);
        }
    };
    // The last chunk runs block by block, all taps of a group of blocks at a
    // time, and stores each group as soon as its sums are complete: the
    // 25 MB of a deep stage's fp32 output then leaves while the chunk still
    // computes, instead of in one burst at the end.  Every fragment of the
    // chunk is in registers by then (the ring holds taps 0 .. T-2, tap T-1
    // is loaded here) and every block's tap-0 B fragment was read in the
    // previous chunk's last tap (or in the set-up).  Groups are pairs of
    // blocks (a triple last when NB is odd), so each accumulator's MFMAs
    // are at least four apart.
    auto run_last = [&](const int chunk, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        fa[T - 1][0] = aload(chunk, T - 1, 0);
        fa[T - 1][1] = aload(chunk, T - 1, 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        constexpr int NG = NB / 2;
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) {
            const int b0 = 2 * gr;
            const int nbk = gr == NG - 1 ? NB - b0 : 2;
            v8bf x[2][3];
#pragma unroll
            for (int k = 0; k < 3; ++k)
                if (k < nbk) x[0][k] = fb[b0 + k];
#pragma unroll
            for (int tp = 0; tp < T; ++tp) {
                if (tp + 1 < T) {
#pragma unroll
                    for (int k = 0; k < 3; ++k)
                        if (k < nbk)
                            x[(tp + 1) & 1][k] =
                                *(const v8bf *)(smem + bbase[b0 + k] + tap_offset(ST, tp + 1));
                }
#pragma unroll
                for (int k = 0; k < 3; ++k)
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb)
                        if (k < nbk) {
                            if constexpr (F16)
                                acc[cb][b0 + k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    __builtin_bit_cast(v8h, x[tp & 1][k]),
                                    __builtin_bit_cast(v8h, fa[tp][cb]), acc[cb][b0 + k], 0, 0, 0);
                            else
                                acc[cb][b0 + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    x[tp & 1][k], fa[tp][cb], acc[cb][b0 + k], 0, 0, 0);
                        }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int k = 0; k < 3; ++k)
                if (k < nbk) store_block(b0 + k);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto step = [&](const int chunk, auto st_c) {
        if (chunk + 1 < A.nchunks)
            run_chunk(chunk, st_c);
        else
            run_last(chunk, st_c);
    };
    for (int chunk = 0; chunk < A.nchunks; chunk += kStages) {
        step(chunk, std::integral_constant<int, 0>{});
        if (chunk + 1 < A.nchunks) step(chunk + 1, std::integral_constant<int, 1>{});
        if (chunk + 2 < A.nchunks) step(chunk + 2, std::integral_constant<int, 2>{});
    }
}

template <bool F16, int NB, int T, int KW, int HPT, int HRT>
hipError_t launch_one(const Img16Args &a, size_t lds, hipStream_t s, const KernelEvents &ev) {
    if (a.kW != KW || a.kH * a.kW != T || a.HP != HPT || a.HR > HRT ||
        a.PS != img16_plane_bytes<HRT, HPT>() || lds != (size_t)img16_lds_bytes<HRT, HPT>() ||
        a.rcp_w != recip16(a.W) || a.rcp_ow != recip16(a.oW) || a.W > 256 || a.oW > 256 ||
        a.H * a.W > 16 * NB || (a.H * a.W) % 4 != 0 || a.nq > 64 || 4 * a.nq != a.oH * a.oW ||
        8 + 16 * a.oH * a.oW > kLand)
        return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)gi_img16<F16, NB, T, KW, HPT, HRT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int64_t wgs = (int64_t)a.N * a.ci_tiles;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL((gi_img16<F16, NB, T, KW, HPT, HRT>), dim3((unsigned)wgs), dim3(256),
                          (uint32_t)lds, s, ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

// Instantiations: (pixel blocks of 16 per wave, taps, kernel width, halo
// pitch, most halo rows).  The first serves 3 x 3 kernels on images of up to
// 14 rows and 14 columns (pitch 30 = 14 mod 16, at least 16 columns).
constexpr int kCfg[][5] = {{13, 9, 3, 30, 16}};

// Weight [Co][Ci][T] -> fragment image wk[ci tile of 64][chunk][tap][block of
// 16][lane][8] (gi_common.h), zero past Ci and Co.  Work-group (chunk of 32
// output channels, block of 16 input channels): the 32 rows of the block's
// 16*T contiguous (ci, tap) elements are copied into LDS with 16-byte loads,
// then each thread gathers one lane's 8 output channels at one (ci, tap) from
// LDS and writes it; consecutive threads write consecutive lanes, so every
// tap's 1 KB fragment block is stored whole.
// VEC: every row of the weight is a whole number of 16-byte pieces (Ci*T a
// multiple of 8), read with range-checked 16-byte buffer loads (w_bytes <
// 2^31); else 2-byte reads.
template <bool VEC>
__global__ __launch_bounds__(256) void weight_frag16(const uint16_t *__restrict__ w,
                                                     uint16_t *__restrict__ wk, int Co, int Ci,
                                                     int T, int nchunks, uint32_t w_bytes) {
    extern __shared__ uint16_t raw[];   // [32 rows][16*T + 8]
    const int chunk = blockIdx.x, blk = blockIdx.y;
    const int pitch = 16 * T + 8;
    const int64_t rowlen = (int64_t)Ci * T;
    const int64_t e0 = (int64_t)blk * 16 * T;   // first element of the block in a row
    const int pieces = 2 * T;                  // 8-element pieces per row of the block
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(w, w_bytes);
    // Four pieces per thread per pass, all loaded before any is stored, so a
    // pass costs one memory round trip (a 3x3 kernel's block is one pass).
    constexpr int kPer = 4;
    for (int i0 = threadIdx.x; i0 < 32 * pieces; i0 += 256 * kPer) {
        v4u v[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = i0 + 256 * u;
            const int r = i / pieces, pc = i - (i / pieces) * pieces;
            const int co = chunk * 32 + r;
            const int64_t e = e0 + 8 * pc;
            const bool ok = i < 32 * pieces && co < Co && e < rowlen;
            if (VEC) {
                v[u] = __builtin_bit_cast(
                    v4u, __builtin_amdgcn_raw_buffer_load_b128(
                             wrs, ok ? (int)(((int64_t)co * rowlen + e) * 2) : kOOB, 0, 0));
            } else {
                v[u] = v4u{0u, 0u, 0u, 0u};
                if (ok) {
                    const uint16_t *src = w + (int64_t)co * rowlen + e;
                    unsigned h[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) h[k] = e + k < rowlen ? src[k] : 0u;
                    v[u] = v4u{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16,
                               h[6] | h[7] << 16};
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = i0 + 256 * u;
            const int r = i / pieces, pc = i - (i / pieces) * pieces;
            if (i < 32 * pieces) *(v4u *)(raw + r * pitch + 8 * pc) = v[u];
        }
    }
    __syncthreads();
    const int ct = blk >> 2, cb = blk & 3;
    for (int o = threadIdx.x; o < T * 64; o += 256) {
        const int tap = o >> 6, ln = o & 63;
        const int gq = ln >> 4, l16 = ln & 15;
        const uint16_t *col = raw + 8 * gq * pitch + l16 * T + tap;
        v4u v;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            v[m] = (unsigned)col[(2 * m) * pitch] | (unsigned)col[(2 * m + 1) * pitch] << 16;
        ((v4u *)wk)[((((int64_t)ct * nchunks + chunk) * T + tap) * 4 + cb) * 64 + ln] = v;
    }
}

}  // namespace

int img16_config(int nb, int kH, int kW, int hp, int hr) {
    for (int i = 0; i < (int)(sizeof(kCfg) / sizeof(kCfg[0])); ++i)
        if (kCfg[i][0] == nb && kCfg[i][1] == kH * kW && kCfg[i][2] == kW && kCfg[i][3] == hp &&
            hr <= kCfg[i][4])
            return i;
    return -1;
}

int img16_plane(int cfg) {
    switch (cfg) {
        case 0: return img16_plane_bytes<16, 30>();
        default: return 0;
    }
}

size_t img16_lds(int cfg) {
    switch (cfg) {
        case 0: return img16_lds_bytes<16, 30>();
        default: return 0;
    }
}

int img16_blocks(int cfg) { return cfg >= 0 ? kCfg[cfg][0] : 0; }

hipError_t launch_img16(const Img16Args &a, int cfg, bool f16, size_t lds, hipStream_t s,
                        const KernelEvents &ev) {
    switch (cfg) {
        case 0:
            return f16 ? launch_one<true, 13, 9, 3, 30, 16>(a, lds, s, ev)
                       : launch_one<false, 13, 9, 3, 30, 16>(a, lds, s, ev);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_weight_frag16(const uint16_t *w, uint16_t *wk, int Co, int Ci, int kHW,
                                int nchunks, int wtiles, hipStream_t s) {
    // One work-group per (chunk, block of 16 input channels) of the image,
    // including the zero blocks past Ci up to wtiles*64 channels.
    const size_t lds = (size_t)32 * (16 * kHW + 8) * sizeof(uint16_t);
    if (lds > 160 * 1024 || wtiles * 4 > 65535) return hipErrorInvalidValue;
    const int64_t wbytes = (int64_t)Co * Ci * kHW * 2;
    // 16-byte buffer loads where rows are whole pieces and byte offsets fit
    // (kOOB stays past the range).
    const bool vec = ((int64_t)Ci * kHW) % 8 == 0 && wbytes < 0x7fff0000LL;
    const void *fn = vec ? (const void *)weight_frag16<true> : (const void *)weight_frag16<false>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const uint32_t wb = vec ? (uint32_t)wbytes : 0u;
    if (vec)
        hipLaunchKernelGGL(weight_frag16<true>, dim3(nchunks, wtiles * 4), dim3(256), lds, s, w, wk,
                           Co, Ci, kHW, nchunks, wb);
    else
        hipLaunchKernelGGL(weight_frag16<false>, dim3(nchunks, wtiles * 4), dim3(256), lds, s, w,
                           wk, Co, Ci, kHW, nchunks, wb);
    return hipGetLastError();
}

}  // namespace gi
