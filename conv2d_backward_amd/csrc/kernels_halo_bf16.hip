// kernels_halo_bf16.hip -- bf16-input halo-tile implicit-GEMM kernel for
// gfx950 (stride 1), fp32 accumulation and output.
//
// The contraction is the implicit GEMM of meganeura conv2d_grad_input_gemm.wgsl
// (header comment: C[Ci, pixels] = A[Ci, K] x B[K, pixels], K = Co*kH*kW),
// with K ordered (chunk of 32 output channels, tap, channel).  The bf16 matrix
// cores take 8 consecutive k per lane from both operands, so both operands are
// laid out output-channel-minor by two prologues:
//   * grad_out -> zero-padded planes of 8 channels (gi_common.h): the zero
//     border is the transposed padding kH-1-pad of the shader's header
//     comment, and a plane row is one contiguous run of 16-byte positions;
//   * weight   -> the exact lane order of the MFMA A fragments.
//
// Work-group: 256 threads = 2 x 2 waves over 64 input channels x a TR x TC
// pixel tile of one image.  Wave (wm, wn) owns input-channel blocks 2wm, 2wm+1
// (16 each) and pixel blocks wn*NBW .. wn*NBW + NBW - 1 (16 pixels each).
// Per chunk of 32 output channels the tile's halo, (TR+kH-1) x (TC+kW-1)
// positions, is copied into LDS by direct global -> LDS loads (double-
// buffered; wave w copies channel plane w), and tap (kh, kw) reads its B
// fragments as the halo shifted by (kH-1-kh, kW-1-kw) positions.  A fragments
// are loaded from the weight image straight into registers, several taps
// ahead.  The loop carries almost no vector arithmetic: a B read is a per-lane
// base address plus the tap's shift, a compile-time immediate when the halo
// pitch and kernel width are template parameters; the chunk parts of the
// global offsets are scalar.
//
// LDS banks: a 16-byte-per-lane LDS read is served 16 lanes per cycle (64
// banks of 4 bytes, i.e. 16 bank groups of 16 bytes).  Measured on gfx950:
// within each half of the wave, the lanes whose index bits 2, 3 and 4 have
// even parity form one cycle and the odd ones the other.  LDS holds each
// channel plane separately (plane offsets a multiple of 256 bytes) with halo
// rows HP positions apart, HP = TC (mod 16): the 16 pixels of a block (which
// may wrap to the next tile row) sit at 16 positions that are consecutive mod
// 16 whatever the tap shift, so every cycle's 16 lanes (8 of one channel
// plane, 8 of the other, covering all 16 pixels) touch 16 different bank
// groups.
//
// V_MFMA_F32_16X16X32_BF16: lane l = 16*g + i supplies A[i][k = 8g .. 8g+7]
// and B[k = 8g .. 8g+7][i] and receives D[4g + r][i], r = 0..3.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_common.h"
#include "gi_launch.h"
#include "half_launch.h"

namespace gi {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

namespace {

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9)
constexpr int kOOB = 0x7ffffff0;         // byte offset past the end of every buffer
constexpr int kQW = kHaloBf16Loads;      // halo direct loads per wave per chunk

typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (long)bytes, kRsrcWord3);
}

// F16: the 16-bit inputs are fp16 (V_MFMA_F32_16X16X32_F16), else bf16; the
// data path is the same bits either way.  NBW pixel blocks per wave, T taps;
// KW > 0: kernel width and HPT halo pitch known at compile time (they must
// equal A.kW and A.HP), else read from A.
template <bool F16, int NBW, int T, int KW, int HPT>
__global__ __launch_bounds__(256, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void gi_halo_bf16(
    const HaloBf16Args A) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j16 = lane & 15, g = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const int HP = HPT > 0 ? HPT : A.HP;
    const int kW = KW > 0 ? KW : A.kW;
    const int kH = KW > 0 ? T / KW : A.kH;

    // Logical order: input-channel tile fastest, then column, row, image.
    const int J = xcd_order(blockIdx.x, gridDim.x);
    const int ci_tile = J % A.ci_tiles;
    int t = J / A.ci_tiles;
    const int ct = t % A.col_tiles;
    t /= A.col_tiles;
    const int rt = t % A.row_tiles;
    const int n = t / A.row_tiles;
    const int a0 = rt * A.TR, b0 = ct * A.TC;
    const int stage = 4 * A.PS;              // bytes per LDS stage: 4 planes
    unsigned char *const dummy = smem + 2 * stage;

    const __amdgpu_buffer_rsrc_t grs = make_rsrc(A.gp, A.gp_bytes);
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(A.wk, A.wk_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(A.dst, A.d_bytes);

    // Halo direct loads: wave w copies plane w (channels 8w .. 8w+7 of the
    // chunk); its load k covers LDS positions 64k .. 64k+63 of the plane,
    // lane -> position 64k + lane = (row, column) with pitch HP.  Positions
    // past the halo's columns or the padded image read zeros.  The chunk part
    // of the offset is scalar.
    int goff[kQW];
#pragma unroll
    for (int k = 0; k < kQW; ++k) {
        const int pos = 64 * k + lane;
        const int hr = pos / HP, hc = pos - (pos / HP) * HP;
        const int y = a0 + hr, x = b0 + hc;
        const bool v = hr < A.HR && hc < A.HC && y < A.YP && x < A.XP;
        goff[k] = v ? (((n * A.nchunks * 4 + wave) * A.YP + y) * A.XP + x) * 16 : kOOB;
    }
    const int chunk_bytes = 4 * A.YP * A.XP * 16;
    // Every wave issues exactly kQW loads per chunk, also past the last chunk
    // (the surplus ones read zeros into a scratch kilobyte of LDS nobody
    // reads), so the number of loads in flight is known at compile time and
    // the compiler's wait counts stay exact.
    auto issue = [&](int chunk, int buf) {
        const bool live = chunk < A.nchunks;
        const int soff = live ? chunk * chunk_bytes : 0;
#pragma unroll
        for (int k = 0; k < kQW; ++k) {
            const bool real = live && k < A.nql;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                grs, (lds_ptr_t)(real ? smem + buf * stage + wave * A.PS + k * 1024 : dummy), 16,
                real ? goff[k] : kOOB, soff, 0, 0);
        }
    };

    // A fragments: weight image offset of (chunk, tap, block 2wm + cb); the
    // per-lane part is the vector offset, the rest scalar.  Past the last
    // chunk the offset is out of range (the load returns zeros): every
    // prefetch is issued unconditionally, so the compiler's wait counts stay
    // exact (a conditional load it cannot count would make it wait for every
    // later load too).
    const int wlane = (ci_tile * A.nchunks * T * 4 + 2 * wm) * 1024 + lane * 16;
    auto aload = [&](int chunk, int tap, int cb) {
        const int soff = chunk < A.nchunks ? ((chunk * T + tap) * 4 + cb) * 1024 : kOOB;
        return __builtin_bit_cast(v8bf, __builtin_amdgcn_raw_buffer_load_b128(wrs, wlane, soff, 0));
    };

    // This lane's pixel in each of its blocks: LDS byte offset of its halo
    // position in plane g of stage 0.  Outside the tile or image the lane reads
    // position j16 (its column is never stored; distinct positions keep the
    // read conflict-free) when every tap's shift keeps that inside the plane,
    // else position 0.
    const int max_shift = (kH - 1) * HP + (kW - 1);
    const int inv = j16 + max_shift < A.nql * 64 ? j16 : 0;
    int bbase[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        const int p = (wn * NBW + b) * 16 + j16;
        const int r = p / A.TC, c = p - (p / A.TC) * A.TC;
        const bool v = p < A.TR * A.TC && a0 + r < A.H && b0 + c < A.W;
        bbase[b] = g * A.PS + (v ? r * HP + c : inv) * 16;
    }

    v4f acc[2][NBW];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int b = 0; b < NBW; ++b) acc[cb][b] = v4f{0.f, 0.f, 0.f, 0.f};

    // Byte shift of tap tp: (kH-1-kh) rows and (kW-1-kw) columns.
    auto shift_bytes = [&](int tp) {
        const int kh = tp / kW, kw = tp - (tp / kW) * kW;
        return ((kH - 1 - kh) * HP + (kW - 1 - kw)) * 16;
    };

    // A ring of T slots indexed by tap: step s = chunk*T + tap uses slot
    // s % T = tap (a compile-time index), and step s + AD is loaded while step
    // s computes (A comes from L2, so it is fetched several taps ahead).
    constexpr int AD = T >= 9 ? 4 : T - 1;
    static_assert(AD >= 1 && AD < T, "prefetch distance");
    v8bf fa[T][2];
#pragma unroll
    for (int s0 = 0; s0 < AD; ++s0) {
        fa[s0][0] = aload(0, s0, 0);
        fa[s0][1] = aload(0, s0, 1);
    }

    issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int chunk = 0; chunk < A.nchunks; ++chunk) {
        const int cur = chunk & 1;
        issue(chunk + 1, cur ^ 1);
        // Per-lane addresses of this stage, opaque to the optimiser so the
        // tap x block addresses are a base register plus an immediate instead
        // of registers held across the loop.
        int bb[NBW];
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
            bb[b] = bbase[b] + cur * stage;
            asm volatile("" : "+v"(bb[b]));
        }
        v8bf fb[2][NBW];
        auto bfetch = [&](int tp, int sl) {
            const int sh = shift_bytes(tp);
#pragma unroll
            for (int b = 0; b < NBW; ++b) fb[sl][b] = *(const v8bf *)(smem + bb[b] + sh);
        };
        bfetch(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tp = 0; tp < T; ++tp) {
            const int sl = tp & 1;
            // Prefetch: A of step + AD, B of the next tap.
            {
                const int t2 = tp + AD;
                const int c2 = t2 < T ? chunk : chunk + 1;
                const int t2m = t2 < T ? t2 : t2 - T;
                fa[t2m][0] = aload(c2, t2m, 0);
                fa[t2m][1] = aload(c2, t2m, 1);
            }
            if (tp + 1 < T) bfetch(tp + 1, sl ^ 1);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int b = 0; b < NBW; ++b)
                    if constexpr (F16)
                        acc[cb][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(v8h, fa[tp][cb]), __builtin_bit_cast(v8h, fb[sl][b]),
                            acc[cb][b], 0, 0, 0);
                    else
                        acc[cb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            fa[tp][cb], fb[sl][b], acc[cb][b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The next chunk's halo must have landed before the barrier.  Loads
        // complete in issue order and the halo loads were issued before this
        // chunk's A prefetches, so it is enough that at most the 2*AD most
        // recent loads (the A fragments of the next chunk's first AD taps)
        // are still in flight: they stay in flight across the barrier.
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * AD) : "memory");
        __syncthreads();
    }
    // Nothing may still write this work-group's LDS when it ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Epilogue: D[4g + r][j16] of each block, NCHW fp32.
    const int plane = A.H * A.W;
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        const int p = (wn * NBW + b) * 16 + j16;
        const int r = p / A.TC, c = p - (p / A.TC) * A.TC;
        const bool pv = p < A.TR * A.TC && a0 + r < A.H && b0 + c < A.W;
        const int pix = (a0 + r) * A.W + b0 + c;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int ci = ci_tile * 64 + (2 * wm + cb) * 16 + 4 * g + rr;
                const int off = (pv && ci < A.Ci) ? ((n * A.Ci + ci) * plane + pix) * 4 : kOOB;
                const float v = acc[cb][b][rr];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), drs, off, 0, 0);
            }
        }
    }
}

template <bool F16, int NBW, int T, int KW, int HPT>
hipError_t launch_one(const HaloBf16Args &a, int tiles, int ci_tiles, size_t lds, hipStream_t s,
                      const KernelEvents &ev) {
    if ((KW > 0 && (a.kW != KW || a.kH * a.kW != T)) || (HPT > 0 && a.HP != HPT))
        return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)gi_halo_bf16<F16, NBW, T, KW, HPT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (a.ci_tiles != ci_tiles) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL((gi_halo_bf16<F16, NBW, T, KW, HPT>), dim3(tiles * ci_tiles), dim3(256),
                          (uint32_t)lds, s, ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

// Instantiations: pixel blocks per wave, taps, and (kernel width, halo pitch)
// when fixed at compile time (0: read at run time).  The first serves 3 x 3
// kernels on 14-wide tiles (pitch 30).
constexpr int kCfg[][4] = {{7, 9, 3, 30}, {7, 9, 0, 0}, {4, 9, 0, 0}, {7, 3, 0, 0}, {4, 3, 0, 0}};

// grad_out NCHW bf16 -> zero-padded channel planes (gi_common.h).  One
// thread per 16-byte position of one plane (8 channels): 8 two-byte loads
// from the 8 channel images, one store.  Consecutive threads take consecutive
// positions of a plane row, so every load and the store are coalesced along
// the row; positions in the padding border load nothing.  `plane` is
// (n * nchunks + chunk) * 4 + g, `pos` the position in the YP x XP plane.
__device__ __forceinline__ void pad_planes_bf16(const uint16_t *__restrict__ g,
                                                uint16_t *__restrict__ gp, const HaloBf16Args &A,
                                                int oH, int oW, int pad_h, int pad_w, int plane,
                                                int pos) {
    if (pos >= A.YP * A.XP) return;
    const int y = pos / A.XP, x = pos - (pos / A.XP) * A.XP;
    const int oh = y - (A.kH - 1 - pad_h), ow = x - (A.kW - 1 - pad_w);
    const int gq = plane & 3, nc = plane >> 2;
    const int n = nc / A.nchunks, chunk = nc - (nc / A.nchunks) * A.nchunks;
    const int co0 = chunk * 32 + 8 * gq;
    uint32_t h[4] = {0u, 0u, 0u, 0u};
    if (oh >= 0 && oh < oH && ow >= 0 && ow < oW) {
        const int64_t img = (int64_t)oH * oW;
        const uint16_t *src = g + ((int64_t)n * A.Co + co0) * img + (int64_t)oh * oW + ow;
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = co0 + e < A.Co ? src[e * img] : (uint16_t)0;
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = (uint32_t)v[2 * q] | ((uint32_t)v[2 * q + 1] << 16);
    }
    *(uint4 *)(gp + ((int64_t)plane * A.YP * A.XP + pos) * 8) = uint4{h[0], h[1], h[2], h[3]};
}

// Weights [Co][Ci][kH][kW] bf16 -> A-fragment lane order (gi_common.h).  One
// work-group per (chunk of 32 output channels, ci tile, lane group g): it
// reads the 8 output channels 8g .. 8g+7 of the chunk for the tile's input
// channels and every tap (one contiguous run per channel, coalesced) into
// LDS, and each thread then writes one lane's 16 bytes.
__device__ __forceinline__ void weight_frag_bf16(const uint16_t *__restrict__ w,
                                                 uint16_t *__restrict__ wk, const HaloBf16Args &A,
                                                 int chunk, int ct, int g, uint16_t *slab) {
    // slab: [8 co][64 ci * T]
    const int T = A.kH * A.kW;
    const int run = 64 * T;
    const int ci_rows = min(64, A.Ci - ct * 64);
    if ((A.Ci * T) % 8 == 0 && (ci_rows * T) % 8 == 0) {
        // Every channel's run starts 16-byte aligned and has whole 8-element
        // pieces: 16-byte loads and stores.
        const int pieces = run / 8;
        for (int i = threadIdx.x; i < 8 * pieces; i += 256) {
            const int c = i / pieces, r8 = i - (i / pieces) * pieces;
            const int co = chunk * 32 + 8 * g + c;
            uint4 v = {0u, 0u, 0u, 0u};
            if (co < A.Co && r8 * 8 < ci_rows * T)
                v = *(const uint4 *)(w + ((int64_t)co * A.Ci + (int64_t)ct * 64) * T + r8 * 8);
            *(uint4 *)(slab + c * run + r8 * 8) = v;
        }
    } else {
    // Thread -> offsets r, r + 256, ... of each channel's run (no division).
    for (int r0 = 0; r0 < run; r0 += 256 * 2) {
        uint16_t v[2][8];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r = r0 + u * 256 + threadIdx.x;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int co = chunk * 32 + 8 * g + c;
                v[u][c] = (r < ci_rows * T && co < A.Co)
                              ? w[((int64_t)co * A.Ci + (int64_t)ct * 64) * T + r]
                              : (uint16_t)0;
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r = r0 + u * 256 + threadIdx.x;
            if (r < run) {
#pragma unroll
                for (int c = 0; c < 8; ++c) slab[c * run + r] = v[u][c];
            }
        }
    }
    }
    __syncthreads();
    // Lanes 16g .. 16g+15 of every (tap, ci block) of this (ci tile, chunk).
    uint4 *out = (uint4 *)(wk + ((int64_t)ct * A.nchunks + chunk) * T * 2048);
    for (int f = threadIdx.x; f < T * 64; f += 256) {
        const int tap = f >> 6, cb = (f >> 4) & 3, l16 = f & 15;
        const int ci = cb * 16 + l16;
        uint32_t h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            h[q] = (uint32_t)slab[(2 * q) * run + ci * T + tap] |
                   ((uint32_t)slab[(2 * q + 1) * run + ci * T + tap] << 16);
        out[(tap * 4 + cb) * 64 + 16 * g + l16] = uint4{h[0], h[1], h[2], h[3]};
    }
}

// Both prologues in one launch (they are independent, so they overlap and
// share one dispatch): the first frag_wgs work-groups reorder the weight
// (the longer-lived ones, dispatched first), the rest pad grad_out (pad_bpp
// per plane).
__global__ __launch_bounds__(256) void prologues_bf16(const uint16_t *__restrict__ g,
                                                      uint16_t *__restrict__ gp,
                                                      const uint16_t *__restrict__ w,
                                                      uint16_t *__restrict__ wk,
                                                      const HaloBf16Args A, int oH, int oW,
                                                      int pad_h, int pad_w, int pad_bpp,
                                                      int frag_wgs, int ci_tiles) {
    extern __shared__ uint16_t slab[];
    int b = blockIdx.x;
    if (b < frag_wgs) {
        const int gq = b & 3;
        b >>= 2;
        weight_frag_bf16(w, wk, A, b / ci_tiles, b % ci_tiles, gq, slab);
    } else {
        b -= frag_wgs;
        const int plane = b / pad_bpp, pb = b - (b / pad_bpp) * pad_bpp;
        pad_planes_bf16(g, gp, A, oH, oW, pad_h, pad_w, plane, pb * 256 + threadIdx.x);
    }
}

}  // namespace

int halo_bf16_config(int nbw, int kH, int kW, int hp) {
    for (int i = 0; i < (int)(sizeof(kCfg) / sizeof(kCfg[0])); ++i) {
        if (kCfg[i][0] != nbw || kCfg[i][1] != kH * kW) continue;
        if (kCfg[i][2] == 0 || (kCfg[i][2] == kW && kCfg[i][3] == hp)) return i;
    }
    return -1;
}

template <bool F16>
hipError_t launch_halo_16(const HaloBf16Args &a, int cfg, int tiles, int ci_tiles, size_t lds,
                          hipStream_t s, const KernelEvents &ev) {
    switch (cfg) {
        case 0: return launch_one<F16, 7, 9, 3, 30>(a, tiles, ci_tiles, lds, s, ev);
        case 1: return launch_one<F16, 7, 9, 0, 0>(a, tiles, ci_tiles, lds, s, ev);
        case 2: return launch_one<F16, 4, 9, 0, 0>(a, tiles, ci_tiles, lds, s, ev);
        case 3: return launch_one<F16, 7, 3, 0, 0>(a, tiles, ci_tiles, lds, s, ev);
        case 4: return launch_one<F16, 4, 3, 0, 0>(a, tiles, ci_tiles, lds, s, ev);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_halo_bf16(const HaloBf16Args &a, int cfg, int tiles, int ci_tiles, size_t lds,
                            hipStream_t s, const KernelEvents &ev) {
    return launch_halo_16<false>(a, cfg, tiles, ci_tiles, lds, s, ev);
}

hipError_t launch_halo_f16(const HaloBf16Args &a, int cfg, int tiles, int ci_tiles, size_t lds,
                           hipStream_t s, const KernelEvents &ev) {
    return launch_halo_16<true>(a, cfg, tiles, ci_tiles, lds, s, ev);
}

hipError_t launch_prologues_bf16(const uint16_t *g, uint16_t *gp, const uint16_t *w, uint16_t *wk,
                                 const HaloBf16Args &a, int oH, int oW, int pad_h, int pad_w,
                                 int ci_tiles, hipStream_t s) {
    const int pad_bpp = (a.YP * a.XP + 255) / 256;
    const int64_t pad_wgs = (int64_t)a.N * a.nchunks * 4 * pad_bpp;
    const int64_t frag_wgs = (int64_t)a.nchunks * ci_tiles * 4;
    const int64_t wgs = pad_wgs + frag_wgs;
    const size_t lds = (size_t)8 * 64 * a.kH * a.kW * sizeof(uint16_t);
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)prologues_bf16,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(prologues_bf16, dim3((unsigned)wgs), dim3(256), lds, s, g, gp, w, wk, a, oH,
                       oW, pad_h, pad_w, pad_bpp, (int)frag_wgs, ci_tiles);
    return hipGetLastError();
}

}  // namespace gi
