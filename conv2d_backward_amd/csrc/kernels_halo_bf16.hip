// kernels_halo_bf16.hip -- bf16-input halo-tile implicit-GEMM kernel for
// gfx950 (stride 1), fp32 accumulation and output.
//
// The contraction is the implicit GEMM of meganeura conv2d_grad_input_gemm.wgsl
// (header comment: C[Ci, pixels] = A[Ci, K] x B[K, pixels], K = Co*kH*kW),
// with K ordered (chunk of 32 output channels, tap, channel).  The bf16 matrix
// cores take 8 consecutive k per lane from both operands, so both operands are
// laid out output-channel-minor by two prologues:
//   * grad_out -> zero-padded NHWC copy (the zero border is the transposed
//     padding kH-1-pad of the shader's header comment), so a halo position's
//     32 channels of a chunk are one 64-byte run;
//   * weight   -> the exact lane order of the MFMA A fragments.
//
// Work-group: 256 threads = 2 x 2 waves over 64 input channels x a TR x TC
// pixel tile of one image.  Wave (wm, wn) owns input-channel blocks 2wm, 2wm+1
// (16 each) and pixel blocks wn*NBW .. wn*NBW + NBW - 1 (16 pixels each).
// Per chunk the tile's halo, (TR+kH-1) x (TC+kW-1) positions x 32 channels,
// is copied into LDS by direct global -> LDS loads (double-buffered), and tap
// (kh, kw) reads its B fragments as the halo shifted by (kH-1-kh, kW-1-kw).
// A fragments are loaded from the weight image straight into registers,
// several taps ahead.  LDS holds a position's four 16-byte channel groups in slots
// permuted by (position / 4) mod 4, and halo rows sit HP positions apart with
// HP = TC (mod 16): 16 lanes reading 16 consecutive pixels of the tile (which
// may wrap to the next tile row) then read 16 positions that are consecutive
// mod 16, i.e. 16 different bank groups.
//
// V_MFMA_F32_16X16X32_BF16: lane l = 16*g + i supplies A[i][k = 8g .. 8g+7]
// and B[k = 8g .. 8g+7][i] and receives D[4g + r][i], r = 0..3.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_common.h"
#include "gi_launch.h"

namespace gi {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9)
constexpr int kOOB = 0x7ffffff0;         // byte offset past the end of every buffer
constexpr int kQW = 8;                   // halo direct loads per wave per chunk (<= 32 rows)

typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (long)bytes, kRsrcWord3);
}

template <int NBW, int T>
__global__ __launch_bounds__(256, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void gi_halo_bf16(
    const HaloBf16Args A) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j16 = lane & 15, g = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;

    // Logical order: input-channel tile fastest, then column, row, image.
    const int J = xcd_order(blockIdx.x, gridDim.x);
    const int ci_tile = J % A.ci_tiles;
    int t = J / A.ci_tiles;
    const int ct = t % A.col_tiles;
    t /= A.col_tiles;
    const int rt = t % A.row_tiles;
    const int n = t / A.row_tiles;
    const int a0 = rt * A.TR, b0 = ct * A.TC;
    const int nq = A.HR * A.QR;           // direct loads per chunk (16 positions each)
    const int stage = A.HR * A.HP * 64;  // bytes per LDS stage

    const __amdgpu_buffer_rsrc_t grs = make_rsrc(A.gp, A.gp_bytes);
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(A.wk, A.wk_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(A.dst, A.d_bytes);

    // This lane's pixel in each of its blocks: halo position (0 outside the
    // tile or image: a valid position whose column is never stored).
    int ppos[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        const int p = (wn * NBW + b) * 16 + j16;
        const int r = p / A.TC, c = p - (p / A.TC) * A.TC;
        const bool v = p < A.TR * A.TC && a0 + r < A.H && b0 + c < A.W;
        ppos[b] = v ? r * A.HP + c : 0;
    }

    // Halo DMA: load q covers halo row q / QR, columns 16 (q % QR) .. +15;
    // lane -> (column + lane/4, slot lane%4) loads channel group
    // slot ^ ((lds position / 4) & 3).
    int goff[kQW];
#pragma unroll
    for (int i = 0; i < kQW; ++i) {
        const int q = wave + 4 * i;
        const int hr = q / A.QR, hc = (q - (q / A.QR) * A.QR) * 16 + (lane >> 2);
        const int lpos = hr * A.HP + hc;
        const int slot = lane & 3;
        const int kg = slot ^ ((lpos >> 2) & 3);
        const int y = a0 + hr, x = b0 + hc;
        const bool v = q < nq && hc < A.HC && y < A.YP && x < A.XP;
        goff[i] = v ? (((n * A.YP + y) * A.XP + x) * A.Cop + 8 * kg) * 2 : kOOB;
    }
    auto issue = [&](int chunk, int buf) {
#pragma unroll
        for (int i = 0; i < kQW; ++i) {
            const int q = wave + 4 * i;
            if (q < nq) {
                const int hr = q / A.QR, u = q - (q / A.QR) * A.QR;
                const int off = goff[i] == kOOB ? kOOB : goff[i] + chunk * 64;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    grs, (lds_ptr_t)(smem + buf * stage + (hr * A.HP + u * 16) * 64), 16, off, 0,
                    0, 0);
            }
        }
    };

    // A fragments: weight image offset of (chunk, tap, block 2wm + cb).
    const int wlane = (ci_tile * A.nchunks * T * 4 + 2 * wm) * 1024 + lane * 16;
    auto aload = [&](int chunk, int tap, int cb) {
        const int off = wlane + ((chunk * T + tap) * 4 + cb) * 1024;
        return __builtin_bit_cast(v8bf, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0));
    };

    v4f acc[2][NBW];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int b = 0; b < NBW; ++b) acc[cb][b] = v4f{0.f, 0.f, 0.f, 0.f};

    // Tap shifts in halo positions.
    int shift[T];
#pragma unroll
    for (int tp = 0; tp < T; ++tp) {
        const int kh = tp / A.kW, kw = tp - (tp / A.kW) * A.kW;
        shift[tp] = (A.kH - 1 - kh) * A.HP + (A.kW - 1 - kw);
    }

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
        if (chunk + 1 < A.nchunks) issue(chunk + 1, cur ^ 1);
        const unsigned char *hs = smem + cur * stage;
        // Per-lane positions, opaque to the optimiser so the tap x block
        // addresses are formed inside the chunk instead of being hoisted out of
        // the loop and held in registers.
        int pp[NBW];
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
            pp[b] = ppos[b];
            asm volatile("" : "+v"(pp[b]));
        }
        v8bf fb[2][NBW];
        auto bfetch = [&](int tp, int sl) {
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                const int pos = pp[b] + shift[tp];
                const int slot = g ^ ((pos >> 2) & 3);
                fb[sl][b] = *(const v8bf *)(hs + (pos * 4 + slot) * 16);
            }
        };
        bfetch(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tp = 0; tp < T; ++tp) {
            const int sl = tp & 1;
            const int as = tp;
            // Prefetch: A of step + AD, B of the next tap.
            {
                const int t2 = tp + AD;
                const int c2 = t2 < T ? chunk : chunk + 1;
                const int t2m = t2 < T ? t2 : t2 - T;
                if (c2 < A.nchunks) {
                    fa[t2m][0] = aload(c2, t2m, 0);
                    fa[t2m][1] = aload(c2, t2m, 1);
                }
            }
            if (tp + 1 < T) bfetch(tp + 1, sl ^ 1);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int b = 0; b < NBW; ++b)
                    acc[cb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[as][cb], fb[sl][b],
                                                                         acc[cb][b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

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

template <int NBW, int T>
hipError_t launch_one(const HaloBf16Args &a, int tiles, int ci_tiles, size_t lds, hipStream_t s,
                      const KernelEvents &ev) {
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)gi_halo_bf16<NBW, T>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (a.ci_tiles != ci_tiles) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL((gi_halo_bf16<NBW, T>), dim3(tiles * ci_tiles), dim3(256), (uint32_t)lds,
                          s, ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

constexpr int kCfg[][2] = {{7, 9}, {4, 9}, {7, 3}, {4, 3}};

// grad_out NCHW bf16 -> zero-padded NHWC bf16.  One work-group per (image n,
// block of 64 channels, band of RB rows of gp): the band is read along ow
// (coalesced), packed into channel pairs in LDS, and written as 16-byte runs
// of 8 channels per position.
__global__ __launch_bounds__(256) void pad_nhwc_bf16(const uint16_t *__restrict__ g,
                                                     uint16_t *__restrict__ gp,
                                                     const HaloBf16Args A, int oH, int oW,
                                                     int pad_h, int pad_w, int RB) {
    extern __shared__ uint32_t band[];  // [RB][oW][33] channel pairs
    const int n = blockIdx.x, co0 = blockIdx.y * 64, y0 = blockIdx.z * RB;
    const int yoff = A.kH - 1 - pad_h;  // oh = y - yoff
    const int xoff = A.kW - 1 - pad_w;  // ow = x - xoff
    // Thread -> one position of the band (fixed), looping over channel pairs:
    // no division per element.
    const int PB = RB * oW;
    const int PBc = PB < 256 ? PB : 256;
    const int cstep = 256 / PBc;
    const int64_t plane = (int64_t)oH * oW;
    for (int p0 = 0; p0 < PB; p0 += PBc) {
        const int pos = p0 + threadIdx.x % PBc;
        const int cp0 = threadIdx.x / PBc;
        if (cp0 >= cstep || pos >= PB) continue;
        const int ry = pos / oW, ow = pos - (pos / oW) * oW;
        const int oh = y0 + ry - yoff;
        const bool row_ok = y0 + ry < A.YP && oh >= 0 && oh < oH;
        const int64_t base = ((int64_t)n * A.Co * oH + oh) * oW + ow;
        uint32_t *dstb = band + pos * 33;
        for (int cp = cp0; cp < 32; cp += 4 * cstep) {
            uint32_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c2 = cp + u * cstep;
                const int co = co0 + 2 * c2;
                uint32_t lo = 0, hi = 0;
                if (row_ok && c2 < 32) {
                    if (co < A.Co) lo = g[base + co * plane];
                    if (co + 1 < A.Co) hi = g[base + (co + 1) * plane];
                }
                v[u] = lo | (hi << 16);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (cp + u * cstep < 32) dstb[cp + u * cstep] = v[u];
        }
    }
    __syncthreads();
    const int groups = min(8, (A.Cop - co0) / 8);  // 16-byte groups of 8 channels
    const int nstore = RB * A.XP * 8;
    for (int e = threadIdx.x; e < nstore; e += 256) {
        const int q = e & 7, pos = e >> 3;
        const int ry = pos / A.XP, x = pos - (pos / A.XP) * A.XP;
        const int y = y0 + ry;
        if (q >= groups || y >= A.YP) continue;
        const int ow = x - xoff;
        uint4 v = {0u, 0u, 0u, 0u};
        if (ow >= 0 && ow < oW) {
            const uint32_t *src = band + (ry * oW + ow) * 33 + 4 * q;
            v = uint4{src[0], src[1], src[2], src[3]};
        }
        *(uint4 *)(gp + (((int64_t)n * A.YP + y) * A.XP + x) * A.Cop + co0 + 8 * q) = v;
    }
}

// Weights [Co][Ci][kH][kW] bf16 -> A-fragment lane order (gi_common.h).  One
// work-group per (chunk of 32 output channels, ci tile, lane group g): it
// reads the 8 output channels 8g .. 8g+7 of the chunk for the tile's input
// channels and every tap (one contiguous run per channel) into LDS, and each
// thread then writes one lane's 16 bytes.
__global__ __launch_bounds__(256) void weight_frag_bf16(const uint16_t *__restrict__ w,
                                                        uint16_t *__restrict__ wk,
                                                        const HaloBf16Args A) {
    extern __shared__ uint16_t slab[];  // [8 co][64 ci * T]
    const int chunk = blockIdx.x, ct = blockIdx.y, g = blockIdx.z;
    const int T = A.kH * A.kW;
    const int run = 64 * T;
    const int ci_rows = min(64, A.Ci - ct * 64);
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

}  // namespace

int halo_bf16_config(int nbw, int taps) {
    for (int i = 0; i < (int)(sizeof(kCfg) / sizeof(kCfg[0])); ++i)
        if (kCfg[i][0] == nbw && kCfg[i][1] == taps) return i;
    return -1;
}

hipError_t launch_halo_bf16(const HaloBf16Args &a, int cfg, int tiles, int ci_tiles, size_t lds,
                            hipStream_t s, const KernelEvents &ev) {
    switch (cfg) {
        case 0: return launch_one<7, 9>(a, tiles, ci_tiles, lds, s, ev);
        case 1: return launch_one<4, 9>(a, tiles, ci_tiles, lds, s, ev);
        case 2: return launch_one<7, 3>(a, tiles, ci_tiles, lds, s, ev);
        case 3: return launch_one<4, 3>(a, tiles, ci_tiles, lds, s, ev);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_pad_nhwc_bf16(const uint16_t *g, uint16_t *gp, const HaloBf16Args &a, int oH,
                                int oW, int pad_h, int pad_w, hipStream_t s) {
    // Rows per work-group: at most what fits 16 KB of LDS, and few enough that
    // the grid has some 2048 work-groups to keep loads in flight.
    int RB = (int)(16384 / ((size_t)oW * 33 * sizeof(uint32_t)));
    const int64_t others = (int64_t)a.N * ((a.Cop + 63) / 64);
    const int want = (int)((a.YP * others + 2047) / 2048);
    if (want < RB) RB = want;
    RB = RB < 1 ? 1 : (RB > a.YP ? a.YP : RB);
    const size_t lds = (size_t)RB * oW * 33 * sizeof(uint32_t);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)pad_nhwc_bf16,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(pad_nhwc_bf16, dim3(a.N, (a.Cop + 63) / 64, (a.YP + RB - 1) / RB),
                       dim3(256), lds, s, g, gp, a, oH, oW, pad_h, pad_w, RB);
    return hipGetLastError();
}

hipError_t launch_weight_frag_bf16(const uint16_t *w, uint16_t *wk, const HaloBf16Args &a,
                                   int ci_tiles, hipStream_t s) {
    const size_t lds = (size_t)8 * 64 * a.kH * a.kW * sizeof(uint16_t);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)weight_frag_bf16,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(weight_frag_bf16, dim3(a.nchunks, ci_tiles, 4), dim3(256), lds, s, w, wk,
                       a);
    return hipGetLastError();
}

}  // namespace gi
