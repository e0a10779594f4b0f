// kernels_generic.hip -- weight reorder prologues and the generic
// phase-split implicit-GEMM kernels (fp32 and bf16 inputs) for gfx950.
//
// The GEMM per phase (see gi_common.h for the phase split):
//   C[ci, pixel] = sum over k of A[ci, k] * B[k, pixel]
//   k = (tap (j, jw), co)            tap-major, co fastest
//   A[ci, k] = weight[co, ci, r_h + s*j, r_w + s*jw]
//   B[k, pixel (n, a, b)] = grad_out[n, co, a + q_h - j, b + q_w - jw]  (0 outside)
// which is the implicit GEMM of meganeura conv2d_grad_input_gemm.wgsl (header
// comment: C[Ci, H*W] = A[Ci, K] x B[K, H*W]) restricted to the taps of one
// residue class, with the K axis ordered tap-major instead of co-major (the
// sum is the same).  Pixels of all batch items are folded into the GEMM's
// column axis; the B tile is gathered from HBM on the fly (no im2col buffer).
//
// These kernels handle every shape the library accepts and are the fallback
// of the planner; they favour simplicity over speed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_common.h"
#include "gi_launch.h"
#include "half_launch.h"

namespace gi {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Weight reorder prologues: one thread per output element, writes coalesced.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void weight_tap_co_ci_f32(const float *__restrict__ w,
                                                            float *__restrict__ wt, int Co,
                                                            int Ci, int kHW, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        int64_t ci = i % Ci;
        int64_t co = (i / Ci) % Co;
        int64_t tap = i / ((int64_t)Ci * Co);
        wt[i] = w[(co * Ci + ci) * kHW + tap];
    }
}

__global__ __launch_bounds__(256) void weight_tap_ci_co_bf16(const uint16_t *__restrict__ w,
                                                             uint16_t *__restrict__ wt, int Co,
                                                             int Ci, int kHW, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        int64_t co = i % Co;
        int64_t ci = (i / Co) % Ci;
        int64_t tap = i / ((int64_t)Ci * Co);
        wt[i] = w[(co * Ci + ci) * kHW + tap];
    }
}

static int prologue_blocks(int64_t total) {
    int64_t b = (total + 255) / 256;
    return (int)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

hipError_t launch_weight_tap_co_ci_f32(const float *w, float *wt, int Co, int Ci, int kHW,
                                       hipStream_t s) {
    int64_t total = (int64_t)Co * Ci * kHW;
    hipLaunchKernelGGL(weight_tap_co_ci_f32, dim3(prologue_blocks(total)), dim3(256), 0, s, w,
                       wt, Co, Ci, kHW, total);
    return hipGetLastError();
}

hipError_t launch_weight_tap_ci_co_bf16(const uint16_t *w, uint16_t *wt, int Co, int Ci,
                                        int kHW, hipStream_t s) {
    int64_t total = (int64_t)Co * Ci * kHW;
    hipLaunchKernelGGL(weight_tap_ci_co_bf16, dim3(prologue_blocks(total)), dim3(256), 0, s, w,
                       wt, Co, Ci, kHW, total);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Shared pieces of the generic kernels.
// ---------------------------------------------------------------------------

// Phase owning pixel tile `tile` (phases are few; a linear scan is enough).
__device__ __forceinline__ int find_phase(const GemmArgs &A, int tile) {
    int p = 0;
    for (int i = 1; i < A.nphases; ++i)
        if (tile >= A.ph[i].tile_begin) p = i;
    return p;
}

// Output row of MFMA 32x32 accumulator register r for lane `lane`: the 32x32
// result is held as 4-row groups, the two half-waves interleaved by 4 rows.
__device__ __forceinline__ int acc_row32(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Store a 32(ci) x 32(pixel) accumulator block into NCHW dst.
__device__ __forceinline__ void store_block(const GemmArgs &A, const Phase &P, const v16f &acc,
                                            int ci_base, int pcol, int npix, int lane) {
    if (pcol >= npix) return;
    const int HaWb = P.Ha * P.Wb;
    const int n = pcol / HaWb;
    const int rem = pcol - n * HaWb;
    const int a = rem / P.Wb;
    const int b = rem - a * P.Wb;
    const int ih = P.rho_h + A.stride * a;
    const int iw = P.rho_w + A.stride * b;
    const int64_t plane = (int64_t)A.H * A.W;
    float *d = A.dst + (int64_t)n * A.Ci * plane + (int64_t)ih * A.W + iw;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int ci = ci_base + acc_row32(r, lane);
        if (ci < A.Ci) d[(int64_t)ci * plane] = acc[r];
    }
}

// ---------------------------------------------------------------------------
// fp32 generic kernel: 256 threads, tile 64 ci x 128 pixels, K step 16 (one
// tap, 16 output channels).  Waves form 2 x 2; each owns 32 ci x 64 pixels =
// two 32x32x2 MFMA accumulators.  Global tiles are prefetched into registers
// one K step ahead and double-buffered in LDS.
// ---------------------------------------------------------------------------
template <int BK>
__global__ __launch_bounds__(256) void gi_generic_f32(const GemmArgs A) {
    constexpr int BM = kGenericBM, BN = kGenericBN, NT = 256;
    constexpr int LDA = BM + 32, LDB = BN + 32;  // row pads keep half-waves on distinct banks
    constexpr int B_RPP = NT / BN, B_PT = BK / B_RPP;
    constexpr int A_RPP = NT / BM, A_PT = BK / A_RPP;
    __shared__ float As[2][BK][LDA];
    __shared__ float Bs[2][BK][LDB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile = blockIdx.x;
    const int ci0 = blockIdx.y * BM;
    const Phase P = A.ph[find_phase(A, tile)];
    const int HaWb = P.Ha * P.Wb;
    const int npix = A.N * HaWb;
    const int pix0 = (tile - P.tile_begin) * BN;
    const int oHW = A.oH * A.oW;
    const int nco = (A.Co + BK - 1) / BK;
    const int T = P.J_h * P.J_w * nco;

    // B gather assignment: one pixel column, rows kb0, kb0 + B_RPP, ...
    const int pc = tid % BN, kb0 = tid / BN;
    const int pix = pix0 + pc;
    const bool pin = pix < npix;
    int n = 0, a = 0, b = 0;
    if (pin) {
        n = pix / HaWb;
        const int rem = pix - n * HaWb;
        a = rem / P.Wb;
        b = rem - a * P.Wb;
    }
    const float *gimg = (const float *)A.grad_out + (int64_t)n * A.Co * oHW;
    // A load assignment: one ci column, rows ka0, ka0 + A_RPP, ...
    const int ac = tid % BM, ka0 = tid / BM;
    const bool ain = ci0 + ac < A.Ci;
    const float *wt = (const float *)A.wt;

    float ra[A_PT], rb[B_PT];
    auto gload = [&](int it) {
        const int tap = it / nco;
        const int co0 = (it - tap * nco) * BK;
        const int j = tap / P.J_w, jw = tap - j * P.J_w;
        const int oh = a + P.q_h - j, ow = b + P.q_w - jw;
        const bool v = pin && oh >= 0 && oh < A.oH && ow >= 0 && ow < A.oW;
        const int off = v ? oh * A.oW + ow : 0;
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            const int co = co0 + kb0 + i * B_RPP;
            rb[i] = (v && co < A.Co) ? gimg[co * oHW + off] : 0.f;
        }
        const int kh = P.r_h + A.stride * j, kw = P.r_w + A.stride * jw;
        const float *ws = wt + (int64_t)(kh * A.kW + kw) * A.Co * A.Ci + ci0 + ac;
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
            const int co = co0 + ka0 + i * A_RPP;
            ra[i] = (ain && co < A.Co) ? ws[(int64_t)co * A.Ci] : 0.f;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PT; ++i) As[buf][ka0 + i * A_RPP][ac] = ra[i];
#pragma unroll
        for (int i = 0; i < B_PT; ++i) Bs[buf][kb0 + i * B_RPP][pc] = rb[i];
    };

    v16f acc0 = {}, acc1 = {};
    const int wm = wave >> 1, wn = wave & 1;
    const int kl = lane >> 5, ml = lane & 31;
    if (T > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int it = 0; it < T; ++it) {
            const int cur = it & 1;
            if (it + 1 < T) gload(it + 1);
#pragma unroll
            for (int kk = 0; kk < BK; kk += 2) {
                const float af = As[cur][kk + kl][wm * 32 + ml];
                const float b0 = Bs[cur][kk + kl][wn * 64 + ml];
                const float b1 = Bs[cur][kk + kl][wn * 64 + 32 + ml];
                acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(af, b0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(af, b1, acc1, 0, 0, 0);
            }
            if (it + 1 < T) sstore(cur ^ 1);
            __syncthreads();
        }
    }
    store_block(A, P, acc0, ci0 + wm * 32, pix0 + wn * 64 + ml, npix, lane);
    store_block(A, P, acc1, ci0 + wm * 32, pix0 + wn * 64 + 32 + ml, npix, lane);
}

// ---------------------------------------------------------------------------
// bf16 generic kernel: same tiling, K step 16 = one 32x32x16 bf16 MFMA.  The
// bf16 operand layout wants 8 consecutive k (= 8 consecutive co of one tap)
// per lane, so tiles sit in LDS k-fastest: As[ci][k], Bs[pixel][k].  The
// weight prologue stores co fastest, so A rows are contiguous in HBM; the B
// gather reads co rows of grad_out and transposes them on the LDS write.
// ---------------------------------------------------------------------------
// F16: fp16 inputs (V_MFMA_F32_32X32X16_F16), else bf16; same data path.
template <bool F16>
__global__ __launch_bounds__(256) void gi_generic_bf16(const GemmArgs A) {
    constexpr int BM = kGenericBM, BN = kGenericBN, BK = 16, NT = 256;
    constexpr int LDK = BK + 8;  // 48-byte rows: 16-byte aligned fragments
    constexpr int B_RPP = NT / BN, B_PT = BK / B_RPP;  // 2 rows per pass, 8 per thread
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile = blockIdx.x;
    const int ci0 = blockIdx.y * BM;
    const Phase P = A.ph[find_phase(A, tile)];
    const int HaWb = P.Ha * P.Wb;
    const int npix = A.N * HaWb;
    const int pix0 = (tile - P.tile_begin) * BN;
    const int oHW = A.oH * A.oW;
    const int nco = (A.Co + BK - 1) / BK;
    const int T = P.J_h * P.J_w * nco;

    const int pc = tid % BN, kb0 = tid / BN;
    const int pix = pix0 + pc;
    const bool pin = pix < npix;
    int n = 0, a = 0, b = 0;
    if (pin) {
        n = pix / HaWb;
        const int rem = pix - n * HaWb;
        a = rem / P.Wb;
        b = rem - a * P.Wb;
    }
    const uint16_t *gimg = (const uint16_t *)A.grad_out + (int64_t)n * A.Co * oHW;
    // A: thread -> ci row (tid / 4), 4 consecutive k at (tid % 4) * 4.
    const int ar = tid >> 2, ak = (tid & 3) * 4;
    const bool ain = ci0 + ar < A.Ci;
    const uint16_t *wt = (const uint16_t *)A.wt;

    uint16_t ra[4], rb[B_PT];
    auto gload = [&](int it) {
        const int tap = it / nco;
        const int co0 = (it - tap * nco) * BK;
        const int j = tap / P.J_w, jw = tap - j * P.J_w;
        const int oh = a + P.q_h - j, ow = b + P.q_w - jw;
        const bool v = pin && oh >= 0 && oh < A.oH && ow >= 0 && ow < A.oW;
        const int off = v ? oh * A.oW + ow : 0;
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            const int co = co0 + kb0 + i * B_RPP;
            rb[i] = (v && co < A.Co) ? gimg[co * oHW + off] : (uint16_t)0;
        }
        const int kh = P.r_h + A.stride * j, kw = P.r_w + A.stride * jw;
        const uint16_t *ws = wt + ((int64_t)(kh * A.kW + kw) * A.Ci + ci0 + ar) * A.Co;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int co = co0 + ak + i;
            ra[i] = (ain && co < A.Co) ? ws[co] : (uint16_t)0;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) As[buf][ar][ak + i] = ra[i];
#pragma unroll
        for (int i = 0; i < B_PT; ++i) Bs[buf][pc][kb0 + i * B_RPP] = rb[i];
    };

    v16f acc0 = {}, acc1 = {};
    const int wm = wave >> 1, wn = wave & 1;
    const int kl = (lane >> 5) * 8, ml = lane & 31;
    if (T > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int it = 0; it < T; ++it) {
            const int cur = it & 1;
            if (it + 1 < T) gload(it + 1);
            const v8bf af = *(const v8bf *)&As[cur][wm * 32 + ml][kl];
            const v8bf b0 = *(const v8bf *)&Bs[cur][wn * 64 + ml][kl];
            const v8bf b1 = *(const v8bf *)&Bs[cur][wn * 64 + 32 + ml][kl];
            if constexpr (F16) {
                const v8h ah = __builtin_bit_cast(v8h, af);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, __builtin_bit_cast(v8h, b0), acc0,
                                                              0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, __builtin_bit_cast(v8h, b1), acc1,
                                                              0, 0, 0);
            } else {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b1, acc1, 0, 0, 0);
            }
            if (it + 1 < T) sstore(cur ^ 1);
            __syncthreads();
        }
    }
    store_block(A, P, acc0, ci0 + wm * 32, pix0 + wn * 64 + ml, npix, lane);
    store_block(A, P, acc1, ci0 + wm * 32, pix0 + wn * 64 + 32 + ml, npix, lane);
}

hipError_t launch_generic_f32(const GemmArgs &a, int tiles_x, hipStream_t s,
                              const KernelEvents &ev) {
    hipExtLaunchKernelGGL(gi_generic_f32<16>, dim3(tiles_x, a.ci_tiles), dim3(256), 0, s,
                          ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

hipError_t launch_generic_bf16(const GemmArgs &a, int tiles_x, hipStream_t s,
                               const KernelEvents &ev) {
    hipExtLaunchKernelGGL(gi_generic_bf16<false>, dim3(tiles_x, a.ci_tiles), dim3(256), 0, s,
                          ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

hipError_t launch_generic_f16(const GemmArgs &a, int tiles_x, hipStream_t s,
                              const KernelEvents &ev) {
    hipExtLaunchKernelGGL(gi_generic_bf16<true>, dim3(tiles_x, a.ci_tiles), dim3(256), 0, s,
                          ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

}  // namespace gi
