// kernels_fwd_f32.hip -- the forward convolution (fp32) for gfx950: weight
// reorders and the generic implicit-GEMM kernel.  Stride-1 forwards run on
// the grad_input kernels instead (a forward correlation with pad p is the
// grad_input sum of the transposed, tap-reversed weight with pad k-1-p); the
// generic kernel serves every stride.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_common.h"

namespace gi {

typedef float v16f __attribute__((ext_vector_type(16)));

namespace {

// wt[(tap*Ci + ci)*Co + co] = w[(co*Ci + ci)*kHW + tap], then kFwdZeroTail
// zeros; one thread per output element, writes coalesced.
__global__ __launch_bounds__(256) void fwd_weight_tap_ci_co_f32(const float *__restrict__ w,
                                                                float *__restrict__ wt, int Co,
                                                                int Ci, int kHW, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total + kFwdZeroTail;
         i += (int64_t)gridDim.x * 256) {
        if (i >= total) {
            wt[i] = 0.f;
            continue;
        }
        const int64_t co = i % Co;
        const int64_t ci = (i / Co) % Ci;
        const int64_t tap = i / ((int64_t)Ci * Co);
        wt[i] = w[(co * Ci + ci) * kHW + tap];
    }
}

// wf[((ci*Co + co)*kHW) + t] = w[(co*Ci + ci)*kHW + kHW-1-t]: [Ci][Co][kH][kW]
// with both kernel axes reversed.
__global__ __launch_bounds__(256) void fwd_weight_flip_f32(const float *__restrict__ w,
                                                           float *__restrict__ wf, int Co, int Ci,
                                                           int kHW, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int64_t t = i % kHW;
        const int64_t co = (i / kHW) % Co;
        const int64_t ci = i / ((int64_t)kHW * Co);
        wf[i] = w[(co * Ci + ci) * kHW + (kHW - 1 - t)];
    }
}

// wt[k*Co + co] = w[co*K + k] (K = Ci*kH*kW): the weight as [K][Co] with k in
// the caller's (ci, kh, kw) order, for the flattened K axis; then
// kFwdZeroTail zeros.
__global__ __launch_bounds__(256) void fwd_weight_k_co_f32(const float *__restrict__ w,
                                                           float *__restrict__ wt, int Co, int K,
                                                           int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total + kFwdZeroTail;
         i += (int64_t)gridDim.x * 256) {
        if (i >= total) {
            wt[i] = 0.f;
            continue;
        }
        const int64_t co = i % Co;
        const int64_t k = i / Co;
        wt[i] = w[co * K + k];
    }
}

int reorder_blocks(int64_t total) {
    const int64_t b = (total + 255) / 256;
    return (int)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

// Output row of 32x32 accumulator register r for lane `lane`.
__device__ __forceinline__ int acc_row32(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// ---------------------------------------------------------------------------
// Generic forward kernel: 256 threads, tile 64 co x 128 pixels, K step 16.
// Waves form 2 x 2; each owns 32 co x 64 pixels = two V_MFMA_F32_32X32X2_F32
// accumulators.  Global tiles are prefetched into registers one K step ahead
// and double-buffered in LDS.  K order: FLATK = false, (ci block of 16, tap)
// with a K step = one tap x 16 input channels (one bounds test per pixel and
// step); FLATK = true, the caller's (ci, kh, kw) order (few input channels:
// no padding of Ci to 16), each k's plane offset and tap read from an LDS
// table.  VECA (Co % 4 == 0): the weight tile is loaded 16 bytes per thread.
// ---------------------------------------------------------------------------
template <bool FLATK, bool VECA>
__global__ __launch_bounds__(256) void gi_fwd_f32(const FwdArgs A) {
    constexpr int BM = kFwdBM, BN = kFwdBN, BK = 16, NT = 256;
    constexpr int B_RPP = NT / BN, B_PT = BK / B_RPP;
    constexpr int A_RPP = NT / BM, A_PT = BK / A_RPP;
    // No row pads: odd k rows store their columns XOR 32, so the two half
    // waves of an MFMA operand read (rows k and k+1, same columns) fall on
    // opposite halves of the 64 banks; a row write stays a bank permutation.
    __shared__ __attribute__((aligned(16))) float As[2][BK][BM];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK][BN];
    // FLATK: (ci*H*W + kh*W + kw, kh << 16 | kw) per k, sized K at launch.
    extern __shared__ int2 ktab[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Logical order: output-channel tile fastest, so the work-groups that
    // gather the same input pixels run together on one XCD's L2.
    const int co_tiles = (A.Co + BM - 1) / BM;
    const int J = xcd_order(blockIdx.x, gridDim.x);
    const int pix0 = (J / co_tiles) * BN;
    const int co0 = (J % co_tiles) * BM;
    const int oHW = A.oH * A.oW;
    const int npix = A.N * oHW;
    const int HW = A.H * A.W;
    const int kHW = A.kH * A.kW;
    const int nci = (A.Ci + BK - 1) / BK;
    const int K = A.Ci * kHW;
    const int T = FLATK ? (K + BK - 1) / BK : kHW * nci;
    if (FLATK) {
        for (int k = tid; k < K; k += NT) {
            const int ci = k / kHW, r = k - (k / kHW) * kHW;
            const int kh = r / A.kW, kw = r - (r / A.kW) * A.kW;
            ktab[k] = make_int2(ci * HW + kh * A.W + kw, (kh << 16) | kw);
        }
        __syncthreads();
    }

    // B gather assignment: one pixel column, rows kb0, kb0 + B_RPP, ...
    const int pc = tid % BN, kb0 = tid / BN;
    const int pix = pix0 + pc;
    const bool pin = pix < npix;
    int n = 0, oh = 0, ow = 0;
    if (pin) {
        n = pix / oHW;
        const int rem = pix - n * oHW;
        oh = rem / A.oW;
        ow = rem - oh * A.oW;
    }
    const int ih0 = oh * A.stride - A.pad_h, iw0 = ow * A.stride - A.pad_w;
    const float *ximg = A.x + (int64_t)n * A.Ci * HW;
    // A load assignment.  Co % 4 == 0 (VECA): four consecutive co of row
    // ka4, one 16-byte load (a group lies wholly below or above Co, and the
    // weight rows and the zero tail are 16-byte aligned).  Otherwise one co
    // column at rows ka0, ka0 + A_RPP, ...: four 4-byte loads.
    const int ac = tid % BM, ka0 = tid / BM;
    const bool ain = co0 + ac < A.Co;
    constexpr int A_CG = BM / 4;
    static_assert(A_PT == 4 && NT / A_CG == BK, "one 16-byte A load per thread and step");
    const int ac4 = (tid % A_CG) * 4, ka4 = tid / A_CG;
    const bool ain4 = co0 + ac4 < A.Co;

    // Every global load is issued unconditionally; an out-of-range lane
    // loads from the zeros after the reordered weight, so nothing touches the
    // loaded registers until they are stored to LDS after the step's MFMAs
    // (a select on the loaded value would make the compiler wait for the
    // loads in the middle of them).
    typedef float RegA[A_PT];
    typedef float RegB[B_PT];
    struct {
        int kh, kw, ci0;
    } nk = {0, 0, 0};   // position of the next step to load (FLATK = false)
    auto gload = [&](int it, RegA &ra, RegB &rb) {
        if (FLATK) {
            const int base = ih0 * A.W + iw0;
            // k is the same across a wave: the step's table entries are read
            // up front (broadcast reads, one wait), not one per load.  The
            // empty asm statement uses both halves of each entry, so the
            // compiler cannot sink a half of the read into the branch of the
            // lanes that need it (which made one LDS wait per element).
            int2 e[B_PT];
#pragma unroll
            for (int i = 0; i < B_PT; ++i) {
                const int k = it * BK + kb0 + i * B_RPP;
                e[i] = ktab[k < K ? k : K - 1];
                __asm__ volatile("" : : "v"(e[i].x), "v"(e[i].y));
            }
#pragma unroll
            for (int i = 0; i < B_PT; ++i) {
                const int k = it * BK + kb0 + i * B_RPP;
                const int kh = e[i].y >> 16, kw = e[i].y & 0xffff;
                const bool ok = pin && k < K && (unsigned)(ih0 + kh) < (unsigned)A.H &&
                                (unsigned)(iw0 + kw) < (unsigned)A.W;
                rb[i] = *(ok ? ximg + (e[i].x + base) : A.zero);
            }
            if (VECA) {
                const int k = it * BK + ka4;
                const bool ok = ain4 && k < K;
                const float4 w4 = *(const float4 *)(ok ? A.wt + ((int64_t)k * A.Co + co0 + ac4)
                                                       : A.zero);
                ra[0] = w4.x;
                ra[1] = w4.y;
                ra[2] = w4.z;
                ra[3] = w4.w;
                return;
            }
#pragma unroll
            for (int i = 0; i < A_PT; ++i) {
                const int k = it * BK + ka0 + i * A_RPP;
                const bool ok = ain && k < K;
                ra[i] = *(ok ? A.wt + ((int64_t)k * A.Co + co0 + ac) : A.zero);
            }
            return;
        }
        // Steps are loaded in order, channel block outer and tap inner: the
        // kH*kW consecutive steps of one block gather from the same input
        // rows, which stay in cache (tap-major order swept every channel
        // between two taps and re-fetched the input from HBM per tap).
        // (kh, kw, ci0) advance per call instead of being divided out of it.
        const bool live = it < T;
        const int kh = nk.kh, kw = nk.kw, ci0 = nk.ci0, tap = kh * A.kW + kw;
        if (++nk.kw == A.kW) {
            nk.kw = 0;
            if (++nk.kh == A.kH) {
                nk.kh = 0;
                nk.ci0 += BK;
            }
        }
        const int ih = ih0 + kh, iw = iw0 + kw;
        const bool v = live && pin && ih >= 0 && ih < A.H && iw >= 0 && iw < A.W;
        const int off = v ? ih * A.W + iw : 0;
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            const int ci = ci0 + kb0 + i * B_RPP;
            const bool ok = v && ci < A.Ci;
            rb[i] = *(ok ? ximg + ((int64_t)ci * HW + off) : A.zero);
        }
        if (VECA) {
            const int ci = ci0 + ka4;
            const bool ok = live && ain4 && ci < A.Ci;
            const float4 w4 = *(const float4 *)(
                ok ? A.wt + (((int64_t)tap * A.Ci + ci) * A.Co + co0 + ac4) : A.zero);
            ra[0] = w4.x;
            ra[1] = w4.y;
            ra[2] = w4.z;
            ra[3] = w4.w;
            return;
        }
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
            const int ci = ci0 + ka0 + i * A_RPP;
            const bool ok = live && ain && ci < A.Ci;
            ra[i] = *(ok ? A.wt + (((int64_t)tap * A.Ci + ci) * A.Co + co0 + ac) : A.zero);
        }
    };
    auto sw = [](int row, int col) { return col ^ ((row & 1) << 5); };
    auto sstore = [&](int buf, const RegA &ra, const RegB &rb) {
        if (VECA) {
            *(float4 *)&As[buf][ka4][sw(ka4, ac4)] = make_float4(ra[0], ra[1], ra[2], ra[3]);
        } else {
#pragma unroll
            for (int i = 0; i < A_PT; ++i) {
                const int r = ka0 + i * A_RPP;
                As[buf][r][sw(r, ac)] = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            const int r = kb0 + i * B_RPP;
            Bs[buf][r][sw(r, pc)] = rb[i];
        }
    };

    v16f acc0 = {}, acc1 = {};
    const int wm = wave >> 1, wn = wave & 1;
    const int kl = lane >> 5, ml = lane & 31;
    auto mma = [&](int cur) {
#pragma unroll
        for (int kk = 0; kk < BK; kk += 2) {
            // Row kk + kl with kk even: the swizzle is XOR 32 for kl = 1.
            const int x = kl << 5;
            const float af = As[cur][kk + kl][(wm * 32 + ml) ^ x];
            const float b0 = Bs[cur][kk + kl][(wn * 64 + ml) ^ x];
            const float b1 = Bs[cur][kk + kl][(wn * 64 + 32 + ml) ^ x];
            acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(af, b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(af, b1, acc1, 0, 0, 0);
        }
    };
    // Two register sets: step it + 2 is loaded while step it multiplies out
    // of one LDS buffer and step it + 1 moves into the other.
    if (T > 0) {
        RegA ra;
        RegB rb;
        gload(0, ra, rb);
        sstore(0, ra, rb);
        __syncthreads();
        for (int it = 0; it < T; ++it) {
            gload(it + 1, ra, rb);
            // Keep every load of the next step above this step's MFMAs (the
            // scheduler otherwise sinks some next to their LDS store, where
            // the wait for them exposes their whole latency).
            __builtin_amdgcn_sched_barrier(0);
            mma(it & 1);
            sstore((it & 1) ^ 1, ra, rb);
            __syncthreads();
        }
    }
    // Store: rows = output channels, column = this lane's pixel.
    auto store = [&](const v16f &acc, int pcol) {
        if (pcol >= npix) return;
        const int nn = pcol / oHW;
        const int rem = pcol - nn * oHW;
        float *d = A.y + (int64_t)nn * A.Co * oHW + rem;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int co = co0 + wm * 32 + acc_row32(r, lane);
            if (co < A.Co) d[(int64_t)co * oHW] = acc[r];
        }
    };
    store(acc0, pix0 + wn * 64 + ml);
    store(acc1, pix0 + wn * 64 + 32 + ml);
}

}  // namespace

hipError_t launch_fwd_weight_tap_ci_co_f32(const float *w, float *wt, int Co, int Ci, int kHW,
                                           hipStream_t s) {
    const int64_t total = (int64_t)Co * Ci * kHW;
    hipLaunchKernelGGL(fwd_weight_tap_ci_co_f32, dim3(reorder_blocks(total + kFwdZeroTail)),
                       dim3(256), 0, s, w, wt, Co, Ci, kHW, total);
    return hipGetLastError();
}

hipError_t launch_fwd_weight_flip_f32(const float *w, float *wf, int Co, int Ci, int kHW,
                                      hipStream_t s) {
    const int64_t total = (int64_t)Co * Ci * kHW;
    hipLaunchKernelGGL(fwd_weight_flip_f32, dim3(reorder_blocks(total)), dim3(256), 0, s, w, wf,
                       Co, Ci, kHW, total);
    return hipGetLastError();
}

hipError_t launch_fwd_weight_k_co_f32(const float *w, float *wt, int Co, int K, hipStream_t s) {
    const int64_t total = (int64_t)Co * K;
    hipLaunchKernelGGL(fwd_weight_k_co_f32, dim3(reorder_blocks(total + kFwdZeroTail)),
                       dim3(256), 0, s, w, wt, Co, K, total);
    return hipGetLastError();
}

bool fwd_flat_k(const FwdArgs &a) {
    return a.Ci < 16 && (int64_t)a.Ci * a.kH * a.kW <= kFwdMaxFlatK;
}

hipError_t launch_fwd_generic_f32(const FwdArgs &a, hipStream_t s, const KernelEvents &ev) {
    const int64_t npix = (int64_t)a.N * a.oH * a.oW;
    if (npix == 0 || a.Co == 0) return hipSuccess;
    const int64_t wgs = (npix + kFwdBN - 1) / kFwdBN * ((a.Co + kFwdBM - 1) / kFwdBM);
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs);
    const bool veca = a.Co % 4 == 0;
    if (fwd_flat_k(a)) {
        const size_t ktab = (size_t)a.Ci * a.kH * a.kW * sizeof(int2);
        if (veca)
            hipExtLaunchKernelGGL(gi_fwd_f32<true, true>, grid, dim3(256), ktab, s, ev.start,
                                  ev.stop, 0, a);
        else
            hipExtLaunchKernelGGL(gi_fwd_f32<true, false>, grid, dim3(256), ktab, s, ev.start,
                                  ev.stop, 0, a);
    } else if (veca) {
        hipExtLaunchKernelGGL(gi_fwd_f32<false, true>, grid, dim3(256), 0, s, ev.start, ev.stop,
                              0, a);
    } else {
        hipExtLaunchKernelGGL(gi_fwd_f32<false, false>, grid, dim3(256), 0, s, ev.start, ev.stop,
                              0, a);
    }
    return hipGetLastError();
}

}  // namespace gi
