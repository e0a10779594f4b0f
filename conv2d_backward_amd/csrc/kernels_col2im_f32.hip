// kernels_col2im_f32.hip -- fp32 column kernel for few input channels (gfx950).
//
// The gradient is the sum over (co, kh, kw) of weight x grad_out that the
// implicit GEMM of meganeura conv2d_grad_input_gemm.wgsl (header comment:
// C[Ci, pixels] = A[Ci, K] x B[K, pixels], K = Co*kH*kW) contracts in one
// go.  With Ci <= 4 that GEMM has at most 4 rows, so any matrix-core shape
// but the 4x4 blocks is mostly padding.  This kernel takes the same sum in
// two steps instead:
//   * columns: Y[q][c] = sum_co grad_out[co][q] * w[co][c] for every
//     grad_out position q = (oh, ow) and every column c = (ci, kh, kw): a
//     GEMM with M = positions, N = Ci*kH*kW (147 for an RGB 7x7 stem) and
//     K = Co, on V_MFMA_F32_16X16X4_F32;
//   * fold: Y[q][c] is added to input pixel (s*oh - pad_h + kh,
//     s*ow - pad_w + kw) of channel ci, the pixel whose gradient that
//     product belongs to (doppler conv2d_backward_input.wgsl: an input pixel
//     sums the contributions of every output pixel it fed).  Each column
//     lands on exactly one pixel, so taps that the stride rules out are never
//     formed.
//
// Work-group: 4 waves (one per SIMD) own a TH x TW tile of one image, held
// in LDS for every input channel with a border of kH-1 rows and at least
// kW-1 columns, and compute the columns of every grad_out position whose
// footprint meets the tile (positions on the border are also computed by
// the neighbouring work-group; each keeps what falls on its own tile).
//
// Matrix cores: lane l = 16g + i supplies A[i][k=g] = grad_out[4c+g][q_i]
// and B[k=g][i] = w[4c+g][16nb+i] for k step c and column block nb, and
// receives Y[q_{4g+r}][16nb+i] in register r.  The weight is staged once in
// LDS and its B fragments of every (c, nb) held in registers (16 x 10 for
// Co <= 64 and 160 columns); grad_out is read as blocks of 16 positions of
// one row.
//
// Fold: the accumulators of a block start as the tile values its columns
// land on (read from LDS), the block's 16 k steps add its products onto
// them, and they are written back: the fold costs LDS reads and writes but
// no vector ALU work, which on one wave per SIMD would hold up the matrix
// cores.  That needs the 64 pixels x 16 columns of a block to be distinct
// pixels, so a block's 16 positions are spread out: 8 positions 4 apart of
// grad_out row k (slots u = 0..7, column 4u + class) and the same 8 columns
// of row k + RW/2 (4*stride >= kW and (RW/2)*stride >= kH, so no two of
// them feed a common pixel).  D row 4g + r (lane group g, register r) is
// row k + RW/2 for g >= 2 and slot 4 (g & 1) + r at stride 1, (g & 1) + 2r
// at stride 2; lane i loads the position of D row i as its A row.  A pair of
// rows takes 4 such blocks (column classes 0..3, 32 positions of each row).
//
// LDS banks (64 of 4 bytes; a single-word read serves 32 lanes a cycle and
// needs their words distinct mod 32, a write serves 16): the tile's pitch and
// channel plane (kW and kH * kW mod 32) put column (ci, kh, kw) on bank
// (column index) + a per-lane constant, mod 32.  At stride 1 a block holds 16 consecutive
// columns and lane groups 0 and 1 are 16 words apart; at stride 2 they are 8
// apart and a pair of blocks splits 32 consecutive columns into alternate
// runs of 8.  Either way the 32 lanes of a half wave hit 32 distinct banks
// in every fold read and write.  Columns of one (ci, kh) still lie in one
// block or two adjacent ones.
//
// Order: between two blocks of a pair the last k step of one and the first
// of the next run back to back, with the first block's writes issued two
// MFMAs after the MFMA that finishes each column block, and each of the
// next block's reads after the write of the column block above it (a pixel
// is only reached by columns of one (ci, kh), i.e. of at most two adjacent
// column blocks).  The next block's loads are issued during the current
// block's middle k steps.  The four waves' rows are RW apart: wave w's pair
// k can only meet pixels of wave w + 1's earlier pairs, so wave w starts
// pair k once wave w + 1 has finished pair k - 1 (a count per wave in LDS),
// and the waves run staggered by an eighth of a block, so that their folds
// reach the LDS at different moments.  A pixel that two waves reach receives wave
// w + 1's columns first; every pixel receives its columns in a fixed order
// and the result is deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_common.h"
#include "gi_launch.h"

namespace gi {

typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9)
constexpr int kOOB = 0x7ffffff0;        // byte offset past the end of every buffer
constexpr int kSteps = kCol2imMaxCo / 4;  // k steps of 4 output channels
constexpr int kDephaseSleep = 10;         // s_sleep units (64 cycles): an eighth of a block

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (long)bytes, kRsrcWord3);
}

// Load at byte offset voff (per lane) + soff (uniform).
__device__ __forceinline__ float load_f32s(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// NBN: column blocks of 16 (Ci*kH*kW <= 16*NBN); S: the stride; CO: 64 when
// Co is 64 (every k step whole), 4 when Co is another multiple of 4 (k
// steps wholly inside or past Co), 0 otherwise.  Every grad_out row of a
// tile takes kCol2imBlocksPerRow = 2 windows of 16 positions.
template <int NBN, int S, int CO>
__global__ __launch_bounds__(256, 1) void gi_col2im_f32(const Col2imArgs A) {
    extern __shared__ __attribute__((aligned(16))) float tile[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i = lane & 15;
    // Position slots between a lane group's registers r and r + 1.
    constexpr int DELTA = S == 2 ? 2 : 1;

    // Logical order: tile column fastest, then tile row, image.
    int bid = xcd_order(blockIdx.x, gridDim.x);
    const int tc = bid % A.tiles_c;
    bid /= A.tiles_c;
    const int tr = bid % A.tiles_r;
    const int n = bid / A.tiles_r;
    const int ih0 = tr * A.TH, iw0 = tc * A.TW;

    // grad_out rows and columns whose footprint meets the tile: position oh
    // feeds input rows S*oh - pad_h .. S*oh - pad_h + kH - 1.
    const int xr = ih0 + A.pad_h - A.kH + 1, xc = iw0 + A.pad_w - A.kW + 1;
    const int oh_lo = xr <= 0 ? 0 : (xr + S - 1) / S;
    const int ow_lo = xc <= 0 ? 0 : (xc + S - 1) / S;
    const int oh_hi = min(A.oH - 1, (ih0 + A.TH - 1 + A.pad_h) / S);
    const int ow_hi = min(A.oW - 1, (iw0 + A.TW - 1 + A.pad_w) / S);
    const int row0 = oh_lo + wave * A.RW;
    const int rows_w = max(0, min(A.RW, oh_hi - row0 + 1));  // this wave's rows

    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(A.w, A.w_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(A.dst, A.d_bytes);

    // LDS: the tile [Ci][plane] (rows of LP floats), 32 slots (plus the
    // fold's position and class offsets) on 32 banks for columns past the
    // last and missing rows, then the weight staged as [kCol2imMaxCo][ws]
    // (rows past Co and columns past ncols zero).
    const int plane = A.plane;
    const int tfl = A.Ci * plane;
    const int dbase = (tfl + 31) / 32 * 32;
    float *const wst = tile + A.wofs;
    // Pairs finished per wave (LDS), past the dummy slots.
    volatile int *const done = (volatile int *)(tile + dbase + 96);
    if (tid < 4) done[tid] = 0;
    // grad_out of a block: lane i loads the position of D row i (row k of
    // the pair for i < 8, row k + RW/2 for i >= 8), output channel 4c + g at
    // byte offset vo (the pair and the lane) + 4 class + c * 16 * oH * oW
    // (uniform); zeros past the wave's rows, the tile's positions or Co.
    // Steps wholly past Co are not loaded; with CO = 0 the channels of the
    // last step past Co take the kOOB offset.
    const int oHW = A.oH * A.oW;
    const int csteps = (A.Co + 3) / 4;
    const int RWh = A.RW / 2;
    // This lane's position column (class 0): D row i's slot.
    const int owl = ow_lo + 4 * (DELTA == 1 ? (i & 7) : ((i >> 2) & 1) + 2 * (i & 3));
    auto pair_vo = [&](int k) {
        const int row = k + (i >= 8 ? RWh : 0);
        return row < rows_w ? (((n * A.Co + g) * A.oH + row0 + row) * A.oW + owl) * 4 : kOOB;
    };
    // k step c reads through one descriptor over all of grad_out with the
    // step's 4 output channels (c * 16 * oH * oW bytes) as the load's scalar
    // offset; the class is part of the lane offset.  Steps wholly past Co are
    // never loaded (their weights are zero and x keeps its zero).  A lane
    // offset of kOOB is past the range whether or not the range check counts
    // the scalar offset (kOOB plus any step offset stays below 2^32).
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(A.grad_out, A.g_bytes);
    const uint32_t step_bytes = 16u * (uint32_t)oHW;  // 4 output channels
    auto gload1 = [&](int c, int vo, int cls, float &x) {
        if (CO != 64 && c >= csteps) return;
        const int lo = CO != 0 || 4 * c + g < A.Co ? vo + 4 * cls : kOOB;
        x = load_f32s(grs, lo, (int)((uint32_t)c * step_bytes));
    };
    // The lane's load offset for class cls (kOOB past the tile's positions).
    auto class_vo = [&](int vo, int cls) { return owl + cls <= ow_hi ? vo : kOOB; };
    float gA[kSteps], gB[kSteps];
#pragma unroll
    for (int c = 0; c < kSteps; ++c) gA[c] = gB[c] = 0.f;
    // Weight rows: four lanes per row of output channel co = tid / 4, 16
    // bytes each at columns j = 4 (tid mod 4) + 16 m; these loads and the
    // first block's grad_out are issued before the tile is cleared.  Buffer
    // loads need 4-byte alignment only; words of a quad past ncols (the next
    // row's) are replaced by zeros.
    // (Columns j < 16 NBN: every column block's; pass m covers 16.)
    const int sco = tid >> 2, sj = 4 * (tid & 3);
    v4f wq[NBN];
#pragma unroll
    for (int m = 0; m < NBN; ++m) {
        const int j = sj + 16 * m;
        wq[m] = v4f{0.f, 0.f, 0.f, 0.f};
        if (sco < A.Co && j < A.ncols)
            wq[m] = __builtin_bit_cast(
                v4f, __builtin_amdgcn_raw_buffer_load_b128(wrs, (sco * A.ncols + j) * 4, 0, 0));
    }
    {
        const int vo = class_vo(pair_vo(0), 0);
#pragma unroll
        for (int c = 0; c < kSteps; ++c) gload1(c, vo, 0, gA[c]);
    }
    for (int k = tid * 4; k < tfl; k += 1024) *(v4f *)(tile + k) = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NBN; ++m) {
        const int j = sj + 16 * m;
        v4f v = wq[m];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j + e >= A.ncols) v[e] = 0.f;
        *(v4f *)(wst + sco * A.ws + j) = v;
    }

    __syncthreads();  // the tile is zero and the weight staged

    // Column of lane i in block nb: at stride 2, blocks 2q and 2q + 1 take
    // the alternate runs of 8 of columns 32q .. 32q + 31 (a last unpaired
    // block takes 16 consecutive ones).
    auto column = [&](int nb) {
        if (S == 2 && nb < (NBN & ~1)) return 32 * (nb >> 1) + 8 * (nb & 1) + (i & 7) + 16 * (i >> 3);
        return 16 * nb + i;
    };
    // B fragments of every k step and column block (zero past Co and
    // ncols, as staged).
    float wv[kSteps][NBN];
#pragma unroll
    for (int c = 0; c < kSteps; ++c)
#pragma unroll
        for (int nb = 0; nb < NBN; ++nb) wv[c][nb] = wst[(4 * c + g) * A.ws + column(nb)];

    // Tile offset of this lane's column in block nb relative to its
    // position's first pixel: channel plane, kh rows, kw columns (the same
    // arithmetic past the last column gives the bank its slot takes).
    const int khw = A.kH * A.kW;
    int cbase[NBN];
    unsigned colok = 0;
#pragma unroll
    for (int nb = 0; nb < NBN; ++nb) {
        // (x * ceil(2^16 / d)) >> 16 = x / d for x, d < 256.
        const int col = column(nb);
        const int ci = (int)(((uint32_t)col * A.magic_khw) >> 16), rem = col - ci * khw;
        const int kh = (int)(((uint32_t)rem * A.magic_kw) >> 16), kw = rem - kh * A.kW;
        cbase[nb] = ci * plane + kh * A.LP + kw;
        if (col < A.ncols) colok |= 1u << nb;
    }

    // Fold byte addresses of the pair of rows (k, k + RW/2), class 0, r = 0
    // (D row 4g + r: row k + RW/2 for g >= 2, slot u0 + DELTA r); r and the
    // class are immediate offsets (4 DELTA S r + S class floats).  Columns
    // past the last and a missing second row go to the slot past the tile
    // on the bank the real address would take.
    int ad[NBN];
    auto pair_addr = [&](int k) {
        const bool hi = g >= 2;
        const bool rv = !hi || k + RWh < rows_w;
        const int u0 = DELTA == 1 ? 4 * (g & 1) : (g & 1);
        const int qoff = (S * (row0 + k + (hi ? RWh : 0)) - A.pad_h - ih0 + A.r0) * A.LP +
                         S * (ow_lo + 4 * u0) - A.pad_w - iw0 + A.c0;
#pragma unroll
        for (int nb = 0; nb < NBN; ++nb) {
            const int real = cbase[nb] + qoff;
            ad[nb] = (rv && (colok >> nb & 1u) ? real : dbase + (real & 31)) * 4;
        }
    };
    // Tile reads and writes of column block nb for class cls, r = 0..3.
    auto tread = [&](int nb, int cls, v4f(&acc)[NBN]) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc[nb][r] = *(const float *)((const char *)tile + ad[nb] +
                                          (4 * DELTA * S * r + S * cls) * 4);
    };
    auto twrite = [&](int nb, int cls, const v4f(&acc)[NBN]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            *(float *)((char *)tile + ad[nb] + (4 * DELTA * S * r + S * cls) * 4) = acc[nb][r];
            asm volatile("" ::: "memory");  // single-word writes, straight from the accumulators
        }
    };
    auto mfma = [&](const float(&gc)[kSteps], int c, int nb, v4f(&acc)[NBN]) {
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(gc[c], wv[c][nb], acc[nb], 0, 0, 0);
    };

    // The middle k steps 1..14 of a block (operands gc), with the loads of
    // the next block (class ncls at pair offset nvo, into gn) among them.
    auto middle = [&](const float(&gc)[kSteps], v4f(&acc)[NBN], float(&gn)[kSteps], int nvo,
                      int ncls) {
        const int vo = class_vo(nvo, ncls);
#pragma unroll
        for (int c = 1; c < kSteps - 1; ++c) {
#pragma unroll
            for (int nb = 0; nb < NBN; ++nb) {
                mfma(gc, c, nb, acc);
                if (nb == 0) gload1(c - 1, vo, ncls, gn[c - 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        gload1(kSteps - 2, vo, ncls, gn[kSteps - 2]);
        gload1(kSteps - 1, vo, ncls, gn[kSteps - 1]);
    };
    // The last k step of class cls (operands gc) and the first of class
    // cls + 1 (operands gn), with the writes of cls and the reads of cls + 1.
    auto boundary = [&](const float(&gc)[kSteps], const float(&gn)[kSteps], int cls,
                        v4f(&acc)[NBN]) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < NBN; ++t) {
            mfma(gc, kSteps - 1, t, acc);
            if (t >= 2) twrite(t - 2, cls, acc);
            if (t >= 3) tread(t - 3, cls + 1, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int w = NBN - 2; w < NBN; ++w)
            if (w >= 0) twrite(w, cls, acc);
#pragma unroll
        for (int r = NBN - 3; r < NBN; ++r)
            if (r >= 0) tread(r, cls + 1, acc);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < NBN; ++nb) {
            mfma(gn, 0, nb, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    v4f acc[NBN];
    // Pairs of rows (k, k + RW/2): four blocks (classes 0..3).  gA holds
    // class 0 of the pair when it starts.  Wave w's pair k meets another
    // wave's pixels only where wave w + 1 is still on an earlier pair (rows
    // RW apart, RW/2 >= ceil(kH / S)), so before pair k >= 1 wave w waits
    // until wave w + 1 has finished pair k - 1 (its count in LDS); wave 3
    // never waits and no wave waits on a lower one, so every wait ends.  The
    // waves start staggered, wave w + 1 an eighth of a block ahead of wave w,
    // so that their folds do not reach the LDS at the same moments (measured
    // on the stem: no stagger 48.7 us, an eighth 46.8, a quarter 47.6).
    for (int z = wave; z < 3; ++z) __builtin_amdgcn_s_sleep(kDephaseSleep);
    for (int k = 0; k < RWh; ++k) {
        if (wave < 3 && k > 0) {
            // (Bounded: far past any wait the protocol allows.)
            for (int spin = 0; spin < (1 << 22) &&
                               __builtin_amdgcn_readfirstlane(done[wave + 1]) < k;
                 ++spin)
                __builtin_amdgcn_s_sleep(1);
            asm volatile("" ::: "memory");
        }
        if (k < rows_w) {
            pair_addr(k);
            const int vo = pair_vo(k);
            const int vo_next = pair_vo(k + 1);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int nb = 0; nb < NBN; ++nb) tread(nb, 0, acc);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int nb = 0; nb < NBN; ++nb) mfma(gA, 0, nb, acc);
            middle(gA, acc, gB, vo, 1);
            boundary(gA, gB, 0, acc);
            middle(gB, acc, gA, vo, 2);
            boundary(gB, gA, 1, acc);
            middle(gA, acc, gB, vo, 3);
            boundary(gA, gB, 2, acc);
            middle(gB, acc, gA, vo_next, 0);
#pragma unroll
            for (int nb = 0; nb < NBN; ++nb) mfma(gB, kSteps - 1, nb, acc);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int nb = 0; nb < NBN; ++nb) twrite(nb, 3, acc);
            asm volatile("" ::: "memory");
        }
        // The pair's writes are complete before its count goes up.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane == 0) done[wave] = k + 1;
        asm volatile("" ::: "memory");
    }
    __syncthreads();  // every wave's fold is in the tile

    // Epilogue: the tile's pixels inside the image, 16 bytes per lane where
    // rows are whole quads (lanes: 16 quads of a row, 16 rows at a time; the
    // LDS rows need not be 16-byte aligned, so four single-word reads).
    const int H = A.H, W = A.W;
    if ((W & 3) == 0 && (A.TW & 3) == 0) {
        const int qr = A.TW / 4;
        for (int qc = tid & 15; qc < qr; qc += 16)
            for (int ci = 0; ci < A.Ci; ++ci)
                for (int row = tid >> 4; row < A.TH; row += 16) {
                    const int ih = ih0 + row, iw = iw0 + 4 * qc;
                    const float *t = tile + ci * plane + (A.r0 + row) * A.LP + A.c0 + 4 * qc;
                    const v4f v = v4f{t[0], t[1], t[2], t[3]};
                    const int off =
                        (ih < H && iw < W) ? (((n * A.Ci + ci) * H + ih) * W + iw) * 4 : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), drs,
                        off, 0, 0);
                }
    } else {
        for (int col = tid & 15; col < A.TW; col += 16)
            for (int ci = 0; ci < A.Ci; ++ci)
                for (int row = tid >> 4; row < A.TH; row += 16) {
                    const int ih = ih0 + row, iw = iw0 + col;
                    const float v = tile[ci * plane + (A.r0 + row) * A.LP + A.c0 + col];
                    const int off =
                        (ih < H && iw < W) ? (((n * A.Ci + ci) * H + ih) * W + iw) * 4 : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), drs, off, 0, 0);
                }
    }
}

// Work-groups of this kernel run one per compute unit: its four waves take
// a SIMD each, and asking for more than half the CU's LDS keeps a second
// work-group from sharing it.
constexpr size_t kOnePerCuLds = 80 * 1024 + 256;

}  // namespace

int col2im_f32_weight_offset(const Col2imArgs &a) {
    // The tile, then 32 slots on 32 banks plus the fold's largest immediate
    // offset (4 DELTA S * 3 + S * 3 <= 54 floats) for columns past the last,
    // then the 4 waves' pair counts; the weight stage starts 16-byte aligned.
    return (a.Ci * a.plane + 31) / 32 * 32 + 96 + 8;
}

size_t col2im_f32_lds_bytes(const Col2imArgs &a) {
    const size_t bytes =
        ((size_t)col2im_f32_weight_offset(a) + (size_t)kCol2imMaxCo * a.ws) * sizeof(float);
    return bytes > kOnePerCuLds ? bytes : kOnePerCuLds;
}

namespace {

template <int S, int CO>
const void *col2im_fn(int nbn) {
    switch (nbn) {
        case 1: return (const void *)gi_col2im_f32<1, S, CO>;
        case 2: return (const void *)gi_col2im_f32<2, S, CO>;
        case 3: return (const void *)gi_col2im_f32<3, S, CO>;
        case 4: return (const void *)gi_col2im_f32<4, S, CO>;
        case 5: return (const void *)gi_col2im_f32<5, S, CO>;
        case 6: return (const void *)gi_col2im_f32<6, S, CO>;
        case 7: return (const void *)gi_col2im_f32<7, S, CO>;
        case 8: return (const void *)gi_col2im_f32<8, S, CO>;
        case 9: return (const void *)gi_col2im_f32<9, S, CO>;
        case 10: return (const void *)gi_col2im_f32<10, S, CO>;
        default: return nullptr;
    }
}

template <int S>
const void *col2im_fn_co(int nbn, int Co) {
    return Co == 64 ? col2im_fn<S, 64>(nbn) : Co % 4 == 0 ? col2im_fn<S, 4>(nbn) : col2im_fn<S, 0>(nbn);
}

}  // namespace

hipError_t launch_col2im_f32(const Col2imArgs &a, hipStream_t s, const KernelEvents &ev) {
    const int nbn = (a.ncols + 15) / 16;
    // The shapes the kernel's indexing assumes.
    if (a.ncols != a.Ci * a.kH * a.kW || nbn < 1 || nbn > kCol2imMaxBlocks)
        return hipErrorInvalidValue;
    if (a.Co <= kCol2imMinCo || a.Co > kCol2imMaxCo || a.stride < 1 ||
        a.stride > kCol2imMaxStride || a.kW > 4 * a.stride)
        return hipErrorInvalidValue;
    // Every tile's grad_out rows fit the four waves' RW rows each, a wave's
    // two row sets are D apart (RW even, RW/2 >= D), and every row's
    // positions fit its blocks.
    const int D = (a.kH + a.stride - 1) / a.stride;
    if ((a.RW & 1) || a.RW / 2 < D || 4 * a.RW < (a.TH + a.kH - 2) / a.stride + 1)
        return hipErrorInvalidValue;
    if (a.wofs != col2im_f32_weight_offset(a)) return hipErrorInvalidValue;
    // Staged weight rows hold every column block; the divisions by
    // reciprocal are exact for the column indices (< 256) and divisors.
    if (a.ws < 16 * nbn || (a.ws & 3) || a.kH * a.kW > 255 ||
        a.magic_khw != recip16(a.kH * a.kW) || a.magic_kw != recip16(a.kW))
        return hipErrorInvalidValue;
    if ((a.TW + a.kW - 2) / a.stride + 1 > 16 * kCol2imBlocksPerRow) return hipErrorInvalidValue;
    // Border and alignment of the LDS tile; its row pitch holds the pixels of
    // every position of a row's blocks (those past the tile's positions fold
    // zeros into the border).
    if (a.r0 < a.kH - 1 || a.LR < a.r0 + a.TH + a.kH - 1 || a.c0 < a.kW - 1 ||
        a.LP < a.c0 + 16 * a.stride * kCol2imBlocksPerRow + a.kW ||
        a.LP < a.c0 + a.TW + a.kW - 1 || a.plane < a.LR * a.LP)
        return hipErrorInvalidValue;
    if ((int64_t)a.tiles_r * a.TH < a.H || (int64_t)a.tiles_c * a.TW < a.W)
        return hipErrorInvalidValue;
    const size_t lds = col2im_f32_lds_bytes(a);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const int64_t wgs = (int64_t)a.N * a.tiles_r * a.tiles_c;
    if (wgs < 1 || wgs > INT32_MAX) return hipErrorInvalidValue;
    const void *fn = a.stride == 1 ? col2im_fn_co<1>(nbn, a.Co) : col2im_fn_co<2>(nbn, a.Co);
    if (!fn) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    void *args[] = {const_cast<Col2imArgs *>(&a)};
    return hipExtLaunchKernel(fn, dim3((unsigned)wgs), dim3(256), args, lds, s, ev.start, ev.stop,
                              0);
}

}  // namespace gi
