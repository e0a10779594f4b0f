/*
 * oracle.c -- plain CPU reference for the gradient of a 2-D convolution with
 * respect to its input, and a separately written forward convolution.
 *
 * TEST INFRASTRUCTURE.  This file is the checker, not the product: only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark load it.  It
 * shares no source, header, table or helper with the GPU library.
 *
 * Everything is accumulated in IEEE double, in one fixed order per output
 * element, with no fast-math, so a result does not depend on the thread count.
 *
 * Definitions followed
 * --------------------
 * grad_input (doppler conv2d_backward_input.wgsl, the direct kernel and its
 * header comment; meganeura conv2d_grad_input_gemm.wgsl, the general-stride
 * branch of the B-tile gather).  Each input pixel (n, ci, ih, iw) collects
 * every output-gradient value it fed in the forward pass:
 *
 *   grad_input[n,ci,ih,iw] = sum over co < Co, kh < kH, kw < kW of
 *                            grad_out[n,co,oh,ow] * weight[co,ci,kh,kw]
 *   where a = ih + pad_h - kh and b = iw + pad_w - kw must both be >= 0,
 *   divisible by the stride, and give oh = a/stride < oH, ow = b/stride < oW.
 *   Terms that fail a condition are absent; an element with none is 0.
 *
 * The doppler kernel has one batch item and one pad; meganeura carries the
 * batch on the grid and separate pad_h / pad_w.  Both are merged here: N
 * independent batch items, per-dimension symmetric zero padding, one stride
 * for both dimensions.  Rather than testing every tap against the three
 * conditions, each element enumerates the output rows and columns whose
 * forward window covered it (a range per dimension, from the forward mapping
 * below) and recovers each term's tap from that mapping: the same terms, so
 * the same sum.
 *
 * abs_sum[n,ci,ih,iw] = the same sum of |grad_out * weight| (used to scale the
 * floating-point tolerance of a GPU result).
 *
 * Forward convolution (the forward mapping stated in the doppler direct
 * kernel's comment: an output pixel oy reads input row oy*stride - pad + ky):
 *
 *   y[n,co,oh,ow] = sum over ci, kh, kw of
 *                   x[n,ci,oh*stride-pad_h+kh, ow*stride-pad_w+kw] * w[co,ci,kh,kw]
 *   with x taken as 0 outside [0,H) x [0,W).
 *
 * It is written from the forward side on purpose (a loop over output pixels),
 * so the adjoint identity <conv(x,w), g> = <x, grad_input(g,w)> checks the two
 * against each other rather than against a shared index formula.
 *
 * grad_weight (doppler conv2d_backward.js, the computeGradWeight branch: a
 * [outChannels, inChannels, kernelH, kernelW] result computed from gradOutput
 * and the forward input; its shader is not on the pages, so the definition is
 * the derivative of the forward mapping above with respect to w):
 *
 *   grad_weight[co,ci,kh,kw] = sum over n < N, oh < oH, ow < oW of
 *                              grad_out[n,co,oh,ow] * x[n,ci,ih,iw]
 *   with ih = oh*stride - pad_h + kh, iw = ow*stride - pad_w + kw; terms with
 *   (ih, iw) outside [0,H) x [0,W) are absent.
 *
 * It is written from the weight side (a loop over the output pixels each
 * weight element touched), so <conv(x,w), g> = <w, grad_weight(x,g)> checks
 * it against the forward function, and <x, grad_input(g,w)> = <w,
 * grad_weight(x,g)> against grad_input.  abs_sum is the same sum of
 * |grad_out * x|.
 *
 * grad_bias (doppler bias_add_backward.wgsl: the bias gradient is the output
 * gradient summed over every position the bias was added to; for a
 * convolution's per-output-channel bias those are all (n, oh, ow)):
 *
 *   grad_bias[co] = sum over n < N, oh < oH, ow < oW of grad_out[n,co,oh,ow]
 *
 * in the order n, oh, ow; abs_sum is the sum of |grad_out|.
 *
 * The forward function also comes with the sum of |x * w| per output element
 * (the scale of a GPU forward result's tolerance) and a sampled form, both
 * from one per-element routine that sums in the same order as the full loop.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH, oW;
} shape_t;

static shape_t make_shape(int N, int Ci, int H, int W, int Co, int kH, int kW,
                          int stride, int pad_h, int pad_w, int oH, int oW)
{
    shape_t s = {N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH, oW};
    return s;
}

/*
 * Along one dimension: the output positions whose forward window covered
 * input index i.  Output position o reads input index o*stride - pad + k for
 * the taps k in [0, K), so o covers i exactly when k = i + pad - o*stride
 * lies in [0, K), i.e. when i + pad - K < o*stride <= i + pad.  The first
 * such o is ceil((i + pad - K + 1) / stride), at least 0; the last is
 * floor((i + pad) / stride), at most out - 1.  lo > hi means none.
 */
static void covering_outputs(int64_t i, int64_t pad, int64_t K, int64_t stride,
                             int64_t out, int64_t *lo, int64_t *hi)
{
    const int64_t top = i + pad;          /* >= 0: i and pad are */
    const int64_t bottom = top - K + 1;   /* may be negative */
    *lo = bottom <= 0 ? 0 : (bottom + stride - 1) / stride;
    *hi = top / stride;
    if (*hi > out - 1) *hi = out - 1;
}

/*
 * One grad_input element: the sum over output channels of every output
 * gradient value this input pixel fed in the forward pass, each times the
 * weight tap that carried it.  The covering output rows and columns come
 * from covering_outputs; the tap is recovered from the forward mapping.
 */
static void grad_input_element(const double *grad_out, const double *weight,
                               const shape_t *s, int64_t n, int64_t ci,
                               int64_t ih, int64_t iw, double *value,
                               double *abs_value)
{
    int64_t oh_lo, oh_hi, ow_lo, ow_hi;
    covering_outputs(ih, s->pad_h, s->kH, s->stride, s->oH, &oh_lo, &oh_hi);
    covering_outputs(iw, s->pad_w, s->kW, s->stride, s->oW, &ow_lo, &ow_hi);
    double acc = 0.0, acc_abs = 0.0;
    for (int64_t co = 0; co < s->Co; ++co) {
        const double *g_plane = grad_out + (n * s->Co + co) * s->oH * s->oW;
        const double *w_taps = weight + (co * s->Ci + ci) * s->kH * s->kW;
        for (int64_t oh = oh_lo; oh <= oh_hi; ++oh) {
            const int64_t kh = ih + s->pad_h - oh * s->stride;
            for (int64_t ow = ow_lo; ow <= ow_hi; ++ow) {
                const int64_t kw = iw + s->pad_w - ow * s->stride;
                const double t = g_plane[oh * s->oW + ow] * w_taps[kh * s->kW + kw];
                acc += t;
                acc_abs += fabs(t);
            }
        }
    }
    *value = acc;
    *abs_value = acc_abs;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Full grad_input.  grad_out [N,Co,oH,oW], weight [Co,Ci,kH,kW], out and
 * abs_sum [N,Ci,H,W]; all contiguous doubles.  abs_sum may be NULL.
 */
void oracle_grad_input_f64(const double *grad_out, const double *weight,
                           double *out, double *abs_sum, int N, int Ci, int H,
                           int W, int Co, int kH, int kW, int stride,
                           int pad_h, int pad_w, int oH, int oW)
{
    shape_t s = make_shape(N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH, oW);
    int64_t rows = s.N * s.Ci * s.H;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t row = 0; row < rows; ++row) {
        int64_t ih = row % s.H;
        int64_t ci = (row / s.H) % s.Ci;
        int64_t n = row / (s.H * s.Ci);
        for (int64_t iw = 0; iw < s.W; ++iw) {
            double v, va;
            grad_input_element(grad_out, weight, &s, n, ci, ih, iw, &v, &va);
            out[row * s.W + iw] = v;
            if (abs_sum) abs_sum[row * s.W + iw] = va;
        }
    }
}

/*
 * The same result at chosen elements only: flat_idx[i] indexes the
 * [N,Ci,H,W] tensor.  Used where the full tensor would take the CPU too long.
 * Indices outside the tensor give NaN.
 */
void oracle_grad_input_at_f64(const double *grad_out, const double *weight,
                              const int64_t *flat_idx, int64_t count,
                              double *out, double *abs_sum, int N, int Ci,
                              int H, int W, int Co, int kH, int kW, int stride,
                              int pad_h, int pad_w, int oH, int oW)
{
    shape_t s = make_shape(N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH, oW);
    int64_t total = s.N * s.Ci * s.H * s.W;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t f = flat_idx[i];
        if (f < 0 || f >= total) {
            out[i] = NAN;
            if (abs_sum) abs_sum[i] = NAN;
            continue;
        }
        int64_t iw = f % s.W;
        int64_t ih = (f / s.W) % s.H;
        int64_t ci = (f / (s.W * s.H)) % s.Ci;
        int64_t n = f / (s.W * s.H * s.Ci);
        double v, va;
        grad_input_element(grad_out, weight, &s, n, ci, ih, iw, &v, &va);
        out[i] = v;
        if (abs_sum) abs_sum[i] = va;
    }
}

/*
 * Forward cross-correlation, written from the output side.  x [N,Ci,H,W],
 * w [Co,Ci,kH,kW], y [N,Co,oH,oW]; all contiguous doubles.
 */
void oracle_conv2d_fwd_f64(const double *x, const double *w, double *y, int N,
                           int Ci, int H, int W, int Co, int kH, int kW,
                           int stride, int pad_h, int pad_w, int oH, int oW)
{
    int64_t planes = (int64_t)N * Co;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t plane = 0; plane < planes; ++plane) {
        int64_t n = plane / Co, co = plane % Co;
        for (int64_t oh = 0; oh < oH; ++oh) {
            for (int64_t ow = 0; ow < oW; ++ow) {
                double acc = 0.0;
                for (int64_t ci = 0; ci < Ci; ++ci) {
                    const double *xp = x + (n * Ci + ci) * H * W;
                    const double *wp = w + (co * Ci + ci) * kH * kW;
                    for (int64_t kh = 0; kh < kH; ++kh) {
                        int64_t ih = oh * stride - pad_h + kh;
                        if (ih < 0 || ih >= H) continue;
                        for (int64_t kw = 0; kw < kW; ++kw) {
                            int64_t iw = ow * stride - pad_w + kw;
                            if (iw < 0 || iw >= W) continue;
                            acc += xp[ih * W + iw] * wp[kh * kW + kw];
                        }
                    }
                }
                y[(plane * oH + oh) * oW + ow] = acc;
            }
        }
    }
}

/* One forward element and its sum of |x * w|, in the order ci, kh, kw. */
static void forward_element(const double *x, const double *w, const shape_t *s,
                            int64_t n, int64_t co, int64_t oh, int64_t ow,
                            double *value, double *abs_value)
{
    double acc = 0.0, acc_abs = 0.0;
    for (int64_t ci = 0; ci < s->Ci; ++ci) {
        const double *xp = x + (n * s->Ci + ci) * s->H * s->W;
        const double *wp = w + (co * s->Ci + ci) * s->kH * s->kW;
        for (int64_t kh = 0; kh < s->kH; ++kh) {
            int64_t ih = oh * s->stride - s->pad_h + kh;
            if (ih < 0 || ih >= s->H) continue;
            for (int64_t kw = 0; kw < s->kW; ++kw) {
                int64_t iw = ow * s->stride - s->pad_w + kw;
                if (iw < 0 || iw >= s->W) continue;
                double t = xp[ih * s->W + iw] * wp[kh * s->kW + kw];
                acc += t;
                acc_abs += fabs(t);
            }
        }
    }
    *value = acc;
    *abs_value = acc_abs;
}

/*
 * Forward cross-correlation with the sum of |x * w| per output element.
 * x [N,Ci,H,W], w [Co,Ci,kH,kW], y and abs_sum [N,Co,oH,oW]; abs_sum may be
 * NULL.
 */
void oracle_conv2d_fwd_abs_f64(const double *x, const double *w, double *y, double *abs_sum,
                               int N, int Ci, int H, int W, int Co, int kH, int kW,
                               int stride, int pad_h, int pad_w, int oH, int oW)
{
    shape_t s = make_shape(N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH, oW);
    int64_t planes = s.N * s.Co;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t plane = 0; plane < planes; ++plane) {
        int64_t n = plane / s.Co, co = plane % s.Co;
        for (int64_t oh = 0; oh < s.oH; ++oh)
            for (int64_t ow = 0; ow < s.oW; ++ow) {
                double v, va;
                forward_element(x, w, &s, n, co, oh, ow, &v, &va);
                y[(plane * s.oH + oh) * s.oW + ow] = v;
                if (abs_sum) abs_sum[(plane * s.oH + oh) * s.oW + ow] = va;
            }
    }
}

/*
 * The forward result and its abs-sum at chosen elements: flat_idx[i] indexes
 * the [N,Co,oH,oW] tensor; indices outside it give NaN.
 */
void oracle_conv2d_fwd_at_f64(const double *x, const double *w, const int64_t *flat_idx,
                              int64_t count, double *out, double *abs_sum, int N, int Ci,
                              int H, int W, int Co, int kH, int kW, int stride, int pad_h,
                              int pad_w, int oH, int oW)
{
    shape_t s = make_shape(N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH, oW);
    int64_t total = s.N * s.Co * s.oH * s.oW;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; ++i) {
        int64_t f = flat_idx[i];
        if (f < 0 || f >= total) {
            out[i] = NAN;
            if (abs_sum) abs_sum[i] = NAN;
            continue;
        }
        int64_t ow = f % s.oW;
        int64_t oh = (f / s.oW) % s.oH;
        int64_t co = (f / (s.oW * s.oH)) % s.Co;
        int64_t n = f / (s.oW * s.oH * s.Co);
        double v, va;
        forward_element(x, w, &s, n, co, oh, ow, &v, &va);
        out[i] = v;
        if (abs_sum) abs_sum[i] = va;
    }
}

/*
 * grad_bias [Co] from grad_out [N,Co,oH,oW]; abs_sum [Co] may be NULL.
 */
void oracle_grad_bias_f64(const double *grad_out, double *out, double *abs_sum, int N,
                          int Co, int oH, int oW)
{
    int64_t plane = (int64_t)oH * oW;
#pragma omp parallel for schedule(static)
    for (int64_t co = 0; co < Co; ++co) {
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double *gp = grad_out + (n * Co + co) * plane;
            for (int64_t p = 0; p < plane; ++p) {
                acc += gp[p];
                acc_abs += fabs(gp[p]);
            }
        }
        out[co] = acc;
        if (abs_sum) abs_sum[co] = acc_abs;
    }
}

/* One grad_weight element, straight from the definition above. */
static void grad_weight_element(const double *x, const double *grad_out,
                                const shape_t *s, int64_t co, int64_t ci,
                                int64_t kh, int64_t kw, double *value,
                                double *abs_value)
{
    double acc = 0.0, acc_abs = 0.0;
    for (int64_t n = 0; n < s->N; ++n) {
        const double *gp = grad_out + (n * s->Co + co) * s->oH * s->oW;
        const double *xp = x + (n * s->Ci + ci) * s->H * s->W;
        for (int64_t oh = 0; oh < s->oH; ++oh) {
            int64_t ih = oh * s->stride - s->pad_h + kh;
            if (ih < 0 || ih >= s->H) continue;
            for (int64_t ow = 0; ow < s->oW; ++ow) {
                int64_t iw = ow * s->stride - s->pad_w + kw;
                if (iw < 0 || iw >= s->W) continue;
                double t = gp[oh * s->oW + ow] * xp[ih * s->W + iw];
                acc += t;
                acc_abs += fabs(t);
            }
        }
    }
    *value = acc;
    *abs_value = acc_abs;
}

/*
 * Full grad_weight.  x [N,Ci,H,W], grad_out [N,Co,oH,oW], out and abs_sum
 * [Co,Ci,kH,kW]; all contiguous doubles.  abs_sum may be NULL.
 */
void oracle_grad_weight_f64(const double *x, const double *grad_out, double *out,
                            double *abs_sum, int N, int Ci, int H, int W, int Co,
                            int kH, int kW, int stride, int pad_h, int pad_w, int oH,
                            int oW)
{
    shape_t s = make_shape(N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH, oW);
    int64_t total = s.Co * s.Ci * s.kH * s.kW;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t e = 0; e < total; ++e) {
        int64_t kw = e % s.kW;
        int64_t kh = (e / s.kW) % s.kH;
        int64_t ci = (e / (s.kW * s.kH)) % s.Ci;
        int64_t co = e / (s.kW * s.kH * s.Ci);
        double v, va;
        grad_weight_element(x, grad_out, &s, co, ci, kh, kw, &v, &va);
        out[e] = v;
        if (abs_sum) abs_sum[e] = va;
    }
}

/*
 * The same result at chosen elements only: flat_idx[i] indexes the
 * [Co,Ci,kH,kW] tensor; indices outside it give NaN.
 */
void oracle_grad_weight_at_f64(const double *x, const double *grad_out,
                               const int64_t *flat_idx, int64_t count, double *out,
                               double *abs_sum, int N, int Ci, int H, int W, int Co,
                               int kH, int kW, int stride, int pad_h, int pad_w, int oH,
                               int oW)
{
    shape_t s = make_shape(N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH, oW);
    int64_t total = s.Co * s.Ci * s.kH * s.kW;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; ++i) {
        int64_t f = flat_idx[i];
        if (f < 0 || f >= total) {
            out[i] = NAN;
            if (abs_sum) abs_sum[i] = NAN;
            continue;
        }
        int64_t kw = f % s.kW;
        int64_t kh = (f / s.kW) % s.kH;
        int64_t ci = (f / (s.kW * s.kH)) % s.Ci;
        int64_t co = f / (s.kW * s.kH * s.Ci);
        double v, va;
        grad_weight_element(x, grad_out, &s, co, ci, kh, kw, &v, &va);
        out[i] = v;
        if (abs_sum) abs_sum[i] = va;
    }
}
