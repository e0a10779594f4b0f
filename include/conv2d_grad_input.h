/*
 * conv2d_grad_input.h -- C ABI of the MI355X (gfx950) conv2d grad_input library.
 *
 * The operation
 * -------------
 * The gradient of a 2-D convolution (cross-correlation, no dilation, one group)
 * with respect to its input.  For every batch item n, input channel ci and
 * input pixel (ih, iw):
 *
 *   dst[n,ci,ih,iw] = sum over co < Co, kh < kH, kw < kW of
 *                     grad_out[n,co,oh,ow] * weight[co,ci,kh,kw]
 *
 * where a = ih + pad_h - kh and b = iw + pad_w - kw are both >= 0 and
 * divisible by the stride, and oh = a / stride < oH, ow = b / stride < oW.
 * Terms that fail a condition are absent; a pixel with none gets 0.
 *
 * This is the direct kernel of doppler conv2d_backward_input.wgsl (an input
 * pixel sums the output gradients it fed in the forward pass, the transposed
 * convolution of its header comment), batched and with per-dimension padding,
 * and the general-stride branch of the B-tile gather of meganeura
 * conv2d_grad_input_gemm.wgsl.  The library computes it as the implicit GEMM
 * of that shader's header comment, C[Ci, H*W] = A[Ci, Co*kH*kW] x
 * B[Co*kH*kW, H*W] per batch item with A the weight read as [Ci, Co*kH*kW]
 * and B the on-the-fly im2col of grad_out, after splitting a strided problem
 * into stride*stride dense sub-problems (one per input-pixel residue), so
 * that taps that would land between output pixels are never multiplied.
 *
 * Layouts and ownership
 * ---------------------
 * All tensors are dense, row-major, on the device the call runs on:
 *   grad_out [N, Co, oH, oW]   read only
 *   weight   [Co, Ci, kH, kW]  read only
 *   dst      [N, Ci, H, W]     fp32, written (every element, never accumulated)
 * The caller allocates and owns all three; the library never frees them.  dst
 * must not overlap either input.  Both convolution stride dimensions take
 * `stride`; padding is symmetric per dimension (pad_h top and bottom, pad_w
 * left and right).
 *
 * Library scratch
 * ---------------
 * Some plans need device scratch: the weight reordered into the order a kernel
 * reads it (about Co*Ci*kH*kW elements), grad_weight's partial sums, the
 * forward's tap-reversed weight.  The library keeps one buffer per (device,
 * stream, purpose), allocated stream-ordered on `stream` (hipMallocAsync) by
 * the first call that needs it, grown when a later call needs more (the old
 * one is freed stream-ordered), and reused by later calls on that stream;
 * stream order keeps the calls apart.  Nothing is carried from one call to the
 * next: every call rewrites what it reads.  An internal lock is held while a
 * call enqueues, so calls from several host threads on one stream are safe
 * (they run in the order they took the lock), and calls on different streams
 * share no buffer.  The cache is keyed by the stream handle, so a stream the
 * library ran on must outlive its buffers: call conv2d_gi_release_workspaces
 * (which waits for each stream's queued work, then frees) before destroying
 * it, or a new stream that receives the same handle would inherit them.
 * conv2d_grad_input_noalloc (below) allocates nothing and uses a fixed
 * per-device buffer instead.

 * Asynchrony and errors
 * ---------------------
 * Calls enqueue work on `stream` (0 = the device's null stream) and return
 * without waiting; dst is valid once the stream has reached that point.  The
 * current HIP device must own the buffers.  All arguments are checked on the
 * host before anything is enqueued: on CONV2D_GI_EINVAL or
 * CONV2D_GI_EUNSUPPORTED nothing is launched and dst is untouched.  Zero or
 * negative sizes are invalid (as the doppler wrappers throw on a missing or
 * zero size): every tensor of a valid call has elements.
 * CONV2D_GI_EHIP reports a HIP runtime error from an allocation or launch
 * (the error string of the last one is kept for conv2d_gi_last_hip_error).
 */
#ifndef CONV2D_GRAD_INPUT_H
#define CONV2D_GRAD_INPUT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define CONV2D_GI_API __attribute__((visibility("default")))
#else
#define CONV2D_GI_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Problem shape.  Field names follow the Params block of meganeura
 * conv2d_grad_input_gemm.wgsl (batch, in_channels, in_h, in_w, out_channels,
 * kernel_h, kernel_w, stride, padding_h, padding_w, out_h, out_w).  H and W
 * are given, not derived, because with stride > 1 several input sizes give the
 * same oH and oW.
 */
typedef struct conv2d_gi_params {
    int32_t N;        /* batch items, >= 1                                    */
    int32_t Ci;       /* input channels = channels of dst, >= 1               */
    int32_t H, W;     /* input (dst) spatial size, >= 1                       */
    int32_t Co;       /* output channels, >= 1                                */
    int32_t kH, kW;   /* kernel size, >= 1                                    */
    int32_t stride;   /* one stride for both dimensions, >= 1                 */
    int32_t pad_h;    /* zero padding above and below, >= 0                   */
    int32_t pad_w;    /* zero padding left and right, >= 0                    */
    int32_t oH, oW;   /* grad_out spatial size; must equal
                         (H + 2*pad_h - kH)/stride + 1 and
                         (W + 2*pad_w - kW)/stride + 1 (floor division), >= 1 */
} conv2d_gi_params;   /* passed by value to every entry point */

/* Status codes returned by every entry point. */
enum {
    CONV2D_GI_OK = 0,
    CONV2D_GI_EINVAL = 1,       /* null pointer or bad shape; nothing launched */
    CONV2D_GI_EUNSUPPORTED = 2, /* valid but beyond the library's limits (index
                                   width, the no-alloc scratch size)          */
    CONV2D_GI_EHIP = 3          /* HIP runtime error from allocation or launch */
};

/*
 * fp32 grad_input.  grad_out and weight fp32, dst fp32 (layouts above).
 * Contraction on the fp32 matrix cores, fp32 accumulation.  No pointer may
 * be NULL.
 */
CONV2D_GI_API int conv2d_grad_input(const float *grad_out, const float *weight, float *dst,
                      conv2d_gi_params p, hipStream_t stream);

/*
 * bf16-input grad_input.  grad_out and weight hold bf16 bit patterns (the top
 * 16 bits of an IEEE float32); dst is fp32.  Products of two bf16 values are
 * exact in fp32; accumulation is fp32 on the bf16 matrix cores.
 */
CONV2D_GI_API int conv2d_grad_input_bf16(const uint16_t *grad_out, const uint16_t *weight,
                           float *dst, conv2d_gi_params p,
                           hipStream_t stream);

/*
 * fp16 inputs: grad_out and weight as IEEE binary16 bit patterns (uint16_t,
 * same layouts), fp32 accumulation, fp32 dst.  The same plans, prologues and
 * kernels as the bf16 entry point with the fp16 MFMA (16x16x32 / 32x32x16
 * f16); the products of two fp16 values are exact in fp32.  This is the
 * fp16 precision the pages cast to (doppler ensureF32 and the f16 casts of
 * the other pages), taken as an input type.  Same validation and status
 * codes as conv2d_grad_input.
 */
CONV2D_GI_API int conv2d_grad_input_f16(const uint16_t *grad_out, const uint16_t *weight,
                                        float *dst, conv2d_gi_params p,
                                        hipStream_t stream);

/*
 * fp32 grad_input that allocates nothing: for callers that cannot call
 * hipMalloc (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, result and validation as
 * conv2d_grad_input; the caller still passes every input and output.
 *
 * The scratch the fp32 plans need (the weight reordered into kernel order,
 * about Co*Ci*kH*kW floats; the Ci <= 4 plan needs none) is a fixed
 * CONV2D_GI_NOALLOC_SCRATCH_BYTES device array inside the library, one copy
 * per GPU, held until the process ends.  A shape whose plan needs more returns
 * CONV2D_GI_EUNSUPPORTED before anything is enqueued.  Every call on one GPU
 * uses that GPU's array: calls that can overlap on a GPU (different streams
 * with no ordering between them) race, so callers keep them on one stream or
 * order them with events.  Nothing is carried from one call to the next.
 * The first call on a device looks the array's device address up
 * (hipGetSymbolAddress); a failure there returns CONV2D_GI_EHIP.
 */
#define CONV2D_GI_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
CONV2D_GI_API int conv2d_grad_input_noalloc(const float *grad_out, const float *weight,
                                            float *dst, conv2d_gi_params p,
                                            hipStream_t stream);

/* Host-only check of a shape, as done by the entry points (no HIP call). */
CONV2D_GI_API int conv2d_gi_validate(conv2d_gi_params p);

/* Static text for a status code. */
CONV2D_GI_API const char *conv2d_gi_strerror(int code);

/* Text of the last HIP error seen by this thread's calls ("" if none). */
CONV2D_GI_API const char *conv2d_gi_last_hip_error(void);

/*
 * Gradient with respect to the weight (the next step of the same backward
 * pass; the computeGradWeight branch of doppler conv2d_backward.js, whose
 * shader is not on the pages, so the definition is the derivative of the
 * forward mapping):
 *
 *   dw[co,ci,kh,kw] = sum over n, oh, ow of grad_out[n,co,oh,ow] * x[n,ci,ih,iw]
 *   with ih = oh*stride - pad_h + kh, iw = ow*stride - pad_w + kw and x = 0
 *   outside [0,H) x [0,W).
 *
 * grad_out: device [N, Co, oH, oW] fp32; x: device [N, Ci, H, W] fp32 (the
 * forward input); dw: device [Co, Ci, kH, kW] fp32, fully overwritten (no
 * accumulation into it).  p: the same shape struct as conv2d_grad_input,
 * validated the same way.  Enqueued on `stream` (asynchronous).  The
 * partial sums of the split pixel axis live in the library's per-stream
 * scratch buffer and are added in a fixed order, so the result does not
 * depend on scheduling.  Returns CONV2D_GI_OK, CONV2D_GI_EINVAL (null pointer,
 * inconsistent shape), CONV2D_GI_EUNSUPPORTED (kernel
 * width above 16, output rows wider than 256 pixels, tensors of 2 GiB or more)
 * or CONV2D_GI_EHIP.
 */
CONV2D_GI_API int conv2d_grad_weight(const float *grad_out, const float *x, float *dw,
                                     conv2d_gi_params p, hipStream_t stream);

/*
 * The whole backward pass of a convolution layer in one call, after the
 * doppler conv2d_backward.js wrapper (its computeGradInput and
 * computeGradWeight options become "output pointer not NULL") with the
 * per-channel bias gradient of bias_add_backward.wgsl beside them:
 *
 *   dx = conv2d_grad_input(grad_out, weight)     (when dx is not NULL)
 *   dw = conv2d_grad_weight(grad_out, x)         (when dw is not NULL)
 *   db[co] = sum over n, oh, ow of grad_out[n,co,oh,ow]   (when db is not NULL)
 *
 * Same shapes, layouts and validation as the single calls; db is device
 * [Co] fp32.  weight may be NULL when dx is, x when dw is; grad_out is
 * required when any output is asked for.  With dw, the
 * bias sums come from the grad_out values the grad_weight kernel already
 * reads (no second pass over grad_out where the 16-byte-load kernel runs);
 * without dw a per-channel reduction computes them.  All sums are in a fixed
 * order (deterministic).  Every output is overwritten.  Returns the first
 * failing step's status; the steps before it have been enqueued.
 */
CONV2D_GI_API int conv2d_backward(const float *grad_out, const float *x, const float *weight,
                                  float *dx, float *dw, float *db, conv2d_gi_params p,
                                  hipStream_t stream);

/*
 * The bias gradient alone: db[co] = sum over n, oh, ow of grad_out[n,co,oh,ow]
 * (bias_add_backward.wgsl's sum over the positions the bias was added to).
 * grad_out: device [N, Co, oH, oW] fp32; db: device [Co] fp32, overwritten.
 * p is validated as for the other calls.
 * Returns CONV2D_GI_OK, CONV2D_GI_EINVAL or CONV2D_GI_EHIP.
 */
CONV2D_GI_API int conv2d_grad_bias(const float *grad_out, float *db, conv2d_gi_params p,
                                   hipStream_t stream);

/*
 * The forward convolution (cross-correlation), the mapping the doppler direct
 * grad_input kernel's comment states (output pixel oh reads input row
 * oh*stride - pad + kh):
 *
 *   y[n,co,oh,ow] = sum over ci, kh, kw of
 *                   x[n,ci,oh*stride-pad_h+kh, ow*stride-pad_w+kw] * w[co,ci,kh,kw]
 *   with x = 0 outside [0,H) x [0,W).
 *
 * x: device [N, Ci, H, W] fp32; w: device [Co, Ci, kH, kW] fp32; y: device
 * [N, Co, oH, oW] fp32, fully overwritten.  p: the same shape struct as the
 * gradient calls, validated the same way.  Stride 1 (pad <= kernel size - 1)
 * runs on the grad_input kernels with the weight transposed and its taps
 * reversed into library scratch (a second per-stream buffer); other shapes
 * on a generic implicit-GEMM kernel.  Enqueued on `stream`.  Returns
 * CONV2D_GI_OK, CONV2D_GI_EINVAL, CONV2D_GI_EUNSUPPORTED (forced variant that
 * does not apply) or CONV2D_GI_EHIP.
 */
CONV2D_GI_API int conv2d_forward(const float *x, const float *w, float *y,
                                 conv2d_gi_params p, hipStream_t stream);

/*
 * Host-only: describe the launches conv2d_forward would make for this shape,
 * as text written into buf (NUL-terminated, truncated to len).
 */
CONV2D_GI_API int conv2d_fwd_plan(conv2d_gi_params p, char *buf, size_t len);

/*
 * Host-only: describe the launch conv2d_grad_weight would make for this shape,
 * as text written into buf (NUL-terminated, truncated to len).
 */
CONV2D_GI_API int conv2d_gw_plan(conv2d_gi_params p, char *buf, size_t len);

/*
 * Host-only: describe the plan the entry point would run for this shape
 * (dtype_bf16 = 0 for fp32 inputs, 1 for bf16, 2 for fp16), as text written
 * into buf (NUL-terminated, truncated to len).  Returns a status code.  The
 * test and diagnostic hooks of conv2d_grad_input_testing.h (this thread's
 * settings) apply.
 */
CONV2D_GI_API int conv2d_gi_plan(conv2d_gi_params p, int dtype_bf16, char *buf,
                   size_t len);

/*
 * Free every cached scratch buffer (each after the work queued on its stream
 * has finished).  Returns a status code.  Later calls allocate again.
 */
CONV2D_GI_API int conv2d_gi_release_workspaces(void);

/* Library version as "major.minor.patch". */
CONV2D_GI_API const char *conv2d_gi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONV2D_GRAD_INPUT_H */
