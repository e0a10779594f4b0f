/*
 * conv2d_grad_input_testing.h -- test and diagnostic hooks of the conv2d
 * grad_input library (same shared library as conv2d_grad_input.h).
 *
 * Not for production callers.  The hooks force a kernel variant, tile or
 * split so that tests can reach every compiled kernel instance on small
 * shapes, and let a benchmark time the contraction kernels apart from their
 * prologues.  Every setting is THREAD-LOCAL: it changes the plans of later
 * calls made from the thread that set it, and no other thread's.  A forced
 * choice that does not apply to a shape falls back as each hook states.
 */
#ifndef CONV2D_GRAD_INPUT_TESTING_H
#define CONV2D_GRAD_INPUT_TESTING_H

#include "conv2d_grad_input.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel variants, for conv2d_gi_set_variant. */
enum {
    CONV2D_GI_VARIANT_AUTO = 0,    /* the planner chooses                      */
    CONV2D_GI_VARIANT_GENERIC = 1, /* any shape: phase split, gathered B tile  */
    CONV2D_GI_VARIANT_HALO = 2,    /* Ci >= 16 (bf16: stride 1): grad_out halo
                                      tile in LDS, every tap a shifted view of
                                      it; other shapes fall back to GENERIC    */
    CONV2D_GI_VARIANT_STEM = 3,    /* fp32, Ci <= 4: 4x4 matrix-core blocks with
                                      the input channels on one side; other
                                      shapes fall back to GENERIC              */
    CONV2D_GI_VARIANT_COL2IM = 4   /* fp32, Ci*kH*kW <= 160, 48 < Co <= 64,
                                      kW <= 4*stride: per grad_out position the
                                      products with every (ci, kh, kw) column
                                      on the matrix cores, folded onto their
                                      input pixels in LDS; other shapes fall
                                      back to GENERIC                          */
};

/*
 * Force a kernel variant for this thread's later grad_input calls
 * (CONV2D_GI_VARIANT_AUTO restores the planner).  Returns the previous
 * setting, or -1 for an unknown variant (setting unchanged).
 */
CONV2D_GI_API int conv2d_gi_set_variant(int variant);

/*
 * Force the pixel tile of the HALO variant for this thread's later calls.
 * fp32: nb pixel blocks of 16 per work-group (4, 8 or 13), a tile of
 * tile_rows x tile_cols pixels of the stride-phase grid (at most nb*16
 * pixels) and the LDS pipeline depth (2 or 3 stages; 0 lets the planner
 * choose).  bf16 / fp16: nb pixel blocks of 16 per wave (4 or 7; two waves
 * share the tile, so at most 2*nb*16 pixels), or 13 for the whole-image
 * kernel (a work-group per image and 128 input channels; the tile is then
 * the image); stages is ignored.  A shape the
 * forced tile does not fit (LDS, halo size) is planned with GENERIC instead.
 * nb = 0 restores the planner.  Returns CONV2D_GI_OK, or CONV2D_GI_EINVAL for
 * values out of range.
 */
CONV2D_GI_API int conv2d_gi_set_halo_tile(int nb, int tile_rows, int tile_cols, int stages);

/*
 * Force how many thread groups of 256 split the output channels of a
 * work-group of the fp32 HALO variant for this thread's later calls (1 or 2;
 * each group stages its own share of the chunks and the first sums both
 * before storing).  A shape no instance
 * with that split serves is planned without it.  0 restores the planner.
 * Returns CONV2D_GI_OK, or CONV2D_GI_EINVAL for other values.
 */
CONV2D_GI_API int conv2d_gi_set_halo_split(int groups);

/*
 * How the fp32 HALO variant runs the stride phases of a work-group's tile for
 * this thread's later calls: 1 one phase after another (each over its own
 * grad_out halo), 2 all phases per chunk of output channels over one shared
 * halo (four phases of tap grids up to 2 x 2 only; other shapes are planned
 * phase at a time).  0 restores the planner.  Returns CONV2D_GI_OK, or
 * CONV2D_GI_EINVAL for other values.
 */
CONV2D_GI_API int conv2d_gi_set_halo_fusion(int mode);

/*
 * Which path this thread's later conv2d_forward calls take: 1 the grad_input
 * kernels (stride 1 only; other shapes return CONV2D_GI_EUNSUPPORTED), 2 the
 * generic forward kernel, 0 restores the planner.  Returns CONV2D_GI_OK, or
 * CONV2D_GI_EINVAL for other values.
 */
CONV2D_GI_API int conv2d_fwd_set_variant(int mode);

/*
 * Which grad_weight kernel this thread's later calls use: 1 the one with
 * 4-byte direct loads (any shape the entry point accepts), 2 the one with
 * 16-byte direct loads (shapes it does not cover return
 * CONV2D_GI_EUNSUPPORTED), 0 restores the planner (16-byte loads where they
 * apply).  Returns CONV2D_GI_OK, or CONV2D_GI_EINVAL for other values.
 */
CONV2D_GI_API int conv2d_gw_set_variant(int mode);

/*
 * For the 16-byte-load grad_weight kernel: output rows per pixel group
 * (clamped to oH), LDS stages (1 or 2) and the most slices of the pixel axis,
 * for this thread's later calls; 0 leaves each to the planner.  A shape whose
 * forced tile does not fit in LDS is planned on the 4-byte-load kernel.
 * Returns CONV2D_GI_OK, or CONV2D_GI_EINVAL for negative values or stages
 * above 2.
 */
CONV2D_GI_API int conv2d_gw_set_tile(int rows, int stages, int max_slices);

/*
 * Measurement hook: when both events are non-NULL, this thread's later calls
 * launch their first contraction kernel so that it records `begin` with the
 * dispatch's own start time and their last one so that it records `end` with
 * its completion time (hipExtLaunchKernelGGL), so the caller can time the
 * contraction kernels apart from the reorder prologues before them.  For
 * conv2d_grad_weight both events bracket its contraction kernel alone,
 * without the slice reduction that follows it.  NULL, NULL switches it off.
 * The events (hipEvent_t) stay the caller's.
 */
CONV2D_GI_API void conv2d_gi_set_profile_events(hipEvent_t begin, hipEvent_t end);

/*
 * Measurement probe: enqueue a kernel of `workgroups` work-groups of 4
 * waves that each issue `iters` rounds of 8 independent matrix-core
 * instructions on varied data (kind 0: fp32 V_MFMA_F32_16X16X4_F32, kind 1:
 * bf16 V_MFMA_F32_16X16X32_BF16), so that timing it with events on `stream`
 * gives the matrix-core rate the chip sustains at the clock it settles to.
 * *flops receives the kernel's flop count.  scratch: device memory of at
 * least `workgroups` floats (written only in a case that does not occur;
 * it keeps the work from being optimised away).  Returns CONV2D_GI_OK,
 * CONV2D_GI_EINVAL or CONV2D_GI_EHIP.
 */
CONV2D_GI_API int conv2d_gi_mfma_peak_probe(int kind, int workgroups, int iters, float *scratch,
                                            hipStream_t stream, double *flops);

#ifdef __cplusplus
}
#endif

#endif /* CONV2D_GRAD_INPUT_TESTING_H */
