/*
 * gnsilu.h -- C ABI of the MI355X (gfx950) channels-last GroupNorm(+SiLU)
 * library, libgnsilu.so.
 *
 * The operation is the one defined in "FLUX.2 VAE decoder fast path behind
 * quality=high", Modifications section 1 "Kernel": GroupNorm over
 * channels-last activations viewed as (N, L = H*W, C) rows with C innermost,
 * computed in three steps -- per-(batch, channel) partial sum / sum of
 * squares over the rows, a finalize to per-(batch, group) fp32 mean/rstd
 * with gamma/beta folded into per-(batch, channel) scale/shift, and a fused
 * elementwise apply with an optional SiLU.  The same section gives the
 * public pair group_norm_silu_4d / group_norm_silu_rows and the inputs for
 * which that kernel declines, leaving the caller to fall back: C not a power
 * of two, C > 2048, a layout that is not channels-last.  This library keeps
 * the decline for layouts that are not channels-last but widens the channel
 * counts it takes (see "Supported set" below), and also takes 5-D NDHWC
 * activations through the rows form (L = D*H*W): the HunyuanVAE-style 5-D
 * call sites, which the same section leaves on the older general kernel.
 *
 * For each sample n and group g (channels g*Cg .. g*Cg+Cg-1, Cg = C/G),
 * over the M = L*Cg elements of the group:
 *     mean = sum(x)/M,  var = sum((x-mean)^2)/M  (biased),
 *     rstd = 1/sqrt(var + eps)
 *     t    = gamma[c]*(x - mean)*rstd + beta[c]
 *     y    = apply_silu ? t*sigmoid(t) : t
 * Statistics are accumulated in fp32 (shifted by one sample of the group,
 * which leaves the result unchanged in exact arithmetic); y is rounded once
 * to bf16, round-to-nearest-even.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors: x and y hold bf16 values as raw 16-bit patterns (uint16 storage)
 *   -- or, through the *_dtype entry points, IEEE fp16 or fp32 values, the
 *   same type for x and y -- dense, element (n, l, c) at offset
 *   (n*L + l)*C + c.  gamma and beta are
 *   fp32[C]; either may be NULL (all ones / all zeros, i.e. GroupNorm
 *   without affine).  All tensor pointers are DEVICE pointers on the device
 *   that owns `stream`.  x and y must be 16-byte aligned.
 * stream: a hipStream_t passed as an opaque pointer; NULL is the null
 *   stream of the current device.
 * Ownership: the caller owns x, y, gamma, beta and the statistics buffers;
 *   they must stay valid until the stream has executed the call.  The
 *   library owns a scratch buffer per (device, stream) for the partial sums
 *   and per-sample arrival counters (tens of KiB for the decoder shapes,
 *   grown on demand by doubling; a buffer that is outgrown is kept, not
 *   freed, and every buffer is held until the process ends, so work already
 *   enqueued and HIP graphs captured with these calls stay valid).  Calls
 *   enqueued on one stream from several host threads are serialised by the
 *   library; calls on different streams use different scratch buffers.  A
 *   captured graph uses the scratch of the stream it was captured on:
 *   replay it on that stream, or ordered with that stream's work.  A call
 *   under capture must not need a larger buffer than that stream already
 *   has (make one call of the same shape on the stream before capturing).
 *   Calls that overlap on one stream's buffer (such a graph replayed on
 *   another stream while a call on the first is running) give undefined
 *   results for those calls; the calls after them are unaffected, because
 *   step 3 clears the arrival counters step 1 used.  The buffer is found by
 *   the stream handle's value: synchronise a stream before destroying it, or
 *   a new stream that receives the same handle shares the buffer with work
 *   still pending on the old one.
 * Synchrony: every compute call is asynchronous on `stream` and returns once
 *   the kernels are enqueued; a fault inside a kernel surfaces at the
 *   caller's next synchronisation (gn_profile_rows excepted, which
 *   synchronises).
 * Aliasing: y == x (in place) is allowed.  Any other overlap is undefined.
 * Determinism: the reduction order is a pure function of (N, L, C, G) and
 *   the dtype, so the same input gives bitwise-identical output on every
 *   call.
 * Supported set: C <= GN_MAX_CHANNELS for which a tile layout exists.  Let
 *   Wd = 8 for 16-bit types and 4 for fp32, W = Wd when L*C % Wd == 0 and 1
 *   otherwise; a layout exists when C / gcd(C, W*NV) <= 256 for some NV in
 *   {1, 2, 4} (NV in {2, 4} for fp32 with W = 4).  In particular every
 *   C <= 256; every multiple of 8 up to 2048 (16-bit) or of 4 up to 1024
 *   (fp32) with L*C % Wd == 0; and multiples of 32 up to 8192 (16-bit) or of
 *   16 up to 4096 (fp32) with L*C % Wd == 0.  gn_plan_rows_dtype reports
 *   whether a shape is in the set without touching the GPU.
 * Errors (checked in this order; nothing is enqueued unless GN_OK):
 *   GN_INVALID_ARGUMENT -- input no GroupNorm accepts: x or y NULL; N, L, H
 *     or W negative; C <= 0; G <= 0; C % G != 0; eps negative, infinite or
 *     NaN; apply_silu not 0 or 1; a dtype outside gn_dtype; the tensor's byte
 *     size overflowing int64.
 *   GN_UNSUPPORTED -- a valid GroupNorm this library declines, so the caller
 *     falls back: C outside the supported set below; (strided forms) a
 *     layout that is not dense channels-last; x or y not 16-byte aligned; a
 *     tensor pointer that is not device memory of the stream's device.
 *   GN_OK is returned without touching the GPU when N*L == 0.
 *   GN_DEVICE_ERROR -- a HIP call failed (scratch allocation, launch).
 */
#ifndef GNSILU_H
#define GNSILU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gn_status {
    GN_OK = 0,
    GN_UNSUPPORTED = 1,
    GN_INVALID_ARGUMENT = 2,
    GN_DEVICE_ERROR = 3,
    GN_SCRATCH_TOO_SMALL = 4  /* gn_silu_rows_noalloc only: see there */
} gn_status;

/* Element type of x and y for the *_dtype entry points.  The page's kernel
 * tests cover fp32 and bf16 activations (Accuracy section, unit tests). */
typedef enum gn_dtype {
    GN_DTYPE_BF16 = 0,
    GN_DTYPE_F16 = 1,
    GN_DTYPE_F32 = 2
} gn_dtype;

/* Element type of gamma and beta, or-ed into the dtype argument of the
 * *_dtype entry points that take them (gn_silu_*_dtype, gn_apply_rows_dtype,
 * gn_profile_rows_dtype; the others accept and ignore it).  The decoder
 * fast path folds its weights in fp32 ("FLUX.2 VAE decoder fast path behind
 * quality=high", the summary after Motivation) and the GroupNorm affine
 * parameters into fp32 scale/shift (Modifications, the kernel item), while
 * a model cast to bf16 or fp16 holds gamma and beta in that type: with
 * GN_AFFINE_BF16 or GN_AFFINE_F16 the gamma and beta
 * pointers (declared const float *) point at C 16-bit values of that type,
 * 2-byte aligned, each widened exactly to fp32 before the fold; without a
 * GN_AFFINE_* value, or with GN_AFFINE_F32, they point at C fp32 values,
 * 4-byte aligned.  A misaligned gamma or beta is GN_UNSUPPORTED; a dtype
 * argument with other bits set, or two GN_AFFINE_* values, is
 * GN_INVALID_ARGUMENT.  The kernels read each 16-bit value through the
 * aligned 4-byte word that holds it, so the 2 bytes just before the first
 * or after the last value of a 16-bit array may be read (never written, and
 * never across a page). */
enum {
    GN_AFFINE_F32 = 0x10,
    GN_AFFINE_BF16 = 0x20,
    GN_AFFINE_F16 = 0x30,
    GN_AFFINE_MASK = 0x30
};

/* Largest channel count the library accepts.  The pages' kernel stops at
 * 2048 (Modifications section 1); the tile layout here reaches 8192. */
#define GN_MAX_CHANNELS 8192

/* group_norm_silu_4d: NHWC 4-D activation of logical shape (N, C, H, W)
 * stored channels-last, i.e. the rows form with L = H*W (the "free permute
 * view" of Modifications section 1). */
gn_status gn_silu_nhwc(const void *x, const float *gamma, const float *beta, void *y,
                       int64_t N, int64_t H, int64_t W, int64_t C, int64_t G,
                       float eps, int apply_silu, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the full
 * path of gn_silu_rows_dtype (same arguments, same checks, same kernels and
 * launch plan, so bitwise the same output), with the library's scratch (the
 * arrival counters, partial sums and statistics) taken from a fixed buffer of
 * GN_NOALLOC_SCRATCH_BYTES compiled into the library instead of the
 * per-(device, stream) buffer the other entry points allocate.  Each device
 * the library runs on holds one such buffer, reserved when the library's
 * code is loaded on it and kept until the process ends.  The call allocates
 * and frees nothing (no hipMalloc / hipFree); its first call on a device
 * looks up that device's buffer address once.
 * Sharing: every call of this entry point on one device uses the same
 * buffer, which keeps the last call's contents; each call first clears the
 * arrival counters it uses (a fill kernel on `stream`, no memset), so nothing
 * an earlier call left behind is read.  Calls ordered on one stream are safe;
 * calls that may overlap on one device (enqueued on different streams without
 * ordering between them, or from several host threads at once) race on the
 * buffer and give undefined results.
 * Errors: as gn_silu_rows_dtype; then, still before any HIP call,
 * GN_SCRATCH_TOO_SMALL when the shape needs more scratch than the buffer
 * holds (gn_plan_rows_dtype's plan_out[7] gives a shape's need: about 80 KiB
 * at the decoder shapes). */
#define GN_NOALLOC_SCRATCH_BYTES (1 << 20)
gn_status gn_silu_rows_noalloc(const void *x, const float *gamma, const float *beta, void *y,
                               int64_t N, int64_t L, int64_t C, int64_t G,
                               float eps, int apply_silu, int dtype, void *stream);

/* Diagnostics (tests): the device address of device `device`'s fixed
 * no-allocation buffer and its size in bytes.  Its layout for a call is the
 * one gn_plan_rows_dtype's scratch_bytes counts: arrival counters from the
 * start, then the partial sums, the partial squares, read-only padding and
 * mean/rstd; a call writes nothing past its scratch_bytes.  Writing into the
 * buffer while a call runs is undefined.  GN_INVALID_ARGUMENT for a null
 * output or a negative device, GN_DEVICE_ERROR when the device cannot be
 * selected. */
gn_status gn_noalloc_scratch(int device, void **ptr_out, int64_t *bytes_out);

/* group_norm_silu_rows: (N, L, C) rows with C innermost, the form the pages'
 * tests exercise "as used by attention" (Accuracy section, unit tests). */
gn_status gn_silu_rows(const void *x, const float *gamma, const float *beta, void *y,
                       int64_t N, int64_t L, int64_t C, int64_t G,
                       float eps, int apply_silu, void *stream);

/* Strided form of gn_silu_nhwc.  x_strides / y_strides give the element
 * strides of the logical (N, C, H, W) dimensions.  Only dense channels-last
 * storage is accepted -- strides (H*W*C, 1, W*C, C), where a dimension of
 * extent 1 may carry any stride -- anything else is GN_UNSUPPORTED
 * (Modifications section 1: no NCHW variant). */
gn_status gn_silu_nhwc_strided(const void *x, const int64_t x_strides[4],
                               const float *gamma, const float *beta,
                               void *y, const int64_t y_strides[4],
                               int64_t N, int64_t H, int64_t W, int64_t C, int64_t G,
                               float eps, int apply_silu, void *stream);

/* NDHWC 5-D activation of logical shape (N, C, D, H, W) stored channels-last
 * (torch.channels_last_3d): the rows form with L = D*H*W.  The same
 * normalisation applies, each group's statistics taken over all D*H*W
 * positions (Modifications section 1 names 5-D call sites such as the
 * HunyuanVAE decoder). */
gn_status gn_silu_ndhwc(const void *x, const float *gamma, const float *beta, void *y,
                        int64_t N, int64_t D, int64_t H, int64_t W, int64_t C, int64_t G,
                        float eps, int apply_silu, void *stream);

/* Steps one and two alone: writes the fp32 per-(n, g) mean and rstd, index
 * n*G + g, to the device buffers mean_out / rstd_out (N*G floats each) --
 * the finalize output of Modifications section 1.  Same checks as
 * gn_silu_rows (y is not used). */
gn_status gn_stats_rows(const void *x, int64_t N, int64_t L, int64_t C, int64_t G,
                        float eps, float *mean_out, float *rstd_out, void *stream);

/* Step three alone: the fused elementwise apply (+ optional SiLU) given
 * per-(n, g) mean / rstd in device memory (N*G floats each, as written by
 * gn_stats_rows); scale = gamma*rstd and shift = beta - mean*scale are
 * formed per (n, c) inside the kernel. */
gn_status gn_apply_rows(const void *x, const float *mean, const float *rstd,
                        const float *gamma, const float *beta, void *y,
                        int64_t N, int64_t L, int64_t C, int64_t G,
                        int apply_silu, void *stream);

/* Measurement helper: runs gn_silu_rows `iters` times on `stream` with a
 * pair of HIP events around every kernel launch, synchronises, and writes
 * the mean duration in milliseconds of each kernel slot of the path to
 * kernel_ms[0 .. *n_kernels-1] (capacity 4); gn_kernel_name(i) names the
 * slots: 0 statistics, 1 separate finalize, 2 apply, 3 the single launch.  A slot whose kernel is
 * not launched for this shape (the separate finalize, when the statistics
 * kernel finishes the groups itself) reads -1.
 * iters must be in [1, 100000]. */
gn_status gn_profile_rows(const void *x, const float *gamma, const float *beta, void *y,
                          int64_t N, int64_t L, int64_t C, int64_t G,
                          float eps, int apply_silu, void *stream,
                          int iters, float *kernel_ms, int *n_kernels);

/* Launch plan of the rows path for a shape, for inspection and tests; no
 * HIP call.  Writes 8 values to plan_out:
 *   [0] slots   values each active lane holds per tile (W*NV)
 *   [1] tiles   tiles per sample (last one may be partial); a tile is whole
 *               rows, T elements (plan_out[11] of gn_plan_rows_dtype)
 *   [2] full    tiles per sample lying wholly inside the sample
 *   [3] tpc1    tiles per workgroup, statistics pass
 *   [4] K1      workgroups per sample, statistics pass (N*K1 launched)
 *   [5] tpc2    tiles per workgroup, apply pass (the first tiles % K2
 *               workgroups of each sample take one tile more)
 *   [6] K2      workgroups per sample, apply pass (N*K2 launched)
 *   [7] scratch bytes of library-owned scratch the call needs
 * Returns the status gn_silu_rows would return from its argument checks
 * for 16-byte-aligned pointers. */
gn_status gn_plan_rows(int64_t N, int64_t L, int64_t C, int64_t G, int64_t plan_out[8]);

/* Whether the full path of a shape runs as a single launch, and its shape;
 * no HIP call.  Steps 1-3 run in one kernel -- one workgroup of 1024 lanes
 * per strip of whole, consecutive groups of a sample, which reduces its
 * groups itself, holds the strip in registers and needs no scratch -- when
 * the tensor is at most 4 MiB, its rows are 16-byte multiples (C times the
 * element size a multiple of 16), Cg is a multiple of W (8 for 16-bit types,
 * 4 for fp32) with Cg/W a power of two up to 64 or a divisor of W, at most
 * 256 workgroups result (one per CU) and each lane holds at most two 16-byte
 * pieces (L * pieces per row <= 2048): the short strips where one launch
 * beats three steps.  Writes 6 values:
 *   [0] 1 when the single launch runs, else 0 (and [1]-[5] are 0)
 *   [1] groups per workgroup (a strip of consecutive groups)
 *   [2] 16-byte pieces per row of a strip (a power of two)
 *   [3] workgroups, N * G / [1]
 *   [4] lanes per workgroup
 *   [5] pieces each lane holds in registers
 * Returns the status gn_silu_rows_dtype would return from its argument
 * checks for aligned pointers.  gn_stats_rows takes the single launch's
 * statistics for such shapes, so steps 1-2 then step 3 still give the full
 * path's output bit for bit. */
gn_status gn_plan_single_launch(int64_t N, int64_t L, int64_t C, int64_t G, int dtype,
                                int64_t plan_out[6]);

/* The same calls for x and y of element type `dtype` (a gn_dtype value);
 * the bf16 entry points above are these with dtype = GN_DTYPE_BF16.
 * gn_plan_rows_dtype writes 15 values, the 8 above and
 *   [8]  1 when step 3 reads x with nontemporal loads (tensors larger than
 *        the 256 MB Infinity Cache), else 0
 *   [9]  W, elements per lane access (16 bytes' worth, or 1)
 *   [10] A, lanes of the workgroup ([14] lanes) that hold slots
 *   [11] T, elements per tile (= A*W*NV, a multiple of C)
 *   [12] the last tiles of each statistics chunk read with plain loads (the
 *        rest nontemporal): all of the chunk when the tensor fits the
 *        Infinity Cache, else the chunk's share of one cache's worth
 *   [13] 1 when step 2 runs in step 3 (the late finalize: x of at most
 *        16 MiB whose sample's step-1 partials number at most
 *        16 * floor(256 / G) chunks, G <= 256): step 1 only writes its
 *        partials and every step-3 workgroup reduces its sample's partials
 *        in the fused finalize's order, so mean/rstd are bitwise the same
 *   [14] lanes per workgroup of steps 1 and 3: 256, or 320 for a tensor above
 *        16 MiB whose channel count's 256-lane layout leaves a quarter or
 *        more of the lanes idle or needs more accesses per lane, when 320
 *        lanes are all busy with the minimal accesses per lane (C = 1280,
 *        2560, ...: one row of 2560 or two of 1280 per tile)
 * gn_silu_ndhwc_strided_dtype is the strided form for 5-D: strides of the
 * logical (N, C, D, H, W) dimensions, dense channels-last only
 * ((D*H*W*C, 1, H*W*C, W*C, C), extent-1 dimensions free). */
gn_status gn_silu_nhwc_dtype(const void *x, const float *gamma, const float *beta, void *y,
                             int64_t N, int64_t H, int64_t W, int64_t C, int64_t G,
                             float eps, int apply_silu, int dtype, void *stream);
gn_status gn_silu_rows_dtype(const void *x, const float *gamma, const float *beta, void *y,
                             int64_t N, int64_t L, int64_t C, int64_t G,
                             float eps, int apply_silu, int dtype, void *stream);
gn_status gn_silu_nhwc_strided_dtype(const void *x, const int64_t x_strides[4],
                                     const float *gamma, const float *beta,
                                     void *y, const int64_t y_strides[4],
                                     int64_t N, int64_t H, int64_t W, int64_t C, int64_t G,
                                     float eps, int apply_silu, int dtype, void *stream);
gn_status gn_silu_ndhwc_dtype(const void *x, const float *gamma, const float *beta, void *y,
                              int64_t N, int64_t D, int64_t H, int64_t W, int64_t C, int64_t G,
                              float eps, int apply_silu, int dtype, void *stream);
gn_status gn_silu_ndhwc_strided_dtype(const void *x, const int64_t x_strides[5],
                                      const float *gamma, const float *beta,
                                      void *y, const int64_t y_strides[5],
                                      int64_t N, int64_t D, int64_t H, int64_t W, int64_t C,
                                      int64_t G, float eps, int apply_silu, int dtype,
                                      void *stream);
gn_status gn_stats_rows_dtype(const void *x, int64_t N, int64_t L, int64_t C, int64_t G,
                              float eps, int dtype, float *mean_out, float *rstd_out,
                              void *stream);
gn_status gn_apply_rows_dtype(const void *x, const float *mean, const float *rstd,
                              const float *gamma, const float *beta, void *y,
                              int64_t N, int64_t L, int64_t C, int64_t G,
                              int apply_silu, int dtype, void *stream);
gn_status gn_profile_rows_dtype(const void *x, const float *gamma, const float *beta, void *y,
                                int64_t N, int64_t L, int64_t C, int64_t G,
                                float eps, int apply_silu, int dtype, void *stream,
                                int iters, float *kernel_ms, int *n_kernels);
gn_status gn_plan_rows_dtype(int64_t N, int64_t L, int64_t C, int64_t G, int dtype,
                             int64_t plan_out[15]);

/* The GroupNorm(+SiLU) fused into the neighbouring 3x3 convolution of the
 * decoder's ResnetBlock2D (Modifications section 2: "ResnetBlock2D
 * norm1/norm2 + SiLU chains" around Conv2d(3x3, p1)):
 *
 *   y = apply_silu ? SiLU(t) : t,   t = gamma[c]*(x - mean[n,g])*rstd[n,g] + beta[c]
 *       (t = x when norm_mean is NULL)
 *   z[n,h,w,co] = bias[co] + res[n,h,w,co]
 *               + sum_{kh,kw in 0..2} sum_{ci} wt[co,kh,kw,ci] * y[n,h+kh-1,w+kw-1,ci]
 *   with y = 0 outside the image (zero padding 1, stride 1), and, when
 *   mean2_out is given, the statistics of z for the next GroupNorm: per
 *   (n, g2) over the G2 contiguous groups of Co, the fp32 mean and
 *   1/sqrt(var + eps2) (biased variance) of the stored bf16 values of z.
 *
 * x: bf16 [N][H][W][Ci] (NHWC); norm_mean / norm_rstd: fp32 [N][G] as written
 * by gn_stats_rows (or by the statistics output of a previous call), both or
 * neither; gamma / beta: fp32 [Ci] or NULL; wt: bf16 [Co][3][3][Ci] (the
 * channels-last layout of a [Co, Ci, 3, 3] weight); bias: fp32 [Co] or NULL;
 * res: bf16 [N][H][W][Co] or NULL (added before rounding: the ResnetBlock2D
 * shortcut); z: bf16 [N][H][W][Co], must not overlap x or res; mean2_out /
 * rstd2_out: fp32 [N][G2] device buffers, both or neither.  The products are
 * of bf16 operands (y is rounded once to bf16 on its way to the matrix
 * cores), accumulated in fp32; z is rounded once to bf16.
 * Supported: Ci a multiple of 32 up to 1024, Co a multiple of 128, and with
 * statistics Co/G2 dividing 64; pointers 16-byte aligned; else
 * GN_UNSUPPORTED.  INVALID as for gn_silu_rows (NULL x/wt/z, negative sizes,
 * Ci % G, Co % G2, eps2, apply_silu, one of a pointer pair missing).  N*H*W
 * == 0 enqueues nothing.  With statistics, the library's scratch buffer of
 * the stream holds per-tile partials (16 bytes per 8x16 pixel tile and
 * output group) and a second kernel merges them; the result is bitwise
 * reproducible. */
gn_status gn_conv3x3_nhwc(const void *x, const float *norm_mean, const float *norm_rstd,
                          const float *gamma, const float *beta, int64_t G, int apply_silu,
                          const void *wt, const float *bias, const void *res, void *z,
                          int64_t N, int64_t H, int64_t W, int64_t Ci, int64_t Co,
                          int64_t G2, float eps2, float *mean2_out, float *rstd2_out,
                          void *stream);

/* The weights of gn_conv3x3_nhwc reach the matrix cores in a packed order
 * (per 128 output channels, per chunk of 32 input channels and tap, the
 * 16-byte fragments of each wave next to each other); gn_conv3x3_nhwc packs
 * them into the stream's scratch buffer on every call (one extra kernel,
 * 2*Co*9*Ci bytes read and written).  A caller whose weights do not change
 * packs them once with gn_conv3x3_pack_weights -- wt: bf16 [Co][3][3][Ci],
 * packed: a device buffer of the same size (Co*9*Ci bf16), 16-byte aligned;
 * same support checks as the convolution -- and passes the packed buffer to
 * gn_conv3x3_nhwc_packed, which is gn_conv3x3_nhwc without the packing
 * step.  The packed order is internal to this library version. */
gn_status gn_conv3x3_pack_weights(const void *wt, void *packed, int64_t Ci, int64_t Co,
                                  void *stream);
gn_status gn_conv3x3_nhwc_packed(const void *x, const float *norm_mean, const float *norm_rstd,
                                 const float *gamma, const float *beta, int64_t G,
                                 int apply_silu, const void *packed_wt, const float *bias,
                                 const void *res, void *z, int64_t N, int64_t H, int64_t W,
                                 int64_t Ci, int64_t Co, int64_t G2, float eps2,
                                 float *mean2_out, float *rstd2_out, void *stream);

/* Launch shape of gn_conv3x3_nhwc for a problem, for inspection and tests;
 * no HIP call.  G2 > 0 asks for the statistics output.  Writes 7 values:
 * [0] tiles_h = ceil(H/8), [1] tiles_w = ceil(W/16) (output tiles of 8x16
 * pixels), [2] nb = Co/(64*wn) output-channel blocks, [3] 1 when the
 * XCD-aware block order is used (nb divides 8), [4] workgroups with work
 * (N*tiles_h*tiles_w*nb), [5] workgroups launched, [6] wn: waves along the
 * output channels of a workgroup of 256 lanes (4 when Co is a multiple of
 * 256: 4 waves of 128 pixels x 64 channels; else 2: 2 x 2 waves of 64 pixels
 * x 64 channels).  Returns
 * the status
 * gn_conv3x3_nhwc would return from its argument checks for aligned
 * pointers. */
gn_status gn_conv3x3_plan(int64_t N, int64_t H, int64_t W, int64_t Ci, int64_t Co, int64_t G2,
                          int64_t plan_out[7]);

/* Name of kernel slot i of gn_profile_rows, or NULL. */
const char *gn_kernel_name(int i);

/* Static description of a status code. */
const char *gn_status_string(gn_status s);

/* Library version, major*10000 + minor*100 + patch. */
int gn_version(void);

/* Facts about HIP device `device` for measurement reports (hipGetDeviceProperties):
 * info_out[0] compute units, [1] peak engine clock in kHz, [2] peak memory
 * clock in kHz, [3] memory bus width in bits, [4] device memory in bytes,
 * [5] wavefront size.  GN_INVALID_ARGUMENT for a null info_out or a negative
 * device, GN_DEVICE_ERROR when the HIP call fails (no device there).  Writes
 * nothing on error. */
gn_status gn_device_info(int device, int64_t info_out[6]);

#ifdef __cplusplus
}
#endif

#endif /* GNSILU_H */
