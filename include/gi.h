/*
 * gi.h -- C ABI of libgi.so: tile-based rasterization of 2D Gaussians on
 * AMD Instinct MI355X (gfx950), forward and backward, with a fused Adam step.
 *
 * Method (as the pages state it; they print no formulas, the readings are
 * given with each call):
 *   - "GaussianImage" (Overview): an image is represented by 2D Gaussians of
 *     8 parameters each -- position, covariance, colour -- and rendered by
 *     accumulated summation.  The covariance is held as a Cholesky factor
 *     (the "gaussianimage_cholesky" scripts of its quick start).
 *   - "Drawing with Gaussians" (Overview, 2D fitting): anisotropic 2D
 *     Gaussians alpha-composited over a trainable background; covariance from
 *     a lower-triangular L (MLX-specific notes).
 *   - "FlashImgs" (Commands: train, --loss l2; Python API): image fitting with
 *     an L2 loss, rendering and training kernels behind tensor-level calls.
 *   - fvdb radiance_fields page (GaussianSplatReconstructionConfig: tile_size
 *     = 16, eps_2d bounding-box padding; GaussianSplatOptimizer: Adam).
 *
 * Conventions shared by every call
 *   - Pointers marked "device" are device memory (hipMalloc, or a torch CUDA
 *     tensor's data pointer) owned by the caller; the library never allocates,
 *     frees or retains them, and keeps no global state.  "host" pointers are
 *     read synchronously during the call.
 *   - `stream` is a hipStream_t (NULL: the legacy default stream).  Every call
 *     only enqueues work on it and returns; results are ready when the stream
 *     reaches them.  Calls on different streams that share buffers race.
 *   - Arguments are checked before anything is enqueued; a bad argument
 *     returns GI_ERR_INVALID_ARG and enqueues nothing.  A failed launch returns
 *     GI_ERR_HIP.  gi_status_string() names a status.
 *   - float arrays are IEEE fp32; device arrays must be 16-byte aligned.
 *   - Pixel (row i, column j) samples the point (j + 0.5, i + 0.5); images are
 *     planar [3][H][W] (channel, row, column).  Tiles are 16x16 pixels, tile
 *     id = ty * ceil(W/16) + tx.  1 <= W, H <= 32768.
 *
 * Gaussian parameters ("params", device float [n][8]):
 *     mux, muy, l11, l21, l22, cr, cg, cb
 *   mean in pixels; covariance Sigma = L L^T with L = [[l11, 0], [l21, l22]]
 *   (signs free, det Sigma = (l11 l22)^2); colour = weighted colour (the
 *   Gaussian's peak amplitude; opacity is folded into it in the sum mode).
 *   Alpha mode adds "logit" (device float [n]): o = sigmoid(min(logit, ln 999)).
 *
 * Cutoff (the 3-sigma rule; its fp32 evaluation is part of the contract so
 * that binning and pixel coverage are reproducible bit for bit):
 *     i11 = 1/l11, i22 = 1/l22, k = -((l21*i11)*i22)            (L^-1 rows)
 *     a = i11*S, b = k*S, c = i22*S,   S = fp32(sqrt(log2(e)/2))
 *     dx = (j+0.5) - mux, dy = (i+0.5) - muy
 *     u = a*dx, t = b*dx, v = fma(c, dy, t), e = fma(v, v, u*u)
 *     the pair (Gaussian, pixel) contributes iff e <= fp32(4.5*log2(e)),
 *   i.e. iff d^T Sigma^-1 d <= 9 up to fp32 rounding; its weight is
 *   w = exp(-d^T Sigma^-1 d / 2) = 2^-e.  A Gaussian with a non-finite
 *   parameter (or logit), l11 == 0, l22 == 0, or non-finite i11/i22/k is
 *   culled: it covers no tile and no pixel, and its gradient is 0.
 */
#ifndef GI_H
#define GI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GI_OK = 0,
    GI_ERR_INVALID_ARG = 1,
    GI_ERR_HIP = 2,
    GI_ERR_CAPACITY = 3,
    GI_ERR_UNSUPPORTED = 4   /* a size beyond a fixed limit of the call (gi_render_image_noalloc) */
} gi_status;

typedef enum {
    GI_MODE_SUM = 0,     /* accumulated summation ("GaussianImage", Overview)            */
    GI_MODE_ALPHA = 1    /* front-to-back alpha over a background ("Drawing with Gaussians") */
} gi_mode;

typedef struct {
    int32_t width;       /* W, pixels */
    int32_t height;      /* H, pixels */
    int32_t mode;        /* gi_mode */
    int32_t reserved;    /* must be 0 */
} gi_desc;

/* Name of a status code (static string). */
const char *gi_status_string(gi_status s);

/* Library version, e.g. "gi 1.0 gfx950". */
const char *gi_version(void);

/* Number of 16x16 tiles, ceil(W/16)*ceil(H/16); 0 for an invalid desc. */
int64_t gi_num_tiles(const gi_desc *desc);

/*
 * gi_preprocess -- per-Gaussian set-up for binning and rasterization.
 *   Reading of "GaussianImage" (8 parameters, Cholesky covariance) and the
 *   fvdb config's eps_2d (pixel padding of the screen-space box).
 *
 *   n        number of Gaussians, 0 <= n < 2^27 (every call that takes n).
 *   params   device float [n][8], as above.
 *   logit    device float [n] (alpha mode) or NULL (sum mode).
 *   records  device float [n][8] out: mux, muy, a, b, c, cr, cg, cb
 *            (a, b, c as in the cutoff rule; zeros for a culled Gaussian).
 *   opacity  device float [n] out (alpha mode): o = 1/(1+exp(-min(logit, ln 999)));
 *            NULL in sum mode.
 *   pixbox   device uint16 [n][4] out: j0, i0, j1, i1, the inclusive pixel box
 *            of the 3-sigma ellipse, clipped to the image:
 *              rx = 3|l11| + 1/256, ry = 3 sqrt(fma(l21, l21, l22*l22)) + 1/256,
 *              j0 = max(0, ceil((mux-0.5) - rx)), j1 = min(W-1, floor((mux-0.5) + rx)),
 *              i0, i1 likewise with muy, ry (fp32).  An empty box (off-image or
 *              culled) is written as (1, 1, 0, 0).
 *   counts   device uint32 [n] out: tiles covered, (j1/16 - j0/16 + 1)(i1/16 - i0/16 + 1),
 *            0 for an empty box.
 */
gi_status gi_preprocess(const gi_desc *desc, int64_t n, const float *params, const float *logit,
                        float *records, float *opacity, uint16_t *pixbox, uint32_t *counts,
                        void *stream);

/*
 * gi_bin_sort -- tile lists: every (tile, Gaussian) pair of the pixel boxes,
 *   ordered by tile and, within a tile, by ascending Gaussian index.  Pairs are
 *   emitted per Gaussian in (index, tile row, tile column) order and sorted by
 *   tile id with a stable radix sort, so each tile's list is in index order
 *   (the summation order of the sum image and the front-to-back order of the
 *   alpha image).  Reading: tile binning is what the FlashImgs viewer calls
 *   "tile-binned compute" (Web viewer) with fvdb's 16-pixel tiles.
 *
 *   pixbox, counts  from gi_preprocess (device).
 *   offsets   device uint32 [n+1] out: exclusive prefix sum of counts; offsets[n] = M.
 *   keys      device uint32 [capacity] out: tile id of pair m (m < M), ascending.
 *   vals      device uint32 [capacity] out: Gaussian index of pair m.
 *   ranges    device uint32 [T][2] out: [start, end) of tile t in keys/vals;
 *             (0, 0) for a tile with no pair.
 *   tile_order device uint32 [T] out, or NULL: a permutation of the tiles for
 *             the raster calls.  The tiles are ranked by decreasing list length
 *             (lengths of 1023 or more count as equal; ties in no particular
 *             order) and rank p goes to launch position serp(p): positions come
 *             in layers of P = the device's CU count, layer k holding ranks
 *             kP .. kP+P-1, in reverse order in odd layers (a last, partial layer
 *             of width r reversed within its r positions).  The hardware deals
 *             consecutive workgroups round-robin over the CUs, so each CU then
 *             gets a mix of long and short lists, which balances the CUs when the
 *             whole grid of tiles is resident at once (a few thousand tiles); it
 *             never changes a result.  Costs one single-workgroup launch; an order from an
 *             earlier binning is as valid (any permutation of the tiles is),
 *             so a caller may refresh it only now and then.
 *   capacity  length of keys/vals, 0 <= capacity < 2^31.
 *   d_num     device uint32 [1] out: M (saturated at 2^32-1).  When M > capacity
 *             no pair is written, every range is (0, 0) and *d_num still holds M.
 *   h_num     host int64 [1] or NULL.  If given, the call waits for the stream,
 *             stores M there, and returns GI_ERR_CAPACITY when M > capacity;
 *             if NULL the call never waits and overflow shows only in *d_num.
 *   workspace device scratch of at least gi_bin_sort_workspace_bytes() bytes,
 *             256-byte aligned; its contents need no initialisation and are
 *             garbage afterwards.
 */
size_t gi_bin_sort_workspace_bytes(const gi_desc *desc, int64_t n, int64_t capacity);
gi_status gi_bin_sort(const gi_desc *desc, int64_t n, const uint16_t *pixbox, const uint32_t *counts,
                      uint32_t *offsets, uint32_t *keys, uint32_t *vals, uint32_t *ranges,
                      uint32_t *tile_order, int64_t capacity, uint32_t *d_num, int64_t *h_num,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * gi_preprocess_bin_sort -- gi_preprocess followed by gi_bin_sort on the same
 *   stream, with identical outputs, in one call that saves a launch: the
 *   preprocess kernel also writes the per-group pair totals the binning would
 *   otherwise compute in a kernel of its own and clears ranges.  Arguments as in
 *   the two calls (the preprocess outputs pixbox and counts are written and then
 *   read by the binning); the same errors, checked before anything is launched.
 *   workspace must hold gi_bin_sort_workspace_bytes() bytes.
 */
gi_status gi_preprocess_bin_sort(const gi_desc *desc, int64_t n, const float *params, const float *logit,
                                 float *records, float *opacity, uint16_t *pixbox, uint32_t *counts,
                                 uint32_t *offsets, uint32_t *keys, uint32_t *vals, uint32_t *ranges,
                                 uint32_t *tile_order, int64_t capacity, uint32_t *d_num, int64_t *h_num,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * gi_render_fwd -- rasterize the binned Gaussians into an image.
 *   Sum mode ("GaussianImage", accumulated summation):
 *       I_k(p) = sum over the tile's list, in list order, of c_k * 2^-e
 *     over pairs admitted by the cutoff; no background, no clamping.  The fp32
 *     sum is formed in list order, so the image is bitwise reproducible.
 *   Alpha mode ("Drawing with Gaussians", alpha-composited over a background):
 *       alpha = o * 2^-e, C_k += c_k * alpha * T, T -= alpha * T, in list order;
 *     after the first Gaussian that leaves T < 1e-4 the pixel stops;
 *       image_k = C_k + T * background_k.
 *
 *   n                 number of Gaussians given to gi_preprocess.
 *   records, opacity, pixbox  from gi_preprocess (opacity NULL in sum mode);
 *                     the pixel boxes let each 8x8 quadrant of a tile skip the
 *                     Gaussians that cannot reach it (no effect on the result).
 *   ranges, vals      from gi_bin_sort.
 *   tile_order        from gi_bin_sort, or NULL (tiles in index order).
 *   background device float [3] (alpha mode) or NULL.
 *   image      device float [3][H][W] out.
 *   t_final    device float [H][W] out (alpha mode): final T; NULL in sum mode.
 *   last       device uint32 [H][W] out (alpha mode): one past the list position
 *              (index into vals) of the last Gaussian composited at the pixel, or
 *              the tile's range start if none; NULL in sum mode.
 */
gi_status gi_render_fwd(const gi_desc *desc, int64_t n, const float *records, const float *opacity,
                        const uint16_t *pixbox, const uint32_t *ranges, const uint32_t *tile_order,
                        const uint32_t *vals,
                        const float *background, float *image, float *t_final, uint32_t *last,
                        void *stream);

/* Flags of gi_render_image and gi_fit_step_sum (see there). */
#define GI_FIT_PREPARED 1u
#define GI_FIT_ORDER 2u
#define GI_FIT_USE_ORDER 4u
#define GI_FIT_NO_UPDATE 8u
#define GI_FIT_TRACK_MAX 16u

/*
 * gi_render_image -- gi_preprocess_bin_sort followed by gi_render_fwd in one
 *   call: params (and logit) in, image (and t_final, last) out, with every
 *   intermediate written as those calls write it.  In sum mode, when each
 *   first-pass bucket holds at most 16 tiles (see gi_fit_step_sum), the
 *   raster's workgroups finish the sort themselves and the bucket pass is not
 *   launched; keys, vals, ranges and every output are still bit-identical to
 *   the two calls.
 *   flags     GI_FIT_ORDER: (re)write tile_order from this binning (possibly
 *             after this call's raster pass); GI_FIT_USE_ORDER: the raster pass
 *             takes the tiles in tile_order, which must hold a valid order.
 *   h_num     as in gi_bin_sort (waits; GI_ERR_CAPACITY when M > capacity, the
 *             image then being empty).
 *   Other arguments as in gi_preprocess_bin_sort and gi_render_fwd.
 */
gi_status gi_render_image(const gi_desc *desc, int64_t n, const float *params, const float *logit,
                          const float *background, float *records, float *opacity, uint16_t *pixbox, uint32_t *counts,
                          uint32_t *offsets, uint32_t *keys, uint32_t *vals, uint32_t *ranges, uint32_t *tile_order,
                          uint32_t flags, int64_t capacity, uint32_t *d_num, int64_t *h_num, void *workspace,
                          size_t workspace_bytes, float *image, float *t_final, uint32_t *last, void *stream);

/*
 * gi_render_image_noalloc -- gi_render_image without a workspace argument, for
 *   callers that cannot allocate device memory (code under HIP graph capture,
 *   tight serving loops, harnesses that forbid allocation).  The bin workspace
 *   is a fixed device array inside the library, 64 MiB, of which each GPU the
 *   library runs on holds its own copy until the process ends; the call itself
 *   allocates and frees nothing.  Every call on one GPU uses that GPU's copy:
 *   calls that may overlap on one GPU (different streams, or different host
 *   threads, without ordering between them) race and give wrong results; calls
 *   ordered on one stream are fine.  The array needs no clearing (every call
 *   writes what it reads).
 *   A problem whose bin workspace (gi_bin_sort_workspace_bytes(desc, n,
 *   capacity)) exceeds gi_render_image_noalloc_max_bytes() returns
 *   GI_ERR_UNSUPPORTED before anything is enqueued (e.g. 2048x2048 with 500,000
 *   Gaussians fits up to about 8 million pairs of capacity).  Otherwise the
 *   arguments, results and errors are gi_render_image's, bit for bit.
 */
size_t gi_render_image_noalloc_max_bytes(void);
gi_status gi_render_image_noalloc(const gi_desc *desc, int64_t n, const float *params, const float *logit,
                                  const float *background, float *records, float *opacity, uint16_t *pixbox,
                                  uint32_t *counts, uint32_t *offsets, uint32_t *keys, uint32_t *vals,
                                  uint32_t *ranges, uint32_t *tile_order, uint32_t flags, int64_t capacity,
                                  uint32_t *d_num, int64_t *h_num, float *image, float *t_final, uint32_t *last,
                                  void *stream);

/*
 * gi_render_fwd_l2 -- gi_render_fwd (sum mode) fused with the L2 loss of
 *   "FlashImgs" (train --loss l2): besides the image it writes
 *     dL_dimage = 2 (image - target) / (3 W H)
 *   and loss_partials[t] = sum over tile t's pixels and channels of
 *   (image - target)^2 (fp32, a fixed order); gi_loss_reduce turns the partials
 *   into the loss.  Same image bits as gi_render_fwd.
 *   target      device float [3][H][W].
 *   dL_dimage   device float [3][H][W] out.
 *   loss_partials device float [T] out (T = gi_num_tiles).
 */
gi_status gi_render_fwd_l2(const gi_desc *desc, int64_t n, const float *records, const uint16_t *pixbox,
                           const uint32_t *ranges, const uint32_t *tile_order, const uint32_t *vals,
                           const float *target, float *image, float *dL_dimage, float *loss_partials,
                           void *stream);

/* d_loss (device float [1]) = (sum of the nparts partials, in fp64, fixed order) / count. */
gi_status gi_loss_reduce(int64_t nparts, const float *loss_partials, int64_t count, float *d_loss,
                         void *stream);

/*
 * gi_render_bwd -- gradients of a scalar loss L given dL/dimage.
 *   Reading of "Drawing with Gaussians" (fused rasterization kernels with
 *   custom VJPs): the exact derivative of gi_render_fwd's image, with the
 *   cutoff held fixed (almost-everywhere derivative) and, in alpha mode, each
 *   pixel's stopping point held fixed.  Per admitted pair with w = 2^-e:
 *     sum:   dL/dc_k += g_k w,  dL/dw = sum_k g_k c_k
 *     alpha: dL/dc_k += g_k alpha T_j,
 *            dL/dalpha = sum_k g_k (T_j c_k - S_k / (1 - alpha)),
 *            S_k = sum over later contributors of c alpha T, plus T_final bg_k,
 *            dL/dlogit += dL/dalpha * w * o (1 - o)  (0 when logit >= ln 999),
 *            dL/dbg_k += g_k T_final.
 *     w -> (mean, L) through d^T Sigma^-1 d.
 *
 *   records, opacity, pixbox: from gi_preprocess (opacity NULL in sum mode).
 *   offsets, ranges, vals, capacity: from / as given to gi_bin_sort.
 *   tile_order from gi_bin_sort, or NULL (tiles in index order).
 *   logit     device float [n] (alpha mode, for the clamp test) or NULL.
 *   background, t_final, last: as given to / produced by gi_render_fwd (alpha
 *             mode; NULL in sum mode).
 *   dL_dimage device float [3][H][W].
 *   dparams   device float [n][8], ACCUMULATED (+=) in the params layout; it may
 *             be NULL, which leaves the pair slots in the workspace for
 *             gi_adam_step_pairs[_rs|_alpha] or gi_grad_gather (no gather pass).
 *   dlogit    device float [n], accumulated (alpha mode) or NULL.
 *   dbackground device float [3], accumulated (alpha mode) or NULL.
 *   loss_partials, loss_count, d_loss (sum mode, optional): when d_loss is not
 *             NULL, a spare workgroup of the same launch also does what
 *             gi_loss_reduce(T, loss_partials, loss_count, d_loss) does (the
 *             partials of gi_render_fwd_l2; one launch fewer per training step);
 *             NULL in alpha mode.
 *   workspace device scratch of gi_render_bwd_workspace_bytes() bytes, 256-byte
 *             aligned, no initialisation needed (alpha mode: it also holds a
 *             64-byte copy of each Gaussian's record, opacity, box and offset,
 *             so that the backward reads one 64-byte line per list entry).
 *   Each (Gaussian, tile) pair's sums (its pixels' terms in the Gaussian's
 *   whitened frame, as gi_grad_gather describes) are formed in the tile's
 *   workgroup, its per-pixel terms added in a fixed order, and stored at the
 *   pair's emission slot offsets[g] + (position of the tile in g's tile
 *   rectangle); a second pass adds each Gaussian's slots in that order and
 *   maps the total to the gradient w.r.t. (mean, L, colour) with the record's
 *   rows (a, b, c).  No atomics: the gradients are bitwise reproducible.  If gi_bin_sort overflowed
 *   (M > capacity) nothing is accumulated.
 */
size_t gi_render_bwd_workspace_bytes(const gi_desc *desc, int64_t n, int64_t capacity);
gi_status gi_render_bwd(const gi_desc *desc, int64_t n, const float *records, const float *opacity,
                        const float *logit, const uint16_t *pixbox, const uint32_t *offsets,
                        const uint32_t *ranges, const uint32_t *tile_order, const uint32_t *vals,
                        int64_t capacity,
                        const float *background, const float *t_final, const uint32_t *last,
                        const float *dL_dimage, float *dparams, float *dlogit, float *dbackground,
                        const float *loss_partials, int64_t loss_count, float *d_loss,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * gi_render_fwd_bwd_l2 -- gi_render_fwd_l2 and then gi_render_bwd (sum mode,
 *   dparams NULL, dL_dimage = the L2 gradient just formed) in one launch: each
 *   tile's workgroup renders the tile, forms its dL/dimage and immediately
 *   back-propagates it, so dL/dimage never goes through device memory and the
 *   tile list is staged once.  Outputs are bit-identical to the two calls:
 *   image, loss_partials (and dL_dimage when not NULL) as gi_render_fwd_l2, the
 *   pair slots in the workspace as gi_render_bwd, ready for
 *   gi_adam_step_pairs (or gi_grad_gather).  Arguments as in those two calls; the
 *   workspace is gi_render_bwd's.  Sum mode only.
 */
gi_status gi_render_fwd_bwd_l2(const gi_desc *desc, int64_t n, const float *records, const uint16_t *pixbox,
                               const uint32_t *offsets, const uint32_t *ranges, const uint32_t *tile_order,
                               const uint32_t *vals, int64_t capacity, const float *target, float *image,
                               float *dL_dimage, float *loss_partials, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * gi_loss_l2 -- L = mean over the 3HW entries of (image - target)^2 and
 *   dL/dimage = 2 (image - target) / (3HW)  ("FlashImgs", --loss l2).
 *   count      number of entries (3*H*W), >= 1.
 *   dL_dimage  device float [count] out (may be NULL).
 *   d_loss     device float [1] out (may be NULL); summed in fp64 per block and
 *              over blocks in a fixed order (reproducible).
 *   workspace  device scratch of gi_loss_workspace_bytes(count) bytes.
 */
size_t gi_loss_workspace_bytes(int64_t count);
gi_status gi_loss_l2(int64_t count, const float *image, const float *target, float *dL_dimage,
                     float *d_loss, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gi_adam_step -- one fused Adam step over rows x row_len fp32 entries
 *   (fvdb GaussianSplatOptimizer: Adam; "Drawing with Gaussians": fused
 *   optimizer kernels).  With t = step >= 1:
 *     m = b1 m + (1-b1) g,  v = b2 v + (1-b2) g^2,
 *     p -= lr[slot] * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps),
 *   slot = column within the row; no weight decay.  zero_grad != 0 also sets
 *   g = 0 afterwards (ready for the next accumulation).
 *   p, g, m, v  device float [rows][row_len], updated in place.
 *   lr          host float [row_len], 1 <= row_len <= 16.
 *   beta1, beta2, eps  host doubles: 1 - beta and the bias corrections are formed
 *               in double before rounding to fp32 (1 - 0.999f is 1.3e-5 off 0.001).
 */
gi_status gi_adam_step(int64_t rows, int32_t row_len, float *p, float *g, float *m, float *v,
                       const float *lr, double beta1, double beta2, double eps, int32_t step,
                       int32_t zero_grad, void *stream);

/*
 * gi_adam_step_pairs -- gi_adam_step (rows of 8, sum mode) whose gradient is
 *   read straight from the per-pair slots that gi_render_bwd(dparams = NULL)
 *   left in its workspace: each Gaussian's slots offsets[g] .. offsets[g+1]
 *   are added in emission order (the gather), mapped to the Cholesky-form
 *   gradient as gi_render_bwd does (with (a, b, c) formed from p, which must
 *   be the params the records were made from), and the Adam update applied in
 *   the same pass.  Same arguments as gi_render_bwd for the slots (desc, n,
 *   offsets, capacity, workspace) and as gi_adam_step for the update (p, m, v
 *   device float [n][8]; lr host float [8]).  A binning overflow gives a zero
 *   gradient.
 *   d_step    device int32 [1] or NULL.  If given, the step t is read from it on
 *             the device (and `step` is ignored; t < 1 counts as 1), so that one
 *             captured graph of a training step stays right on every replay
 *             when the caller advances *d_step in the same graph.  The bias
 *             corrections 1/(1-b1^t), 1/sqrt(1-b2^t) are formed on the device in
 *             fp64 either way (the same bits for the same t).
 *   loss_partials, loss_count, d_loss (optional): when d_loss is not NULL, one
 *             more workgroup of the launch does what gi_loss_reduce(T,
 *             loss_partials, loss_count, d_loss) does (T = gi_num_tiles), for the
 *             partials of gi_render_fwd_bwd_l2: the training step's loss
 *             without a launch of its own.
 */
gi_status gi_adam_step_pairs(const gi_desc *desc, int64_t n, const uint32_t *offsets, int64_t capacity,
                             const void *workspace, size_t workspace_bytes, float *p, float *m, float *v,
                             const float *lr, double beta1, double beta2, double eps, int32_t step,
                             const int32_t *d_step, const float *loss_partials, int64_t loss_count,
                             float *d_loss, void *stream);

/*
 * gi_fit_step_sum -- one training step of the accumulated-sum fit (sum mode,
 *   L2 loss, Adam) in one call: the tile binning of the parameters, the fused
 *   forward + L2 gradient + backward (gi_render_fwd_bwd_l2), and the Adam step
 *   with the gathered gradient (gi_adam_step_pairs, with the loss reduced into
 *   d_loss).  The Adam kernel then goes on to set up the updated parameters
 *   for the next step's binning -- what gi_preprocess_bin_sort's preprocess
 *   kernel does (records, pixbox, counts, the binning's group totals and digit
 *   histogram in the bin workspace, ranges cleared) -- so that the next call can
 *   start with the sort (GI_FIT_PREPARED): one launch and one pass over the
 *   parameters fewer per step.  Every result is bit-identical to the sequence
 *   gi_preprocess_bin_sort, gi_render_fwd_bwd_l2, gi_adam_step_pairs.
 *   Reading: "FlashImgs" (train --loss l2, max_steps; Performance) and fvdb's
 *   Adam (GaussianSplatOptimizer), run as one step.
 *
 *   b         the buffers (gi_fit_buffers), as in the calls above; after the
 *             call params / m / v hold the updated values, image and *d_loss
 *             the forward of this step (before the update), offsets / keys /
 *             vals / d_num this step's binning, records / pixbox / counts the
 *             set-up of the UPDATED parameters, and ranges are cleared (ready for
 *             the next binning).
 *   hp        Adam hyperparameters (host), as gi_adam_step_pairs'.
 *   step, d_step  Adam's step t, as gi_adam_step_pairs'.
 *   flags     GI_FIT_PREPARED: the previous gi_fit_step_sum on the same buffers,
 *             desc, n and capacity left the set-up (skip the preprocess kernel);
 *             without it the call preprocesses params first.  Only valid if
 *             params were not changed in between.
 *             GI_FIT_ORDER: also (re)write b->tile_order from this binning (as
 *             gi_bin_sort's tile_order; it may be written after this call's
 *             raster pass, i.e. take effect from the next call).
 *             GI_FIT_USE_ORDER: the raster pass takes the tiles in b->tile_order,
 *             which must hold a valid order (an earlier call's GI_FIT_ORDER, or
 *             gi_bin_sort); any permutation gives the same results.
 *             GI_FIT_NO_UPDATE: binning and the fused raster only -- the
 *             pair slots stay in b->bwd_workspace and the loss
 *             partials in b->loss_partials for the caller's own update pass
 *             (e.g. gi_adam_step_pairs_rs of another parameter form whose
 *             Cholesky form is b->params); hp (may be NULL), step, d_step, m, v
 *             and d_loss are unused, and the next call must not pass GI_FIT_PREPARED.
 *             GI_FIT_TRACK_MAX: b->d_num points to 2 uint32; besides M in
 *             d_num[0], d_num[1] = max(d_num[1], M) (the caller clears it): one
 *             read after many asynchronous steps tells whether any of their
 *             binnings overflowed (M > capacity renders nothing and gives a
 *             zero gradient for that step).
 *   When each first-pass bucket holds at most 16 tiles (plans whose low digit
 *   has at most 4 bits, e.g. 768x512), the raster's
 *   workgroups finish the sort themselves -- each reads its tile's bucket and
 *   picks its entries out in bucket order, writing keys, vals and the range
 *   exactly where the bucket pass would -- and that pass is not launched.
 *   Errors as the calls above; a binning overflow (M > capacity) shows in
 *   *d_num and gives a zero gradient (the Adam step still runs).
 */

typedef struct gi_fit_buffers {
    float *params, *m, *v;          /* device float [n][8]: parameters and Adam moments, in place */
    const float *target;            /* device float [3][H][W] */
    float *image;                   /* device float [3][H][W] out */
    float *loss_partials;           /* device float [T] (scratch) */
    float *d_loss;                  /* device float [1] out, or NULL */
    float *records;                 /* device float [n][8] */
    uint16_t *pixbox;               /* device uint16 [n][4] */
    uint32_t *counts;               /* device uint32 [n] */
    uint32_t *offsets;              /* device uint32 [n+1] */
    uint32_t *keys, *vals;          /* device uint32 [capacity] */
    uint32_t *ranges;               /* device uint32 [T][2] */
    uint32_t *tile_order;           /* device uint32 [T], or NULL */
    uint32_t *d_num;                /* device uint32 [1] out: M */
    int64_t capacity;
    void *bin_workspace;            /* gi_bin_sort_workspace_bytes(desc, n, capacity) bytes */
    size_t bin_workspace_bytes;
    void *bwd_workspace;            /* gi_render_bwd_workspace_bytes(desc, n, capacity) bytes */
    size_t bwd_workspace_bytes;
} gi_fit_buffers;

typedef struct gi_adam_hparams {
    float lr[8];                    /* per parameter slot */
    double beta1, beta2, eps;
} gi_adam_hparams;

gi_status gi_fit_step_sum(const gi_desc *desc, int64_t n, const gi_fit_buffers *b, const gi_adam_hparams *hp,
                          int32_t step, const int32_t *d_step, uint32_t flags, void *stream);

/*
 * gi_fit_step_sum_ssim -- gi_fit_step_sum with the pixel loss of gi_loss_ssim
 *   (w1 mean|I - T| + w2 mean (I - T)^2 + ws (1 - SSIM); "Drawing with
 *   Gaussians", 2D fitting; "FlashImgs", Training features / --loss) in place
 *   of the L2 loss.  The SSIM gradient at a pixel needs the rendered image
 *   around it, so the raster pass is the forward (finishing the sort as the
 *   fused pass does), gi_loss_ssim with GI_SSIM_TARGET_PREPARED, and the
 *   backward into the pair slots; the binning before and the Adam step with
 *   the set-up for the next call after are gi_fit_step_sum's.  Every result
 *   is bit-identical to the sequence gi_preprocess_bin_sort, gi_render_fwd,
 *   gi_loss_ssim, gi_render_bwd (dparams = NULL), gi_adam_step_pairs.
 *   b->loss_partials is not used (may be NULL); b->d_loss (or NULL) receives
 *   the loss.  Flags, buffers and errors as gi_fit_step_sum, and:
 *   w1, w2, ws      finite loss weights.
 *   dL_dimage       device float [3][H][W] (scratch: dL/dI), 16-byte aligned,
 *                   not the image or the target.
 *   ssim_workspace  >= gi_loss_ssim_workspace_bytes(W, H) bytes, 256-byte
 *                   aligned, holding b->target's statistics from
 *                   gi_loss_ssim_target.
 */
gi_status gi_fit_step_sum_ssim(const gi_desc *desc, int64_t n, const gi_fit_buffers *b, const gi_adam_hparams *hp,
                               float w1, float w2, float ws, float *dL_dimage, void *ssim_workspace,
                               size_t ssim_workspace_bytes, int32_t step, const int32_t *d_step, uint32_t flags,
                               void *stream);

/*
 * Parameter forms ("GaussianImage", Overview and its training scripts: the
 * covariance as a Cholesky factor or as a rotation and two scales;
 * "FlashImgs", Library API: xy / scale / rot tensors, and rendering a trained
 * set at any output size).
 *   GI_PARAMS_CHOLESKY  the params above.
 *   GI_PARAMS_RS        mux, muy, sx, sy, theta, cr, cg, cb (theta in radians):
 *                       Sigma = R diag(sx^2, sy^2) R^T,
 *                       R = [[cos theta, -sin theta], [sin theta, cos theta]].
 */
typedef enum { GI_PARAMS_CHOLESKY = 0, GI_PARAMS_RS = 1 } gi_param_kind;

/*
 * gi_params_to_cholesky -- the Cholesky-form params (the form every other call
 *   takes) of n Gaussians given in form `kind`, with the image plane scaled by
 *   D = diag(fx, fy): mean D mu, covariance D Sigma D, i.e. L -> D L.  To render
 *   a set at another size W' x H', pass fx = W'/W, fy = H'/H; fx = fy = 1 only
 *   converts.  RS, in fp32 with (cs, sn) = sincosf(theta), ax = |sx|, ay = |sy|:
 *     l11 = sqrt(fma(cs ax, cs ax, (sn ay)^2)),
 *     l21 = (cs sn) ((ax - ay)(ax + ay)) / l11,   l22 = (ax ay) / l11
 *   (the Cholesky factor of Sigma; l22 from det Sigma = (ax ay)^2 without
 *   cancellation), then (fx l11, fy l21, fy l22).  A zero scale gives l22 = 0,
 *   which the raster culls.  The cutoff rule above then applies to these
 *   Cholesky params.
 *   params  device float [n][8] in form `kind`.
 *   out     device float [n][8]; may alias params only for GI_PARAMS_CHOLESKY.
 *   fx, fy  > 0 and finite.
 */
gi_status gi_params_to_cholesky(int32_t kind, int64_t n, const float *params, float fx, float fy, float *out,
                                void *stream);

/*
 * gi_params_to_cholesky_grad -- the chain rule of gi_params_to_cholesky:
 *   dparams = J^T dout, J its Jacobian at params (same kind, fx, fy).
 *   dout       device float [n][8]: gradient w.r.t. the Cholesky-form params
 *              (e.g. gi_render_bwd's dparams).
 *   dparams    device float [n][8], must not alias params; overwritten, or added
 *              to when accumulate != 0.  A Gaussian whose Cholesky form has
 *              l11 == 0 or a non-finite entry gets a zero gradient.
 */
gi_status gi_params_to_cholesky_grad(int32_t kind, int64_t n, const float *params, float fx, float fy,
                                     const float *dout, float *dparams, int32_t accumulate, void *stream);

/*
 * gi_grad_gather -- the gradient w.r.t. params of form `kind` straight from
 *   the backward's pair slots: what gi_render_bwd's dparams gives followed by
 *   gi_params_to_cholesky_grad, without going through the Cholesky-form
 *   gradient ("GaussianImage", Overview and its "gaussianimage_rs" scripts;
 *   "FlashImgs", Library API: scale / rot tensors, rendering at any size).
 *   The slots hold each pair's sums in the Gaussian's whitened frame
 *   (u, v) = (a dx, b dx + c dy) of its record: with h = (dL/dw) w, the sums
 *   of h u, h v, h u^2, h u v, h v^2 and of g_k w.  Any parameterisation's
 *   gradient is a linear map of a Gaussian's total; for the rotation-scale
 *   form that map (to the Gaussian's own axes) is orthogonal up to the scales,
 *   computed in fp64, so the result keeps the accuracy of the per-pixel terms
 *   -- unlike the chain rule applied to the Cholesky-form gradient, which for
 *   a rotated, elongated Gaussian is a difference of much larger terms.
 *   desc       the rendered image (sum or alpha mode; only the 8 parameters are
 *              gathered here).
 *   kind       gi_param_kind of params.
 *   params     device float [n][8] in form `kind`, whose Cholesky form at scale
 *              (fx, fy) (gi_params_to_cholesky) made `records`.
 *   records    device float [n][8]: gi_preprocess's records of that form, as
 *              given to the backward.
 *   offsets, capacity: as given to gi_render_bwd.
 *   workspace  gi_render_bwd's workspace after gi_render_bwd with dparams NULL,
 *              or gi_render_fwd_bwd_l2 (the slots are read, not changed).
 *   dparams    device float [n][8], ACCUMULATED (+=), not aliasing params.
 *   Gaussians without pairs (culled, off-image) and every Gaussian after an
 *   overflowed binning get nothing added.
 */
gi_status gi_grad_gather(const gi_desc *desc, int32_t kind, int64_t n, const float *params, float fx, float fy,
                         const float *records, const uint32_t *offsets, int64_t capacity, const void *workspace,
                         size_t workspace_bytes, float *dparams, void *stream);

/*
 * gi_loss_ssim -- the pixel loss
 *     L = w1 mean|I - T| + w2 mean (I - T)^2 + ws (1 - SSIM)
 *   over the 3HW entries, and dL/dI ("Drawing with Gaussians", 2D fitting:
 *   (1 - w) L1 + w (1 - SSIM) with w = 0.2; "FlashImgs", Commands: --loss l2,
 *   l1, l2+ssim, l1+ssim, and parse_loss's (l1, l2, ssim) ratios; fvdb:
 *   ssim_lambda).  SSIM (a reading: the pages give no formula) is the mean
 *   over the 3HW entries of the structural similarity map: per channel, the
 *   local statistics under an 11x11 Gaussian window (sigma 1.5, weights
 *   normalised to 1; pixels outside the image count as 0, the map has the
 *   image's size),
 *     SSIM(p) = (2 mx my + C1)(2 sxy + C2) / ((mx^2 + my^2 + C1)(sxx + syy + C2)),
 *   C1 = 0.01^2, C2 = 0.03^2 (x = I, y = T).  d|e|/de = sign(e), 0 at 0.
 *   One fused stencil kernel (fp32) per call; the loss is added up in fp64 in
 *   a fixed order by the workgroup that finishes last.
 *   image, target  device float [3][H][W].
 *   dL_dimage      device float [3][H][W], written; must not alias the inputs.
 *   d_loss         device float [1] (written: L) or NULL.
 *   workspace      device, >= gi_loss_ssim_workspace_bytes(W, H), 256-byte aligned;
 *                  calls that share a workspace must not overlap.
 *   flags          0: the call first forms this target's window statistics in
 *                  the workspace (as gi_loss_ssim_target does), replacing any
 *                  there.  GI_SSIM_TARGET_PREPARED: the workspace holds them
 *                  from gi_loss_ssim_target (or an unflagged call) with this
 *                  target, unchanged since, and the workspace has not been
 *                  written by the caller since; the call then skips that step.
 *                  Same results, bit for bit, either way.
 *
 * gi_loss_ssim_target -- the target's window statistics (its local means of T
 *   and T^2, the fitting loop's constant half of SSIM) into the workspace, for
 *   later gi_loss_ssim calls with GI_SSIM_TARGET_PREPARED; it also resets the
 *   workspace's count of finished tiles that the loss reduction uses.  Same
 *   arguments as above.
 */
#define GI_SSIM_TARGET_PREPARED 1u
size_t gi_loss_ssim_workspace_bytes(int32_t width, int32_t height);
gi_status gi_loss_ssim_target(int32_t width, int32_t height, const float *target, void *workspace,
                              size_t workspace_bytes, void *stream);
gi_status gi_loss_ssim(int32_t width, int32_t height, const float *image, const float *target, float w1, float w2,
                       float ws, float *dL_dimage, float *d_loss, void *workspace, size_t workspace_bytes,
                       uint32_t flags, void *stream);

/*
 * gi_adam_step_pairs_rs -- gi_adam_step_pairs for rotation-scale params (the
 *   "gaussianimage_rs" form of "GaussianImage"): each Gaussian's per-pair
 *   gradient slots (left by gi_render_fwd_bwd_l2, or gi_render_bwd with
 *   dparams = NULL, for the Cholesky params gi_params_to_cholesky made with
 *   fx = fy = 1) are added in emission order, mapped to the
 *   rotation-scale gradient as gi_grad_gather does (kind GI_PARAMS_RS,
 *   fx = fy = 1, the records' rows formed from p) and applied to p by the Adam
 *   step, in one pass.  Arguments as gi_adam_step_pairs (no device step counter);
 *   p, m, v device float [n][8] in the rotation-scale form.
 *   chol_out  device float [n][8] or NULL: also the updated Gaussians'
 *             Cholesky form (what gi_params_to_cholesky with fx = fy = 1
 *             writes, bit for bit), ready for the next step's binning.
 */
gi_status gi_adam_step_pairs_rs(const gi_desc *desc, int64_t n, const uint32_t *offsets, int64_t capacity,
                                const void *workspace, size_t workspace_bytes, float *p, float *m, float *v,
                                const float *lr, double beta1, double beta2, double eps, int32_t step,
                                const float *loss_partials, int64_t loss_count, float *d_loss, float *chol_out,
                                void *stream);

/*
 * gi_merge_pairs -- moment-matching merge of Gaussian pairs ("FlashImgs",
 *   Commands: merge, an overcomplete set merged down (80K -> 50K) by moment
 *   matching; Library API: merge_gaussians).  A reading, as the pages give no
 *   formula: Gaussian n is the function c_n exp(-q_n/2) with per-channel
 *   integral 2 pi |det L_n| c_{n,k} and mass w_n = |det L_n| sum_k |c_{n,k}|;
 *   pair (i, j) becomes the Gaussian with the mean and covariance of the
 *   mass-weighted mixture,
 *     mu = (w_i mu_i + w_j mu_j)/W,  Sigma = sum (w/W)(Sigma_n + d_n d_n^T),
 *     d_n = mu_n - mu, W = w_i + w_j (equal weights when W = 0),
 *   L = chol(Sigma) with a positive diagonal, and the colour that keeps each
 *   channel's integral: c_k = (|det L_i| c_{i,k} + |det L_j| c_{j,k}) / |det L|.
 *   Computed in fp64, rounded to fp32.  Which pairs to merge is the caller's.
 *   pairs   device int32 [n_pairs][2], 8-byte aligned: indices into params; a
 *           pair with an index outside [0, n) gives an all-NaN row.
 *   params  device float [n][8] (Cholesky form); out device float [n_pairs][8],
 *           not aliasing params.
 */
gi_status gi_merge_pairs(int64_t n_pairs, const int32_t *pairs, int64_t n, const float *params, float *out,
                         void *stream);

/*
 * gi_merge_round / gi_merge_apply / gi_merge_to -- merging a set down to a
 *   target count ("FlashImgs", Commands: merge -- an overcomplete set, 80K ->
 *   50K, "merges similar ones down" by moment matching; Library API:
 *   Session.merge_to).  The pages name no similarity or pair rule; the reading:
 *   - cost of merging Gaussians i < j: Runnalls' bound on the increase of the
 *     Kullback-Leibler divergence when two mixture components are replaced by
 *     their moment-matched merge ("Kullback-Leibler approach to Gaussian mixture
 *     reduction", IEEE Trans. AES 2007), in fp64, in this order (p = i's params,
 *     q = j's, each converted to fp64; no fused multiply-add):
 *       da = |l11 l22|_p, wa = da ((|c0| + |c1|) + |c2|)_p, db, wb likewise,
 *       W = wa + wb, fa = wa/W (0.5 if W = 0), fb likewise,
 *       mx = fa px + fb qx, my likewise; ax = px - mx, ay, bx, by likewise,
 *       s11 = fa (l11p l11p + ax ax) + fb (l11q l11q + bx bx),
 *       s21 = fa (l11p l21p + ax ay) + fb (l11q l21q + bx by),
 *       s22 = fa ((l21p l21p + l22p l22p) + ay ay) + fb ((...)q + by by),
 *       dm = s11 s22 - s21 s21;  cost = +inf if not dm > 0, else 0 if W = 0,
 *       else 0.5 (W log dm - wa log(da da) - wb log(db db));
 *   - candidates of i: the other mergeable Gaussians (all params finite, l11
 *     and l22 nonzero) whose cell -- the 16x16 tile of the mean's pixel, the
 *     mean clamped to the image -- is i's or a neighbour (3x3);
 *   - a round: each Gaussian picks its cheapest candidate (ties: the smaller
 *     index); the pairs (i, j), i < j, that pick each other are merged, all of
 *     them or, if more than max_pairs, the max_pairs with the smallest
 *     (fp32 rounding of the cost, i);
 *   - apply: the merged Gaussian (gi_merge_pairs) takes the smaller index's
 *     place, every other Gaussian keeps its params and relative order;
 *   - gi_merge_to: rounds (each asking for at most the count still to remove)
 *     until target is reached or a round finds no pair.
 *   The cost uses the platform's fp64 log on each side of a comparison, so two
 *   costs equal to within an ulp or two could order differently elsewhere; no
 *   other floating-point step decides an index.
 *   n          0 <= n < 2^30 (Cholesky-form params [n][8], device).
 *   workspace  device, >= gi_merge_workspace_bytes(desc, n), 256-byte aligned;
 *              no initialisation needed.  All three calls take a workspace of the
 *              size for their n (gi_merge_to: for the starting n).
 *   gi_merge_round: pairs device int32 [n/2][2] out, 8-byte aligned;
 *              *h_npairs (host) = their count.  Waits for the count.
 *   gi_merge_apply: the n_pairs disjoint pairs (as gi_merge_round writes them)
 *              merged: out device [n - n_pairs][8], not aliasing params.
 *              Asynchronous.
 *   gi_merge_to: out device [n][8] (the first *h_n_out rows are the result), not
 *              aliasing params; *h_rounds (host, may be NULL) = rounds done.
 *              Waits for each round's count.
 */
size_t gi_merge_workspace_bytes(const gi_desc *desc, int64_t n);
gi_status gi_merge_round(const gi_desc *desc, int64_t n, const float *params, int64_t max_pairs, int32_t *pairs,
                         int64_t *h_npairs, void *workspace, size_t workspace_bytes, void *stream);
gi_status gi_merge_apply(const gi_desc *desc, int64_t n, const float *params, int64_t n_pairs, const int32_t *pairs,
                         float *out, void *workspace, size_t workspace_bytes, void *stream);
gi_status gi_merge_to(const gi_desc *desc, int64_t n, const float *params, int64_t target, float *out,
                      int64_t *h_n_out, int32_t *h_rounds, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gi_adc -- adaptive density control ("FlashImgs", Training features: every
 *   300 steps from step 150, dead, out-of-bounds and bloated Gaussians are
 *   relocated to high-error pixels; Library API: Session.densify).  The pages
 *   give no thresholds; the reading (sum mode):
 *   - flags (fp64 decisions): 1 dead -- a non-finite parameter, l11 or l22
 *     zero, or max_k |c_k| < 1/255 (cannot move a pixel by one 8-bit level);
 *     2 out of bounds -- the mean outside [0, W) x [0, H); 4 bloated -- the
 *     larger eigenvalue of Sigma above t = (max(W, H)/16)^2, decided as
 *     not (s11 <= t and s22 <= t and (t - s11)(t - s22) >= s21^2) with
 *     s11 = l11 l11, s21 = l11 l21, s22 = l21 l21 + l22 l22;
 *   - pixel error (fp32): r = target - image, e = fma(r_b, r_b, fma(r_g, r_g,
 *     r_r r_r)), a NaN counting as 0;
 *   - the K = min(#flagged, W H) pixels of largest e (ties: the smaller pixel
 *     index), in ascending pixel index, go to the flagged Gaussians in
 *     ascending index: mean = the pixel centre, l11 = l22 = s0, l21 = 0,
 *     colour = r at the pixel (the Gaussian fills the residual at its centre).
 *   params     device float [n][8], updated in place (sum mode, Cholesky form).
 *   m, v       device float [n][8] or NULL: Adam moments; a relocated
 *              Gaussian's rows are zeroed.
 *   image, target  device float [3][H][W] (the current render and the target).
 *   flags      device int32 [n] out (the flags above, 0 = kept) or NULL.
 *   d_moved    device uint32 [1] out (K) or NULL.
 *   workspace  device, >= gi_adc_workspace_bytes(desc, n), 256-byte aligned;
 *              no initialisation needed.  Asynchronous (no host wait).
 */
size_t gi_adc_workspace_bytes(const gi_desc *desc, int64_t n);
gi_status gi_adc(const gi_desc *desc, int64_t n, float *params, float *m, float *v, const float *image,
                 const float *target, float s0, int32_t *flags, uint32_t *d_moved, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * gi_render_bwd_absgrad -- gi_render_bwd in the sum mode (dparams accumulated,
 *   no loss) that also accumulates each Gaussian's "absgrad" ("Drawing with
 *   Gaussians", 3D densification: the backward accumulates the per-pixel
 *   absolute screen-space mean-gradient contributions, which do not cancel):
 *     dabs[g] += ( sum_p |dL_p/dmux|, sum_p |dL_p/dmuy| )
 *   over the pixels p the Gaussian is summed at, dL_p/dmu being pixel p's term
 *   of dL/dmu (p's own 3 channels).  dparams equals gi_render_bwd's bit for bit.
 *   dabs   device float [n][2], 8-byte aligned, accumulated (+=).
 *   Other arguments as gi_render_bwd (workspace from
 *   gi_render_bwd_workspace_bytes).
 */
gi_status gi_render_bwd_absgrad(const gi_desc *desc, int64_t n, const float *records, const uint16_t *pixbox,
                                const uint32_t *offsets, const uint32_t *ranges, const uint32_t *tile_order,
                                const uint32_t *vals, int64_t capacity, const float *dL_dimage, float *dparams,
                                float *dabs, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gi_render_fwd_alpha_l2 -- gi_render_fwd in the alpha mode that also writes
 *   the L2 loss gradient dL/dI = 2 (I - T) / (3HW) (what gi_loss_l2 writes,
 *   bit for bit) and each tile's sum of squared residuals to loss_partials
 *   ("Drawing with Gaussians", Overview: fused kernels for the alpha
 *   compositing fit; "FlashImgs", --loss l2).
 *   target, dL_dimage  device float [3][H][W] (dL_dimage written; no aliasing).
 *   loss_partials      device float [gi_num_tiles] (written).
 *   Other arguments as gi_render_fwd (alpha mode).
 */
gi_status gi_render_fwd_alpha_l2(const gi_desc *desc, int64_t n, const float *records, const float *opacity,
                                 const uint16_t *pixbox, const uint32_t *ranges, const uint32_t *tile_order,
                                 const uint32_t *vals, const float *background, const float *target, float *image,
                                 float *t_final, uint32_t *last, float *dL_dimage, float *loss_partials,
                                 void *stream);

/*
 * gi_adam_step_pairs_alpha -- the alpha mode's update in one pass: the
 *   per-pair slots that gi_render_bwd (alpha, dparams = NULL) left in its
 *   workspace are added per Gaussian in emission order and mapped to the
 *   gradient (as its gather does, with the records' rows formed from p) and
 *   the Adam step (as gi_adam_step) applied to the 8 params and the logit
 *   of every Gaussian, and to the background's 3 channels from the tiles'
 *   background partials; d_loss (optional) also gets the loss of
 *   gi_render_fwd_alpha_l2's partials (as gi_loss_reduce).
 *   p, m, v              device float [n][8];  lr host float [8].
 *   logit, m_logit, v_logit  device float [n];  lr_logit.
 *   background, m_bg, v_bg   device float [3] (at least);  lr_bg.
 *   Other arguments as gi_adam_step_pairs.  A binning overflow gives zero gradients.
 */
gi_status gi_adam_step_pairs_alpha(const gi_desc *desc, int64_t n, const uint32_t *offsets, int64_t capacity,
                                   const void *workspace, size_t workspace_bytes, float *p, float *m, float *v,
                                   const float *lr, float *logit, float *m_logit, float *v_logit, float lr_logit,
                                   float *background, float *m_bg, float *v_bg, float lr_bg, double beta1,
                                   double beta2, double eps, int32_t step, const float *loss_partials,
                                   int64_t loss_count, float *d_loss, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GI_H */
