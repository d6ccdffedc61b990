// gi_launch.hpp -- host-side launchers of the gfx950 kernels (internal to libgi).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gi {

// The binning's first-pass digit histogram, one table column per 256-Gaussian
// segment, written by the kernel that forms the tile counts (table NULL: not
// written; the binning then counts in a kernel of its own).
struct BinHist {
    uint32_t *table;
    int tiles_x, shift, bits;
    int redundant;         // layout [column][digit] (read raw), else [digit][ncols_cap] (scanned)
    int ncols_cap;
};

// Adam hyperparameters as the kernels take them (1 - beta formed in fp64 on the host).
struct AdamHP {
    float lr[8];
    float b1, omb1, b2, omb2, eps;
    double b1d, b2d;                 // for the bias corrections formed on the device (d_step set)
    float bc1, bc2;                  // the corrections for `step`, formed on the host (d_step NULL)
    int step;                        // used when d_step is NULL
    const int32_t *d_step;           // device step count (graph replays), or NULL
};
AdamHP make_adam_hp(const float *lr, double beta1, double beta2, double eps, int step, const int32_t *d_step);

// k_preprocess.hip
// group_sums / ranges (or NULL): the binning's group sums and cleared ranges (gi_preprocess_bin_sort),
// and the digit histogram when hist.table is set.
hipError_t launch_preprocess(int n, int W, int H, const float *params, const float *logit, float *records,
                             float *opacity, uint16_t *pixbox, uint32_t *counts, unsigned long long *group_sums,
                             uint32_t *ranges, BinHist hist, hipStream_t s);

// Adam from the pair slots (as launch_adam_pairs), then the set-up of the updated Gaussians
// for the next binning (as launch_preprocess with group_sums); d_loss: also the loss reduction.
hipError_t launch_adam_preprocess(int n, int W, int H, const uint32_t *offsets, int64_t capacity, const void *bwd_ws,
                                  float *p, float *m, float *v, const AdamHP &a, float *records, uint16_t *pixbox,
                                  uint32_t *counts, unsigned long long *group_sums, uint32_t *ranges, BinHist hist,
                                  const float *loss_partials, int64_t loss_count, float *d_loss, hipStream_t s);

// k_binning.hip
struct BinPlan {
    int n, W, H, tiles_x, ntiles;
    int64_t capacity;
    int order_kind;        // 0: one pass (<= 8 key bits); 1: high digit, then buckets (<= 16); 2: LSD
    int passes;            // sort passes over all pairs (>= 1; a single tile takes one 0-bit pass)
    int bits[4];           // digit width of each pass
    int shift0;            // first pass: digit = (key >> shift0) & (2^bits[0] - 1)
    int lo_bits;           // bucket pass: low digit width (order_kind 1)
    int bucket_lanes;      // bucket pass: keys per lane per chunk (4, 8 or 16)
    int nb_g;              // Gaussian groups of 256
    int redundant_groups;  // group bases summed by each block (no group-scan kernel)
    int seg_groups, nseg;  // groups per first-pass segment, number of segments
    int pass_lanes;        // keys per lane in the later passes' blocks (4, 8 or 16)
    int nbs;               // sort blocks of 256 * pass_lanes keys over the capacity (later passes)
    int ncols_cap[4];      // digit-table columns of each pass
    int table_redundant[4];// digit table read raw by every block (no scan kernel)
    size_t off_part, off_kalt, off_valt, off_table, off_tsp, off_bstart, bytes;
};
BinPlan make_bin_plan(int n, int W, int H, int64_t capacity);
// groups_done: the preprocess kernel already wrote the group sums and cleared the ranges.
// first_pass_only: stop after the first sort pass (bucket_list_mode plans; the raster finishes the sort).
// d_max (or NULL): device running maximum of M, raised to this binning's M.
hipError_t launch_bin_sort(const BinPlan &p, const uint16_t *pixbox, const uint32_t *counts, uint32_t *offsets,
                           uint32_t *keys, uint32_t *vals, uint32_t *ranges, uint32_t *tile_order, uint32_t *d_num,
                           void *ws, hipStream_t s, bool groups_done = false, bool first_pass_only = false,
                           uint32_t *d_max = nullptr);
// The tile order from the ranges (as gi_bin_sort's tile_order).
hipError_t launch_tile_order(const BinPlan &p, const uint32_t *ranges, uint32_t *tile_order, hipStream_t s);

// The second sort pass done by the raster's own workgroups: the first pass left each bucket
// (tiles sharing the high digit) in emission order; tile t's workgroup picks its entries out of
// its bucket and writes them, and its range, where the bucket pass would have.
struct BucketList {
    const uint32_t *kin, *vin;     // first-pass output
    const uint32_t *bstart;        // bucket starts [2^hi + 1]
    const uint32_t *m_eff;         // M, or 0 when nothing was binned
    int lo_bits;
    uint32_t *kout, *vout;         // final keys / vals
    uint32_t *ranges;              // final ranges [T][2]
};
// Plans whose buckets hold at most 16 tiles (MSD order, low digit <= 4 bits).
bool bucket_list_mode(const BinPlan &p);
BucketList bin_bucket_list(const BinPlan &p, void *ws, uint32_t *keys, uint32_t *vals, uint32_t *ranges);
// device address of the group sums inside the bin workspace
unsigned long long *bin_group_sums(const BinPlan &p, void *ws);
// what gi_preprocess_bin_sort's preprocess kernel histograms for the plan (table NULL when the
// plan counts in a kernel of its own)
BinHist bin_hist(const BinPlan &p, void *ws);
// device address of the 64-bit instance total inside the workspace
const void *bin_total_ptr(const void *ws);

// k_raster_sum.hip

hipError_t launch_loss_reduce(int nparts, const float *partials, int64_t count, float *d_loss, hipStream_t s);
// d_loss (or NULL): also reduce the raster pass's per-tile loss partials into it (one more workgroup).
hipError_t launch_adam_pairs(int n, int W, int H, const uint32_t *offsets, int64_t capacity, const void *ws, float *p,
                             float *m, float *v, const float *lr, double beta1, double beta2, double eps, int step,
                             const int32_t *d_step, const float *loss_partials, int64_t loss_count, float *d_loss,
                             hipStream_t s);

// Backward workspace: per (Gaussian, tile) gradient at its emission slot.
struct BwdPlan {
    size_t off_part;    // float4 [capacity][2]: the pair's sums (slot layout: gi_device.hpp)
    size_t off_logit;   // float [capacity]: dlogit (alpha)
    size_t off_bg;      // float4 [ntiles]: dbackground per tile (alpha)
    size_t off_abs;     // float2 [capacity]: sum |d mux|, sum |d muy| over the pair's pixels (absgrad)
    size_t bytes;
};
BwdPlan make_bwd_plan(int W, int H, int64_t capacity);
hipError_t launch_render_sum_bwd(int W, int H, const float *records, const uint16_t *pixbox,
                                 const uint32_t *offsets, const uint32_t *ranges, const uint32_t *order,
                                 const uint32_t *vals, int64_t capacity, const float *dL_dimage, void *ws,
                                 const float *loss_partials, int64_t loss_count, float *d_loss, hipStream_t s,
                                 bool absgrad = false);
// Forward (target: also the L2 gradient and loss partials).  With bl, each tile's list is taken
// from its bucket (and written out) instead of ranges / vals.
hipError_t launch_render_sum_fwd(int W, int H, const float *records, const uint16_t *pixbox,
                                 const uint32_t *ranges, const uint32_t *order, const uint32_t *vals, float *image,
                                 const float *target, float *dL_dimage, float *loss_partials, hipStream_t s,
                                 const BucketList *bl = nullptr);
// Forward with the L2 loss and backward of each tile in one launch (dL_dimage may be NULL).  With
// bl, each tile's list is taken from its bucket (and written out) instead of ranges / vals.
hipError_t launch_render_sum_fused(int W, int H, const float *records, const uint16_t *pixbox,
                                   const uint32_t *offsets, const uint32_t *ranges, const uint32_t *order,
                                   const uint32_t *vals, int64_t capacity, float *image, const float *target,
                                   float *dL_dimage, float *loss_partials, void *ws, hipStream_t s,
                                   const BucketList *bl = nullptr);
// Adds each Gaussian's slots (offsets[g] .. offsets[g+1]) in order to dparams / dlogit, and the
// per-tile background partials to dbackground.
hipError_t launch_grad_gather(int n, int W, int H, int ntiles, const uint32_t *offsets, int64_t capacity,
                              const void *ws, const float *records, int alpha, float *dparams, float *dlogit,
                              float *dbackground, hipStream_t s, float *dabs = nullptr);

// k_raster_alpha.hip
hipError_t launch_render_alpha_fwd(int W, int H, const float *records, const float *opacity,
                                   const uint16_t *pixbox, const uint32_t *ranges, const uint32_t *order,
                                   const uint32_t *vals, const float *background, float *image, float *t_final,
                                   uint32_t *last, hipStream_t s, const float *target = nullptr,
                                   float *dL = nullptr, float *loss_part = nullptr);
hipError_t launch_adam_pairs_alpha(int n, int W, int H, const uint32_t *offsets, int64_t capacity, const void *ws,
                                   float *p, float *m, float *v, const float *lr, float *logit, float *ml, float *vl,
                                   float lr_logit, float *bg, float *mbg, float *vbg, float lr_bg, double beta1,
                                   double beta2, double eps, int step, const float *loss_partials, int64_t loss_count,
                                   float *d_loss, hipStream_t s);
size_t alpha_bwd_workspace_bytes(int W, int H, int64_t n, int64_t capacity);
hipError_t launch_render_alpha_bwd(int W, int H, int64_t n, const float *records, const float *opacity,
                                   const float *logit, const uint16_t *pixbox, const uint32_t *offsets,
                                   const uint32_t *ranges, const uint32_t *order, const uint32_t *vals,
                                   int64_t capacity, const float *background, const float *t_final,
                                   const uint32_t *last, const float *dL_dimage, void *ws, hipStream_t s);

// k_optim.hip
size_t loss_workspace_bytes(int64_t count);
hipError_t launch_loss_l2(int64_t count, const float *image, const float *target, float *dL_dimage, float *d_loss,
                          void *ws, hipStream_t s);
hipError_t launch_adam(int64_t rows, int row_len, float *p, float *g, float *m, float *v, const float *lr,
                       double beta1, double beta2, double eps, int step, int zero_grad, hipStream_t s);

// k_ssim.hip
size_t ssim_workspace_bytes(int W, int H);
hipError_t launch_ssim_target(int W, int H, const float *y, void *ws_ptr, hipStream_t s);
hipError_t launch_loss_ssim(int W, int H, const float *x, const float *y, float w1, float w2, float ws, float *dL,
                            float *loss, void *ws_ptr, bool target_prepared, hipStream_t s);

// k_adapt.hip
hipError_t launch_merge_pairs(int64_t np, int64_t n, const float *params, const int32_t *pairs, float *out,
                              hipStream_t s);
size_t merge_workspace_bytes(int W, int H, int64_t n);
// One merge round: the pairs (ascending smaller index, at most max_pairs) and their count to
// d_count (ws laid out for n_cap >= n Gaussians).
hipError_t launch_merge_round(int W, int H, int n_cap, int n, const float *params, uint32_t max_pairs,
                              int32_t *pairs_out, uint32_t *d_count, void *ws, hipStream_t s);
// params with the disjoint pairs merged, index order kept: out [n - np][8].
hipError_t launch_merge_apply(int n_cap, int n, const float *params, int64_t np, const int32_t *pairs, float *out,
                              void *ws, int W, int H, hipStream_t s);
float *merge_tmp_params(void *ws, int W, int H, int64_t n);       // a second [n][8] params buffer
int32_t *merge_pairs_buffer(void *ws, int W, int H, int64_t n);   // [n/2 + 1][2]
uint32_t *merge_count_ptr(void *ws, int W, int H, int64_t n);     // a device counter
size_t adc_workspace_bytes(int W, int H, int64_t n);
hipError_t launch_adc(int W, int H, int n, float *params, float *m, float *v, const float *image,
                      const float *target, float s0, int32_t *flags_out, uint32_t *d_moved, void *ws, hipStream_t s);
hipError_t launch_params_to_cholesky(int kind, int64_t n, const float *in, float fx, float fy, float *out,
                                     hipStream_t s);
hipError_t launch_params_to_cholesky_grad(int kind, int64_t n, const float *in, float fx, float fy,
                                          const float *dout, float *din, int accumulate, hipStream_t s);
hipError_t launch_adam_pairs_rs(int n, int W, int H, const uint32_t *offsets, int64_t capacity, const void *ws,
                                float *p, float *m, float *v, const float *lr, double beta1, double beta2, double eps,
                                int step, const float *loss_partials, int64_t loss_count, float *d_loss, float *chol,
                                hipStream_t s);
// dparams (+)= the gradient w.r.t. params of form `kind` whose Cholesky form at scale (fx, fy) made
// `records`, from the pair slots the backward left in ws.
hipError_t launch_grad_gather_params(int kind, int n, int W, int H, const float *params, float fx, float fy,
                                     const float *records, const uint32_t *offsets, int64_t capacity, const void *ws,
                                     float *dparams, hipStream_t s);

}  // namespace gi
