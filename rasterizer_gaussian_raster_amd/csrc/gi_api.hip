// gi_api.hip -- the extern "C" entry points declared in include/gi.h: argument
// checks, launch of the gfx950 kernels on the caller's stream, status codes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "../../include/gi.h"
#include "gi_launch.hpp"

namespace {

constexpr int kMaxDim = 32768;
// Gaussians per call: the update kernels index up to 8 lanes and 4 float4 per Gaussian in 32-bit
// arithmetic, which stays in range below 2^27 Gaussians.
constexpr int64_t kMaxGaussians = 1ll << 27;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

bool desc_ok(const gi_desc *d) {
    return d && d->width >= 1 && d->height >= 1 && d->width <= kMaxDim && d->height <= kMaxDim &&
           (d->mode == GI_MODE_SUM || d->mode == GI_MODE_ALPHA) && d->reserved == 0;
}

gi_status hip_status(hipError_t e) { return e == hipSuccess ? GI_OK : GI_ERR_HIP; }

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char *gi_status_string(gi_status s) {
    switch (s) {
    case GI_OK: return "GI_OK";
    case GI_ERR_INVALID_ARG: return "GI_ERR_INVALID_ARG";
    case GI_ERR_HIP: return "GI_ERR_HIP";
    case GI_ERR_CAPACITY: return "GI_ERR_CAPACITY";
    case GI_ERR_UNSUPPORTED: return "GI_ERR_UNSUPPORTED";
    default: return "GI_UNKNOWN_STATUS";
    }
}

const char *gi_version(void) { return "gi 1.0 gfx950"; }

int64_t gi_num_tiles(const gi_desc *desc) {
    if (!desc_ok(desc)) return 0;
    return (int64_t)((desc->width + 15) / 16) * ((desc->height + 15) / 16);
}

}  // extern "C"

namespace {
bool preprocess_args_ok(const gi_desc *desc, int64_t n, const float *params, const float *logit,
                        const float *records, const float *opacity, const uint16_t *pixbox, const uint32_t *counts) {
    if (!desc_ok(desc) || n < 0 || n >= kMaxGaussians) return false;
    const bool alpha = desc->mode == GI_MODE_ALPHA;
    if (n > 0) {
        if (!params || !records || !pixbox || !counts) return false;
        if (!aligned16(params) || !aligned16(records) || !aligned16(pixbox) || !aligned16(counts)) return false;
        if (alpha != (logit != nullptr) || alpha != (opacity != nullptr)) return false;
    }
    return true;
}

bool bin_args_ok(const gi_desc *desc, int64_t n, const uint16_t *pixbox, const uint32_t *counts,
                 const uint32_t *offsets, const uint32_t *keys, const uint32_t *vals, const uint32_t *ranges,
                 int64_t capacity, const uint32_t *d_num, const void *workspace, size_t workspace_bytes) {
    if (!desc_ok(desc) || n < 0 || n >= kMaxGaussians || capacity < 0 || capacity >= (1ll << 31)) return false;
    if (!offsets || !ranges || !d_num || !workspace || !aligned256(workspace)) return false;
    if (n > 0 && (!pixbox || !counts)) return false;
    if (capacity > 0 && (!keys || !vals)) return false;
    return workspace_bytes >= gi::make_bin_plan((int)n, desc->width, desc->height, capacity).bytes;
}

// M back to the host (one wait on the stream) and the overflow status.
gi_status read_total(const void *workspace, int64_t capacity, int64_t *h_num, hipStream_t s) {
    unsigned long long total = 0;
    hipError_t e = hipMemcpyAsync(&total, gi::bin_total_ptr(workspace), sizeof(total), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return GI_ERR_HIP;
    *h_num = (int64_t)total;
    return (int64_t)total > capacity ? GI_ERR_CAPACITY : GI_OK;
}
}  // namespace

extern "C" {

gi_status gi_preprocess(const gi_desc *desc, int64_t n, const float *params, const float *logit, float *records,
                        float *opacity, uint16_t *pixbox, uint32_t *counts, void *stream) {
    if (!preprocess_args_ok(desc, n, params, logit, records, opacity, pixbox, counts)) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_preprocess((int)n, desc->width, desc->height, params, logit, records, opacity,
                                            pixbox, counts, nullptr, nullptr, gi::BinHist{}, as_stream(stream)));
}

size_t gi_bin_sort_workspace_bytes(const gi_desc *desc, int64_t n, int64_t capacity) {
    if (!desc_ok(desc) || n < 0 || n >= kMaxGaussians || capacity < 0 || capacity >= (1ll << 31)) return 0;
    return gi::make_bin_plan((int)n, desc->width, desc->height, capacity).bytes;
}

gi_status gi_bin_sort(const gi_desc *desc, int64_t n, const uint16_t *pixbox, const uint32_t *counts,
                      uint32_t *offsets, uint32_t *keys, uint32_t *vals, uint32_t *ranges, uint32_t *tile_order,
                      int64_t capacity, uint32_t *d_num, int64_t *h_num, void *workspace, size_t workspace_bytes,
                      void *stream) {
    if (!bin_args_ok(desc, n, pixbox, counts, offsets, keys, vals, ranges, capacity, d_num, workspace,
                     workspace_bytes))
        return GI_ERR_INVALID_ARG;
    const gi::BinPlan plan = gi::make_bin_plan((int)n, desc->width, desc->height, capacity);
    hipStream_t s = as_stream(stream);
    if (gi::launch_bin_sort(plan, pixbox, counts, offsets, keys, vals, ranges, tile_order, d_num, workspace, s) !=
        hipSuccess)
        return GI_ERR_HIP;
    return h_num ? read_total(workspace, capacity, h_num, s) : GI_OK;
}

gi_status gi_preprocess_bin_sort(const gi_desc *desc, int64_t n, const float *params, const float *logit,
                                 float *records, float *opacity, uint16_t *pixbox, uint32_t *counts,
                                 uint32_t *offsets, uint32_t *keys, uint32_t *vals, uint32_t *ranges,
                                 uint32_t *tile_order, int64_t capacity, uint32_t *d_num, int64_t *h_num,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    if (!preprocess_args_ok(desc, n, params, logit, records, opacity, pixbox, counts) ||
        !bin_args_ok(desc, n, pixbox, counts, offsets, keys, vals, ranges, capacity, d_num, workspace,
                     workspace_bytes))
        return GI_ERR_INVALID_ARG;
    const gi::BinPlan plan = gi::make_bin_plan((int)n, desc->width, desc->height, capacity);
    hipStream_t s = as_stream(stream);
    hipError_t e = gi::launch_preprocess((int)n, desc->width, desc->height, params, logit, records, opacity,
                                         pixbox, counts, gi::bin_group_sums(plan, workspace), ranges,
                                         gi::bin_hist(plan, workspace), s);
    if (e == hipSuccess)
        e = gi::launch_bin_sort(plan, pixbox, counts, offsets, keys, vals, ranges, tile_order, d_num, workspace, s,
                                true);
    if (e != hipSuccess) return GI_ERR_HIP;
    return h_num ? read_total(workspace, capacity, h_num, s) : GI_OK;
}

}  // extern "C"

namespace {

// gi_render_image's arguments other than the workspace.
bool render_image_args_ok(const gi_desc *desc, int64_t n, const float *params, const float *logit,
                          const float *background, const float *records, const float *opacity,
                          const uint16_t *pixbox, const uint32_t *counts, const uint32_t *tile_order, uint32_t flags,
                          const float *image, const float *t_final, const uint32_t *last) {
    if (!preprocess_args_ok(desc, n, params, logit, records, opacity, pixbox, counts)) return false;
    if ((flags & ~(uint32_t)(GI_FIT_ORDER | GI_FIT_USE_ORDER)) != 0u) return false;
    if ((flags & (GI_FIT_ORDER | GI_FIT_USE_ORDER)) && !tile_order) return false;
    if (!image || !aligned16(image)) return false;
    const bool alpha = desc->mode == GI_MODE_ALPHA;
    if (alpha && (!background || !t_final || !last)) return false;
    if (!alpha && (background || t_final || last)) return false;
    return true;
}

// The work of gi_render_image on checked arguments, with the bin workspace at `workspace`.
gi_status render_image_run(const gi_desc *desc, int64_t n, const float *params, const float *logit,
                           const float *background, float *records, float *opacity, uint16_t *pixbox,
                           uint32_t *counts, uint32_t *offsets, uint32_t *keys, uint32_t *vals, uint32_t *ranges,
                           uint32_t *tile_order, uint32_t flags, int64_t capacity, uint32_t *d_num, int64_t *h_num,
                           void *workspace, float *image, float *t_final, uint32_t *last, void *stream) {
    const bool alpha = desc->mode == GI_MODE_ALPHA;
    const int W = desc->width, H = desc->height;
    const gi::BinPlan plan = gi::make_bin_plan((int)n, W, H, capacity);
    hipStream_t s = as_stream(stream);
    const uint32_t *order = (flags & GI_FIT_USE_ORDER) ? tile_order : nullptr;
    // sum mode with buckets of at most 16 tiles: the raster finishes the sort (no bucket pass)
    const bool bucket = !alpha && gi::bucket_list_mode(plan);
    hipError_t e = gi::launch_preprocess((int)n, W, H, params, logit, records, opacity, pixbox, counts,
                                         gi::bin_group_sums(plan, workspace), ranges,
                                         gi::bin_hist(plan, workspace), s);
    if (e == hipSuccess)
        e = gi::launch_bin_sort(plan, pixbox, counts, offsets, keys, vals, ranges,
                                (!bucket && (flags & GI_FIT_ORDER)) ? tile_order : nullptr, d_num, workspace, s,
                                true, bucket);
    if (e == hipSuccess) {
        if (alpha) {
            e = gi::launch_render_alpha_fwd(W, H, records, opacity, pixbox, ranges, order, vals, background, image,
                                            t_final, last, s);
        } else {
            const gi::BucketList bl = gi::bin_bucket_list(plan, workspace, keys, vals, ranges);
            e = gi::launch_render_sum_fwd(W, H, records, pixbox, ranges, order, vals, image, nullptr, nullptr,
                                          nullptr, s, bucket ? &bl : nullptr);
        }
    }
    if (e == hipSuccess && bucket && (flags & GI_FIT_ORDER)) e = gi::launch_tile_order(plan, ranges, tile_order, s);
    if (e != hipSuccess) return GI_ERR_HIP;
    return h_num ? read_total(workspace, capacity, h_num, s) : GI_OK;
}

// The bin workspace of gi_render_image_noalloc: one file-scope device array, a copy of which every
// GPU the library runs on holds until the process ends.  Its name is a host-side stand-in in host
// code; the address of each device's copy comes from hipGetSymbolAddress, taken once per device
// (with that device current) and kept in scratch_ptr.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on that device).
gi_status scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GI_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GI_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return GI_OK;
}

}  // namespace

extern "C" {

gi_status gi_render_image(const gi_desc *desc, int64_t n, const float *params, const float *logit,
                          const float *background, float *records, float *opacity, uint16_t *pixbox, uint32_t *counts,
                          uint32_t *offsets, uint32_t *keys, uint32_t *vals, uint32_t *ranges, uint32_t *tile_order,
                          uint32_t flags, int64_t capacity, uint32_t *d_num, int64_t *h_num, void *workspace,
                          size_t workspace_bytes, float *image, float *t_final, uint32_t *last, void *stream) {
    if (!render_image_args_ok(desc, n, params, logit, background, records, opacity, pixbox, counts, tile_order, flags,
                              image, t_final, last) ||
        !bin_args_ok(desc, n, pixbox, counts, offsets, keys, vals, ranges, capacity, d_num, workspace,
                     workspace_bytes))
        return GI_ERR_INVALID_ARG;
    return render_image_run(desc, n, params, logit, background, records, opacity, pixbox, counts, offsets, keys, vals,
                            ranges, tile_order, flags, capacity, d_num, h_num, workspace, image, t_final, last,
                            stream);
}

size_t gi_render_image_noalloc_max_bytes(void) { return kScratchBytes; }

gi_status gi_render_image_noalloc(const gi_desc *desc, int64_t n, const float *params, const float *logit,
                                  const float *background, float *records, float *opacity, uint16_t *pixbox,
                                  uint32_t *counts, uint32_t *offsets, uint32_t *keys, uint32_t *vals,
                                  uint32_t *ranges, uint32_t *tile_order, uint32_t flags, int64_t capacity,
                                  uint32_t *d_num, int64_t *h_num, float *image, float *t_final, uint32_t *last,
                                  void *stream) {
    if (!render_image_args_ok(desc, n, params, logit, background, records, opacity, pixbox, counts, tile_order, flags,
                              image, t_final, last))
        return GI_ERR_INVALID_ARG;
    if (capacity < 0 || capacity >= (1ll << 31)) return GI_ERR_INVALID_ARG;
    if (gi::make_bin_plan((int)n, desc->width, desc->height, capacity).bytes > kScratchBytes)
        return GI_ERR_UNSUPPORTED;                        // beyond the fixed scratch: checked before any device call
    void *ws = nullptr;
    const gi_status st = scratch_address(&ws);
    if (st != GI_OK) return st;
    if (!bin_args_ok(desc, n, pixbox, counts, offsets, keys, vals, ranges, capacity, d_num, ws, kScratchBytes))
        return GI_ERR_INVALID_ARG;
    return render_image_run(desc, n, params, logit, background, records, opacity, pixbox, counts, offsets, keys, vals,
                            ranges, tile_order, flags, capacity, d_num, h_num, ws, image, t_final, last, stream);
}

gi_status gi_render_fwd(const gi_desc *desc, int64_t n, const float *records, const float *opacity,
                        const uint16_t *pixbox, const uint32_t *ranges, const uint32_t *tile_order,
                        const uint32_t *vals, const float *background, float *image, float *t_final, uint32_t *last,
                        void *stream) {
    if (!desc_ok(desc) || n < 0 || n >= kMaxGaussians) return GI_ERR_INVALID_ARG;
    if (!ranges || !vals || !image || !aligned16(image)) return GI_ERR_INVALID_ARG;
    if (n > 0 && (!records || !pixbox || !aligned16(records))) return GI_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    if (desc->mode == GI_MODE_SUM) {
        if (opacity || background || t_final || last) return GI_ERR_INVALID_ARG;
        return hip_status(gi::launch_render_sum_fwd(desc->width, desc->height, records, pixbox, ranges, tile_order,
                                                    vals, image, nullptr, nullptr, nullptr, s));
    }
    if (!background || !t_final || !last || (n > 0 && !opacity)) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_render_alpha_fwd(desc->width, desc->height, records, opacity, pixbox, ranges,
                                                  tile_order, vals, background, image, t_final, last, s));
}

gi_status gi_render_fwd_l2(const gi_desc *desc, int64_t n, const float *records, const uint16_t *pixbox,
                           const uint32_t *ranges, const uint32_t *tile_order, const uint32_t *vals,
                           const float *target, float *image, float *dL_dimage, float *loss_partials,
                           void *stream) {
    if (!desc_ok(desc) || desc->mode != GI_MODE_SUM || n < 0 || n >= kMaxGaussians) return GI_ERR_INVALID_ARG;
    if (!ranges || !vals || !image || !target || !dL_dimage || !loss_partials || !aligned16(image))
        return GI_ERR_INVALID_ARG;
    if (n > 0 && (!records || !pixbox || !aligned16(records))) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_render_sum_fwd(desc->width, desc->height, records, pixbox, ranges, tile_order,
                                                vals, image, target, dL_dimage, loss_partials, as_stream(stream)));
}

gi_status gi_loss_reduce(int64_t nparts, const float *loss_partials, int64_t count, float *d_loss, void *stream) {
    if (nparts < 1 || nparts >= (1ll << 31) || count < 1 || !loss_partials || !d_loss) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_loss_reduce((int)nparts, loss_partials, count, d_loss, as_stream(stream)));
}

size_t gi_render_bwd_workspace_bytes(const gi_desc *desc, int64_t n, int64_t capacity) {
    if (!desc_ok(desc) || n < 0 || n >= kMaxGaussians || capacity < 0 || capacity >= (1ll << 31)) return 0;
    if (desc->mode == GI_MODE_ALPHA) return gi::alpha_bwd_workspace_bytes(desc->width, desc->height, n, capacity);
    return gi::make_bwd_plan(desc->width, desc->height, capacity).bytes;
}

gi_status gi_render_bwd(const gi_desc *desc, int64_t n, const float *records, const float *opacity,
                        const float *logit, const uint16_t *pixbox, const uint32_t *offsets,
                        const uint32_t *ranges, const uint32_t *tile_order, const uint32_t *vals, int64_t capacity,
                        const float *background, const float *t_final, const uint32_t *last,
                        const float *dL_dimage, float *dparams, float *dlogit, float *dbackground,
                        const float *loss_partials, int64_t loss_count, float *d_loss,
                        void *workspace, size_t workspace_bytes, void *stream) {
    if (!desc_ok(desc) || n < 0 || n >= kMaxGaussians || capacity < 0 || capacity >= (1ll << 31))
        return GI_ERR_INVALID_ARG;
    if (d_loss && (desc->mode != GI_MODE_SUM || !loss_partials || loss_count < 1)) return GI_ERR_INVALID_ARG;
    if (!offsets || !ranges || !vals || !dL_dimage || !workspace || !aligned256(workspace))
        return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::make_bwd_plan(desc->width, desc->height, capacity).bytes) return GI_ERR_INVALID_ARG;
    if (n > 0 && (!records || !pixbox || !aligned16(records) || (dparams && !aligned16(dparams))))
        return GI_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    const int W = desc->width, H = desc->height;
    const int ntiles = (int)gi_num_tiles(desc);
    hipError_t e;
    if (desc->mode == GI_MODE_SUM) {
        if (opacity || logit || background || t_final || last || dlogit || dbackground) return GI_ERR_INVALID_ARG;
        e = gi::launch_render_sum_bwd(W, H, records, pixbox, offsets, ranges, tile_order, vals, capacity, dL_dimage,
                                      workspace, loss_partials, loss_count, d_loss, s);
        if (e == hipSuccess && dparams)
            e = gi::launch_grad_gather((int)n, W, H, ntiles, offsets, capacity, workspace, records, 0, dparams, nullptr,
                                       nullptr, s);
        return hip_status(e);
    }
    if (!background || !t_final || !last || (n > 0 && (!opacity || !logit))) return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::alpha_bwd_workspace_bytes(W, H, n, capacity)) return GI_ERR_INVALID_ARG;
    e = gi::launch_render_alpha_bwd(W, H, n, records, opacity, logit, pixbox, offsets, ranges, tile_order, vals,
                                    capacity, background, t_final, last, dL_dimage, workspace, s);
    if (e == hipSuccess && dparams)               // dparams = NULL: the slots stay for gi_adam_step_pairs_alpha
        e = gi::launch_grad_gather((int)n, W, H, ntiles, offsets, capacity, workspace, records, 1, dparams, dlogit,
                                   dbackground, s);
    return hip_status(e);
}

gi_status gi_render_fwd_bwd_l2(const gi_desc *desc, int64_t n, const float *records, const uint16_t *pixbox,
                               const uint32_t *offsets, const uint32_t *ranges, const uint32_t *tile_order,
                               const uint32_t *vals, int64_t capacity, const float *target, float *image,
                               float *dL_dimage, float *loss_partials, void *workspace, size_t workspace_bytes,
                               void *stream) {
    if (!desc_ok(desc) || desc->mode != GI_MODE_SUM || n < 0 || n >= kMaxGaussians || capacity < 0 ||
        capacity >= (1ll << 31))
        return GI_ERR_INVALID_ARG;
    if (!offsets || !ranges || !vals || !target || !image || !loss_partials || !aligned16(image) || !workspace ||
        !aligned256(workspace))
        return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::make_bwd_plan(desc->width, desc->height, capacity).bytes) return GI_ERR_INVALID_ARG;
    if (n > 0 && (!records || !pixbox || !aligned16(records))) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_render_sum_fused(desc->width, desc->height, records, pixbox, offsets, ranges,
                                                  tile_order, vals, capacity, image, target, dL_dimage,
                                                  loss_partials, workspace, as_stream(stream)));
}

namespace {
// The SSIM loss of gi_fit_step_sum_ssim (NULL: the L2 loss of gi_fit_step_sum).
struct FitSsim {
    float w1, w2, ws;
    float *dL;
    void *workspace;
    size_t workspace_bytes;
};

gi_status fit_step_sum(const gi_desc *desc, int64_t n, const gi_fit_buffers *b, const gi_adam_hparams *hp,
                       int32_t step, const int32_t *d_step, uint32_t flags, void *stream, const FitSsim *ssim) {
    if (!desc_ok(desc) || desc->mode != GI_MODE_SUM || !b || n < 0 || n >= kMaxGaussians) return GI_ERR_INVALID_ARG;
    if ((flags & ~(uint32_t)(GI_FIT_PREPARED | GI_FIT_ORDER | GI_FIT_USE_ORDER | GI_FIT_NO_UPDATE |
                             GI_FIT_TRACK_MAX)) != 0u)
        return GI_ERR_INVALID_ARG;
    const bool update = !(flags & GI_FIT_NO_UPDATE);
    if (update) {                                         // hp is only read by the update pass
        if (!hp || (!d_step && step < 1)) return GI_ERR_INVALID_ARG;
        if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !(hp->eps >= 0.0))
            return GI_ERR_INVALID_ARG;
    }
    if (!preprocess_args_ok(desc, n, b->params, nullptr, b->records, nullptr, b->pixbox, b->counts) ||
        !bin_args_ok(desc, n, b->pixbox, b->counts, b->offsets, b->keys, b->vals, b->ranges, b->capacity, b->d_num,
                     b->bin_workspace, b->bin_workspace_bytes))
        return GI_ERR_INVALID_ARG;
    if ((flags & (GI_FIT_ORDER | GI_FIT_USE_ORDER)) && !b->tile_order) return GI_ERR_INVALID_ARG;
    if (!b->target || !b->image || !aligned16(b->image) || (!ssim && !b->loss_partials) || !b->bwd_workspace ||
        !aligned256(b->bwd_workspace))
        return GI_ERR_INVALID_ARG;
    const int W = desc->width, H = desc->height;
    if (b->bwd_workspace_bytes < gi::make_bwd_plan(W, H, b->capacity).bytes) return GI_ERR_INVALID_ARG;
    if (ssim) {
        if (!std::isfinite(ssim->w1) || !std::isfinite(ssim->w2) || !std::isfinite(ssim->ws)) return GI_ERR_INVALID_ARG;
        if (!ssim->dL || !aligned16(ssim->dL) || ssim->dL == b->image || ssim->dL == b->target ||
            !ssim->workspace || !aligned256(ssim->workspace) ||
            ssim->workspace_bytes < gi::ssim_workspace_bytes(W, H))
            return GI_ERR_INVALID_ARG;
    }
    if (update && n > 0 && (!b->m || !b->v || !aligned16(b->m) || !aligned16(b->v))) return GI_ERR_INVALID_ARG;
    const gi::BinPlan plan = gi::make_bin_plan((int)n, W, H, b->capacity);
    const gi::BinHist hist = gi::bin_hist(plan, b->bin_workspace);
    unsigned long long *groups = gi::bin_group_sums(plan, b->bin_workspace);
    hipStream_t s = as_stream(stream);
    hipError_t e = hipSuccess;
    if (!(flags & GI_FIT_PREPARED))
        e = gi::launch_preprocess((int)n, W, H, b->params, nullptr, b->records, nullptr, b->pixbox, b->counts, groups,
                                  b->ranges, hist, s);
    // Buckets of at most 16 tiles: the raster's workgroups finish the sort themselves (each picks its
    // tile's entries out of its bucket), so the bucket pass is not launched; the tile order, when
    // asked for, is then formed after the raster from the ranges it wrote.
    const bool bucket = gi::bucket_list_mode(plan);
    const uint32_t *order = (flags & GI_FIT_USE_ORDER) ? b->tile_order : nullptr;
    if (e == hipSuccess)
        e = gi::launch_bin_sort(plan, b->pixbox, b->counts, b->offsets, b->keys, b->vals, b->ranges,
                                (!bucket && (flags & GI_FIT_ORDER)) ? b->tile_order : nullptr, b->d_num,
                                b->bin_workspace, s, true, bucket, (flags & GI_FIT_TRACK_MAX) ? b->d_num + 1 : nullptr);
    if (e == hipSuccess) {
        const gi::BucketList bl = gi::bin_bucket_list(plan, b->bin_workspace, b->keys, b->vals, b->ranges);
        if (!ssim) {
            e = gi::launch_render_sum_fused(W, H, b->records, b->pixbox, b->offsets, b->ranges, order, b->vals,
                                            b->capacity, b->image, b->target, nullptr, b->loss_partials,
                                            b->bwd_workspace, s, bucket ? &bl : nullptr);
        } else {
            // the SSIM gradient needs the whole image: forward (finishing the sort), the loss, backward
            e = gi::launch_render_sum_fwd(W, H, b->records, b->pixbox, b->ranges, order, b->vals, b->image, nullptr,
                                          nullptr, nullptr, s, bucket ? &bl : nullptr);
            if (e == hipSuccess)
                e = gi::launch_loss_ssim(W, H, b->image, b->target, ssim->w1, ssim->w2, ssim->ws, ssim->dL, b->d_loss,
                                         ssim->workspace, true, s);
            if (e == hipSuccess)
                e = gi::launch_render_sum_bwd(W, H, b->records, b->pixbox, b->offsets, b->ranges, order, b->vals,
                                              b->capacity, ssim->dL, b->bwd_workspace, nullptr, 0, nullptr, s);
        }
    }
    if (e == hipSuccess && bucket && (flags & GI_FIT_ORDER)) e = gi::launch_tile_order(plan, b->ranges, b->tile_order, s);
    if (e == hipSuccess && update)
        e = gi::launch_adam_preprocess((int)n, W, H, b->offsets, b->capacity, b->bwd_workspace, b->params, b->m, b->v,
                                       gi::make_adam_hp(hp->lr, hp->beta1, hp->beta2, hp->eps, step, d_step),
                                       b->records, b->pixbox, b->counts, groups, b->ranges, hist,
                                       ssim ? nullptr : b->loss_partials, 3ll * W * H, ssim ? nullptr : b->d_loss, s);
    return hip_status(e);
}
}  // namespace

gi_status gi_fit_step_sum(const gi_desc *desc, int64_t n, const gi_fit_buffers *b, const gi_adam_hparams *hp,
                          int32_t step, const int32_t *d_step, uint32_t flags, void *stream) {
    return fit_step_sum(desc, n, b, hp, step, d_step, flags, stream, nullptr);
}

gi_status gi_fit_step_sum_ssim(const gi_desc *desc, int64_t n, const gi_fit_buffers *b, const gi_adam_hparams *hp,
                               float w1, float w2, float ws, float *dL_dimage, void *ssim_workspace,
                               size_t ssim_workspace_bytes, int32_t step, const int32_t *d_step, uint32_t flags,
                               void *stream) {
    const FitSsim f{w1, w2, ws, dL_dimage, ssim_workspace, ssim_workspace_bytes};
    return fit_step_sum(desc, n, b, hp, step, d_step, flags, stream, &f);
}

size_t gi_loss_workspace_bytes(int64_t count) { return count < 1 ? 0 : gi::loss_workspace_bytes(count); }

gi_status gi_loss_l2(int64_t count, const float *image, const float *target, float *dL_dimage, float *d_loss,
                     void *workspace, size_t workspace_bytes, void *stream) {
    if (count < 1 || !image || !target || !workspace) return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::loss_workspace_bytes(count) || (reinterpret_cast<uintptr_t>(workspace) & 7u))
        return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_loss_l2(count, image, target, dL_dimage, d_loss, workspace, as_stream(stream)));
}

gi_status gi_adam_step_pairs(const gi_desc *desc, int64_t n, const uint32_t *offsets, int64_t capacity,
                             const void *workspace, size_t workspace_bytes, float *p, float *m, float *v,
                             const float *lr, double beta1, double beta2, double eps, int32_t step,
                             const int32_t *d_step, const float *loss_partials, int64_t loss_count, float *d_loss,
                             void *stream) {
    if (!desc_ok(desc) || desc->mode != GI_MODE_SUM || n < 0 || n >= kMaxGaussians || capacity < 0 ||
        capacity >= (1ll << 31) || (!d_step && step < 1) || !lr)
        return GI_ERR_INVALID_ARG;
    if (d_loss && (!loss_partials || loss_count < 1)) return GI_ERR_INVALID_ARG;
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps >= 0.0)) return GI_ERR_INVALID_ARG;
    if (!offsets || !workspace || !aligned256(workspace)) return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::make_bwd_plan(desc->width, desc->height, capacity).bytes) return GI_ERR_INVALID_ARG;
    if (n > 0 && (!p || !m || !v || !aligned16(p) || !aligned16(m) || !aligned16(v))) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_adam_pairs((int)n, desc->width, desc->height, offsets, capacity, workspace, p, m, v,
                                            lr, beta1, beta2, eps, step, d_step, loss_partials, loss_count,
                                            d_loss, as_stream(stream)));
}

gi_status gi_adam_step(int64_t rows, int32_t row_len, float *p, float *g, float *m, float *v, const float *lr,
                       double beta1, double beta2, double eps, int32_t step, int32_t zero_grad, void *stream) {
    if (rows < 0 || row_len < 1 || row_len > 16 || step < 1 || !lr) return GI_ERR_INVALID_ARG;
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps >= 0.0))
        return GI_ERR_INVALID_ARG;
    if (rows > 0) {
        if (!p || !g || !m || !v) return GI_ERR_INVALID_ARG;
        if (row_len % 4 == 0 && (!aligned16(p) || !aligned16(g) || !aligned16(m) || !aligned16(v)))
            return GI_ERR_INVALID_ARG;
    }
    return hip_status(gi::launch_adam(rows, row_len, p, g, m, v, lr, beta1, beta2, eps, step, zero_grad,
                                      as_stream(stream)));
}

gi_status gi_params_to_cholesky(int32_t kind, int64_t n, const float *params, float fx, float fy, float *out,
                                void *stream) {
    if ((kind != GI_PARAMS_CHOLESKY && kind != GI_PARAMS_RS) || n < 0) return GI_ERR_INVALID_ARG;
    if (!(fx > 0.0f) || !(fy > 0.0f) || !std::isfinite(fx) || !std::isfinite(fy)) return GI_ERR_INVALID_ARG;
    if (n > 0) {
        if (!params || !out || !aligned16(params) || !aligned16(out)) return GI_ERR_INVALID_ARG;
        if (kind == GI_PARAMS_RS && params == out) return GI_ERR_INVALID_ARG;
    }
    return hip_status(gi::launch_params_to_cholesky(kind, n, params, fx, fy, out, as_stream(stream)));
}

gi_status gi_params_to_cholesky_grad(int32_t kind, int64_t n, const float *params, float fx, float fy,
                                     const float *dout, float *dparams, int32_t accumulate, void *stream) {
    if ((kind != GI_PARAMS_CHOLESKY && kind != GI_PARAMS_RS) || n < 0) return GI_ERR_INVALID_ARG;
    if (!(fx > 0.0f) || !(fy > 0.0f) || !std::isfinite(fx) || !std::isfinite(fy)) return GI_ERR_INVALID_ARG;
    if (n > 0) {
        if (!params || !dout || !dparams || !aligned16(params) || !aligned16(dout) || !aligned16(dparams))
            return GI_ERR_INVALID_ARG;
        if (dparams == params) return GI_ERR_INVALID_ARG;
    }
    return hip_status(gi::launch_params_to_cholesky_grad(kind, n, params, fx, fy, dout, dparams, accumulate != 0,
                                                         as_stream(stream)));
}

gi_status gi_grad_gather(const gi_desc *desc, int32_t kind, int64_t n, const float *params, float fx, float fy,
                         const float *records, const uint32_t *offsets, int64_t capacity, const void *workspace,
                         size_t workspace_bytes, float *dparams, void *stream) {
    if (!desc_ok(desc) || (kind != GI_PARAMS_CHOLESKY && kind != GI_PARAMS_RS) || n < 0 || n >= kMaxGaussians ||
        capacity < 0 || capacity >= (1ll << 31))
        return GI_ERR_INVALID_ARG;
    if (!(fx > 0.0f) || !(fy > 0.0f) || !std::isfinite(fx) || !std::isfinite(fy)) return GI_ERR_INVALID_ARG;
    if (!offsets || !workspace || !aligned256(workspace)) return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::make_bwd_plan(desc->width, desc->height, capacity).bytes) return GI_ERR_INVALID_ARG;
    if (n > 0 && (!params || !records || !dparams || !aligned16(params) || !aligned16(records) ||
                  !aligned16(dparams) || dparams == params))
        return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_grad_gather_params(kind, (int)n, desc->width, desc->height, params, fx, fy, records,
                                                    offsets, capacity, workspace, dparams, as_stream(stream)));
}

size_t gi_loss_ssim_workspace_bytes(int32_t width, int32_t height) {
    if (width < 1 || height < 1 || width > kMaxDim || height > kMaxDim) return 0;
    return gi::ssim_workspace_bytes(width, height);
}

gi_status gi_loss_ssim_target(int32_t width, int32_t height, const float *target, void *workspace,
                              size_t workspace_bytes, void *stream) {
    if (width < 1 || height < 1 || width > kMaxDim || height > kMaxDim) return GI_ERR_INVALID_ARG;
    if (!target || !workspace || !aligned256(workspace)) return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::ssim_workspace_bytes(width, height)) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_ssim_target(width, height, target, workspace, as_stream(stream)));
}

gi_status gi_loss_ssim(int32_t width, int32_t height, const float *image, const float *target, float w1, float w2,
                       float ws, float *dL_dimage, float *d_loss, void *workspace, size_t workspace_bytes,
                       uint32_t flags, void *stream) {
    if (width < 1 || height < 1 || width > kMaxDim || height > kMaxDim) return GI_ERR_INVALID_ARG;
    if (!std::isfinite(w1) || !std::isfinite(w2) || !std::isfinite(ws)) return GI_ERR_INVALID_ARG;
    if (!image || !target || !dL_dimage || !workspace || !aligned256(workspace)) return GI_ERR_INVALID_ARG;
    if (flags & ~GI_SSIM_TARGET_PREPARED) return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::ssim_workspace_bytes(width, height)) return GI_ERR_INVALID_ARG;
    if (dL_dimage == image || dL_dimage == target) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_loss_ssim(width, height, image, target, w1, w2, ws, dL_dimage, d_loss, workspace,
                                           (flags & GI_SSIM_TARGET_PREPARED) != 0, as_stream(stream)));
}

gi_status gi_adam_step_pairs_rs(const gi_desc *desc, int64_t n, const uint32_t *offsets, int64_t capacity,
                                const void *workspace, size_t workspace_bytes, float *p, float *m, float *v,
                                const float *lr, double beta1, double beta2, double eps, int32_t step,
                                const float *loss_partials, int64_t loss_count, float *d_loss, float *chol_out,
                                void *stream) {
    if (!desc_ok(desc) || desc->mode != GI_MODE_SUM || n < 0 || n >= kMaxGaussians || capacity < 0 ||
        capacity >= (1ll << 31) || step < 1 || !lr)
        return GI_ERR_INVALID_ARG;
    if (d_loss && (!loss_partials || loss_count < 1)) return GI_ERR_INVALID_ARG;
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps >= 0.0)) return GI_ERR_INVALID_ARG;
    if (!offsets || !workspace || !aligned256(workspace)) return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::make_bwd_plan(desc->width, desc->height, capacity).bytes) return GI_ERR_INVALID_ARG;
    if (n > 0 && (!p || !m || !v || !aligned16(p) || !aligned16(m) || !aligned16(v))) return GI_ERR_INVALID_ARG;
    if (n > 0 && chol_out && (!aligned16(chol_out) || chol_out == p)) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_adam_pairs_rs((int)n, desc->width, desc->height, offsets, capacity, workspace, p, m,
                                               v, lr, beta1, beta2, eps, step, loss_partials, loss_count, d_loss,
                                               chol_out, as_stream(stream)));
}

gi_status gi_merge_pairs(int64_t n_pairs, const int32_t *pairs, int64_t n, const float *params, float *out,
                         void *stream) {
    if (n_pairs < 0 || n < 0 || n >= kMaxGaussians) return GI_ERR_INVALID_ARG;
    if (n_pairs > 0 && (!pairs || !params || !out || !aligned16(params) || !aligned16(out) ||
                        (reinterpret_cast<uintptr_t>(pairs) & 7u) != 0 || out == params))
        return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_merge_pairs(n_pairs, n, params, pairs, out, as_stream(stream)));
}

size_t gi_merge_workspace_bytes(const gi_desc *desc, int64_t n) {
    if (!desc_ok(desc) || n < 0 || n >= (1ll << 30)) return 0;
    return gi::merge_workspace_bytes(desc->width, desc->height, n);
}

namespace {
bool merge_args_ok(const gi_desc *desc, int64_t n, const float *params, const void *workspace,
                   size_t workspace_bytes) {
    if (!desc_ok(desc) || n < 0 || n >= (1ll << 30)) return false;
    if (!workspace || !aligned256(workspace)) return false;
    if (workspace_bytes < gi::merge_workspace_bytes(desc->width, desc->height, n)) return false;
    return n == 0 || (params && aligned16(params));
}

// The count a merge round left in device memory, read back (one wait on the stream).
gi_status read_count(const uint32_t *d_count, int64_t *h, hipStream_t s) {
    uint32_t c = 0;
    hipError_t e = hipMemcpyAsync(&c, d_count, sizeof(c), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return GI_ERR_HIP;
    *h = (int64_t)c;
    return GI_OK;
}
}  // namespace

gi_status gi_merge_round(const gi_desc *desc, int64_t n, const float *params, int64_t max_pairs, int32_t *pairs,
                         int64_t *h_npairs, void *workspace, size_t workspace_bytes, void *stream) {
    if (!merge_args_ok(desc, n, params, workspace, workspace_bytes) || max_pairs < 0 || !h_npairs) return GI_ERR_INVALID_ARG;
    if (n >= 2 && (!pairs || (reinterpret_cast<uintptr_t>(pairs) & 7u))) return GI_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    uint32_t *cnt = gi::merge_count_ptr(workspace, desc->width, desc->height, n);
    int32_t *dst = n >= 2 ? pairs : gi::merge_pairs_buffer(workspace, desc->width, desc->height, n);
    const uint32_t mp = (uint32_t)(max_pairs < n / 2 ? max_pairs : n / 2);
    if (gi::launch_merge_round(desc->width, desc->height, (int)n, (int)n, params, mp, dst, cnt, workspace, s) !=
        hipSuccess)
        return GI_ERR_HIP;
    return read_count(cnt, h_npairs, s);
}

gi_status gi_merge_apply(const gi_desc *desc, int64_t n, const float *params, int64_t n_pairs, const int32_t *pairs,
                         float *out, void *workspace, size_t workspace_bytes, void *stream) {
    if (!merge_args_ok(desc, n, params, workspace, workspace_bytes) || n_pairs < 0 || 2 * n_pairs > n)
        return GI_ERR_INVALID_ARG;
    if (n_pairs > 0 && (!pairs || (reinterpret_cast<uintptr_t>(pairs) & 7u))) return GI_ERR_INVALID_ARG;
    if (n > n_pairs && (!out || !aligned16(out) || out == params)) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_merge_apply((int)n, (int)n, params, n_pairs, pairs, out, workspace, desc->width,
                                             desc->height, as_stream(stream)));
}

gi_status gi_merge_to(const gi_desc *desc, int64_t n, const float *params, int64_t target, float *out,
                      int64_t *h_n_out, int32_t *h_rounds, void *workspace, size_t workspace_bytes, void *stream) {
    if (!merge_args_ok(desc, n, params, workspace, workspace_bytes) || target < 0 || !h_n_out) return GI_ERR_INVALID_ARG;
    if (n > 0 && (!out || !aligned16(out) || out == params)) return GI_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    const int W = desc->width, H = desc->height;
    float *tmp = gi::merge_tmp_params(workspace, W, H, n);
    int32_t *pairs = gi::merge_pairs_buffer(workspace, W, H, n);
    uint32_t *cnt = gi::merge_count_ptr(workspace, W, H, n);
    // rounds alternate between out and tmp; the workspace plan of the first n serves every round
    const float *cur = params;
    float *dst = out;
    int64_t m = n;
    int32_t rounds = 0;
    while (m > target && m >= 2) {
        if (gi::launch_merge_round(W, H, (int)n, (int)m, cur, (uint32_t)((m - target) < m / 2 ? (m - target) : m / 2),
                                   pairs, cnt, workspace, s) != hipSuccess)
            return GI_ERR_HIP;
        int64_t np = 0;
        const gi_status st = read_count(cnt, &np, s);
        if (st != GI_OK) return st;
        if (np == 0) break;
        if (gi::launch_merge_apply((int)n, (int)m, cur, np, pairs, dst, workspace, W, H, s) != hipSuccess)
            return GI_ERR_HIP;
        m -= np;
        ++rounds;
        cur = dst;
        dst = dst == out ? tmp : out;
    }
    if (cur != out && m > 0 &&
        hipMemcpyAsync(out, cur, (size_t)m * 32, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return GI_ERR_HIP;
    *h_n_out = m;
    if (h_rounds) *h_rounds = rounds;
    return GI_OK;
}

size_t gi_adc_workspace_bytes(const gi_desc *desc, int64_t n) {
    if (!desc_ok(desc) || desc->mode != GI_MODE_SUM || n < 0 || n >= kMaxGaussians) return 0;
    return gi::adc_workspace_bytes(desc->width, desc->height, n);
}

gi_status gi_adc(const gi_desc *desc, int64_t n, float *params, float *m, float *v, const float *image,
                 const float *target, float s0, int32_t *flags, uint32_t *d_moved, void *workspace,
                 size_t workspace_bytes, void *stream) {
    if (!desc_ok(desc) || desc->mode != GI_MODE_SUM || n < 0 || n >= kMaxGaussians) return GI_ERR_INVALID_ARG;
    if ((int64_t)desc->width * desc->height >= (1ll << 31)) return GI_ERR_INVALID_ARG;
    if (!std::isfinite(s0) || !image || !target || !workspace || !aligned256(workspace)) return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::adc_workspace_bytes(desc->width, desc->height, n)) return GI_ERR_INVALID_ARG;
    if (n > 0 && (!params || !aligned16(params) || (m && !aligned16(m)) || (v && !aligned16(v))))
        return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_adc(desc->width, desc->height, (int)n, params, m, v, image, target, s0, flags, d_moved,
                                     workspace, as_stream(stream)));
}

gi_status gi_render_bwd_absgrad(const gi_desc *desc, int64_t n, const float *records, const uint16_t *pixbox,
                                const uint32_t *offsets, const uint32_t *ranges, const uint32_t *tile_order,
                                const uint32_t *vals, int64_t capacity, const float *dL_dimage, float *dparams,
                                float *dabs, void *workspace, size_t workspace_bytes, void *stream) {
    if (!desc_ok(desc) || desc->mode != GI_MODE_SUM || n < 0 || n >= kMaxGaussians || capacity < 0 ||
        capacity >= (1ll << 31))
        return GI_ERR_INVALID_ARG;
    if (!offsets || !ranges || !vals || !dL_dimage || !workspace || !aligned256(workspace))
        return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::make_bwd_plan(desc->width, desc->height, capacity).bytes) return GI_ERR_INVALID_ARG;
    if (n > 0 && (!records || !pixbox || !dparams || !dabs || !aligned16(records) || !aligned16(dparams) ||
                  (reinterpret_cast<uintptr_t>(dabs) & 7u) != 0))
        return GI_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    const int W = desc->width, H = desc->height;
    hipError_t e = gi::launch_render_sum_bwd(W, H, records, pixbox, offsets, ranges, tile_order, vals, capacity,
                                             dL_dimage, workspace, nullptr, 0, nullptr, s, true);
    if (e == hipSuccess)
        e = gi::launch_grad_gather((int)n, W, H, (int)gi_num_tiles(desc), offsets, capacity, workspace, records, 0,
                                   dparams,
                                   nullptr, nullptr, s, dabs);
    return hip_status(e);
}

gi_status gi_render_fwd_alpha_l2(const gi_desc *desc, int64_t n, const float *records, const float *opacity,
                                 const uint16_t *pixbox, const uint32_t *ranges, const uint32_t *tile_order,
                                 const uint32_t *vals, const float *background, const float *target, float *image,
                                 float *t_final, uint32_t *last, float *dL_dimage, float *loss_partials,
                                 void *stream) {
    if (!desc_ok(desc) || desc->mode != GI_MODE_ALPHA || n < 0 || n >= kMaxGaussians) return GI_ERR_INVALID_ARG;
    if (!ranges || !vals || !background || !target || !image || !t_final || !last || !dL_dimage || !loss_partials)
        return GI_ERR_INVALID_ARG;
    if (n > 0 && (!records || !opacity || !pixbox || !aligned16(records))) return GI_ERR_INVALID_ARG;
    if (dL_dimage == target || dL_dimage == image) return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_render_alpha_fwd(desc->width, desc->height, records, opacity, pixbox, ranges,
                                                  tile_order, vals, background, image, t_final, last,
                                                  as_stream(stream), target, dL_dimage, loss_partials));
}

gi_status gi_adam_step_pairs_alpha(const gi_desc *desc, int64_t n, const uint32_t *offsets, int64_t capacity,
                                   const void *workspace, size_t workspace_bytes, float *p, float *m, float *v,
                                   const float *lr, float *logit, float *m_logit, float *v_logit, float lr_logit,
                                   float *background, float *m_bg, float *v_bg, float lr_bg, double beta1,
                                   double beta2, double eps, int32_t step, const float *loss_partials,
                                   int64_t loss_count, float *d_loss, void *stream) {
    if (!desc_ok(desc) || desc->mode != GI_MODE_ALPHA || n < 0 || n >= kMaxGaussians || capacity < 0 ||
        capacity >= (1ll << 31) || step < 1 || !lr)
        return GI_ERR_INVALID_ARG;
    if (d_loss && (!loss_partials || loss_count < 1)) return GI_ERR_INVALID_ARG;
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps >= 0.0)) return GI_ERR_INVALID_ARG;
    if (!offsets || !workspace || !aligned256(workspace) || !background || !m_bg || !v_bg) return GI_ERR_INVALID_ARG;
    if (workspace_bytes < gi::make_bwd_plan(desc->width, desc->height, capacity).bytes) return GI_ERR_INVALID_ARG;
    if (n > 0 && (!p || !m || !v || !logit || !m_logit || !v_logit || !aligned16(p) || !aligned16(m) ||
                  !aligned16(v)))
        return GI_ERR_INVALID_ARG;
    return hip_status(gi::launch_adam_pairs_alpha((int)n, desc->width, desc->height, offsets, capacity, workspace, p,
                                                  m, v, lr, logit, m_logit, v_logit, lr_logit, background, m_bg,
                                                  v_bg, lr_bg, beta1, beta2, eps, step, loss_partials, loss_count,
                                                  d_loss, as_stream(stream)));
}

}  // extern "C"
