// k_preprocess.hip -- per-Gaussian set-up: Cholesky factor -> scaled rows of
// L^-1 (the conic used by the cutoff), 3-sigma pixel box, tile count, opacity.
//
// "GaussianImage" (Overview): 8 parameters per Gaussian (position, Cholesky
// covariance, colour).  fvdb GaussianSplatReconstructionConfig (eps_2d): the
// screen-space box is padded by a small pixel margin; here 1/256 px, enough to
// keep every pixel that the fp32 cutoff admits inside the box.
//
// HBM-bound: 32 B read (+4 B logit) and 44 B written (+4 B opacity) per Gaussian.
#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

// One Gaussian's set-up from its parameters p0 = (mux, muy, l11, l21),
// p1 = (l22, cr, cg, cb) and, when has_logit, its logit.
struct Prep {
    float4 rp, rq;     // record
    uint2 box;         // packed pixel box
    uint32_t cnt;      // tiles covered
    float opacity;
};

__device__ __forceinline__ Prep preprocess_gaussian(float4 p0, float4 p1, bool has_logit, float lam, int W, int H) {
    const float l11 = p0.z, l21 = p0.w, l22 = p1.x;
    bool ok = isfinite(p0.x) && isfinite(p0.y) && isfinite(l11) && isfinite(l21) && isfinite(l22) &&
              isfinite(p1.y) && isfinite(p1.z) && isfinite(p1.w);
    if (has_logit) ok = ok && isfinite(lam);
    ok = ok && l11 != 0.0f && l22 != 0.0f;
    float a = 0.0f, b = 0.0f, c = 0.0f;
    if (ok) {
        const float3 r = conic_rows(l11, l21, l22);
        ok = isfinite(r.x) && isfinite(r.y) && isfinite(r.z);
        a = r.x;
        b = r.y;
        c = r.z;
    }
    Prep o;
    o.cnt = 0;
    o.box = make_uint2(1u | (1u << 16), 0u);   // empty: j0 = i0 = 1, j1 = i1 = 0
    if (ok) {
        const float rx = 3.0f * fabsf(l11) + kPad;
        const float ry = 3.0f * sqrtf(fmaf(l21, l21, l22 * l22)) + kPad;
        const float cx = p0.x - 0.5f, cy = p0.y - 0.5f;
        const float fj0 = fmaxf(ceilf(cx - rx), 0.0f);
        const float fj1 = fminf(floorf(cx + rx), (float)(W - 1));
        const float fi0 = fmaxf(ceilf(cy - ry), 0.0f);
        const float fi1 = fminf(floorf(cy + ry), (float)(H - 1));
        if (fj0 <= fj1 && fi0 <= fi1) {
            const uint32_t j0 = (uint32_t)fj0, j1 = (uint32_t)fj1, i0 = (uint32_t)fi0, i1 = (uint32_t)fi1;
            o.box = make_uint2(j0 | (i0 << 16), j1 | (i1 << 16));
            o.cnt = ((j1 >> 4) - (j0 >> 4) + 1) * ((i1 >> 4) - (i0 >> 4) + 1);
        }
    } else {
        a = b = c = 0.0f;
    }
    o.rp = ok ? make_float4(p0.x, p0.y, a, b) : make_float4(0.f, 0.f, 0.f, 0.f);
    o.rq = ok ? make_float4(c, p1.y, p1.z, p1.w) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float l = fminf(lam, kLogitMax);
    o.opacity = ok ? 1.0f / (1.0f + expf(-l)) : 0.0f;
    return o;
}

// One Gaussian: record, pixel box (also returned in *box_out), tile count (returned), opacity.
__device__ __forceinline__ uint32_t preprocess_one(int g, int W, int H, const float4 *__restrict__ params,
                                                   const float *__restrict__ logit, float4 *__restrict__ records,
                                                   float *__restrict__ opacity, uint2 *__restrict__ pixbox,
                                                   uint32_t *__restrict__ counts, uint2 *box_out) {
    const Prep o = preprocess_gaussian(params[2 * g], params[2 * g + 1], logit != nullptr, logit ? logit[g] : 0.0f,
                                       W, H);
    records[2 * g] = o.rp;
    records[2 * g + 1] = o.rq;
    pixbox[g] = o.box;
    counts[g] = o.cnt;
    if (opacity) opacity[g] = o.opacity;
    *box_out = o.box;
    return o.cnt;
}

// The binning's first step for one 256-Gaussian group of a block of NT threads, given each
// thread's tile count c and box: the group's pair total and, when hist.table is set, its
// first-pass digit histogram.  One histogram row per wave (hw: NT/64 rows of 256 u32 of LDS,
// nothing to clear beforehand): each wave clears and fills its own row, so a single barrier
// publishes the rows and the wave sums (ws: NT/64 u64); the row sums go to the table.
template <int NT>
__device__ __forceinline__ void group_totals_waves(uint32_t c, uint2 box, unsigned long long *__restrict__ group_sums,
                                                   BinHist hist, uint32_t *hw, unsigned long long *ws) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int radix = 1 << hist.bits;
    uint32_t *row = hw + wave * 256;
    if (hist.table) {                                     // uniform; LDS ops of a wave stay in order
        for (int d = lane; d < radix; d += 64) row[d] = 0u;
        hist_add_pairs(row, c, box, hist.tiles_x, hist.shift, (uint32_t)(radix - 1));
    }
    unsigned long long x = c;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    if (lane == 0) ws[wave] = x;
    __syncthreads();
    if (tid == 0) {
        unsigned long long t = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) t += ws[w];
        group_sums[blockIdx.x] = t;
    }
    if (hist.table && tid < radix) {
        uint32_t h = 0u;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) h += hw[w * 256 + tid];
        if (hist.redundant) hist.table[(size_t)blockIdx.x * radix + tid] = h;
        else hist.table[(size_t)tid * hist.ncols_cap + blockIdx.x] = h;
    }
}

// With group_sums (binning in the same call): also the sum of each 256-Gaussian
// group's tile counts, the tile ranges cleared and, when hist.table is set, the
// group's first-pass digit histogram -- the binning's first step.
__global__ __launch_bounds__(256) void k_preprocess(int n, int W, int H, const float4 *__restrict__ params,
                                                    const float *__restrict__ logit,
                                                    float4 *__restrict__ records, float *__restrict__ opacity,
                                                    uint2 *__restrict__ pixbox, uint32_t *__restrict__ counts,
                                                    unsigned long long *__restrict__ group_sums,
                                                    uint2 *__restrict__ ranges, int ntiles, BinHist hist) {
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    uint2 box = make_uint2(1u, 0u);
    if (group_sums) {
        __shared__ unsigned long long ws[4];
        __shared__ uint32_t hw[4 * 256];
        for (int t = g; t < ntiles; t += gridDim.x * 256) ranges[t] = make_uint2(0u, 0u);
        const uint32_t c = g < n ? preprocess_one(g, W, H, params, logit, records, opacity, pixbox, counts, &box) : 0u;
        group_totals_waves<256>(c, box, group_sums, hist, hw, ws);
        return;
    }
    if (g >= n) return;
    preprocess_one(g, W, H, params, logit, records, opacity, pixbox, counts, &box);
}

hipError_t launch_preprocess(int n, int W, int H, const float *params, const float *logit, float *records,
                             float *opacity, uint16_t *pixbox, uint32_t *counts, unsigned long long *group_sums,
                             uint32_t *ranges, BinHist hist, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int bs = 256;
    const int ntiles = ((W + kTile - 1) / kTile) * ((H + kTile - 1) / kTile);
    k_preprocess<<<(n + bs - 1) / bs, bs, 0, s>>>(n, W, H, reinterpret_cast<const float4 *>(params), logit,
                                                  reinterpret_cast<float4 *>(records), opacity,
                                                  reinterpret_cast<uint2 *>(pixbox), counts, group_sums,
                                                  reinterpret_cast<uint2 *>(ranges), ntiles, hist);
    return hipGetLastError();
}

// Adam on each Gaussian's 8 parameters with the gradient gathered from its
// pair slots (the arithmetic of k_adam_pairs, so the same bits), then the
// set-up of the updated Gaussian for the next binning, as k_preprocess with
// group_sums: record, pixel box, tile count, the group's pair total and digit
// histogram, and the tile ranges cleared.  With `loss`, the last workgroup
// reduces the loss partials of the raster pass instead.
//
// Two lanes per Gaussian (512 threads per 256-Gaussian group): lane h of the
// pair gathers and updates the parameter half h (float4), so each lane's chain
// of dependent loads and Adam steps is half as long; the pair then swaps
// halves and both form the set-up (the even lane keeps the count).
constexpr int kAdamPrepThreads = 512;
__global__ __launch_bounds__(kAdamPrepThreads) void k_adam_preprocess(
    int n, int W, int H, int ngroups, const uint32_t *__restrict__ offsets, uint32_t capacity,
    const float4 *__restrict__ part, float4 *__restrict__ p, float4 *__restrict__ m, float4 *__restrict__ v, AdamHP a,
    float4 *__restrict__ records, uint2 *__restrict__ pixbox, uint32_t *__restrict__ counts,
    unsigned long long *__restrict__ group_sums, uint2 *__restrict__ ranges, int ntiles, BinHist hist,
    const float *__restrict__ loss_part, int nparts, double inv_count, float *__restrict__ loss) {
    constexpr int NT = kAdamPrepThreads;
    if (loss && (int)blockIdx.x == ngroups) {
        __shared__ double sm[256];
        loss_reduce_block(nparts, loss_part, inv_count, loss, sm);
        return;
    }
    __shared__ unsigned long long ws[NT / 64];
    __shared__ uint32_t hw[NT / 64 * 256];
    const int tid = threadIdx.x, half = tid & 1;
    const int g = blockIdx.x * 256 + (tid >> 1);
    for (int t = blockIdx.x * NT + tid; t < ntiles; t += ngroups * NT) ranges[t] = make_uint2(0u, 0u);
    float c1, c2;
    adam_step_bias(a, c1, c2);
    uint32_t c = 0u;
    uint2 box = make_uint2(1u, 0u);
    if (g < n) {                                          // both lanes of the pair
        const size_t q = 2 * (size_t)g + half;
        float4 P = p[q], Mm = m[q], V = v[q];
        const uint32_t o0 = offsets[g], o1r = offsets[g + 1];   // both loads out with the parameter loads
        const uint32_t o1 = offsets[n] <= capacity ? o1r : o0;  // else the binning overflowed: zero gradient
        float4 gr = make_float4(0.f, 0.f, 0.f, 0.f);
        gather_half(part, o0, o1, half, gr);
        {                                                 // sums -> gradient, with the rows of the old record
            const float4 O = make_float4(__shfl_xor(P.x, 1, 64), __shfl_xor(P.y, 1, 64), __shfl_xor(P.z, 1, 64),
                                         __shfl_xor(P.w, 1, 64));
            const float4 A0 = half ? O : P, A1 = half ? P : O;
            const float3 r = conic_rows(A0.z, A0.w, A1.x);
            gr = o1 > o0 ? slot_grad_half(half, r.x, r.y, r.z, gr) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        const int l0 = 4 * half;
        adam_update(P.x, gr.x, Mm.x, V.x, a.lr[l0], a, c1, c2);
        adam_update(P.y, gr.y, Mm.y, V.y, a.lr[l0 + 1], a, c1, c2);
        adam_update(P.z, gr.z, Mm.z, V.z, a.lr[l0 + 2], a, c1, c2);
        adam_update(P.w, gr.w, Mm.w, V.w, a.lr[l0 + 3], a, c1, c2);
        p[q] = P;
        m[q] = Mm;
        v[q] = V;
        const float4 Q = make_float4(__shfl_xor(P.x, 1, 64), __shfl_xor(P.y, 1, 64), __shfl_xor(P.z, 1, 64),
                                     __shfl_xor(P.w, 1, 64));
        const float4 P0 = half ? Q : P, P1 = half ? P : Q;
        const Prep o = preprocess_gaussian(P0, P1, false, 0.0f, W, H);
        if (half) {
            records[q] = o.rq;
        } else {
            records[q] = o.rp;
            pixbox[g] = o.box;
            counts[g] = o.cnt;
            c = o.cnt;
            box = o.box;
        }
    }
    group_totals_waves<NT>(c, box, group_sums, hist, hw, ws);
}

hipError_t launch_adam_preprocess(int n, int W, int H, const uint32_t *offsets, int64_t capacity, const void *bwd_ws,
                                  float *p, float *m, float *v, const AdamHP &a, float *records, uint16_t *pixbox,
                                  uint32_t *counts, unsigned long long *group_sums, uint32_t *ranges, BinHist hist,
                                  const float *loss_partials, int64_t loss_count, float *d_loss, hipStream_t s) {
    const int ngroups = (n + 255) / 256;
    const int nb = ngroups + (d_loss ? 1 : 0);
    if (nb == 0) return hipSuccess;
    const int ntiles = ((W + kTile - 1) / kTile) * ((H + kTile - 1) / kTile);
    const BwdPlan pl = make_bwd_plan(W, H, capacity);
    k_adam_preprocess<<<nb, kAdamPrepThreads, 0, s>>>(
        n, W, H, ngroups, offsets, (uint32_t)capacity,
        reinterpret_cast<const float4 *>(static_cast<const char *>(bwd_ws) + pl.off_part),
        reinterpret_cast<float4 *>(p), reinterpret_cast<float4 *>(m), reinterpret_cast<float4 *>(v), a,
        reinterpret_cast<float4 *>(records), reinterpret_cast<uint2 *>(pixbox), counts, group_sums,
        reinterpret_cast<uint2 *>(ranges), ntiles, hist, loss_partials, ntiles,
        loss_count > 0 ? 1.0 / (double)loss_count : 0.0, d_loss);
    return hipGetLastError();
}

}  // namespace gi
