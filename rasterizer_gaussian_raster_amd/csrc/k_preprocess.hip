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

// One Gaussian: record, pixel box (also returned in *box_out), tile count (returned), opacity.
__device__ __forceinline__ uint32_t preprocess_one(int g, int W, int H, const float4 *__restrict__ params,
                                                   const float *__restrict__ logit, float4 *__restrict__ records,
                                                   float *__restrict__ opacity, uint2 *__restrict__ pixbox,
                                                   uint32_t *__restrict__ counts, uint2 *box_out) {
    const float4 p0 = params[2 * g];       // mux, muy, l11, l21
    const float4 p1 = params[2 * g + 1];   // l22, cr, cg, cb
    const float l11 = p0.z, l21 = p0.w, l22 = p1.x;
    bool ok = isfinite(p0.x) && isfinite(p0.y) && isfinite(l11) && isfinite(l21) && isfinite(l22) &&
              isfinite(p1.y) && isfinite(p1.z) && isfinite(p1.w);
    float lam = 0.0f;
    if (logit) {
        lam = logit[g];
        ok = ok && isfinite(lam);
    }
    ok = ok && l11 != 0.0f && l22 != 0.0f;
    float a = 0.0f, b = 0.0f, c = 0.0f;
    if (ok) {
        const float i11 = 1.0f / l11;          // correctly rounded (no fast-math)
        const float i22 = 1.0f / l22;
        const float k = -((l21 * i11) * i22);
        ok = isfinite(i11) && isfinite(i22) && isfinite(k);
        a = i11 * kScale;
        b = k * kScale;
        c = i22 * kScale;
    }
    uint32_t cnt = 0;
    uint2 box = make_uint2(1u | (1u << 16), 0u);   // empty: j0 = i0 = 1, j1 = i1 = 0
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
            box = make_uint2(j0 | (i0 << 16), j1 | (i1 << 16));
            cnt = ((j1 >> 4) - (j0 >> 4) + 1) * ((i1 >> 4) - (i0 >> 4) + 1);
        }
    } else {
        a = b = c = 0.0f;
    }
    records[2 * g] = ok ? make_float4(p0.x, p0.y, a, b) : make_float4(0.f, 0.f, 0.f, 0.f);
    records[2 * g + 1] = ok ? make_float4(c, p1.y, p1.z, p1.w) : make_float4(0.f, 0.f, 0.f, 0.f);
    pixbox[g] = box;
    counts[g] = cnt;
    *box_out = box;
    if (opacity) {
        const float l = fminf(lam, kLogitMax);
        opacity[g] = ok ? 1.0f / (1.0f + expf(-l)) : 0.0f;
    }
    return cnt;
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
    uint2 box;
    if (group_sums) {
        __shared__ unsigned long long ws[4];
        __shared__ uint32_t h[256];
        const int radix = 1 << hist.bits;
        if (hist.table && (int)threadIdx.x < radix) h[threadIdx.x] = 0u;
        for (int t = g; t < ntiles; t += gridDim.x * 256) ranges[t] = make_uint2(0u, 0u);
        const uint32_t c = g < n ? preprocess_one(g, W, H, params, logit, records, opacity, pixbox, counts, &box) : 0u;
        // block sum of the counts (u64), waves then the workgroup
        unsigned long long x = c;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
        if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = x;
        __syncthreads();                                  // also publishes the cleared histogram
        if (threadIdx.x == 0) group_sums[blockIdx.x] = ((ws[0] + ws[1]) + ws[2]) + ws[3];
        if (hist.table) {                                 // uniform
            hist_add_pairs(h, c, box, hist.tiles_x, hist.shift, (uint32_t)(radix - 1));
            __syncthreads();
            if ((int)threadIdx.x < radix) {
                if (hist.redundant) hist.table[(size_t)blockIdx.x * radix + threadIdx.x] = h[threadIdx.x];
                else hist.table[(size_t)threadIdx.x * hist.ncols_cap + blockIdx.x] = h[threadIdx.x];
            }
        }
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

}  // namespace gi
