// k_raster_sum.hip -- accumulated-sum rasterization ("GaussianImage", Overview:
// rendering by accumulated summation of 2D Gaussians) and its backward.
//
// Forward (pixel-major).  One workgroup of 4 waves per 16x16 tile; wave w owns
// the 8x8 quadrant (w & 1, w >> 1), one pixel per lane.  The tile's list is
// staged 256 Gaussians at a time with coalesced loads; while staging, each
// thread tests its Gaussian's pixel box against the four quadrants and the
// records are compacted, in list order, into one LDS list per quadrant
// (ballot + popcount ranks).  Each wave then walks only its quadrant's list.
// A Gaussian whose box misses the quadrant cannot pass the cutoff at any of its
// pixels, so the compaction removes no admitted pair and keeps the per-pixel
// summation order: the image is the same bits as a walk of the whole list.
// Per evaluated pair: 7 VALU for the cutoff exponent, compare + select, one
// v_exp_f32, 3 FMA -- FP32-VALU bound.
//
// Backward (Gaussian-major).  Lane = Gaussian of the tile's list (64 per wave),
// the 256 pixels' dL/dI staged in LDS and read as wave-uniform broadcasts.
// Each lane accumulates its Gaussian's gradient over the tile's pixels in
// registers, so no cross-lane reduction is needed; column-invariant factors
// (dx, u, b dx, u^2) are hoisted out of the row loop.  One set of 8 fp32
// atomics per (Gaussian, tile) adds the result to dparams, after applying the
// chain rule from the scaled rows of L^-1 (a, b, c) to (l11, l21, l22).
#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

struct SumRec { float4 p, q; };   // p = (mux, muy, a, b), q = (c, cr, cg, cb)

__global__ __launch_bounds__(256) void k_render_sum_fwd(int W, int H, int tiles_x, int ntiles,
                                                        const float4 *__restrict__ records,
                                                        const uint2 *__restrict__ pixbox,
                                                        const uint2 *__restrict__ ranges,
                                                        const uint32_t *__restrict__ vals,
                                                        float *__restrict__ image) {
    __shared__ SumRec lst[4][256];
    __shared__ int wq[4][4];                      // [wave][quadrant]: staged count this batch
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    if (t >= ntiles) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int x0 = (t % tiles_x) * kTile, y0 = (t / tiles_x) * kTile;
    const int pxi = x0 + (wave & 1) * 8 + (lane & 7);
    const int pyi = y0 + (wave >> 1) * 8 + (lane >> 3);
    const float px = (float)pxi + 0.5f, py = (float)pyi + 0.5f;
    const uint2 rg = ranges[t];
    const uint64_t below = lanes_below();
    float ar = 0.0f, ag = 0.0f, ab = 0.0f;

    for (uint32_t base = rg.x; base < rg.y; base += 256) {
        const uint32_t idx = base + tid;
        uint32_t qm = 0;
        SumRec r;
        r.p = r.q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (idx < rg.y) {
            const uint32_t g = vals[idx];
            r.p = records[2 * g];
            r.q = records[2 * g + 1];
            const uint2 bx = pixbox[g];
            const int j0 = bx.x & 0xffff, i0 = bx.x >> 16, j1 = bx.y & 0xffff, i1 = bx.y >> 16;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int qx0 = x0 + (q & 1) * 8, qy0 = y0 + (q >> 1) * 8;
                qm |= (j0 <= qx0 + 7 && j1 >= qx0 && i0 <= qy0 + 7 && i1 >= qy0) ? (1u << q) : 0u;
            }
        }
        uint32_t rank[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint64_t m = __ballot((qm >> q) & 1u);
            rank[q] = (uint32_t)__popcll(m & below);
            if (lane == 0) wq[wave][q] = __popcll(m);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if ((qm >> q) & 1u) {
                int off = rank[q];
                for (int w = 0; w < wave; ++w) off += wq[w][q];
                lst[q][off] = r;
            }
        }
        const int cnt = __builtin_amdgcn_readfirstlane(wq[0][wave] + wq[1][wave] + wq[2][wave] + wq[3][wave]);
        __syncthreads();
        const SumRec *L = lst[wave];
        for (int k = 0; k < cnt; ++k) {
            const float4 A = L[k].p, B = L[k].q;
            const float dx = px - A.x, dy = py - A.y;
            const float u = A.z * dx;
            const float tb = A.w * dx;
            const float v = fmaf(B.x, dy, tb);
            const float e = fmaf(v, v, u * u);
            const float w = e <= kE9 ? exp2_hw(-e) : 0.0f;   // adding c * 0 leaves the sum's bits unchanged
            ar = fmaf(B.y, w, ar);
            ag = fmaf(B.z, w, ag);
            ab = fmaf(B.w, w, ab);
        }
        if (base + 256 < rg.y) __syncthreads();   // the next batch reuses lst / wq
    }
    if (pxi < W && pyi < H) {
        const size_t o = (size_t)pyi * W + pxi, plane = (size_t)W * H;
        image[o] = ar;
        image[o + plane] = ag;
        image[o + 2 * plane] = ab;
    }
}

__global__ __launch_bounds__(256) void k_render_sum_bwd(int W, int H, int tiles_x, int ntiles,
                                                        const float4 *__restrict__ records,
                                                        const uint2 *__restrict__ pixbox,
                                                        const uint2 *__restrict__ ranges,
                                                        const uint32_t *__restrict__ vals,
                                                        const float *__restrict__ dL,
                                                        float *__restrict__ dparams) {
    __shared__ float4 gp[256];                    // dL/dI of the tile's pixels, row-major
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    if (t >= ntiles) return;
    const uint2 rg = ranges[t];
    if (rg.x == rg.y) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int x0 = (t % tiles_x) * kTile, y0 = (t / tiles_x) * kTile;
    {
        const int xi = x0 + (tid & 15), yi = y0 + (tid >> 4);
        float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
        if (xi < W && yi < H) {
            const size_t o = (size_t)yi * W + xi, plane = (size_t)W * H;
            g = make_float4(dL[o], dL[o + plane], dL[o + 2 * plane], 0.f);
        }
        gp[tid] = g;
    }
    __syncthreads();
    const uint32_t len = rg.y - rg.x;
    for (uint32_t cb = (uint32_t)wave * 64; cb < len; cb += 256) {
        const bool valid = cb + lane < len;
        uint32_t g = 0;
        float4 A = make_float4(0.f, 0.f, 0.f, 0.f), B = make_float4(INFINITY, 0.f, 0.f, 0.f);
        int j0 = 16, j1 = -1, i0 = 16, i1 = -1;           // tile-local box, empty for idle lanes
        if (valid) {
            g = vals[rg.x + cb + lane];
            A = records[2 * g];
            B = records[2 * g + 1];
            const uint2 bx = pixbox[g];
            j0 = max((int)(bx.x & 0xffff) - x0, 0);
            j1 = min((int)(bx.y & 0xffff) - x0, 15);
            i0 = max((int)(bx.x >> 16) - y0, 0);
            i1 = min((int)(bx.y >> 16) - y0, 15);
        }
        // pixel range of the union of the wave's boxes (wave-uniform)
        int cx0 = j0, cx1 = j1, cy0 = i0, cy1 = i1;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            cx0 = min(cx0, __shfl_xor(cx0, d, 64));
            cx1 = max(cx1, __shfl_xor(cx1, d, 64));
            cy0 = min(cy0, __shfl_xor(cy0, d, 64));
            cy1 = max(cy1, __shfl_xor(cy1, d, 64));
        }
        cx0 = __builtin_amdgcn_readfirstlane(cx0);
        cx1 = __builtin_amdgcn_readfirstlane(cx1);
        cy0 = __builtin_amdgcn_readfirstlane(cy0);
        cy1 = __builtin_amdgcn_readfirstlane(cy1);

        float dy[kTile];
#pragma unroll
        for (int r = 0; r < kTile; ++r) dy[r] = ((float)(y0 + r) + 0.5f) - A.y;

        float Hu = 0.f, Hv = 0.f, Hudx = 0.f, Hvdx = 0.f, Hvdy = 0.f, Cr = 0.f, Cg = 0.f, Cb = 0.f;
        for (int col = cx0; col <= cx1; ++col) {
            const float dx = ((float)(x0 + col) + 0.5f) - A.x;
            const float u = A.z * dx;
            const float tb = A.w * dx;
            const float uu = u * u;
            float ch = 0.f, chv = 0.f;
#pragma unroll
            for (int r = 0; r < kTile; ++r) {
                if (r < cy0 || r > cy1) continue;          // uniform
                const float4 gv = gp[r * kTile + col];
                const float v = fmaf(B.x, dy[r], tb);
                const float e = fmaf(v, v, uu);
                if (e <= kE9) {
                    const float w = exp2_hw(-e);
                    Cr = fmaf(gv.x, w, Cr);
                    Cg = fmaf(gv.y, w, Cg);
                    Cb = fmaf(gv.z, w, Cb);
                    const float gc = fmaf(gv.z, B.w, fmaf(gv.y, B.z, gv.x * B.y));
                    const float h = gc * w;
                    const float hv = h * v;
                    ch += h;
                    chv += hv;
                    Hvdy = fmaf(hv, dy[r], Hvdy);
                }
            }
            Hu = fmaf(u, ch, Hu);
            Hudx = fmaf(u * dx, ch, Hudx);
            Hv += chv;
            Hvdx = fmaf(dx, chv, Hvdx);
        }
        if (valid && (Cr != 0.f || Cg != 0.f || Cb != 0.f || Hu != 0.f || Hv != 0.f)) {
            // e = u^2 + v^2, w = 2^-e: dL/de = -ln2 * h summed above through (Hu, Hv, ...).
            const float k2 = 2.0f * kLn2;
            const float a = A.z, b = A.w, c = B.x;
            const float dmx = k2 * fmaf(a, Hu, b * Hv);
            const float dmy = k2 * c * Hv;
            const float da = -k2 * Hudx, db = -k2 * Hvdx, dc = -k2 * Hvdy;
            const float is = 1.0f / kScale;
            // a = S/l11, b = -S l21/(l11 l22), c = S/l22
            const float dl11 = -is * fmaf(a * a, da, a * b * db);
            const float dl21 = -is * (a * c * db);
            const float dl22 = -is * fmaf(b * c, db, c * c * dc);
            float *d = dparams + 8 * (size_t)g;
            atomicAdd(d + 0, dmx);
            atomicAdd(d + 1, dmy);
            atomicAdd(d + 2, dl11);
            atomicAdd(d + 3, dl21);
            atomicAdd(d + 4, dl22);
            atomicAdd(d + 5, Cr);
            atomicAdd(d + 6, Cg);
            atomicAdd(d + 7, Cb);
        }
    }
}

static int padded_tiles(int ntiles) { return (ntiles + 7) & ~7; }

hipError_t launch_render_sum_fwd(int W, int H, const float *records, const uint16_t *pixbox,
                                 const uint32_t *ranges, const uint32_t *vals, float *image, hipStream_t s) {
    const int tiles_x = (W + kTile - 1) / kTile, ntiles = tiles_x * ((H + kTile - 1) / kTile);
    k_render_sum_fwd<<<padded_tiles(ntiles), 256, 0, s>>>(W, H, tiles_x, ntiles,
                                                          reinterpret_cast<const float4 *>(records),
                                                          reinterpret_cast<const uint2 *>(pixbox),
                                                          reinterpret_cast<const uint2 *>(ranges), vals, image);
    return hipGetLastError();
}

hipError_t launch_render_sum_bwd(int W, int H, const float *records, const uint16_t *pixbox,
                                 const uint32_t *ranges, const uint32_t *vals, const float *dL_dimage,
                                 float *dparams, hipStream_t s) {
    const int tiles_x = (W + kTile - 1) / kTile, ntiles = tiles_x * ((H + kTile - 1) / kTile);
    k_render_sum_bwd<<<padded_tiles(ntiles), 256, 0, s>>>(W, H, tiles_x, ntiles,
                                                          reinterpret_cast<const float4 *>(records),
                                                          reinterpret_cast<const uint2 *>(pixbox),
                                                          reinterpret_cast<const uint2 *>(ranges), vals,
                                                          dL_dimage, dparams);
    return hipGetLastError();
}

}  // namespace gi
