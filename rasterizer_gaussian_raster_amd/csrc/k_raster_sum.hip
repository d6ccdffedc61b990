// k_raster_sum.hip -- accumulated-sum rasterization ("GaussianImage", Overview:
// rendering by accumulated summation of 2D Gaussians) and its backward.
//
// Forward (pixel-major).  One workgroup of 4 waves per 16x16 tile; wave w owns
// the 8x8 quadrant (w & 1, w >> 1), one pixel per lane.  The tile's list is
// staged 128 Gaussians at a time with coalesced loads; while staging, each
// thread tests its Gaussian's pixel box against the four quadrants and the
// records are compacted, in list order, into one LDS list per quadrant
// (ballot + popcount ranks).  Each wave then walks only its quadrant's list.
// A Gaussian whose box misses the quadrant cannot pass the cutoff at any of its
// pixels, so the compaction removes no admitted pair and keeps the per-pixel
// summation order: the image is the same bits as a walk of the whole list.
// Per evaluated pair: 7 VALU for the cutoff exponent, compare + select, one
// v_exp_f32, 3 FMA -- FP32-VALU bound.
//
// Backward (work items).  The tile is cut into 16 blocks of 4x4 pixels; every
// list entry yields one work item per block its pixel box overlaps (about 0.4
// of the binned pairs at the benchmark shapes), and the items are packed 64
// per wave, one per lane, so no lane idles on a short list and no pair outside
// the box is evaluated.  A lane walks its block's 16 pixels (dL/dI staged in
// LDS), keeping the Gaussian's partial gradient in registers with the
// column-invariant factors (dx, u, b dx, u^2) hoisted; the chain rule from the
// scaled rows of L^-1 (a, b, c) to (l11, l21, l22) is applied per item, the
// items of an entry meet in LDS float atomics, and each entry then adds its 8
// values to dparams with fp32 global atomics.
#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

struct SumRec { float4 p, q; };   // p = (mux, muy, a, b), q = (c, cr, cg, cb)

constexpr int kFwdBatch = 128;    // list entries staged per round (16 KB of LDS: 8+ workgroups per CU)

// exclusive scan over the 256 threads of a workgroup (wave shuffles + one LDS step)
__device__ __forceinline__ uint32_t block_exclusive_scan_u32(uint32_t x, uint32_t *sm, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(inc, d, 64);
        if (lane >= d) inc += y;
    }
    if (lane == 63) sm[wave] = inc;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t s = sm[w];
        off += (w < wave) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return off + inc - x;
}

__global__ __launch_bounds__(256) void k_render_sum_fwd(int W, int H, int tiles_x, int ntiles,
                                                        const float4 *__restrict__ records,
                                                        const uint2 *__restrict__ pixbox,
                                                        const uint2 *__restrict__ ranges,
                                                        const uint32_t *__restrict__ vals,
                                                        float *__restrict__ image) {
    __shared__ SumRec lst[4][kFwdBatch];
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

    for (uint32_t base = rg.x; base < rg.y; base += kFwdBatch) {
        const uint32_t idx = base + tid;
        uint32_t qm = 0;
        SumRec r;
        r.p = r.q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tid < kFwdBatch && idx < rg.y) {
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
        if (base + kFwdBatch < rg.y) __syncthreads();   // the next batch reuses lst / wq
    }
    if (pxi < W && pyi < H) {
        const size_t o = (size_t)pyi * W + pxi, plane = (size_t)W * H;
        image[o] = ar;
        image[o + plane] = ag;
        image[o + 2 * plane] = ab;
    }
}

// Backward work item: one (list entry, 4x4 pixel block) pair per lane.
__global__ __launch_bounds__(256) void k_render_sum_bwd(int W, int H, int tiles_x, int ntiles,
                                                        const float4 *__restrict__ records,
                                                        const uint2 *__restrict__ pixbox,
                                                        const uint2 *__restrict__ ranges,
                                                        const uint32_t *__restrict__ vals,
                                                        const float *__restrict__ dL,
                                                        float *__restrict__ dparams) {
    __shared__ float4 gp[256];                    // dL/dI of the tile's pixels, row-major
    __shared__ SumRec ent[256];                   // staged list entries
    __shared__ uint32_t eg[256];                  // their Gaussian indices
    __shared__ float acc[256][9];                 // per-entry gradient (params layout), padded row
    __shared__ uint16_t items[256 * 16];          // entry | block << 8
    __shared__ uint32_t sm[4];
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
    const float k2 = 2.0f * kLn2;
    const float is = 1.0f / kScale;
    for (uint32_t base = rg.x; base < rg.y; base += 256) {
        const uint32_t idx = base + tid;
        uint32_t nit = 0, bx0 = 0, by0 = 0, wb = 1;
        if (idx < rg.y) {
            const uint32_t g = vals[idx];
            ent[tid].p = records[2 * g];
            ent[tid].q = records[2 * g + 1];
            eg[tid] = g;
            const uint2 bx = pixbox[g];
            const int j0 = max((int)(bx.x & 0xffff) - x0, 0), j1 = min((int)(bx.y & 0xffff) - x0, 15);
            const int i0 = max((int)(bx.x >> 16) - y0, 0), i1 = min((int)(bx.y >> 16) - y0, 15);
            bx0 = (uint32_t)j0 >> 2;
            by0 = (uint32_t)i0 >> 2;
            wb = ((uint32_t)j1 >> 2) - bx0 + 1;
            nit = wb * (((uint32_t)i1 >> 2) - by0 + 1);
        }
#pragma unroll
        for (int k = 0; k < 9; ++k) acc[tid][k] = 0.0f;
        uint32_t nitems;
        const uint32_t off = block_exclusive_scan_u32(nit, sm, &nitems);
        for (uint32_t k = 0; k < nit; ++k) {
            const uint32_t q = k / wb;
            const uint32_t blk = (by0 + q) * 4 + bx0 + (k - q * wb);
            items[off + k] = (uint16_t)(tid | (blk << 8));
        }
        __syncthreads();
        for (uint32_t cb = (uint32_t)wave * 64; cb < nitems; cb += 256) {
            const uint32_t it = cb + lane;
            const bool active = it < nitems;
            const uint32_t code = active ? items[it] : 0u;
            const uint32_t e = code & 0xffu, blk = code >> 8;
            const int lx = (int)(blk & 3u) * 4, ly = (int)(blk >> 2) * 4;
            const float4 A = ent[e].p, B = ent[e].q;
            float dy[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) dy[rr] = ((float)(y0 + ly + rr) + 0.5f) - A.y;
            float Hu = 0.f, Hv = 0.f, Hudx = 0.f, Hvdx = 0.f, Hvdy = 0.f, Cr = 0.f, Cg = 0.f, Cb = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float dx = ((float)(x0 + lx + c) + 0.5f) - A.x;
                const float u = A.z * dx;
                const float tb = A.w * dx;
                const float uu = u * u;
                float ch = 0.f, chv = 0.f;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float4 gv = gp[(ly + rr) * kTile + lx + c];
                    const float v = fmaf(B.x, dy[rr], tb);
                    const float ee = fmaf(v, v, uu);
                    const float w = (active && ee <= kE9) ? exp2_hw(-ee) : 0.0f;
                    Cr = fmaf(gv.x, w, Cr);
                    Cg = fmaf(gv.y, w, Cg);
                    Cb = fmaf(gv.z, w, Cb);
                    const float h = fmaf(gv.z, B.w, fmaf(gv.y, B.z, gv.x * B.y)) * w;
                    const float hv = h * v;
                    ch += h;
                    chv += hv;
                    Hvdy = fmaf(hv, dy[rr], Hvdy);
                }
                Hu = fmaf(u, ch, Hu);
                Hudx = fmaf(u * dx, ch, Hudx);
                Hv += chv;
                Hvdx = fmaf(dx, chv, Hvdx);
            }
            if (active && (Cr != 0.f || Cg != 0.f || Cb != 0.f || Hu != 0.f || Hv != 0.f)) {
                // e = u^2 + v^2, w = 2^-e: dL/de = -ln2 h, summed through (Hu, Hv, ...); then
                // a = S/l11, b = -S l21/(l11 l22), c = S/l22 -> (l11, l21, l22).
                const float a = A.z, b = A.w, c = B.x;
                const float da = -k2 * Hudx, db = -k2 * Hvdx, dc = -k2 * Hvdy;
                float *d = acc[e];
                atomicAdd(d + 0, k2 * fmaf(a, Hu, b * Hv));
                atomicAdd(d + 1, k2 * c * Hv);
                atomicAdd(d + 2, -is * fmaf(a * a, da, a * b * db));
                atomicAdd(d + 3, -is * (a * c * db));
                atomicAdd(d + 4, -is * fmaf(b * c, db, c * c * dc));
                atomicAdd(d + 5, Cr);
                atomicAdd(d + 6, Cg);
                atomicAdd(d + 7, Cb);
            }
        }
        __syncthreads();
        if (idx < rg.y) {
            float *d = dparams + 8 * (size_t)eg[tid];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float v = acc[tid][k];
                if (v != 0.0f) atomicAdd(d + k, v);
            }
        }
        if (base + 256 < rg.y) __syncthreads();   // the next batch reuses ent / acc / items
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
