// k_raster_alpha.hip -- front-to-back alpha compositing over a background
// ("Drawing with Gaussians", Overview: anisotropic 2D Gaussians alpha-composited
// over a trainable background; fused kernels with custom VJPs) and its backward.
//
// Layout as the sum forward: one workgroup per 16x16 tile, wave w owns the 8x8
// quadrant (w & 1, w >> 1), one pixel per lane, the tile list staged 128 at a
// time and compacted per quadrant in list order.  A Gaussian dropped for a
// quadrant has alpha = 0 at every pixel there, so T and C are unchanged by it:
// compaction keeps the results bit for bit.
//
// Forward per admitted pair: alpha = o 2^-e, C += c alpha T, T -= alpha T; a
// pixel stops after the Gaussian that leaves T < 1e-4 (recorded as `last`, one
// past its list position); a wave leaves the list once all its pixels stopped.
//
// Backward: each pixel walks its list from `last` down to the range start.
// T_j = T_{j+1} / (1 - alpha_j) recovers the transmittance in front of each
// Gaussian, and one scalar suffix accumulator gS = sum_k g_k S_k carries the
// colour behind it (S_k = later contributions + T_final bg_k), so
//   dL/dalpha_j = T_j (g . c_j) - gS / (1 - alpha_j),  gS += (g . c_j) alpha_j T_j.
// The 9 per-pixel contributions of a Gaussian are summed over the wave with
// DPP row ops and broadcasts (skipped when no pixel of the wave is covered) and
// written over the entry's slot in the wave's own quadrant list; each list
// entry then adds its four quadrant results in quadrant order and stores the
// gradient at its emission slot for the per-Gaussian gather.  No atomics: the
// gradients are bitwise reproducible.
#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

struct AlphaRec { float4 p, q, r; };   // p = (mux, muy, a, b), q = (c, cr, cg, cb), r = (o, pos, so, g)

constexpr int kBatch = 128;           // list entries staged per round (24 KB of LDS per workgroup)

__device__ __forceinline__ uint32_t quadrant_mask(uint2 bx, int x0, int y0) {
    const int j0 = bx.x & 0xffff, i0 = bx.x >> 16, j1 = bx.y & 0xffff, i1 = bx.y >> 16;
    uint32_t qm = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int qx0 = x0 + (q & 1) * 8, qy0 = y0 + (q >> 1) * 8;
        qm |= (j0 <= qx0 + 7 && j1 >= qx0 && i0 <= qy0 + 7 && i1 >= qy0) ? (1u << q) : 0u;
    }
    return qm;
}

// Stage list entries [lo, hi) (hi - lo <= kBatch) into the per-quadrant lists; returns this wave's count.
// Backward only (offsets != nullptr): also the entry's emission slot -> eslot[tid]
// and its position in each quadrant list -> qpos[tid][q] (0xff: not in that list).
__device__ __forceinline__ int stage_alpha(AlphaRec (*lst)[kBatch], int (*wq)[4], uint32_t lo, uint32_t hi, int x0,
                                           int y0, const float4 *__restrict__ records,
                                           const float *__restrict__ opacity, const float *__restrict__ logit,
                                           const uint2 *__restrict__ pixbox, const uint32_t *__restrict__ vals,
                                           uint64_t below, const uint32_t *__restrict__ offsets = nullptr,
                                           uint32_t *eslot = nullptr, uint8_t (*qpos)[4] = nullptr) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint32_t idx = lo + tid;
    uint32_t qm = 0;
    float4 rp = make_float4(0.f, 0.f, 0.f, 0.f), rq = rp, rr = rp;
    if (tid < kBatch && idx < hi) {
        const uint32_t g = vals[idx];
        rp = records[2 * g];
        rq = records[2 * g + 1];
        const float o = opacity[g];
        float so = 0.0f;
        if (logit) so = logit[g] < kLogitMax ? o * (1.0f - o) : 0.0f;
        rr = make_float4(o, __uint_as_float(idx), so, __uint_as_float(g));
        const uint2 bx = pixbox[g];
        qm = quadrant_mask(bx, x0, y0);
        if (offsets) eslot[tid] = emit_slot(offsets[g], bx, x0 / kTile, y0 / kTile);
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
            lst[q][off].p = rp;
            lst[q][off].q = rq;
            lst[q][off].r = rr;
            if (qpos) qpos[tid][q] = (uint8_t)off;
        } else if (qpos && tid < kBatch) {
            qpos[tid][q] = 0xff;
        }
    }
    const int cnt = __builtin_amdgcn_readfirstlane(wq[0][wave] + wq[1][wave] + wq[2][wave] + wq[3][wave]);
    __syncthreads();
    return cnt;
}

__global__ __launch_bounds__(256) void k_render_alpha_fwd(int W, int H, int tiles_x, int ntiles,
                                                          const float4 *__restrict__ records,
                                                          const float *__restrict__ opacity,
                                                          const uint2 *__restrict__ pixbox,
                                                          const uint2 *__restrict__ ranges, const uint32_t *__restrict__ order,
                                                          const uint32_t *__restrict__ vals,
                                                          const float *__restrict__ bg,
                                                          float *__restrict__ image, float *__restrict__ t_final,
                                                          uint32_t *__restrict__ last) {
    __shared__ AlphaRec lst[4][kBatch];
    __shared__ int wq[4][4];
    __shared__ int wdone[4];
    const int t = tile_of(blockIdx.x, gridDim.x, ntiles, order);
    if (t >= ntiles) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int x0 = (t % tiles_x) * kTile, y0 = (t / tiles_x) * kTile;
    const int pxi = x0 + (wave & 1) * 8 + (lane & 7);
    const int pyi = y0 + (wave >> 1) * 8 + (lane >> 3);
    const float px = (float)pxi + 0.5f, py = (float)pyi + 0.5f;
    const uint2 rg = ranges[t];
    const uint64_t below = lanes_below();
    float T = 1.0f, cr = 0.f, cg = 0.f, cb = 0.f;
    uint32_t lst_end = rg.x;
    bool done = false;

    for (uint32_t base = rg.x; base < rg.y; base += kBatch) {
        const uint32_t hi = rg.y - base > (uint32_t)kBatch ? base + kBatch : rg.y;
        const int cnt = stage_alpha(lst, wq, base, hi, x0, y0, records, opacity, nullptr, pixbox, vals, below);
        const AlphaRec *L = lst[wave];
        for (int k = 0; k < cnt; ++k) {
            if (__ballot(!done) == 0) break;
            const float4 A = L[k].p, B = L[k].q, R = L[k].r;
            const float dx = px - A.x, dy = py - A.y;
            const float u = A.z * dx;
            const float tb = A.w * dx;
            const float v = fmaf(B.x, dy, tb);
            const float e = fmaf(v, v, u * u);
            if (!done && e <= kE9) {
                const float al = R.x * exp2_hw(-e);
                const float aT = al * T;
                cr = fmaf(B.y, aT, cr);
                cg = fmaf(B.z, aT, cg);
                cb = fmaf(B.w, aT, cb);
                T -= aT;
                lst_end = __float_as_uint(R.y) + 1u;
                done = T < kTmin;
            }
        }
        const bool wave_done = __ballot(!done) == 0;        // all lanes vote (outside any branch)
        if (lane == 0) wdone[wave] = wave_done;
        if (hi >= rg.y) break;
        __syncthreads();
        if (wdone[0] && wdone[1] && wdone[2] && wdone[3]) break;   // uniform
    }
    if (pxi < W && pyi < H) {
        const size_t o = (size_t)pyi * W + pxi, plane = (size_t)W * H;
        image[o] = fmaf(T, bg[0], cr);
        image[o + plane] = fmaf(T, bg[1], cg);
        image[o + 2 * plane] = fmaf(T, bg[2], cb);
        t_final[o] = T;
        last[o] = lst_end;
    }
}

__global__ __launch_bounds__(256) void k_render_alpha_bwd(int W, int H, int tiles_x, int ntiles,
                                                          const float4 *__restrict__ records,
                                                          const float *__restrict__ opacity,
                                                          const float *__restrict__ logit,
                                                          const uint2 *__restrict__ pixbox,
                                                          const uint32_t *__restrict__ offsets,
                                                          const uint2 *__restrict__ ranges, const uint32_t *__restrict__ order,
                                                          const uint32_t *__restrict__ vals, uint32_t capacity,
                                                          const float *__restrict__ bg,
                                                          const float *__restrict__ t_final,
                                                          const uint32_t *__restrict__ last,
                                                          const float *__restrict__ dL,
                                                          float4 *__restrict__ part, float *__restrict__ part_l,
                                                          float4 *__restrict__ part_bg) {
    __shared__ AlphaRec lst[4][kBatch];
    __shared__ int wq[4][4];
    __shared__ uint32_t wmax[4];
    __shared__ float wbg[4][3];
    __shared__ uint32_t eslot[kBatch];
    __shared__ uint8_t qpos[kBatch][4];
    const int t = tile_of(blockIdx.x, gridDim.x, ntiles, order);
    if (t >= ntiles) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int x0 = (t % tiles_x) * kTile, y0 = (t / tiles_x) * kTile;
    const int pxi = x0 + (wave & 1) * 8 + (lane & 7);
    const int pyi = y0 + (wave >> 1) * 8 + (lane >> 3);
    const float px = (float)pxi + 0.5f, py = (float)pyi + 0.5f;
    const uint2 rg = ranges[t];
    const uint64_t below = lanes_below();
    const bool inside = pxi < W && pyi < H;
    float T = 0.f, gr = 0.f, gg = 0.f, gb = 0.f;
    uint32_t lp = rg.x;
    if (inside) {
        const size_t o = (size_t)pyi * W + pxi, plane = (size_t)W * H;
        T = t_final[o];
        lp = min(max(last[o], rg.x), rg.y);     // stays inside the tile's list whatever `last` holds
        gr = dL[o];
        gg = dL[o + plane];
        gb = dL[o + 2 * plane];
    }
    // dL/dbg_k = sum_p g_k T_final: one partial per tile
    {
        const float sr = wave_total(gr * T), sg = wave_total(gg * T), sb = wave_total(gb * T);
        if (lane == 0) { wbg[wave][0] = sr; wbg[wave][1] = sg; wbg[wave][2] = sb; }
        uint32_t m = lp;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
        if (lane == 0) wmax[wave] = m;
    }
    __syncthreads();
    if (tid == 0)
        part_bg[t] = make_float4(((wbg[0][0] + wbg[1][0]) + wbg[2][0]) + wbg[3][0],
                                 ((wbg[0][1] + wbg[1][1]) + wbg[2][1]) + wbg[3][1],
                                 ((wbg[0][2] + wbg[1][2]) + wbg[2][2]) + wbg[3][2], 0.f);
    const uint32_t bend0 = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    // entries behind every pixel's stop contribute nothing: their slots get zeros
    for (uint32_t idx = bend0 + tid; idx < rg.y; idx += 256) {
        const uint32_t g = vals[idx];
        const uint32_t slot = emit_slot(offsets[g], pixbox[g], x0 / kTile, y0 / kTile);
        if (slot < capacity) {
            part[2 * (size_t)slot] = make_float4(0.f, 0.f, 0.f, 0.f);
            part[2 * (size_t)slot + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
            part_l[slot] = 0.f;
        }
    }
    float gS = T * fmaf(gb, bg[2], fmaf(gg, bg[1], gr * bg[0]));
    const float k2 = 2.0f * kLn2;
    const float is = 1.0f / kScale;

    for (uint32_t hi = bend0; hi > rg.x;) {
        const uint32_t lo = hi - rg.x > (uint32_t)kBatch ? hi - kBatch : rg.x;
        __syncthreads();                                   // previous batch fully consumed
        const int cnt = stage_alpha(lst, wq, lo, hi, x0, y0, records, opacity, logit, pixbox, vals, below,
                                    offsets, eslot, qpos);
        const AlphaRec *L = lst[wave];
        for (int k = cnt - 1; k >= 0; --k) {
            const float4 A = L[k].p, B = L[k].q, R = L[k].r;
            const uint32_t pos = __float_as_uint(R.y);
            const float dx = px - A.x, dy = py - A.y;
            const float u = A.z * dx;
            const float tb = A.w * dx;
            const float v = fmaf(B.x, dy, tb);
            const float e = fmaf(v, v, u * u);
            const bool act = pos < lp && e <= kE9;
            float *res = reinterpret_cast<float *>(&lst[wave][k]);   // this wave is done reading entry k
            if (__ballot(act) == 0) {                                  // uniform
                if (lane == 0) {
                    lst[wave][k].p = make_float4(0.f, 0.f, 0.f, 0.f);
                    lst[wave][k].q = make_float4(0.f, 0.f, 0.f, 0.f);
                    res[8] = 0.0f;
                }
                continue;
            }
            float dcr = 0.f, dcg = 0.f, dcb = 0.f, hu = 0.f, hv = 0.f, hudx = 0.f, hvdx = 0.f, hvdy = 0.f, dlg = 0.f;
            if (act) {
                const float w = exp2_hw(-e);
                const float al = R.x * w;
                const float rinv = __builtin_amdgcn_rcpf(1.0f - al);
                const float Tj = T * rinv;
                const float aTj = al * Tj;
                dcr = gr * aTj;
                dcg = gg * aTj;
                dcb = gb * aTj;
                const float gc = fmaf(gb, B.w, fmaf(gg, B.z, gr * B.y));
                const float dal = fmaf(Tj, gc, -(rinv * gS));
                gS = fmaf(gc, aTj, gS);
                T = Tj;
                const float h = dal * al;                  // dL/dw * w, with dL/dw = dal * o
                hu = h * u;
                hv = h * v;
                hudx = hu * dx;
                hvdx = hv * dx;
                hvdy = hv * dy;
                dlg = dal * w * R.z;
            }
            const float Hu = wave_total(hu), Hv = wave_total(hv), Hudx = wave_total(hudx);
            const float Hvdx = wave_total(hvdx), Hvdy = wave_total(hvdy);
            const float Cr = wave_total(dcr), Cg = wave_total(dcg), Cb = wave_total(dcb);
            const float Dl = wave_total(dlg);
            if (lane == 0) {
                const float a = A.z, b = A.w, c = B.x;
                const float da = -k2 * Hudx, db = -k2 * Hvdx, dc = -k2 * Hvdy;
                lst[wave][k].p = make_float4(k2 * fmaf(a, Hu, b * Hv), k2 * c * Hv, -is * fmaf(a * a, da, a * b * db),
                                             -is * (a * c * db));
                lst[wave][k].q = make_float4(-is * fmaf(b * c, db, c * c * dc), Cr, Cg, Cb);
                res[8] = Dl;
            }
        }
        __syncthreads();
        if (tid < kBatch && lo + tid < hi) {      // quadrant results of this entry, added in quadrant order
            float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
            float sl = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = qpos[tid][q];
                if (k != 0xff) {
                    const float4 u0 = lst[q][k].p, u1 = lst[q][k].q;
                    s0.x += u0.x; s0.y += u0.y; s0.z += u0.z; s0.w += u0.w;
                    s1.x += u1.x; s1.y += u1.y; s1.z += u1.z; s1.w += u1.w;
                    sl += lst[q][k].r.x;
                }
            }
            const uint32_t slot = eslot[tid];
            if (slot < capacity) {
                part[2 * (size_t)slot] = s0;
                part[2 * (size_t)slot + 1] = s1;
                part_l[slot] = sl;
            }
        }
        hi = lo;
    }
}

static int padded_tiles(int ntiles) { return (ntiles + 7) & ~7; }

hipError_t launch_render_alpha_fwd(int W, int H, const float *records, const float *opacity,
                                   const uint16_t *pixbox, const uint32_t *ranges, const uint32_t *order,
                                   const uint32_t *vals, const float *background, float *image, float *t_final,
                                   uint32_t *last, hipStream_t s) {
    const int tiles_x = (W + kTile - 1) / kTile, ntiles = tiles_x * ((H + kTile - 1) / kTile);
    k_render_alpha_fwd<<<padded_tiles(ntiles), 256, 0, s>>>(
        W, H, tiles_x, ntiles, reinterpret_cast<const float4 *>(records), opacity,
        reinterpret_cast<const uint2 *>(pixbox), reinterpret_cast<const uint2 *>(ranges), order, vals, background,
        image, t_final, last);
    return hipGetLastError();
}

hipError_t launch_render_alpha_bwd(int W, int H, const float *records, const float *opacity, const float *logit,
                                   const uint16_t *pixbox, const uint32_t *offsets, const uint32_t *ranges,
                                   const uint32_t *order, const uint32_t *vals, int64_t capacity,
                                   const float *background,
                                   const float *t_final, const uint32_t *last, const float *dL_dimage, void *ws,
                                   hipStream_t s) {
    const int tiles_x = (W + kTile - 1) / kTile, ntiles = tiles_x * ((H + kTile - 1) / kTile);
    const BwdPlan p = make_bwd_plan(W, H, capacity);
    char *w = static_cast<char *>(ws);
    k_render_alpha_bwd<<<padded_tiles(ntiles), 256, 0, s>>>(
        W, H, tiles_x, ntiles, reinterpret_cast<const float4 *>(records), opacity, logit,
        reinterpret_cast<const uint2 *>(pixbox), offsets, reinterpret_cast<const uint2 *>(ranges), order, vals,
        (uint32_t)capacity, background, t_final, last, dL_dimage, reinterpret_cast<float4 *>(w + p.off_part),
        reinterpret_cast<float *>(w + p.off_logit), reinterpret_cast<float4 *>(w + p.off_bg));
    return hipGetLastError();
}

}  // namespace gi
