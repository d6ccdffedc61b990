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
// The 9 per-pixel contributions of a Gaussian are summed over the wave for 8
// entries at a time, by one butterfly transpose-reduce (skipped when no pixel of
// the wave is covered), and written over the entries' slots in the wave's own
// quadrant list; each list entry then adds its four quadrant sums in quadrant
// order, turns them into the gradients of its record (linear in the sums) and
// stores them at its emission slot for the per-Gaussian gather.  No atomics: the
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
                                           uint32_t *eslot = nullptr, uint8_t (*qpos)[4] = nullptr,
                                           float4 *own = nullptr) {
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
    if (own) *own = make_float4(rp.z, rp.w, rq.x, rr.z);     // a, b, c, so
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

// Butterfly transpose-reduce over the wave: lane l holds 64 values x[i]; on return lane l holds
// the sum over all 64 lanes of x[l].  Each step sums pairs of values across a lane pair and keeps
// one of them, by the lane's side: upper half / lower half (permlane32 swap), odd / even row
// (permlane16 swap), then row mirror, half-row mirror and two quad permutations (DPP).  63 + 63
// swaps / moves and adds per 64 sums, against 64 x 6 for 64 separate reductions.
template <int N>
__device__ __forceinline__ void bfly_swap32(float (&x)[2 * N], float (&y)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[i]), __float_as_uint(x[i + N]), false, false);
        y[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}
template <int N>
__device__ __forceinline__ void bfly_swap16(float (&x)[2 * N], float (&y)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[i]), __float_as_uint(x[i + N]), false, false);
        y[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}
template <int CTRL, int N>
__device__ __forceinline__ void bfly_dpp(float (&x)[2 * N], float (&y)[N], bool low) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float keep = low ? x[i] : x[i + N], send = low ? x[i + N] : x[i];
        y[i] = keep + dpp_f<CTRL>(send);
    }
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
            // without a branch: alpha = 0 leaves T and the colour unchanged (a running sum from +0
            // never becomes -0, so adding c * 0 keeps its bits)
            const bool act = !done && e <= kE9;
            const float al = act ? R.x * exp2_hw(-e) : 0.0f;
            const float aT = al * T;
            cr = fmaf(B.y, aT, cr);
            cg = fmaf(B.z, aT, cg);
            cb = fmaf(B.w, aT, cb);
            T -= aT;
            lst_end = act ? __float_as_uint(R.y) + 1u : lst_end;
            done = T < kTmin;
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
        float4 own;
        const int cnt = stage_alpha(lst, wq, lo, hi, x0, y0, records, opacity, logit, pixbox, vals, below,
                                    offsets, eslot, qpos, &own);
        const AlphaRec *L = lst[wave];
        float *res = reinterpret_cast<float *>(&lst[wave][0]);   // entry k's results: res[12 k + 0..8]
        // groups of 8 entries, back to front; per pixel and entry 9 values (the pixel's parts of
        // sum h u, h v, h u dx, h v dx, h v dy, g aT (3), dL/dalpha w), reduced over the wave together
        for (int k0 = cnt - 1; k0 >= 0; k0 -= 8) {
            float x[64], xo[8];
            bool any = false;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int k = k0 - j;
                if (k < 0) {                                          // uniform
#pragma unroll
                    for (int c = 0; c < 8; ++c) x[8 * j + c] = 0.0f;
                    xo[j] = 0.0f;
                    continue;
                }
                const float4 A = L[k].p, B = L[k].q, R = L[k].r;
                const uint32_t pos = __float_as_uint(R.y);
                const float dx = px - A.x, dy = py - A.y;
                const float u = A.z * dx;
                const float tb = A.w * dx;
                const float v = fmaf(B.x, dy, tb);
                const float e = fmaf(v, v, u * u);
                const bool act = pos < lp && e <= kE9;
                if (__ballot(act) == 0) {                             // uniform
#pragma unroll
                    for (int c = 0; c < 8; ++c) x[8 * j + c] = 0.0f;
                    xo[j] = 0.0f;
                    continue;
                }
                any = true;
                {   // without a branch: w = 0 gives rinv = 1, T and gS unchanged and zero contributions
                    const float w = act ? exp2_hw(-e) : 0.0f;
                    const float al = R.x * w;
                    const float rinv = __builtin_amdgcn_rcpf(1.0f - al);
                    const float Tj = T * rinv;
                    const float aTj = al * Tj;
                    const float gc = fmaf(gb, B.w, fmaf(gg, B.z, gr * B.y));
                    const float dal = fmaf(Tj, gc, -(rinv * gS));
                    gS = fmaf(gc, aTj, gS);
                    T = Tj;
                    const float h = dal * al;                         // dL/dw * w, with dL/dw = dal * o
                    const float hu = h * u, hv = h * v;
                    x[8 * j + 0] = hu;
                    x[8 * j + 1] = hv;
                    x[8 * j + 2] = hu * dx;
                    x[8 * j + 3] = hv * dx;
                    x[8 * j + 4] = hv * dy;
                    x[8 * j + 5] = gr * aTj;
                    x[8 * j + 6] = gg * aTj;
                    x[8 * j + 7] = gb * aTj;
                    xo[j] = dal * w;
                }
            }
            const int kk = k0 - (lane >> 3);                          // this lane's entry after the reduce
            if (!any) {                                               // uniform: no pixel met these entries
                if (kk >= 0) {
                    res[12 * kk + (lane & 7)] = 0.0f;
                    if ((lane & 7) == 0) res[12 * kk + 8] = 0.0f;
                }
                continue;
            }
            float y32[32], y16[16], y8[8], y4[4], y2[2], y1[1];
            bfly_swap32<32>(x, y32);
            bfly_swap16<16>(y32, y16);
            bfly_dpp<0x140, 8>(y16, y8, (lane & 8) == 0);             // row mirror
            bfly_dpp<0x141, 4>(y8, y4, (lane & 4) == 0);              // half-row mirror
            bfly_dpp<0x4e, 2>(y4, y2, (lane & 2) == 0);               // quad: lanes ^ 2
            bfly_dpp<0xb1, 1>(y2, y1, (lane & 1) == 0);               // quad: lanes ^ 1
            // the entries' dL/dalpha w: 8 values, summed within each 8-lane group after three steps
            float o4[4], o2[2], o1[1];
            bfly_swap32<4>(xo, o4);
            bfly_swap16<2>(o4, o2);
            bfly_dpp<0x140, 1>(o2, o1, (lane & 8) == 0);
            float ot = o1[0];
            ot += dpp_f<0x141>(ot);
            ot += dpp_f<0x4e>(ot);
            ot += dpp_f<0xb1>(ot);
            if (kk >= 0) {                                            // lane l: entry k0 - l/8, value l%8
                res[12 * kk + (lane & 7)] = y1[0];
                if ((lane & 7) == 0) res[12 * kk + 8] = ot;
            }
        }
        __syncthreads();
        if (tid < kBatch && lo + tid < hi) {      // quadrant sums of this entry, added in quadrant order
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
            // e = u^2 + v^2, w = 2^-e: dL/de = -ln2 h, summed through (Hu, Hv, ...); then
            // a = S/l11, b = -S l21/(l11 l22), c = S/l22 -> (l11, l21, l22); dL/dlogit = so sum dL/dalpha w
            const float a = own.x, b = own.y, c = own.z;
            const float da = -k2 * s0.z, db = -k2 * s0.w, dc = -k2 * s1.x;
            const float4 d0 = make_float4(k2 * fmaf(a, s0.x, b * s0.y), k2 * c * s0.y,
                                          -is * fmaf(a * a, da, a * b * db), -is * (a * c * db));
            const float4 d1 = make_float4(-is * fmaf(b * c, db, c * c * dc), s1.y, s1.z, s1.w);
            const uint32_t slot = eslot[tid];
            if (slot < capacity) {
                part[2 * (size_t)slot] = d0;
                part[2 * (size_t)slot + 1] = d1;
                part_l[slot] = own.w * sl;
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
