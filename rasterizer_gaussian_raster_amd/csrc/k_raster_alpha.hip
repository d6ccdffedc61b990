// k_raster_alpha.hip -- front-to-back alpha compositing over a background
// ("Drawing with Gaussians", Overview: anisotropic 2D Gaussians alpha-composited
// over a trainable background; fused kernels with custom VJPs) and its backward.
//
// Layout: one workgroup of two waves per 16x16 tile; wave w owns the 8x16 half
// of columns 8w .. 8w + 7, two pixels per lane (rows r and r + 8 of one column,
// which share the Gaussian's x terms); the tile list is staged 128 entries at a
// time, one per thread, and compacted per half in list order.  A Gaussian
// dropped for a half has alpha = 0 at every pixel there, so T and C are
// unchanged by it: compaction keeps the results bit for bit.
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
// The 9 per-pixel contributions of a Gaussian (the slot sums of gi_device.hpp
// with h = (dL/dalpha) alpha, and dL/dalpha w for the logit) are summed over the
// wave for 8 entries at a time, by one butterfly transpose-reduce (skipped when
// no pixel of the wave is covered), and written over the entries' slots in the
// wave's own half list; each list entry then adds its two halves' sums in order
// and stores them at its emission slot for the per-Gaussian gather, which turns
// a Gaussian's total into its gradient.  No atomics: the gradients are bitwise
// reproducible.
#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

struct AlphaRec { float4 p, q, r; };   // p = (mux, muy, a, b), q = (c, cr, cg, cb), r = (o, pos, so, g)

constexpr int kAlphaThreads = 128;    // two waves per tile
constexpr int kBatch = kAlphaThreads; // list entries staged per round, one per thread (12 KB of LDS)

// Halves of the tile at (x0, y0) that the pixel box meets: bit h for columns x0 + 8h .. x0 + 8h + 7.
__device__ __forceinline__ uint32_t half_mask(uint2 bx, int x0, int y0) {
    const int j0 = bx.x & 0xffff, i0 = bx.x >> 16, j1 = bx.y & 0xffff, i1 = bx.y >> 16;
    if (i0 > y0 + 15 || i1 < y0) return 0u;
    uint32_t m = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int hx0 = x0 + 8 * h;
        m |= (j0 <= hx0 + 7 && j1 >= hx0) ? (1u << h) : 0u;
    }
    return m;
}

// The backward's entry record of Gaussian g (64 bytes, so that a list entry is one aligned 64-byte
// read instead of five scattered ones): [4 g] = (mux, muy, a, b), [4 g + 1] = (c, cr, cg, cb),
// [4 g + 2] = (o, so, pixel box (2 x u32 bits)), [4 g + 3] = (emission offset bits, 0, 0, 0), with
// so = o (1 - o) below the logit clamp, else 0 -- the values the separate arrays hold, bit for bit.
struct AlphaPack { float4 p, q, r, s; };

// Stage list entries [lo, hi) (hi - lo <= kBatch) into the per-half lists; returns this wave's count.
// Backward only (pack != nullptr, the entries read from the packed records): also the entry's
// emission slot -> eslot[tid], its position in each half's list -> qpos[tid][h] (0xff: not in that
// list) and its (a, b, c, so) -> *own.
__device__ __forceinline__ int stage_alpha(AlphaRec (*lst)[kBatch], int (*wq)[2], uint32_t lo, uint32_t hi, int x0,
                                           int y0, const float4 *__restrict__ records,
                                           const float *__restrict__ opacity, const uint2 *__restrict__ pixbox,
                                           const uint32_t *__restrict__ vals, uint64_t below,
                                           const AlphaPack *__restrict__ pack = nullptr, uint32_t *eslot = nullptr,
                                           uint8_t (*qpos)[2] = nullptr, float4 *own = nullptr) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint32_t idx = lo + tid;
    uint32_t hm = 0;
    float4 rp = make_float4(0.f, 0.f, 0.f, 0.f), rq = rp, rr = rp;
    if (idx < hi) {
        const uint32_t g = vals[idx];
        if (pack) {
            const AlphaPack e = pack[g];
            rp = e.p;
            rq = e.q;
            rr = make_float4(e.r.x, __uint_as_float(idx), e.r.y, __uint_as_float(g));
            const uint2 bx = make_uint2(__float_as_uint(e.r.z), __float_as_uint(e.r.w));
            hm = half_mask(bx, x0, y0);
            eslot[tid] = emit_slot(__float_as_uint(e.s.x), bx, x0 / kTile, y0 / kTile);
        } else {
            rp = records[2 * g];
            rq = records[2 * g + 1];
            rr = make_float4(opacity[g], __uint_as_float(idx), 0.0f, __uint_as_float(g));
            hm = half_mask(pixbox[g], x0, y0);
        }
    }
    if (own) *own = make_float4(rp.z, rp.w, rq.x, rr.z);     // a, b, c, so
    uint32_t rank[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint64_t m = __ballot((hm >> h) & 1u);
        rank[h] = (uint32_t)__popcll(m & below);
        if (lane == 0) wq[wave][h] = __popcll(m);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if ((hm >> h) & 1u) {
            const int off = (int)rank[h] + (wave ? wq[0][h] : 0);
            lst[h][off].p = rp;
            lst[h][off].q = rq;
            lst[h][off].r = rr;
            if (qpos) qpos[tid][h] = (uint8_t)off;
        } else if (qpos) {
            qpos[tid][h] = 0xff;
        }
    }
    const int cnt = __builtin_amdgcn_readfirstlane(wq[0][wave] + wq[1][wave]);
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

// L2: also dL/dI = gscale (I - T) (what gi_loss_l2 writes, bit for bit) and the tile's sum of
// squared residuals in loss_part[t] (lanes, then the two waves, in a fixed order).
template <bool L2>
__global__ __launch_bounds__(kAlphaThreads) void k_render_alpha_fwd(int W, int H, int tiles_x, int ntiles,
                                                          const float4 *__restrict__ records,
                                                          const float *__restrict__ opacity,
                                                          const uint2 *__restrict__ pixbox,
                                                          const uint2 *__restrict__ ranges, const uint32_t *__restrict__ order,
                                                          const uint32_t *__restrict__ vals,
                                                          const float *__restrict__ bg,
                                                          float *__restrict__ image, float *__restrict__ t_final,
                                                          uint32_t *__restrict__ last, const float *__restrict__ target,
                                                          float *__restrict__ dL, float gscale,
                                                          float *__restrict__ loss_part) {
    __shared__ AlphaRec lst[2][kBatch];
    __shared__ int wq[2][2];
    __shared__ int wdone[2];
    __shared__ float wsq[2];
    const int t = tile_of(blockIdx.x, gridDim.x, ntiles, order);
    if (t >= ntiles) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int x0 = (t % tiles_x) * kTile, y0 = (t / tiles_x) * kTile;
    const int pxi = x0 + wave * 8 + (lane & 7);
    const int pyi = y0 + (lane >> 3);                     // the lane's upper pixel; the lower one is 8 rows down
    const float px = (float)pxi + 0.5f, py0 = (float)pyi + 0.5f, py1 = (float)(pyi + 8) + 0.5f;
    const uint2 rg = ranges[t];
    const uint64_t below = lanes_below();
    float T0 = 1.0f, r0 = 0.f, g0 = 0.f, b0 = 0.f, T1 = 1.0f, r1 = 0.f, g1 = 0.f, b1 = 0.f;
    uint32_t end0 = rg.x, end1 = rg.x;
    bool done0 = false, done1 = false;

    for (uint32_t base = rg.x; base < rg.y; base += kBatch) {
        const uint32_t hi = rg.y - base > (uint32_t)kBatch ? base + kBatch : rg.y;
        const int cnt = stage_alpha(lst, wq, base, hi, x0, y0, records, opacity, pixbox, vals, below);
        const AlphaRec *L = lst[wave];
        for (int k = 0; k < cnt; ++k) {
            if (__ballot(!(done0 && done1)) == 0) break;
            const float4 A = L[k].p, B = L[k].q, R = L[k].r;
            const float dx = px - A.x;
            const float u = A.z * dx;
            const float tb = A.w * dx;
            const float uu = u * u;
            const float v0 = fmaf(B.x, py0 - A.y, tb), v1 = fmaf(B.x, py1 - A.y, tb);
            const float e0 = fmaf(v0, v0, uu), e1 = fmaf(v1, v1, uu);
            // without a branch: alpha = 0 leaves T and the colour unchanged (a running sum from +0
            // never becomes -0, so adding c * 0 keeps its bits)
            const bool a0 = !done0 && e0 <= kE9, a1 = !done1 && e1 <= kE9;
            const float al0 = a0 ? R.x * exp2_hw(-e0) : 0.0f, al1 = a1 ? R.x * exp2_hw(-e1) : 0.0f;
            const float aT0 = al0 * T0, aT1 = al1 * T1;
            r0 = fmaf(B.y, aT0, r0);
            g0 = fmaf(B.z, aT0, g0);
            b0 = fmaf(B.w, aT0, b0);
            r1 = fmaf(B.y, aT1, r1);
            g1 = fmaf(B.z, aT1, g1);
            b1 = fmaf(B.w, aT1, b1);
            T0 -= aT0;
            T1 -= aT1;
            const uint32_t pe = __float_as_uint(R.y) + 1u;
            end0 = a0 ? pe : end0;
            end1 = a1 ? pe : end1;
            done0 = T0 < kTmin;
            done1 = T1 < kTmin;
        }
        const bool wave_done = __ballot(!(done0 && done1)) == 0;   // all lanes vote (outside any branch)
        if (lane == 0) wdone[wave] = wave_done;
        if (hi >= rg.y) break;
        __syncthreads();
        if (wdone[0] && wdone[1]) break;                   // uniform
    }
    const size_t plane = (size_t)W * H;
    float sq = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int yi = pyi + 8 * h;
        if (pxi < W && yi < H) {
            const size_t o = (size_t)yi * W + pxi;
            const float T = h ? T1 : T0;
            const float ir = fmaf(T, bg[0], h ? r1 : r0), ig = fmaf(T, bg[1], h ? g1 : g0);
            const float ib = fmaf(T, bg[2], h ? b1 : b0);
            image[o] = ir;
            image[o + plane] = ig;
            image[o + 2 * plane] = ib;
            t_final[o] = T;
            last[o] = h ? end1 : end0;
            if (L2) {
                const float rr = ir - target[o], rg = ig - target[o + plane], rb = ib - target[o + 2 * plane];
                dL[o] = gscale * rr;
                dL[o + plane] = gscale * rg;
                dL[o + 2 * plane] = gscale * rb;
                sq += fmaf(rb, rb, fmaf(rg, rg, rr * rr));
            }
        }
    }
    if (L2) {
        const float s = wave_total(sq);
        if (lane == 0) wsq[wave] = s;
        __syncthreads();
        if (tid == 0) loss_part[t] = wsq[0] + wsq[1];
    }
}

// One pixel's step back over entry (A, B, R): w = 0 (not touched, or behind the pixel's stop) gives
// rinv = 1, T and gS unchanged and zero contributions.  Returns h = dL/dw w (dL/dw = dL/dalpha o)
// and the pixel's dL/dalpha w, alpha T (through refs).
__device__ __forceinline__ float alpha_back_pixel(bool act, float e, float o, float gr, float gg, float gb,
                                                  float4 B, float &T, float &gS, float &dalw, float &aT) {
    const float w = act ? exp2_hw(-e) : 0.0f;
    const float al = o * w;
    const float rinv = __builtin_amdgcn_rcpf(1.0f - al);
    const float Tj = T * rinv;
    aT = al * Tj;
    const float gc = fmaf(gb, B.w, fmaf(gg, B.z, gr * B.y));
    const float dal = fmaf(Tj, gc, -(rinv * gS));
    gS = fmaf(gc, aT, gS);
    T = Tj;
    dalw = dal * w;
    return dal * al;
}

// The packed entry records of n Gaussians (AlphaPack above), one float4 per thread: coalesced stores.
__global__ __launch_bounds__(256) void k_alpha_pack(int n, const float4 *__restrict__ records,
                                                    const float *__restrict__ opacity, const float *__restrict__ logit,
                                                    const uint2 *__restrict__ pixbox,
                                                    const uint32_t *__restrict__ offsets, float4 *__restrict__ pack) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // float4 i % 4 of Gaussian i / 4
    const int64_t g = i >> 2;
    if (g >= n) return;
    const int k = (int)(i & 3);
    float4 v;
    if (k < 2) {
        v = records[2 * g + k];
    } else if (k == 2) {
        const float o = opacity[g];
        const float so = logit ? (logit[g] < kLogitMax ? o * (1.0f - o) : 0.0f) : 0.0f;
        const uint2 bx = pixbox[g];
        v = make_float4(o, so, __uint_as_float(bx.x), __uint_as_float(bx.y));
    } else {
        v = make_float4(__uint_as_float(offsets[g]), 0.0f, 0.0f, 0.0f);
    }
    pack[i] = v;
}

__global__ __launch_bounds__(kAlphaThreads) void k_render_alpha_bwd(int W, int H, int tiles_x, int ntiles,
                                                          const AlphaPack *__restrict__ pack,
                                                          const uint2 *__restrict__ ranges, const uint32_t *__restrict__ order,
                                                          const uint32_t *__restrict__ vals, uint32_t capacity,
                                                          const float *__restrict__ bg,
                                                          const float *__restrict__ t_final,
                                                          const uint32_t *__restrict__ last,
                                                          const float *__restrict__ dL,
                                                          float4 *__restrict__ part, float *__restrict__ part_l,
                                                          float4 *__restrict__ part_bg) {
    __shared__ AlphaRec lst[2][kBatch];
    __shared__ int wq[2][2];
    __shared__ uint32_t wmax[2];
    __shared__ float wbg[2][3];
    __shared__ uint32_t eslot[kBatch];
    __shared__ uint8_t qpos[kBatch][2];
    const int t = tile_of(blockIdx.x, gridDim.x, ntiles, order);
    if (t >= ntiles) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int x0 = (t % tiles_x) * kTile, y0 = (t / tiles_x) * kTile;
    const int pxi = x0 + wave * 8 + (lane & 7);
    const int pyi = y0 + (lane >> 3);                     // the lane's upper pixel; the lower one is 8 rows down
    const float px = (float)pxi + 0.5f, py0 = (float)pyi + 0.5f, py1 = (float)(pyi + 8) + 0.5f;
    const uint2 rg = ranges[t];
    const uint64_t below = lanes_below();
    const size_t plane = (size_t)W * H;
    float T0 = 0.f, gr0 = 0.f, gg0 = 0.f, gb0 = 0.f, T1 = 0.f, gr1 = 0.f, gg1 = 0.f, gb1 = 0.f;
    uint32_t lp0 = rg.x, lp1 = rg.x;
    if (pxi < W && pyi < H) {
        const size_t o = (size_t)pyi * W + pxi;
        T0 = t_final[o];
        lp0 = min(max(last[o], rg.x), rg.y);     // stays inside the tile's list whatever `last` holds
        gr0 = dL[o];
        gg0 = dL[o + plane];
        gb0 = dL[o + 2 * plane];
    }
    if (pxi < W && pyi + 8 < H) {
        const size_t o = (size_t)(pyi + 8) * W + pxi;
        T1 = t_final[o];
        lp1 = min(max(last[o], rg.x), rg.y);
        gr1 = dL[o];
        gg1 = dL[o + plane];
        gb1 = dL[o + 2 * plane];
    }
    // dL/dbg_k = sum_p g_k T_final: one partial per tile
    {
        const float sr = wave_total(fmaf(gr1, T1, gr0 * T0)), sg = wave_total(fmaf(gg1, T1, gg0 * T0));
        const float sb = wave_total(fmaf(gb1, T1, gb0 * T0));
        if (lane == 0) { wbg[wave][0] = sr; wbg[wave][1] = sg; wbg[wave][2] = sb; }
        uint32_t m = max(lp0, lp1);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
        if (lane == 0) wmax[wave] = m;
    }
    __syncthreads();
    if (tid == 0)
        part_bg[t] = make_float4(wbg[0][0] + wbg[1][0], wbg[0][1] + wbg[1][1], wbg[0][2] + wbg[1][2], 0.f);
    const uint32_t bend0 = max(wmax[0], wmax[1]);
    // entries behind every pixel's stop contribute nothing: their slots get zeros
    for (uint32_t idx = bend0 + tid; idx < rg.y; idx += kAlphaThreads) {
        const AlphaPack &e = pack[vals[idx]];
        const uint32_t slot = emit_slot(__float_as_uint(e.s.x), make_uint2(__float_as_uint(e.r.z), __float_as_uint(e.r.w)),
                                        x0 / kTile, y0 / kTile);
        if (slot < capacity) {
            part[2 * (size_t)slot] = make_float4(0.f, 0.f, 0.f, 0.f);
            part[2 * (size_t)slot + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
            part_l[slot] = 0.f;
        }
    }
    float gS0 = T0 * fmaf(gb0, bg[2], fmaf(gg0, bg[1], gr0 * bg[0]));
    float gS1 = T1 * fmaf(gb1, bg[2], fmaf(gg1, bg[1], gr1 * bg[0]));

    for (uint32_t hi = bend0; hi > rg.x;) {
        const uint32_t lo = hi - rg.x > (uint32_t)kBatch ? hi - kBatch : rg.x;
        __syncthreads();                                   // previous batch fully consumed
        float4 own;
        const int cnt = stage_alpha(lst, wq, lo, hi, x0, y0, nullptr, nullptr, nullptr, vals, below, pack, eslot,
                                    qpos, &own);
        const AlphaRec *L = lst[wave];
        float *res = reinterpret_cast<float *>(&lst[wave][0]);   // entry k's results: res[12 k + 0..8]
        // groups of 8 entries, back to front; per lane (two pixels) and entry 9 values (the pixels'
        // parts of sum h u, h v, h u dx, h v dx, h v dy, g aT (3), dL/dalpha w), reduced over the
        // wave together
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
                const float dx = px - A.x;
                const float dy0 = py0 - A.y, dy1 = py1 - A.y;
                const float u = A.z * dx;
                const float tb = A.w * dx;
                const float uu = u * u;
                const float v0 = fmaf(B.x, dy0, tb), v1 = fmaf(B.x, dy1, tb);
                const float e0 = fmaf(v0, v0, uu), e1 = fmaf(v1, v1, uu);
                const bool act0 = pos < lp0 && e0 <= kE9, act1 = pos < lp1 && e1 <= kE9;
                if (__ballot(act0 || act1) == 0) {                    // uniform
#pragma unroll
                    for (int c = 0; c < 8; ++c) x[8 * j + c] = 0.0f;
                    xo[j] = 0.0f;
                    continue;
                }
                any = true;
                float dw0, dw1, aT0, aT1;
                const float h0 = alpha_back_pixel(act0, e0, R.x, gr0, gg0, gb0, B, T0, gS0, dw0, aT0);
                const float h1 = alpha_back_pixel(act1, e1, R.x, gr1, gg1, gb1, B, T1, gS1, dw1, aT1);
                const float hu = u * (h0 + h1);                       // u is the two pixels'
                const float hv0 = h0 * v0, hv1 = h1 * v1;
                const float hv = hv0 + hv1;
                x[8 * j + 0] = hu;
                x[8 * j + 1] = hv;
                x[8 * j + 2] = hu * u;
                x[8 * j + 3] = hv * u;
                x[8 * j + 4] = fmaf(hv1, v1, hv0 * v0);
                x[8 * j + 5] = fmaf(gr1, aT1, gr0 * aT0);
                x[8 * j + 6] = fmaf(gg1, aT1, gg0 * aT0);
                x[8 * j + 7] = fmaf(gb1, aT1, gb0 * aT0);
                xo[j] = dw0 + dw1;
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
        if (lo + tid < hi) {                      // the two halves' sums of this entry, added in order
            float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
            float sl = 0.f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = qpos[tid][h];
                if (k != 0xff) {
                    const float4 u0 = lst[h][k].p, u1 = lst[h][k].q;
                    s0.x += u0.x; s0.y += u0.y; s0.z += u0.z; s0.w += u0.w;
                    s1.x += u1.x; s1.y += u1.y; s1.z += u1.z; s1.w += u1.w;
                    sl += lst[h][k].r.x;
                }
            }
            // the pair's sums as they are (slot layout in gi_device.hpp; the gather turns a Gaussian's
            // total into its gradient); dL/dlogit = so sum dL/dalpha w
            const uint32_t slot = eslot[tid];
            if (slot < capacity) {
                part[2 * (size_t)slot] = s0;
                part[2 * (size_t)slot + 1] = s1;
                part_l[slot] = own.w * sl;
            }
        }
        hi = lo;
    }
}

static int padded_tiles(int ntiles) { return (ntiles + 7) & ~7; }

// The alpha training step's update in one pass: each Gaussian's per-pair slots (8 values and the
// logit's) added in emission order (as k_grad_gather; two lanes per Gaussian, four values each),
// and the Adam step of its 8 params and its logit; the second-to-last workgroup adds up the tiles'
// background partials (as k_grad_gather) and steps the background's 3 channels; the last one
// reduces the loss partials.
__global__ __launch_bounds__(256) void k_adam_pairs_alpha(int n, int ntiles, const uint32_t *__restrict__ offsets,
                                                          uint32_t capacity, const float4 *__restrict__ part,
                                                          const float *__restrict__ part_l,
                                                          const float4 *__restrict__ part_bg, float4 *__restrict__ p,
                                                          float4 *__restrict__ m, float4 *__restrict__ v, AdamHP a,
                                                          float *__restrict__ logit, float *__restrict__ ml,
                                                          float *__restrict__ vl, float lr_logit,
                                                          float *__restrict__ bg, float *__restrict__ mbg,
                                                          float *__restrict__ vbg, float lr_bg,
                                                          const float *__restrict__ loss_part, double inv_count,
                                                          float *__restrict__ loss) {
    const int nb = (int)((2 * (int64_t)n + 255) / 256);
    float c1, c2;
    adam_step_bias(a, c1, c2);
    const bool ok = offsets[n] <= capacity;               // else the binning overflowed: zero gradients
    if ((int)blockIdx.x == nb) {                          // the background
        __shared__ float4 sm[256];
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok)
            for (int t = threadIdx.x; t < ntiles; t += 256) {
                const float4 u = part_bg[t];
                s.x += u.x; s.y += u.y; s.z += u.z;
            }
        sm[threadIdx.x] = s;
        __syncthreads();
        for (int o = 128; o > 0; o >>= 1) {
            if (threadIdx.x < o) {
                sm[threadIdx.x].x += sm[threadIdx.x + o].x;
                sm[threadIdx.x].y += sm[threadIdx.x + o].y;
                sm[threadIdx.x].z += sm[threadIdx.x + o].z;
            }
            __syncthreads();
        }
        if (threadIdx.x < 3) {
            const float G = threadIdx.x == 0 ? sm[0].x : threadIdx.x == 1 ? sm[0].y : sm[0].z;
            float P = bg[threadIdx.x], Mo = mbg[threadIdx.x], V = vbg[threadIdx.x];
            adam_update(P, G, Mo, V, lr_bg, a, c1, c2);
            bg[threadIdx.x] = P;
            mbg[threadIdx.x] = Mo;
            vbg[threadIdx.x] = V;
        }
        return;
    }
    if ((int)blockIdx.x == nb + 1) {                      // the loss
        if (loss) {
            __shared__ double sd[256];
            loss_reduce_block(ntiles, loss_part, inv_count, loss, sd);
        }
        return;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // lane h = i & 1 of Gaussian i >> 1: params 4h .. 4h + 3
    const int64_t g = i >> 1;
    const int h = (int)(i & 1);
    if (g >= n) return;
    const uint32_t o0 = offsets[g], o1 = ok ? offsets[g + 1] : o0;
    float4 gr = make_float4(0.f, 0.f, 0.f, 0.f);
    gather_half(reinterpret_cast<const float4 *>(part), o0, o1, h, gr);
    const float4 a4 = p[2 * g + h], m4 = m[2 * g + h], v4 = v[2 * g + h];
    {                                                     // sums -> gradient, with the record's rows
        const float4 o4 = make_float4(__shfl_xor(a4.x, 1, 64), __shfl_xor(a4.y, 1, 64), __shfl_xor(a4.z, 1, 64),
                                      __shfl_xor(a4.w, 1, 64));
        const float4 A0 = h ? o4 : a4, A1 = h ? a4 : o4;
        const float3 r = conic_rows(A0.z, A0.w, A1.x);
        gr = o1 > o0 ? slot_grad_half(h, r.x, r.y, r.z, gr) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float P[4] = {a4.x, a4.y, a4.z, a4.w};
    const float G[4] = {gr.x, gr.y, gr.z, gr.w};
    float M[4] = {m4.x, m4.y, m4.z, m4.w};
    float V[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) adam_update(P[k], G[k], M[k], V[k], a.lr[4 * h + k], a, c1, c2);
    p[2 * g + h] = make_float4(P[0], P[1], P[2], P[3]);
    m[2 * g + h] = make_float4(M[0], M[1], M[2], M[3]);
    v[2 * g + h] = make_float4(V[0], V[1], V[2], V[3]);
    if (h == 1) {
        float dl = 0.f;
        for (uint32_t q = o0; q < o1; ++q) dl += part_l[q];
        float L = logit[g], Ml = ml[g], Vl = vl[g];
        adam_update(L, dl, Ml, Vl, lr_logit, a, c1, c2);
        logit[g] = L;
        ml[g] = Ml;
        vl[g] = Vl;
    }
}

hipError_t launch_adam_pairs_alpha(int n, int W, int H, const uint32_t *offsets, int64_t capacity, const void *ws,
                                   float *p, float *m, float *v, const float *lr, float *logit, float *ml, float *vl,
                                   float lr_logit, float *bg, float *mbg, float *vbg, float lr_bg, double beta1,
                                   double beta2, double eps, int step, const float *loss_partials, int64_t loss_count,
                                   float *d_loss, hipStream_t s) {
    const int ntiles = ((W + kTile - 1) / kTile) * ((H + kTile - 1) / kTile);
    const BwdPlan pl = make_bwd_plan(W, H, capacity);
    const AdamHP a = make_adam_hp(lr, beta1, beta2, eps, step, nullptr);
    const char *w = static_cast<const char *>(ws);
    k_adam_pairs_alpha<<<(unsigned)((2 * (int64_t)n + 255) / 256) + 2, 256, 0, s>>>(
        n, ntiles, offsets, (uint32_t)capacity, reinterpret_cast<const float4 *>(w + pl.off_part),
        reinterpret_cast<const float *>(w + pl.off_logit), reinterpret_cast<const float4 *>(w + pl.off_bg),
        reinterpret_cast<float4 *>(p), reinterpret_cast<float4 *>(m), reinterpret_cast<float4 *>(v), a, logit, ml, vl,
        lr_logit, bg, mbg, vbg, lr_bg, loss_partials, loss_count > 0 ? 1.0 / (double)loss_count : 0.0, d_loss);
    return hipGetLastError();
}

hipError_t launch_render_alpha_fwd(int W, int H, const float *records, const float *opacity,
                                   const uint16_t *pixbox, const uint32_t *ranges, const uint32_t *order,
                                   const uint32_t *vals, const float *background, float *image, float *t_final,
                                   uint32_t *last, hipStream_t s, const float *target, float *dL,
                                   float *loss_part) {
    const int tiles_x = (W + kTile - 1) / kTile, ntiles = tiles_x * ((H + kTile - 1) / kTile);
    if (target) {
        const float gscale = (float)(2.0 / (3.0 * (double)W * (double)H));
        k_render_alpha_fwd<true><<<padded_tiles(ntiles), kAlphaThreads, 0, s>>>(
            W, H, tiles_x, ntiles, reinterpret_cast<const float4 *>(records), opacity,
            reinterpret_cast<const uint2 *>(pixbox), reinterpret_cast<const uint2 *>(ranges), order, vals, background,
            image, t_final, last, target, dL, gscale, loss_part);
    } else {
        k_render_alpha_fwd<false><<<padded_tiles(ntiles), kAlphaThreads, 0, s>>>(
            W, H, tiles_x, ntiles, reinterpret_cast<const float4 *>(records), opacity,
            reinterpret_cast<const uint2 *>(pixbox), reinterpret_cast<const uint2 *>(ranges), order, vals, background,
            image, t_final, last, nullptr, nullptr, 0.0f, nullptr);
    }
    return hipGetLastError();
}

// The alpha backward's workspace: the pair slots of make_bwd_plan, then the packed entry records.
size_t alpha_bwd_workspace_bytes(int W, int H, int64_t n, int64_t capacity) {
    return make_bwd_plan(W, H, capacity).bytes + (((size_t)(n > 0 ? n : 1) * sizeof(AlphaPack) + 255) & ~(size_t)255);
}

hipError_t launch_render_alpha_bwd(int W, int H, int64_t n, const float *records, const float *opacity,
                                   const float *logit, const uint16_t *pixbox, const uint32_t *offsets,
                                   const uint32_t *ranges, const uint32_t *order, const uint32_t *vals,
                                   int64_t capacity, const float *background, const float *t_final,
                                   const uint32_t *last, const float *dL_dimage, void *ws, hipStream_t s) {
    const int tiles_x = (W + kTile - 1) / kTile, ntiles = tiles_x * ((H + kTile - 1) / kTile);
    const BwdPlan p = make_bwd_plan(W, H, capacity);
    char *w = static_cast<char *>(ws);
    AlphaPack *pack = reinterpret_cast<AlphaPack *>(w + p.bytes);
    if (n > 0)
        k_alpha_pack<<<(unsigned)((4 * n + 255) / 256), 256, 0, s>>>(
            (int)n, reinterpret_cast<const float4 *>(records), opacity, logit, reinterpret_cast<const uint2 *>(pixbox),
            offsets, reinterpret_cast<float4 *>(pack));
    k_render_alpha_bwd<<<padded_tiles(ntiles), kAlphaThreads, 0, s>>>(
        W, H, tiles_x, ntiles, pack, reinterpret_cast<const uint2 *>(ranges), order, vals,
        (uint32_t)capacity, background, t_final, last, dL_dimage, reinterpret_cast<float4 *>(w + p.off_part),
        reinterpret_cast<float *>(w + p.off_logit), reinterpret_cast<float4 *>(w + p.off_bg));
    return hipGetLastError();
}

}  // namespace gi
