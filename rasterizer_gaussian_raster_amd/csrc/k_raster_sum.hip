// k_raster_sum.hip -- accumulated-sum rasterization ("GaussianImage", Overview:
// rendering by accumulated summation of 2D Gaussians) and its backward.
//
// Forward (pixel-major).  One workgroup of 4 waves per 16x16 tile; wave w owns
// the 8x8 quadrant q = (w + t) mod 4 of tile t, at (q & 1, q >> 1), one pixel per
// lane (rotated by tile, so that a SIMD's waves hold a mix of the quadrants).  The tile's list is
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
// of the binned pairs at the benchmark shapes).  Each wave takes a quarter of
// the tile's entries and packs their items 64 per round, one per lane, entry
// by entry (no lane idles on a short list and no pair outside the box is
// evaluated); after the tile's dL/dI is in LDS the waves never wait for one
// another.  A lane walks its block's 16 pixels (dL/dI staged in LDS), keeping
// the pair's sums in registers with the column-invariant factors (dx, u, b dx,
// u^2) hoisted.  The sums are taken in the Gaussian's whitened frame (u, v):
// with h = (dL/dw) w, the slot holds (sum h u, sum h v, sum h u^2, sum h u v,
// sum h v^2) and the three colour sums sum g_k w -- the gradient of any
// parameterisation of the covariance is a linear map of these, applied once per
// Gaussian after the gather (slot_grad_cholesky; the rotation-scale form's map
// is orthogonal up to scale factors, so it adds no cancellation).  Each entry
// adds up its items in a fixed order and stores its 8 values at its emission
// slot for the per-Gaussian gather: no atomics anywhere, so the gradients are
// bitwise reproducible.
#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

struct SumRec { float4 p, q; };   // p = (mux, muy, a, b), q = (c, cr, cg, cb)

constexpr int kFwdBatch = 128;    // list entries staged per round (16 KB of LDS: 8+ workgroups per CU)

// Backward work item: one (list entry, 4x4 pixel block) pair.  Each wave takes
// a quarter of every batch of list entries and lists their items entry by entry
// (blocks ascending); with R = ceil(items / 64), lane l takes the run of items
// [l R, l R + R) and adds them up in registers, entry by entry.  A run meets at
// most a few entries and an entry spans few runs: each (entry, run) partial
// goes to an LDS slot -- the entry's first run to slot e, a run that continues
// an entry from the lane before to slot kWaveEnt + l -- and each entry finally
// adds its partials in run order.  No atomics; the result does not depend on
// timing.
constexpr int kBwdBatch = 128;                    // list entries per block round, split over the 4 waves
constexpr int kWaveEnt = kBwdBatch / 4;           // entries a wave takes per round (at most)
constexpr int kBwdWavesPerSimd = 6;              // occupancy the backward kernels are built for (<= 80
                                                  // VGPRs): 6 tile workgroups per CU, all 1536 tiles of a
                                                  // 768x512 image resident at once
constexpr int kGpStride = 17;                     // padded LDS run of one 4x4 block's dL/dI (float4):
                                                  // the 16 blocks' pixels at one offset span all
                                                  // 8 bank groups (at most 2-way conflicts)

// LDS of the two phases; the fused kernel overlays them (the forward's lists
// are dead once the tile's image is formed).
struct FwdLds {
    SumRec lst[4][kFwdBatch];                     // per quadrant: the batch's entries that touch it
    int wq[4][4];                                 // [wave][quadrant]: staged count this batch
};
struct BwdLds {
    float4 entp[4][kWaveEnt], entq[4][kWaveEnt];  // per wave: its staged entries (p, q)
    uint16_t items[4][kWaveEnt * 16];             // per wave: entry | block << 8, entry-major
    float4 part[4][kWaveEnt + 64][2];             // per wave: (entry, run) partial sums
};
constexpr size_t kPhaseLds = sizeof(FwdLds) > sizeof(BwdLds) ? sizeof(FwdLds) : sizeof(BwdLds);

// One lane's entry of a wave's share, loaded into registers.
struct BwdEntry {
    float4 p, q;
    uint2 box;
    uint32_t g;            // the Gaussian (its emission offset is loaded by the backward itself)
};

// List entry i.  fresh: the list was written by this workgroup during this
// launch, so the load bypasses the CU's L1 (agent-scope atomic load).
__device__ __forceinline__ uint32_t load_list(const uint32_t *vals, uint32_t i, bool fresh) {
    return fresh ? __hip_atomic_load(vals + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : vals[i];
}

// This wave's share of the batch at `base`: entries [e0, e0 + ne) (wave-uniform).
__device__ __forceinline__ void bwd_share(uint2 rg, uint32_t base, uint32_t &e0, uint32_t &ne) {
    const uint32_t nb = min((uint32_t)kBwdBatch, rg.y - base);
    const uint32_t q = (nb + 3) >> 2;
    e0 = base + (uint32_t)(threadIdx.x >> 6) * q;
    const uint32_t end = base + nb;
    ne = e0 < end ? min(q, end - e0) : 0u;
}

// Forward of one tile for this thread's pixel (px, py) = pixel centre: the
// three channel sums over the tile's list in list order.  The list is staged
// 128 entries at a time, wave w loading the w-th quarter of the batch (the
// backward's share layout); each entry's pixel box is tested against the four
// 8x8 quadrants and the records are compacted, in list order, into one LDS
// list per quadrant; the wave walks quadrant quad's list.  With `first`, this lane's
// entry of the first batch is also kept there: the backward's first share,
// loaded once for both passes.  With tl0, the first batch's Gaussians come from
// that LDS copy of the list instead of vals.  On return other waves
// may still read S: barrier before reusing it.
__device__ __forceinline__ void sum_fwd_tile(FwdLds &S, int x0, int y0, uint2 rg, const float4 *__restrict__ records,
                                             const uint2 *__restrict__ pixbox, const uint32_t *__restrict__ vals,
                                             const uint32_t *tl0, BwdEntry *first, int quad, float px,
                                             float py, float &ar, float &ag, float &ab) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint64_t below = lanes_below();
    for (uint32_t base = rg.x; base < rg.y; base += kFwdBatch) {
        uint32_t e0, ne;
        bwd_share(rg, base, e0, ne);
        uint32_t qm = 0;
        SumRec r;
        r.p = r.q = make_float4(0.f, 0.f, 0.f, 0.f);
        uint2 bx = make_uint2(1u, 0u);
        uint32_t g = 0u;
        if ((uint32_t)lane < ne) {
            g = (tl0 && base == rg.x) ? tl0[e0 - rg.x + lane] : load_list(vals, e0 + lane, tl0 != nullptr);
            r.p = records[2 * g];
            r.q = records[2 * g + 1];
            bx = pixbox[g];
            const int j0 = bx.x & 0xffff, i0 = bx.x >> 16, j1 = bx.y & 0xffff, i1 = bx.y >> 16;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int qx0 = x0 + (q & 1) * 8, qy0 = y0 + (q >> 1) * 8;
                qm |= (j0 <= qx0 + 7 && j1 >= qx0 && i0 <= qy0 + 7 && i1 >= qy0) ? (1u << q) : 0u;
            }
        }
        if (first && base == rg.x) {
            first->p = r.p;
            first->q = r.q;
            first->box = bx;
            first->g = g;
        }
        uint32_t rank[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint64_t m = __ballot((qm >> q) & 1u);
            rank[q] = (uint32_t)__popcll(m & below);
            if (lane == 0) S.wq[wave][q] = __popcll(m);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if ((qm >> q) & 1u) {
                int o = rank[q];
                for (int w = 0; w < wave; ++w) o += S.wq[w][q];
                S.lst[q][o] = r;
            }
        }
        const int cnt = __builtin_amdgcn_readfirstlane(S.wq[0][quad] + S.wq[1][quad] + S.wq[2][quad] + S.wq[3][quad]);
        __syncthreads();
        const SumRec *L = S.lst[quad];
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
}

// Writes the image (and the L2 terms) of this thread's pixel and, with a
// target, each wave's sum of squared residuals to wsq.  Returns the pixel's
// dL/dI (zero off the image).  The caller's next barrier publishes wsq; then
// loss_part_store writes the tile's sum.
template <bool L2>
__device__ __forceinline__ float4 sum_fwd_store(int W, int H, int pxi, int pyi, int t, float ar, float ag, float ab,
                                                float *__restrict__ image, const float *__restrict__ target,
                                                float *__restrict__ dL, float gscale, float *__restrict__ loss_part,
                                                float *wsq /* LDS [4] */) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float sq = 0.0f;
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
    if (pxi < W && pyi < H) {
        const size_t o = (size_t)pyi * W + pxi, plane = (size_t)W * H;
        image[o] = ar;
        image[o + plane] = ag;
        image[o + 2 * plane] = ab;
        if (L2) {
            const float rr = ar - target[o], rgr = ag - target[o + plane], rbr = ab - target[o + 2 * plane];
            g = make_float4(gscale * rr, gscale * rgr, gscale * rbr, 0.f);
            if (dL) {
                dL[o] = g.x;
                dL[o + plane] = g.y;
                dL[o + 2 * plane] = g.z;
            }
            sq = fmaf(rbr, rbr, fmaf(rgr, rgr, rr * rr));
        }
    }
    if (L2) {
        const float ws = wave_total(sq);
        if (lane == 0) wsq[wave] = ws;
    }
    return g;
}

// The tile's sum of squared residuals, in a fixed order (after the barrier that publishes wsq).
__device__ __forceinline__ void loss_part_store(int t, const float *wsq, float *__restrict__ loss_part) {
    if (threadIdx.x == 0) loss_part[t] = ((wsq[0] + wsq[1]) + wsq[2]) + wsq[3];
}

// Tile t's list from its first-pass bucket (entries of the tiles sharing t's
// high digit, in emission order): the entries with key t, in bucket order, are
// the tile's list (the stable sort), placed after the bucket's entries with
// smaller keys.  Writes them to kout / vout and the range to ranges -- what the
// bucket pass writes -- and the first kFwdBatch Gaussians to tl.  Buckets are
// read 2048 entries at a time (one round for the usual sizes).  sc: LDS
// scratch of 2 + 8 rows of 4.  Ends with a barrier.
constexpr int kBucketPL = 8;
__device__ __forceinline__ uint2 bucket_tile_list(const BucketList &B, int t, uint32_t *tl, uint32_t (*sc)[4]) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint64_t below = lanes_below();
    uint2 *ranges = reinterpret_cast<uint2 *>(B.ranges);
    // the bucket's bounds (always in bounds to read) load together with M: the test below uses both,
    // so the chain of dependent loads is tile -> (M, bounds) -> entries
    const uint32_t b = (uint32_t)t >> B.lo_bits, tt = (uint32_t)t;
    const uint32_t s0 = B.bstart[b], s1 = B.bstart[b + 1];
    if (*B.m_eff == 0u || s1 < s0) {                      // nothing binned (or overflow): uniform
        if (tid == 0) ranges[t] = make_uint2(0u, 0u);
        return make_uint2(0u, 0u);
    }
    constexpr uint32_t CH = 256u * kBucketPL;
    const bool one = s1 - s0 <= CH;                       // uniform: keep the chunk in registers
    uint32_t k[kBucketPL], v[kBucketPL];
    if (one) {                                            // one round of loads, one barrier for counts and ranks
        uint64_t m[kBucketPL];
        uint32_t wl = 0;
#pragma unroll
        for (int i = 0; i < kBucketPL; ++i) {
            const uint32_t idx = s0 + (uint32_t)(i * 256 + tid);
            k[i] = idx < s1 ? B.kin[idx] : 0xffffffffu;
            v[i] = idx < s1 ? B.vin[idx] : 0u;
        }
#pragma unroll
        for (int i = 0; i < kBucketPL; ++i) {
            m[i] = __ballot(k[i] == tt);
            wl += (uint32_t)__popcll(__ballot(k[i] < tt));
            if (lane == 0) sc[2 + i][wave] = (uint32_t)__popcll(m[i]);
        }
        if (lane == 0) sc[0][wave] = wl;
        __syncthreads();
        const uint32_t lt = ((sc[0][0] + sc[0][1]) + sc[0][2]) + sc[0][3];
        uint32_t base = 0;
#pragma unroll
        for (int i = 0; i < kBucketPL; ++i) {
            uint32_t before = 0, all = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t c = sc[2 + i][w];
                before += w < wave ? c : 0u;
                all += c;
            }
            if (k[i] == tt) {
                const uint32_t r = base + before + (uint32_t)__popcll(m[i] & below);
                B.kout[s0 + lt + r] = tt;
                B.vout[s0 + lt + r] = v[i];
                if (r < (uint32_t)kFwdBatch) tl[r] = v[i];
            }
            base += all;
        }
        const uint2 rg = base ? make_uint2(s0 + lt, s0 + lt + base) : make_uint2(0u, 0u);
        if (tid == 0) ranges[t] = rg;
        __syncthreads();                                  // publishes tl / vout
        return rg;
    }
    // pass 1: entries below t and equal to t, per wave
    uint32_t wl = 0, we = 0;
    for (uint32_t c0 = s0; c0 < s1; c0 += CH) {
#pragma unroll
        for (int i = 0; i < kBucketPL; ++i) {
            const uint32_t idx = c0 + (uint32_t)(i * 256 + tid);
            k[i] = idx < s1 ? B.kin[idx] : 0xffffffffu;
            if (one) v[i] = idx < s1 ? B.vin[idx] : 0u;
        }
#pragma unroll
        for (int i = 0; i < kBucketPL; ++i) {
            wl += (uint32_t)__popcll(__ballot(k[i] < tt));
            we += (uint32_t)__popcll(__ballot(k[i] == tt));
        }
    }
    if (lane == 0) { sc[0][wave] = wl; sc[1][wave] = we; }
    __syncthreads();
    const uint32_t lt = ((sc[0][0] + sc[0][1]) + sc[0][2]) + sc[0][3];
    const uint32_t eq = ((sc[1][0] + sc[1][1]) + sc[1][2]) + sc[1][3];
    const uint2 rg = eq ? make_uint2(s0 + lt, s0 + lt + eq) : make_uint2(0u, 0u);
    if (tid == 0) ranges[t] = rg;
    // pass 2: ranks of the tile's entries in bucket order (chunk, register, wave, lane)
    uint32_t r0 = 0;
    for (uint32_t c0 = s0; c0 < s1 && r0 < eq; c0 += CH) {   // uniform
        if (!one) {
#pragma unroll
            for (int i = 0; i < kBucketPL; ++i) {
                const uint32_t idx = c0 + (uint32_t)(i * 256 + tid);
                k[i] = idx < s1 ? B.kin[idx] : 0xffffffffu;
                v[i] = idx < s1 ? B.vin[idx] : 0u;
            }
        }
        uint64_t m[kBucketPL];
#pragma unroll
        for (int i = 0; i < kBucketPL; ++i) {
            m[i] = __ballot(k[i] == tt);
            if (lane == 0) sc[2 + i][wave] = (uint32_t)__popcll(m[i]);
        }
        __syncthreads();
        uint32_t base = r0;
#pragma unroll
        for (int i = 0; i < kBucketPL; ++i) {
            uint32_t before = 0, all = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t c = sc[2 + i][w];
                before += w < wave ? c : 0u;
                all += c;
            }
            if (k[i] == tt) {
                const uint32_t r = base + before + (uint32_t)__popcll(m[i] & below);
                B.kout[rg.x + r] = tt;
                B.vout[rg.x + r] = v[i];
                if (r < (uint32_t)kFwdBatch) tl[r] = v[i];
            }
            base += all;
        }
        r0 = base;
        __syncthreads();                                  // sc is rewritten next chunk; publishes tl / vout
    }
    return rg;
}

// L2 = true also forms the L2 loss gradient 2 (I - T) / (3 W H) from the target
// and each tile's sum of squared residuals (reduced over the tile in a fixed order).
// With bl, each tile's list is taken from its first-pass bucket (and written
// out) instead of ranges / vals.
template <bool L2>
__global__ __launch_bounds__(256) void k_render_sum_fwd(int W, int H, int tiles_x, int ntiles,
                                                        const float4 *__restrict__ records,
                                                        const uint2 *__restrict__ pixbox,
                                                        const uint2 *__restrict__ ranges, const uint32_t *__restrict__ order,
                                                        const uint32_t *vals,
                                                        float *__restrict__ image,
                                                        const float *__restrict__ target,
                                                        float *__restrict__ dL, float gscale,
                                                        float *__restrict__ loss_part, BucketList bl) {
    __shared__ FwdLds S;
    __shared__ float wsq[4];
    __shared__ uint32_t tl[kFwdBatch];
    __shared__ uint32_t sc[2 + kBucketPL][4];
    const int t = tile_of(blockIdx.x, gridDim.x, ntiles, order);
    if (t >= ntiles) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int x0 = (t % tiles_x) * kTile, y0 = (t / tiles_x) * kTile;
    const int quad = (wave + t) & 3;                      // the wave's quadrant, rotated by tile
    const int pxi = x0 + (quad & 1) * 8 + (lane & 7);
    const int pyi = y0 + (quad >> 1) * 8 + (lane >> 3);
    const bool bucket = bl.kin != nullptr;                // uniform
    const uint2 rg = bucket ? bucket_tile_list(bl, t, tl, sc) : ranges[t];
    float ar = 0.0f, ag = 0.0f, ab = 0.0f;
    sum_fwd_tile(S, x0, y0, rg, records, pixbox, bucket ? bl.vout : vals, bucket ? tl : nullptr, nullptr, quad,
                 (float)pxi + 0.5f, (float)pyi + 0.5f, ar, ag, ab);
    sum_fwd_store<L2>(W, H, pxi, pyi, t, ar, ag, ab, image, target, dL, gscale, loss_part, wsq);
    if (L2) {
        __syncthreads();
        loss_part_store(t, wsq, loss_part);
    }
}

__global__ __launch_bounds__(256) void k_loss_reduce(int nparts, const float *__restrict__ part, double inv_count,
                                                     float *__restrict__ loss) {
    __shared__ double sm[256];
    loss_reduce_block(nparts, part, inv_count, loss, sm);
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bwd_load(uint32_t e0, uint32_t ne, const float4 *__restrict__ records,
                                         const uint2 *__restrict__ pixbox, const uint32_t *vals, bool fresh,
                                         BwdEntry &E) {
    const uint32_t lane = threadIdx.x & 63;
    E.p = E.q = make_float4(0.f, 0.f, 0.f, 0.f);
    E.box = make_uint2(1u, 0u);
    E.g = 0u;
    if (lane < ne) {
        const uint32_t g = load_list(vals, e0 + lane, fresh);
        E.p = records[2 * g];
        E.q = records[2 * g + 1];
        E.box = pixbox[g];
        E.g = g;
    }
}

// Stages lane `lane`'s entry: its record in LDS and the rectangle of 4x4
// blocks its pixel box overlaps (empty when none).
__device__ __forceinline__ void bwd_stage(BwdLds &S, uint32_t ne, const BwdEntry &E, int x0, int y0, int &bx0,
                                          int &bx1, int &by0, int &by1) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    bx0 = 4; bx1 = -1; by0 = 4; by1 = -1;
    if ((uint32_t)lane < ne) {
        S.entp[wave][lane] = E.p;
        S.entq[wave][lane] = E.q;
        const uint2 bx = E.box;
        bx0 = max((int)(bx.x & 0xffff) - x0, 0) >> 2;
        bx1 = min((int)(bx.y & 0xffff) - x0, 15) >> 2;
        by0 = max((int)(bx.x >> 16) - y0, 0) >> 2;
        by1 = min((int)(bx.y >> 16) - y0, 15) >> 2;
    }
}

// LDS index of pixel (x, y) of the tile in gp: block (y/4)*4 + x/4, offset (y%4)*4 + x%4.
__device__ __forceinline__ int gp_index(int x, int y) {
    return (((y >> 2) << 2) | (x >> 2)) * kGpStride + ((y & 3) << 2) + (x & 3);
}

// Backward of one tile with its dL/dI published in gp and the first share's
// entries (E0) already loaded; each entry's 8 values go to its emission slot.
// Wave-local from here on (no workgroup barrier).  ABS also forms each pair's
// sums of |per-pixel d mux| and |per-pixel d muy| ("absgrad": run partials in
// pabs [4][kWaveEnt + 64], the pair's total at its slot of part_abs).
template <bool ABS = false>
__device__ __forceinline__ void sum_bwd_tile(BwdLds &S, const float4 *gp, int tx, int ty, uint2 rg, BwdEntry E0,
                                             const float4 *__restrict__ records, const uint2 *__restrict__ pixbox,
                                             const uint32_t *__restrict__ offsets, const uint32_t *vals,
                                             bool fresh_vals, uint32_t capacity, float4 *__restrict__ part,
                                             float2 (*pabs)[kWaveEnt + 64] = nullptr,
                                             float2 *__restrict__ part_abs = nullptr) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int x0 = tx * kTile, y0 = ty * kTile;
    const float fx0 = (float)x0 + 0.5f, fy0 = (float)y0 + 0.5f;   // the tile's first pixel centre
    const float k2 = 2.0f * kLn2;
    for (uint32_t base = rg.x; base < rg.y; base += kBwdBatch) {
        uint32_t e0, ne;
        bwd_share(rg, base, e0, ne);
        if (ne == 0) continue;                              // wave-uniform; no workgroup barrier below
        // wave priority: the staging (loads, then a short LDS pass) before other waves' item loops, so
        // that its loads go out early; the item loop at the default priority
        __builtin_amdgcn_s_setprio(2);
        BwdEntry E = E0;
        if (base != rg.x) bwd_load(e0, ne, records, pixbox, vals, fresh_vals, E);
        int bx0, bx1, by0, by1;
        bwd_stage(S, ne, E, x0, y0, bx0, bx1, by0, by1);
        // the entry's emission offset is only needed for the final store: its load goes out now and
        // its latency hides behind the items (and stays out of the staging loads)
        const uint32_t goff = (uint32_t)lane < ne ? offsets[E.g] : 0u;
        // entry-major item positions: lane e's items are [s_e, s_e + n_e), blocks in
        // ascending order (row-major over its rectangle)
        const uint32_t n_e = (uint32_t)(lane) < ne ? (uint32_t)((bx1 - bx0 + 1) * (by1 - by0 + 1)) : 0u;
        const uint32_t incl = wave_scan_incl(n_e);
        const uint32_t s_e = incl - n_e;
        const uint32_t nitems = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        {
            uint32_t o = s_e;
            for (int by = by0; by <= by1; ++by)
                for (int bx = bx0; bx <= bx1; ++bx) S.items[wave][o++] = (uint16_t)(lane | ((by * 4 + bx) << 8));
        }
        wave_sync();
        __builtin_amdgcn_s_setprio(0);
        const uint32_t R = (nitems + 63u) >> 6;             // items per lane (wave-uniform)
        const uint32_t f = (uint32_t)lane * R, fend = min(f + R, nitems);
        float4 acc0 = make_float4(0.f, 0.f, 0.f, 0.f), acc1 = acc0;   // the current (entry, run) partial
        float2 accA = make_float2(0.f, 0.f);                         // ABS: its sums of |h (a u + b v)|, |h v|
        uint32_t cur = 0xffffffffu, cur_slot = 0u;
        for (uint32_t r = 0; r < R; ++r) {
            const uint32_t it = f + r;
            if (it < fend) {
                const uint32_t code = S.items[wave][it];
                const uint32_t e = code & 0xffu, blk = code >> 8;
                if (e != cur) {                             // a new (entry, run) segment
                    if (cur != 0xffffffffu) {
                        S.part[wave][cur_slot][0] = acc0;
                        S.part[wave][cur_slot][1] = acc1;
                        acc0 = acc1 = make_float4(0.f, 0.f, 0.f, 0.f);
                        if constexpr (ABS) {
                            pabs[wave][cur_slot] = accA;
                            accA = make_float2(0.f, 0.f);
                        }
                    }
                    // the run's first item continues the previous lane's entry, or an entry starts here
                    const bool cont = r == 0 && it > 0 && (S.items[wave][it - 1] & 0xffu) == e;
                    cur = e;
                    cur_slot = cont ? (uint32_t)(kWaveEnt + lane) : e;
                }
                const int lx = (int)(blk & 3u) * 4, ly = (int)(blk >> 2) * 4;
                const float4 A = S.entp[wave][e], B = S.entq[wave][e];
                // pixel centres: the block's first column and row converted once, the others one
                // more each (all exact in fp32, the same values as converting each pixel's index)
                const float cx0 = fx0 + (float)lx, cy0 = fy0 + (float)ly;
                float dy[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) dy[rr] = (cy0 + (float)rr) - A.y;
                // the first column and pixel assign their sums (no addition of a zero)
                float Hu, Hv, Muu, Muv, Mvv, Cr, Cg, Cb;
                float Ax = 0.f, Ay = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float dx = (cx0 + (float)c) - A.x;
                    const float u = A.z * dx;
                    const float tb = A.w * dx;
                    const float uu = u * u;
                    const float au = A.z * u;
                    float ch, chv, chvv;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const float4 gv = gp[blk * kGpStride + rr * 4 + c];
                        const float v = fmaf(B.x, dy[rr], tb);
                        const float ee = fmaf(v, v, uu);
                        const float w = ee <= kE9 ? exp2_hw(-ee) : 0.0f;
                        if (c == 0 && rr == 0) {
                            Cr = gv.x * w;
                            Cg = gv.y * w;
                            Cb = gv.z * w;
                        } else {
                            Cr = fmaf(gv.x, w, Cr);
                            Cg = fmaf(gv.y, w, Cg);
                            Cb = fmaf(gv.z, w, Cb);
                        }
                        const float h = fmaf(gv.z, B.w, fmaf(gv.y, B.z, gv.x * B.y)) * w;
                        const float hv = h * v;
                        if (rr == 0) {
                            ch = h;
                            chv = hv;
                            chvv = hv * v;
                        } else {
                            ch += h;
                            chv += hv;
                            chvv = fmaf(hv, v, chvv);
                        }
                        if constexpr (ABS) {
                            Ax += fabsf(h * fmaf(A.w, v, au));
                            Ay += fabsf(hv);
                        }
                    }
                    if (c == 0) {
                        Hu = u * ch;
                        Muu = uu * ch;
                        Muv = u * chv;
                        Hv = chv;
                        Mvv = chvv;
                    } else {
                        Hu = fmaf(u, ch, Hu);
                        Muu = fmaf(uu, ch, Muu);
                        Muv = fmaf(u, chv, Muv);
                        Hv += chv;
                        Mvv += chvv;
                    }
                }
                // the item's share of the pair's sums (slot_grad_cholesky turns a Gaussian's total
                // into its gradient)
                acc0.x += Hu;
                acc0.y += Hv;
                acc0.z += Muu;
                acc0.w += Muv;
                acc1.x += Mvv;
                acc1.y += Cr;
                acc1.z += Cg;
                acc1.w += Cb;
                if constexpr (ABS) {
                    accA.x += k2 * Ax;
                    accA.y += k2 * fabsf(B.x) * Ay;
                }
            }
        }
        if (cur != 0xffffffffu) {
            S.part[wave][cur_slot][0] = acc0;
            S.part[wave][cur_slot][1] = acc1;
            if constexpr (ABS) pabs[wave][cur_slot] = accA;
        }
        wave_sync();
        // entry e (lane e): its first run's partial, then those of the runs of lanes
        // L0 + 1 .. L1 that continue it, in order
        const uint32_t slot = (uint32_t)lane < ne ? emit_slot(goff, E.box, tx, ty) : 0xffffffffu;
        if ((uint32_t)lane < ne && slot < capacity) {
            float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
            if (n_e > 0u) {                                 // always, for a box that meets the tile
                s0 = S.part[wave][lane][0];
                s1 = S.part[wave][lane][1];
            }
            const uint32_t L0 = s_e / R, L1 = n_e > 0u ? (s_e + n_e - 1u) / R : L0;
            float2 sa = make_float2(0.f, 0.f);
            if constexpr (ABS) {
                if (n_e > 0u) sa = pabs[wave][lane];
            }
            for (uint32_t L = L0 + 1u; L <= L1; ++L) {
                const float4 u0 = S.part[wave][kWaveEnt + L][0], u1 = S.part[wave][kWaveEnt + L][1];
                s0.x += u0.x; s0.y += u0.y; s0.z += u0.z; s0.w += u0.w;
                s1.x += u1.x; s1.y += u1.y; s1.z += u1.z; s1.w += u1.w;
                if constexpr (ABS) {
                    const float2 ua = pabs[wave][kWaveEnt + L];
                    sa.x += ua.x;
                    sa.y += ua.y;
                }
            }
            part[2 * (size_t)slot] = s0;
            part[2 * (size_t)slot + 1] = s1;
            if constexpr (ABS) part_abs[slot] = sa;
        }
        wave_sync();                                        // ent / items are rewritten next batch
    }
}

template <bool ABS>
__global__ __launch_bounds__(256, kBwdWavesPerSimd) void k_render_sum_bwd(int W, int H, int tiles_x, int ntiles,
                                                        const float4 *__restrict__ records,
                                                        const uint2 *__restrict__ pixbox,
                                                        const uint32_t *__restrict__ offsets,
                                                        const uint2 *__restrict__ ranges, const uint32_t *__restrict__ order,
                                                        const uint32_t *__restrict__ vals, uint32_t capacity,
                                                        const float *__restrict__ dL,
                                                        float4 *__restrict__ part,
                                                        const float *__restrict__ loss_part, int nparts,
                                                        double inv_count, float *__restrict__ loss,
                                                        float2 *__restrict__ part_abs) {
    __shared__ float4 gp[16 * kGpStride];               // dL/dI of the tile's pixels, block by block
    __shared__ float2 pabs[ABS ? 4 : 1][kWaveEnt + 64];
    __shared__ __align__(16) unsigned char lds[sizeof(BwdLds)];
    if (loss && blockIdx.x == gridDim.x - 1) {          // the spare last workgroup: the forward's loss
        loss_reduce_block(nparts, loss_part, inv_count, loss, reinterpret_cast<double *>(lds));
        return;
    }
    BwdLds &S = *reinterpret_cast<BwdLds *>(lds);
    const int t = tile_of(blockIdx.x, gridDim.x, ntiles, order);
    if (t >= ntiles) return;
    const uint2 rg = ranges[t];
    if (rg.x == rg.y) return;
    const int tid = threadIdx.x;
    const int tx = t % tiles_x, ty = t / tiles_x;
    const int x0 = tx * kTile, y0 = ty * kTile;
    // dL/dI loads and the first share's loads go out together; one workgroup
    // barrier publishes the tile's dL/dI, everything after it is wave-local.
    uint32_t e0, ne;
    bwd_share(rg, rg.x, e0, ne);
    float4 gv0 = make_float4(0.f, 0.f, 0.f, 0.f);
    {
        const int xi = x0 + (tid & 15), yi = y0 + (tid >> 4);
        if (xi < W && yi < H) {
            const size_t o = (size_t)yi * W + xi, plane = (size_t)W * H;
            gv0 = make_float4(dL[o], dL[o + plane], dL[o + 2 * plane], 0.f);
        }
    }
    BwdEntry E0;
    bwd_load(e0, ne, records, pixbox, vals, false, E0);
    gp[gp_index(tid & 15, tid >> 4)] = gv0;
    __syncthreads();
    sum_bwd_tile<ABS>(S, gp, tx, ty, rg, E0, records, pixbox, offsets, vals, false, capacity, part,
                      ABS ? pabs : nullptr, part_abs);
}

// Forward with the L2 loss, then the backward of the same tile, in one
// workgroup: the tile's dL/dI never leaves LDS, and the backward's first share
// of entries is the forward's own first batch, kept in registers.  Same results, bit for bit, as
// k_render_sum_fwd<true> followed by k_render_sum_bwd.
__global__ __launch_bounds__(256, kBwdWavesPerSimd) void k_render_sum_fused(int W, int H, int tiles_x, int ntiles,
                                                          const float4 *__restrict__ records,
                                                          const uint2 *__restrict__ pixbox,
                                                          const uint32_t *__restrict__ offsets,
                                                          const uint2 *__restrict__ ranges,
                                                          const uint32_t *__restrict__ order,
                                                          const uint32_t *vals, uint32_t capacity,
                                                          float *__restrict__ image, const float *__restrict__ target,
                                                          float *__restrict__ dL, float gscale,
                                                          float *__restrict__ loss_part, float4 *__restrict__ part,
                                                          BucketList bl) {
    __shared__ float4 gp[16 * kGpStride];
    __shared__ __align__(16) unsigned char lds[kPhaseLds];
    __shared__ float wsq[4];
    __shared__ uint32_t tl[kFwdBatch];                    // bucket mode: the list's first batch
    __shared__ uint32_t sc[2 + kBucketPL][4];
    const int t = tile_of(blockIdx.x, gridDim.x, ntiles, order);
    if (t >= ntiles) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tx = t % tiles_x, ty = t / tiles_x;
    const int x0 = tx * kTile, y0 = ty * kTile;
    const int quad = (wave + t) & 3;                      // the wave's quadrant, rotated by tile
    const int pxi = x0 + (quad & 1) * 8 + (lane & 7);
    const int pyi = y0 + (quad >> 1) * 8 + (lane >> 3);
    // Wave priority: the list, its staging and the forward ahead of the backward item loops of
    // the CU's other workgroups (every tile's workgroup is resident from the start; the oldest
    // ones would otherwise hold the issue slots while the others' loads wait to go out).
    __builtin_amdgcn_s_setprio(2);
    const bool bucket = bl.kin != nullptr;                // uniform
    const uint2 rg = bucket ? bucket_tile_list(bl, t, tl, sc) : ranges[t];
    if (bucket) vals = bl.vout;                           // later batches read the list just written
    BwdEntry E0;                                          // the backward's first share, loaded by the forward
    E0.p = E0.q = make_float4(0.f, 0.f, 0.f, 0.f);
    E0.box = make_uint2(1u, 0u);
    E0.g = 0u;
    float ar = 0.0f, ag = 0.0f, ab = 0.0f;
    sum_fwd_tile(*reinterpret_cast<FwdLds *>(lds), x0, y0, rg, records, pixbox, vals, bucket ? tl : nullptr, &E0, quad,
                 (float)pxi + 0.5f, (float)pyi + 0.5f, ar, ag, ab);
    const float4 g = sum_fwd_store<true>(W, H, pxi, pyi, t, ar, ag, ab, image, target, dL, gscale, loss_part, wsq);
    gp[gp_index(pxi - x0, pyi - y0)] = g;
    __syncthreads();                                      // gp and wsq published; the forward's lists are dead
    loss_part_store(t, wsq, loss_part);
    if (rg.x == rg.y) return;                             // uniform
    __builtin_amdgcn_s_setprio(0);
    sum_bwd_tile(*reinterpret_cast<BwdLds *>(lds), gp, tx, ty, rg, E0, records, pixbox, offsets, vals, bucket, capacity,
                 part);
}

// One thread per Gaussian: its pairs' partial gradients sit at offsets[g] ..
// offsets[g+1] in emission order; add them in that order (reproducible).
__global__ __launch_bounds__(256) void k_grad_gather(int n, int ntiles, const uint32_t *__restrict__ offsets,
                                                     uint32_t capacity, const float4 *__restrict__ records,
                                                     const float4 *__restrict__ part,
                                                     const float *__restrict__ part_l,
                                                     const float4 *__restrict__ part_bg,
                                                     float *__restrict__ dparams, float *__restrict__ dlogit,
                                                     float *__restrict__ dbg, const float2 *__restrict__ part_abs,
                                                     float2 *__restrict__ dabs) {
    if (offsets[n] > capacity) return;                  // binning overflowed: nothing was rendered
    if (dbg && blockIdx.x == 0) {
        __shared__ float4 sm[256];
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int t = threadIdx.x; t < ntiles; t += 256) {
            const float4 v = part_bg[t];
            s.x += v.x; s.y += v.y; s.z += v.z;
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
        if (threadIdx.x == 0) { dbg[0] += sm[0].x; dbg[1] += sm[0].y; dbg[2] += sm[0].z; }
    }
    const int g = blockIdx.x * 256 + threadIdx.x;
    if (g >= n) return;
    const uint32_t o0 = offsets[g], o1 = offsets[g + 1];
    if (o1 == o0) return;
    if (dabs) {                                         // absgrad: the pairs' sums, in emission order
        float2 s = dabs[g];
        for (uint32_t q = o0; q < o1; ++q) {
            const float2 u = part_abs[q];
            s.x += u.x;
            s.y += u.y;
        }
        dabs[g] = s;
    }
    float4 *d = reinterpret_cast<float4 *>(dparams) + 2 * (size_t)g;
    float4 d0 = d[0], d1 = d[1];
    const float4 rp = records[2 * (size_t)g], rq = records[2 * (size_t)g + 1];
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    gather_slots(part, o0, o1, a, b);
    float l = 0.f;
    if (part_l)
        for (uint32_t q = o0; q < o1; ++q) l += part_l[q];
    a = slot_grad_half(0, rp.z, rp.w, rq.x, a);
    b = slot_grad_half(1, rp.z, rp.w, rq.x, b);
    d0.x += a.x; d0.y += a.y; d0.z += a.z; d0.w += a.w;
    d1.x += b.x; d1.y += b.y; d1.z += b.z; d1.w += b.w;
    d[0] = d0;
    d[1] = d1;
    if (dlogit) dlogit[g] += l;
}

// Adam on each Gaussian's 8 parameters with the gradient gathered from its
// pairs' slots (offsets[g] .. offsets[g+1], emission order): the gather and
// the optimizer in one pass, no gradient array.  Eight lanes per Gaussian, lane
// j on parameter j: a Gaussian's parameters, moments and each slot are 32
// contiguous bytes read by its 8 lanes together, and up to 8 slots are loaded
// at once.  Each slot entry is added in ascending order, as in gather_slots,
// and the sums are turned into the gradient by slot_grad_entry with the
// record's rows formed from the parameters (same bits as a gather followed by
// the Adam step).
// With `loss`, one more workgroup (the last) reduces the loss partials of the
// raster pass into it.
__global__ __launch_bounds__(256) void k_adam_pairs(int n, const uint32_t *__restrict__ offsets, uint32_t capacity,
                                                    const float *__restrict__ part, float *__restrict__ p,
                                                    float *__restrict__ m, float *__restrict__ v, AdamHP a,
                                                    const float *__restrict__ loss_part, int nparts, double inv_count,
                                                    float *__restrict__ loss) {
    if (loss && blockIdx.x == gridDim.x - 1) {
        __shared__ double sm[256];
        loss_reduce_block(nparts, loss_part, inv_count, loss, sm);
        return;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // parameter i % 8 of Gaussian i / 8
    const int g = (int)(i >> 3), j = (int)(i & 7);
    // the whole group of 8 lanes takes the same branch (the exchange below stays within it)
    if (g >= n) return;
    float c1, c2;
    adam_step_bias(a, c1, c2);
    float P = p[i], Mo = m[i], V = v[i];
    const uint32_t o0 = offsets[g], o1r = offsets[g + 1];
    const uint32_t o1 = offsets[n] <= capacity ? o1r : o0;   // else the binning overflowed: zero gradient
    float S = 0.0f;
    for (uint32_t q = o0; q < o1; q += 8) {
        float u[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) u[k] = part[8 * (size_t)min(q + (uint32_t)k, o1 - 1u) + j];   // repeats not added
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (q + (uint32_t)k < o1) S += u[k];
    }
    const int lane = threadIdx.x & 63, grp = lane & ~7;
    const float3 r = conic_rows(__shfl(P, grp + 2, 64), __shfl(P, grp + 3, 64), __shfl(P, grp + 4, 64));
    const float Sn = __shfl(S, min(lane + 1, grp + 7), 64);
    const float G = o1 > o0 ? slot_grad_entry(j, r.x, r.y, r.z, S, Sn) : 0.0f;   // no pairs: culled, or none
    float lr = a.lr[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) lr = j == k ? a.lr[k] : lr;
    adam_update(P, G, Mo, V, lr, a, c1, c2);
    p[i] = P;
    m[i] = Mo;
    v[i] = V;
}

AdamHP make_adam_hp(const float *lr, double beta1, double beta2, double eps, int step, const int32_t *d_step) {
    AdamHP a{};
    for (int i = 0; i < 8; ++i) a.lr[i] = lr[i];
    a.b1 = (float)beta1;
    a.omb1 = (float)(1.0 - beta1);
    a.b2 = (float)beta2;
    a.omb2 = (float)(1.0 - beta2);
    a.eps = (float)eps;
    a.b1d = beta1;
    a.b2d = beta2;
    a.step = step;
    a.d_step = d_step;
    if (!d_step) adam_bias(beta1, beta2, step, a.bc1, a.bc2);
    return a;
}

static int padded_tiles(int ntiles) { return (ntiles + 7) & ~7; }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdPlan make_bwd_plan(int W, int H, int64_t capacity) {
    const int ntiles = ((W + kTile - 1) / kTile) * ((H + kTile - 1) / kTile);
    const size_t cap = (size_t)(capacity > 0 ? capacity : 1);
    BwdPlan p{};
    size_t off = 0;
    p.off_part = off; off = align256(off + 32 * cap);
    p.off_logit = off; off = align256(off + 4 * cap);
    p.off_bg = off; off = align256(off + 16 * (size_t)ntiles);
    p.off_abs = off; off = align256(off + 8 * cap);
    p.bytes = off;
    return p;
}

hipError_t launch_adam_pairs(int n, int W, int H, const uint32_t *offsets, int64_t capacity, const void *ws, float *p,
                             float *m, float *v, const float *lr, double beta1, double beta2, double eps, int step,
                             const int32_t *d_step, const float *loss_partials, int64_t loss_count, float *d_loss,
                             hipStream_t s) {
    const int nb = (int)(((int64_t)n * 8 + 255) / 256) + (d_loss ? 1 : 0);
    if (nb == 0) return hipSuccess;
    const BwdPlan pl = make_bwd_plan(W, H, capacity);
    const AdamHP a = make_adam_hp(lr, beta1, beta2, eps, step, d_step);
    const int ntiles = ((W + kTile - 1) / kTile) * ((H + kTile - 1) / kTile);
    k_adam_pairs<<<nb, 256, 0, s>>>(
        n, offsets, (uint32_t)capacity, reinterpret_cast<const float *>(static_cast<const char *>(ws) + pl.off_part),
        p, m, v, a,
        loss_partials, ntiles, loss_count > 0 ? 1.0 / (double)loss_count : 0.0, d_loss);
    return hipGetLastError();
}

hipError_t launch_grad_gather(int n, int W, int H, int ntiles, const uint32_t *offsets, int64_t capacity,
                              const void *ws, const float *records, int alpha, float *dparams, float *dlogit,
                              float *dbackground, hipStream_t s, float *dabs) {
    if (n == 0 && !(alpha && dbackground)) return hipSuccess;
    const BwdPlan p = make_bwd_plan(W, H, capacity);
    const char *w = static_cast<const char *>(ws);
    const int nb = (n + 255) / 256;
    k_grad_gather<<<nb > 0 ? nb : 1, 256, 0, s>>>(
        n, ntiles, offsets, (uint32_t)capacity, reinterpret_cast<const float4 *>(records),
        reinterpret_cast<const float4 *>(w + p.off_part), alpha ? reinterpret_cast<const float *>(w + p.off_logit) : nullptr,
        reinterpret_cast<const float4 *>(w + p.off_bg), dparams, alpha ? dlogit : nullptr,
        alpha ? dbackground : nullptr, reinterpret_cast<const float2 *>(w + p.off_abs),
        reinterpret_cast<float2 *>(dabs));
    return hipGetLastError();
}

hipError_t launch_render_sum_fwd(int W, int H, const float *records, const uint16_t *pixbox,
                                 const uint32_t *ranges, const uint32_t *order, const uint32_t *vals, float *image,
                                 const float *target, float *dL_dimage, float *loss_partials, hipStream_t s,
                                 const BucketList *bl) {
    const int tiles_x = (W + kTile - 1) / kTile, ntiles = tiles_x * ((H + kTile - 1) / kTile);
    const BucketList b = bl ? *bl : BucketList{};
    const float4 *rec = reinterpret_cast<const float4 *>(records);
    const uint2 *bx = reinterpret_cast<const uint2 *>(pixbox);
    const uint2 *rg = reinterpret_cast<const uint2 *>(ranges);
    if (target) {
        const float gscale = (float)(2.0 / (3.0 * (double)W * (double)H));
        k_render_sum_fwd<true><<<padded_tiles(ntiles), 256, 0, s>>>(W, H, tiles_x, ntiles, rec, bx, rg, order, vals,
                                                                     image, target, dL_dimage, gscale, loss_partials, b);
    } else {
        k_render_sum_fwd<false><<<padded_tiles(ntiles), 256, 0, s>>>(W, H, tiles_x, ntiles, rec, bx, rg, order, vals,
                                                                      image, nullptr, nullptr, 0.0f, nullptr, b);
    }
    return hipGetLastError();
}

hipError_t launch_loss_reduce(int nparts, const float *partials, int64_t count, float *d_loss, hipStream_t s) {
    k_loss_reduce<<<1, 256, 0, s>>>(nparts, partials, 1.0 / (double)count, d_loss);
    return hipGetLastError();
}

hipError_t launch_render_sum_bwd(int W, int H, const float *records, const uint16_t *pixbox,
                                 const uint32_t *offsets, const uint32_t *ranges, const uint32_t *order,
                                 const uint32_t *vals, int64_t capacity, const float *dL_dimage, void *ws,
                                 const float *loss_partials, int64_t loss_count, float *d_loss, hipStream_t s,
                                 bool absgrad) {
    const int tiles_x = (W + kTile - 1) / kTile, ntiles = tiles_x * ((H + kTile - 1) / kTile);
    const BwdPlan p = make_bwd_plan(W, H, capacity);
    // with d_loss, 8 more workgroups: the last one (no tile under either tile map) reduces the loss
    const int nb = padded_tiles(ntiles) + (d_loss ? 8 : 0);
    const double inv_count = loss_count > 0 ? 1.0 / (double)loss_count : 0.0;
    float4 *part = reinterpret_cast<float4 *>(static_cast<char *>(ws) + p.off_part);
    float2 *pa = reinterpret_cast<float2 *>(static_cast<char *>(ws) + p.off_abs);
    if (absgrad)
        k_render_sum_bwd<true><<<nb, 256, 0, s>>>(
            W, H, tiles_x, ntiles, reinterpret_cast<const float4 *>(records), reinterpret_cast<const uint2 *>(pixbox),
            offsets, reinterpret_cast<const uint2 *>(ranges), order, vals, (uint32_t)capacity, dL_dimage, part,
            loss_partials, ntiles, inv_count, d_loss, pa);
    else
        k_render_sum_bwd<false><<<nb, 256, 0, s>>>(
            W, H, tiles_x, ntiles, reinterpret_cast<const float4 *>(records), reinterpret_cast<const uint2 *>(pixbox),
            offsets, reinterpret_cast<const uint2 *>(ranges), order, vals, (uint32_t)capacity, dL_dimage, part,
            loss_partials, ntiles, inv_count, d_loss, nullptr);
    return hipGetLastError();
}

hipError_t launch_render_sum_fused(int W, int H, const float *records, const uint16_t *pixbox,
                                   const uint32_t *offsets, const uint32_t *ranges, const uint32_t *order,
                                   const uint32_t *vals, int64_t capacity, float *image, const float *target,
                                   float *dL_dimage, float *loss_partials, void *ws, hipStream_t s,
                                   const BucketList *bl) {
    const int tiles_x = (W + kTile - 1) / kTile, ntiles = tiles_x * ((H + kTile - 1) / kTile);
    const BwdPlan p = make_bwd_plan(W, H, capacity);
    const float gscale = (float)(2.0 / (3.0 * (double)W * (double)H));
    const BucketList b = bl ? *bl : BucketList{};
    k_render_sum_fused<<<padded_tiles(ntiles), 256, 0, s>>>(
        W, H, tiles_x, ntiles, reinterpret_cast<const float4 *>(records), reinterpret_cast<const uint2 *>(pixbox),
        offsets, reinterpret_cast<const uint2 *>(ranges), order, vals, (uint32_t)capacity, image, target, dL_dimage,
        gscale, loss_partials, reinterpret_cast<float4 *>(static_cast<char *>(ws) + p.off_part), b);
    return hipGetLastError();
}

}  // namespace gi
