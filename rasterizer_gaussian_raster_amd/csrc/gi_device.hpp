// gi_device.hpp -- device-side helpers shared by the gfx950 kernels of libgi.
//
// Wave64 only (CDNA4).  Cross-lane reductions use DPP row operations and the
// gfx9 row broadcasts, which stay inside the VALU (no LDS round trip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gi_launch.hpp"

namespace gi {

constexpr int kTile = 16;            // tile edge, pixels (fvdb config: tile_size = 16)
constexpr int kWave = 64;

// fp32 constants of the cutoff rule, each the fp32 value nearest its definition.
constexpr float kScale = 0x1.b2da4ep-1f;   // sqrt(log2(e) / 2)
constexpr float kE9 = 0x1.9f7f06p+2f;      // 9 * log2(e) / 2: e <= kE9  <=>  q <= 9
constexpr float kLogitMax = 0x1.ba0846p+2f;// ln(999): opacity clamp at 0.999
constexpr float kTmin = 1e-4f;             // alpha mode: stop once T < kTmin
constexpr float kLn2 = 0x1.62e430p-1f;     // ln 2
constexpr float kPad = 0.00390625f;        // 1/256 px pad of the pixel box

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ __forceinline__ uint64_t lanes_below() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Orders a wave's LDS writes before its later LDS reads by other lanes of the
// same wave (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// b^t (t >= 0) by binary powering in fp64: a short chain of multiplications
// (a few ulps of fp64 from the exact power, far below the fp32 rounding that
// follows) instead of a general pow.
__host__ __device__ __forceinline__ double powi_f64(double b, int t) {
    double r = 1.0, x = b;
    for (unsigned e = (unsigned)t; e != 0u; e >>= 1) {
        if (e & 1u) r *= x;
        x *= x;
    }
    return r;
}

// Adam's bias corrections for step t (t < 1 is taken as 1), formed in fp64 and
// rounded once: 1/(1 - b1^t) and 1/sqrt(1 - b2^t).  The host forms them the
// same way (IEEE fp64 products, quotient and square root: the same bits).
__host__ __device__ __forceinline__ void adam_bias(double b1, double b2, int t, float &inv_bc1,
                                                   float &inv_sqrt_bc2) {
    const int tt = t < 1 ? 1 : t;
    inv_bc1 = (float)(1.0 / (1.0 - powi_f64(b1, tt)));
    inv_sqrt_bc2 = (float)(1.0 / sqrt(1.0 - powi_f64(b2, tt)));
}

// This step's corrections: the host's, or formed here from the device step
// count (graph replays).  Called before any load is issued (the fp64 loop of
// the device path then costs no wait on outstanding loads).
__device__ __forceinline__ void adam_step_bias(const AdamHP &a, float &inv_bc1, float &inv_sqrt_bc2) {
    if (a.d_step) {                                        // uniform
        adam_bias(a.b1d, a.b2d, *a.d_step, inv_bc1, inv_sqrt_bc2);
    } else {
        inv_bc1 = a.bc1;
        inv_sqrt_bc2 = a.bc2;
    }
}

// One Adam update of a scalar: the same expression in every optimizer kernel.
__device__ __forceinline__ void adam_update(float &p, float g, float &m, float &v, float lr, const AdamHP &a,
                                            float inv_bc1, float inv_sqrt_bc2) {
    m = fmaf(a.b1, m, a.omb1 * g);
    v = fmaf(a.b2, v, a.omb2 * g * g);
    p -= lr * (m * inv_bc1) / (sqrtf(v) * inv_sqrt_bc2 + a.eps);
}

// Adds the pair slots q in [o0, o1) (part[2q], part[2q + 1]) into (a, b) in
// ascending q; K slots are loaded at a time so that their latencies overlap.
template <int K = 4>
__device__ __forceinline__ void gather_slots(const float4 *__restrict__ part, uint32_t o0, uint32_t o1, float4 &a,
                                             float4 &b) {
    for (uint32_t q = o0; q < o1; q += K) {
        float4 u[K], w[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t qq = min(q + (uint32_t)k, o1 - 1u);     // in range; repeats are not added
            u[k] = part[2 * (size_t)qq];
            w[k] = part[2 * (size_t)qq + 1];
        }
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (q + (uint32_t)k < o1) {
                a.x += u[k].x; a.y += u[k].y; a.z += u[k].z; a.w += u[k].w;
                b.x += w[k].x; b.y += w[k].y; b.z += w[k].z; b.w += w[k].w;
            }
    }
}

// Half h of the same sum (part[2q + h] for q in [o0, o1), ascending q): the
// value gather_slots forms for that half, bit for bit.
// The first K slots are loaded outside the loop, so that they go out as soon as
// the offsets are in (a loop would wait for every load in flight first).
template <int K = 4>
__device__ __forceinline__ void gather_half(const float4 *__restrict__ part, uint32_t o0, uint32_t o1, int h,
                                            float4 &a) {
    {
        float4 u[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t qq = o1 > o0 ? min(o0 + (uint32_t)k, o1 - 1u) : 0u;   // in range; extras not added
            u[k] = part[2 * (size_t)qq + h];
        }
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (o0 + (uint32_t)k < o1) {
                a.x += u[k].x; a.y += u[k].y; a.z += u[k].z; a.w += u[k].w;
            }
    }
    for (uint32_t q = o0 + K; q < o1; q += K) {
        float4 u[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t qq = min(q + (uint32_t)k, o1 - 1u);     // in range; repeats are not added
            u[k] = part[2 * (size_t)qq + h];
        }
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (q + (uint32_t)k < o1) {
                a.x += u[k].x; a.y += u[k].y; a.z += u[k].z; a.w += u[k].w;
            }
    }
}

// The pair slots of the backward hold, per (Gaussian, tile) pair and summed over the pair's
// pixels, the Gaussian's sums in its scaled whitened frame: with h = (dL/dw) w and
// (u, v) = (a dx, b dx + c dy) (the record's rows, e = u^2 + v^2, w = 2^-e, so dL/de = -ln2 h),
//   s0 = (sum h u, sum h v, sum h u^2, sum h u v),  s1 = (sum h v^2, sum g_r w, sum g_g w, sum g_b w).
// The gradient of any parameterisation is a linear map of a Gaussian's total, applied after the
// gather.  Cholesky form (a = S/l11, b = -S l21/(l11 l22), c = S/l22, W = [[a, 0], [b, c]]):
//   dL/dmu = 2 ln2 W^T (sum h u, sum h v),
//   dL/d(l11, l21, l22) = (2 ln2 / S) (a sum h u^2 + b sum h u v, c sum h u v, c sum h v^2)
// (the lower triangle of dL/dL = (2 ln2 / S) W^T M, M = [[sum h u^2, sum h u v], [sum h u v,
// sum h v^2]]); the colours' gradients are the last three sums.
// The record's rows (a, b, c) = S (1/l11, -(l21/l11)/l22, 1/l22) of a Cholesky factor, in the op
// order of the cutoff rule (the preprocess forms every record with it; a kernel that has the
// params rather than the record gets the same bits).
__device__ __forceinline__ float3 conic_rows(float l11, float l21, float l22) {
    const float i11 = 1.0f / l11;          // correctly rounded (no fast-math)
    const float i22 = 1.0f / l22;
    const float k = -((l21 * i11) * i22);
    return make_float3(i11 * kScale, k * kScale, i22 * kScale);
}

constexpr float kGradMu = 2.0f * kLn2;
constexpr float kGradL = kGradMu / kScale;

// Half h of a Gaussian's Cholesky-form gradient from half h of its gathered sums (h = 0: mux,
// muy, l11, l21; h = 1: l22 and the colours); (a, b, c) its record's rows.  Every kernel that
// turns slots into a gradient uses these expressions, so their results agree bit for bit.
__device__ __forceinline__ float4 slot_grad_half(int h, float a, float b, float c, float4 s) {
    if (h == 0)
        return make_float4(kGradMu * fmaf(a, s.x, b * s.y), kGradMu * (c * s.y), kGradL * fmaf(a, s.z, b * s.w),
                           kGradL * (c * s.w));
    return make_float4(kGradL * (c * s.x), s.y, s.z, s.w);
}

// Entry j of the same gradient from the sums sj (entry j of the total) and sn (entry j + 1).
__device__ __forceinline__ float slot_grad_entry(int j, float a, float b, float c, float sj, float sn) {
    switch (j) {
    case 0: return kGradMu * fmaf(a, sj, b * sn);
    case 1: return kGradMu * (c * sj);
    case 2: return kGradL * fmaf(a, sj, b * sn);
    case 3: return kGradL * (c * sj);
    case 4: return kGradL * (c * sj);
    default: return sj;
    }
}

// Sum of the per-tile partials in a fixed order, divided by the entry count
// (the first 256 threads of a workgroup of 256 or more; sm: 256 doubles of LDS).
__device__ __forceinline__ void loss_reduce_block(int nparts, const float *__restrict__ part, double inv_count,
                                                  float *__restrict__ loss, double *sm) {
    double s = 0.0;
    if (threadIdx.x < 256) {                               // a larger block's other threads only take the barriers
        for (int i = threadIdx.x; i < nparts; i += 256) s += (double)part[i];
        sm[threadIdx.x] = s;
    }
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) sm[threadIdx.x] += sm[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) *loss = (float)(sm[0] * inv_count);
}

// 2^x with the hardware transcendental (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf, bool BOUND_CTRL = false>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, BANK_MASK, BOUND_CTRL));
}

// Sum over the 64 lanes, returned uniform (read from lane 63).
__device__ __forceinline__ float wave_total(float x) {
    x += dpp_f<0xb1>(x);
    x += dpp_f<0x4e>(x);
    x += dpp_f<0x141>(x);
    x += dpp_f<0x140>(x);
    x += dpp_f<0x142, 0xa>(x);
    x += dpp_f<0x143, 0xc>(x);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf, bool BOUND_CTRL = false>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, BANK_MASK, BOUND_CTRL);
}

// Inclusive prefix sum over the 64 lanes with DPP (all lanes active): three
// row_shr steps give sums of 4, then row_shr 4 / 8 on the upper banks finish
// each 16-lane row, and the row_bcast 15 / 31 steps carry rows into rows.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
    uint32_t v = x + dpp_u<0x111, 0xf, 0xf, true>(x);      // row_shr:1
    v += dpp_u<0x112, 0xf, 0xf, true>(x);                   // row_shr:2
    v += dpp_u<0x113, 0xf, 0xf, true>(x);                   // row_shr:3
    v += dpp_u<0x114, 0xf, 0xe>(v);                         // row_shr:4, lanes 4..15 of each row
    v += dpp_u<0x118, 0xf, 0xc>(v);                         // row_shr:8, lanes 8..15 of each row
    v += dpp_u<0x142, 0xa>(v);                              // row_bcast:15 into rows 1 and 3
    v += dpp_u<0x143, 0xc>(v);                              // row_bcast:31 into rows 2 and 3
    return v;
}

// XCD-aware block -> work-item map: the hardware deals consecutive workgroups
// round-robin over the 8 XCDs; give each XCD a contiguous run of work items so
// neighbouring tiles (which share Gaussians) hit the same L2.  The grid must
// be a multiple of 8 blocks; the map is then a bijection of [0, nblocks).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    const int per = nblocks >> 3;
    return (bid & 7) * per + (bid >> 3);
}

// The tile workgroup `bid` of `nblocks` takes: order[bid] when a tile order is
// given (longest list first; workgroups past the tiles get none), else the
// XCD-aware map of bid.
__device__ __forceinline__ int tile_of(int bid, int nblocks, int ntiles, const uint32_t *order) {
    if (order) return bid < ntiles ? (int)order[bid] : ntiles;
    return xcd_remap(bid, nblocks);
}

// Emission slot of the pair (Gaussian g, tile (tx, ty)): offsets[g] plus the
// tile's row-major position in g's tile rectangle (box = packed pixel box).
__device__ __forceinline__ uint32_t emit_slot(uint32_t off_g, uint2 box, int tx, int ty) {
    const int tx0 = (int)(box.x & 0xffffu) >> 4, ty0 = (int)(box.x >> 16) >> 4;
    const int tx1 = (int)(box.y & 0xffffu) >> 4;
    return off_g + (uint32_t)((ty - ty0) * (tx1 - tx0 + 1) + (tx - tx0));
}

// Adds the tile pairs of one Gaussian (count c, packed pixel box bx) to an LDS
// histogram of the digit (tile id >> shift) & dmask.  Each row of its tile
// rectangle is a run of consecutive tile ids, added run by run where the digit
// changes (one atomic per run instead of one per pair).
__device__ __forceinline__ void hist_add_pairs(uint32_t *hist, uint32_t c, uint2 bx, int tiles_x, int shift,
                                               uint32_t dmask) {
    if (c == 0u) return;
    const uint32_t tx0 = (bx.x & 0xffffu) >> 4, ty0 = (bx.x >> 16) >> 4;
    const uint32_t wt = ((bx.y & 0xffffu) >> 4) - tx0 + 1u;
    const uint32_t rows = ((bx.y >> 16) >> 4) - ty0 + 1u;   // c = rows * wt
    for (uint32_t r = 0; r < rows; ++r) {
        const uint32_t lo = (ty0 + r) * (uint32_t)tiles_x + tx0, hi = lo + wt - 1u;
        for (uint32_t a = lo; a <= hi;) {
            const uint32_t e = min(hi, (((a >> shift) + 1u) << shift) - 1u);
            atomicAdd(&hist[(a >> shift) & dmask], e - a + 1u);
            a = e + 1u;
        }
    }
}

}  // namespace gi
