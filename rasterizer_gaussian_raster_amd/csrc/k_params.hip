// k_params.hip -- other forms of a Gaussian's parameters, turned into the
// Cholesky form the raster takes, and the chain rule back ("GaussianImage",
// Overview and its scripts: covariance as a Cholesky factor or as a rotation
// and two scales; "FlashImgs", Library API: xy / scale / rot tensors and
// rendering a trained set at any output size).
//
// Rotation-scale: Sigma = R diag(sx^2, sy^2) R^T, R = [[cos, -sin], [sin, cos]].
// Its Cholesky factor: with A = Sigma11 = (cos ax)^2 + (sin ay)^2,
// B = Sigma21 = cos sin (ax^2 - ay^2), det Sigma = (ax ay)^2:
//   l11 = sqrt(A), l21 = B / l11, l22 = ax ay / l11.
// Scaling the image plane by D = diag(fx, fy) maps mu -> D mu and L -> D L.
// One thread per Gaussian, two 16-byte loads and stores: HBM-bound.
#include <hip/hip_runtime.h>

#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

struct CholRS {
    float cs, sn, ax, ay, l11, l21, l22;
};

__device__ __forceinline__ CholRS rs_cholesky(float sx, float sy, float th) {
    CholRS r;
    sincosf(th, &r.sn, &r.cs);
    r.ax = fabsf(sx);
    r.ay = fabsf(sy);
    const float p = r.cs * r.ax, q = r.sn * r.ay;
    r.l11 = sqrtf(fmaf(p, p, q * q));
    r.l21 = (r.cs * r.sn) * ((r.ax - r.ay) * (r.ax + r.ay)) / r.l11;
    r.l22 = (r.ax * r.ay) / r.l11;
    return r;
}

__global__ __launch_bounds__(256) void k_params_to_cholesky(int kind, int64_t n, const float4 *__restrict__ in,
                                                           float fx, float fy, float4 *__restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= n) return;
    const float4 a = in[2 * g], b = in[2 * g + 1];
    float l11 = a.z, l21 = a.w, l22 = b.x;
    float4 ob = b;
    if (kind == 1) {                                        // (mux, muy, sx, sy), (theta, cr, cg, cb)
        const CholRS r = rs_cholesky(a.z, a.w, b.x);
        l11 = r.l11;
        l21 = r.l21;
        l22 = r.l22;
    }
    ob.x = fy * l22;
    out[2 * g] = make_float4(fx * a.x, fy * a.y, fx * l11, fy * l21);
    out[2 * g + 1] = ob;
}

// d(loss)/d(params in form `kind`) from the gradient (d0, d1) w.r.t. the Cholesky form of the
// Gaussian (a, b) scaled by (fx, fy); rotation-scale in fp64.  This is the chain rule applied to a
// gradient that is already a sum: for a rotated, elongated Gaussian the factor's gradient can be
// much larger than the rotation-scale gradient it carries, and its rounding is carried along
// (slot_grad_rs, which maps the backward's own sums, does not have that loss).
__device__ __forceinline__ void chol_chain(int kind, float4 a, float4 b, float fx, float fy, float4 d0, float4 d1,
                                           float4 &r0, float4 &r1) {
    // gradients w.r.t. the unscaled Cholesky form
    const float gmx = fx * d0.x, gmy = fy * d0.y, g11 = fx * d0.z, g21 = fy * d0.w, g22 = fy * d1.x;
    if (kind == 1) {
        const CholRS c = rs_cholesky(a.z, a.w, b.x);
        if (!(c.l11 > 0.0f) || !isfinite(c.l11) || !isfinite(c.l21) || !isfinite(c.l22)) {
            r0 = make_float4(0.f, 0.f, 0.f, 0.f);
            r1 = r0;
        } else {
            // l21 = B/l11, l22 = P/l11, l11 = sqrt(A): the whole dependence on l11 folded into A
            const double l11 = c.l11, l21 = c.l21, l22 = c.l22, cs = c.cs, sn = c.sn, ax = c.ax, ay = c.ay;
            const double inv = 1.0 / l11;
            const double gl11 = (double)g11 - ((double)g21 * l21 + (double)g22 * l22) * inv;
            const double gA = 0.5 * gl11 * inv, gB = (double)g21 * inv, gP = (double)g22 * inv;
            const double cc = cs * cs, ss = sn * sn, csn = cs * sn;
            const double dsq = (ax - ay) * (ax + ay);
            const double gax = 2.0 * ax * (gA * cc + gB * csn) + gP * ay;
            const double gay = 2.0 * ay * (gA * ss - gB * csn) + gP * ax;
            const double gth = -2.0 * (csn * dsq) * gA + gB * ((cc - ss) * dsq);
            r0 = make_float4(gmx, gmy, copysignf(1.0f, a.z) * (float)gax, copysignf(1.0f, a.w) * (float)gay);
            r1 = make_float4((float)gth, d1.y, d1.z, d1.w);
        }
    } else {
        r0 = make_float4(gmx, gmy, g11, g21);
        r1 = make_float4(g22, d1.y, d1.z, d1.w);
    }
}

// The gradient w.r.t. the rotation-scale params p0 = (mux, muy, sx, sy), p1 = (theta, cr, cg, cb)
// of a Gaussian rendered at scale D = diag(fx, fy) through the record rows (a, b, c), from its
// gathered slot sums s0, s1 (layout in gi_device.hpp), in fp64.  The rendered factor is
// L' = S W^-1, W = [[a, 0], [b, c]] (S = sqrt(log2(e)/2): e = |W d|^2 = q S^2), and
// Z = diag(1/sx, 1/sy) R^T D^-1 whitens D Sigma D along the Gaussian's own axes, so O = Z L' is
// orthogonal and M_z = O M O^T (M = [[sum h u^2, sum h u v], [sum h u v, sum h v^2]]) holds the
// second sums in those axes (z = S Z d).  With dL/dSigma'^-1 = -ln2 L' M L'^T:
//   dL/dsx = 2 ln2 M_z,xx / sx,  dL/dsy = 2 ln2 M_z,yy / sy,
//   dL/dtheta = 2 ln2 (sx/sy - sy/sx) M_z,xy,  dL/dmu = D 2 ln2 W^T (sum h u, sum h v).
// O's entries are at most 1 in size: the map adds no cancellation to the per-pixel terms' own.
__device__ __forceinline__ void slot_grad_rs(float4 p0, float4 p1, float fx, float fy, float a, float b, float c,
                                             float4 s0, float4 s1, float4 &r0, float4 &r1) {
    const double sx = p0.z, sy = p0.w;
    if (a == 0.0f || c == 0.0f || sx == 0.0 || sy == 0.0) {
        r0 = make_float4(0.f, 0.f, 0.f, 0.f);
        r1 = r0;
        return;
    }
    constexpr double kLn2d = 0.69314718055994530942;
    constexpr double kSd = 0.84932180028801904272;       // sqrt(log2(e) / 2)
    float snf, csf;
    sincosf(p1.x, &snf, &csf);                            // as rs_cholesky
    const double cs = csf, sn = snf, da = a, db = b, dc = c, dfx = fx, dfy = fy;
    // D^-1 L' = [[m11, 0], [m21, m22]]; O = diag(1/sx, 1/sy) R^T D^-1 L'
    const double m11 = kSd / (dfx * da), m21 = -kSd * db / (dfy * da * dc), m22 = kSd / (dfy * dc);
    const double o11 = (cs * m11 + sn * m21) / sx, o12 = sn * m22 / sx;
    const double o21 = (cs * m21 - sn * m11) / sy, o22 = cs * m22 / sy;
    const double muu = s0.z, muv = s0.w, mvv = s1.x;
    const double zxx = o11 * o11 * muu + 2.0 * o11 * o12 * muv + o12 * o12 * mvv;
    const double zyy = o21 * o21 * muu + 2.0 * o21 * o22 * muv + o22 * o22 * mvv;
    const double zxy = o11 * o21 * muu + (o11 * o22 + o12 * o21) * muv + o12 * o22 * mvv;
    const double k2 = 2.0 * kLn2d;
    r0 = make_float4((float)(dfx * k2 * (da * (double)s0.x + db * (double)s0.y)), (float)(dfy * k2 * dc * (double)s0.y),
                     (float)(k2 * zxx / sx), (float)(k2 * zyy / sy));
    r1 = make_float4((float)(k2 * (sx / sy - sy / sx) * zxy), s1.y, s1.z, s1.w);
}

__global__ __launch_bounds__(256) void k_params_to_cholesky_grad(int kind, int64_t n, const float4 *__restrict__ in,
                                                                float fx, float fy, const float4 *__restrict__ dout,
                                                                float4 *__restrict__ din, int accumulate) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= n) return;
    const float4 a = in[2 * g], b = in[2 * g + 1];
    const float4 d0 = dout[2 * g], d1 = dout[2 * g + 1];
    float4 r0, r1;
    chol_chain(kind, a, b, fx, fy, d0, d1, r0, r1);
    if (accumulate) {
        const float4 o0 = din[2 * g], o1 = din[2 * g + 1];
        r0 = make_float4(o0.x + r0.x, o0.y + r0.y, o0.z + r0.z, o0.w + r0.w);
        r1 = make_float4(o1.x + r1.x, o1.y + r1.y, o1.z + r1.z, o1.w + r1.w);
    }
    din[2 * g] = r0;
    din[2 * g + 1] = r1;
}

// Rotation-scale training: each Gaussian's pair slots added in emission order (as k_grad_gather
// does), the sums mapped to the rotation-scale gradient (slot_grad_rs, with the rows of the record
// the raster used: the Cholesky form of the params, as k_params_to_cholesky forms it with
// fx = fy = 1, through conic_rows), and the Adam update of the rotation-scale params; two lanes
// per Gaussian (four values each, swapped for the map and the conversion).  The spare last
// workgroup reduces the loss.
__global__ __launch_bounds__(256) void k_adam_pairs_rs(int n, const uint32_t *__restrict__ offsets, uint32_t capacity,
                                                       const float4 *__restrict__ part, float4 *__restrict__ p,
                                                       float4 *__restrict__ m, float4 *__restrict__ v, AdamHP ah,
                                                       const float *__restrict__ loss_part, int nparts,
                                                       double inv_count, float *__restrict__ loss,
                                                       float4 *__restrict__ chol) {
    if (loss && blockIdx.x == gridDim.x - 1) {
        __shared__ double sm[256];
        loss_reduce_block(nparts, loss_part, inv_count, loss, sm);
        return;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // lane h = i & 1 of Gaussian i >> 1: params 4h .. 4h + 3
    const int64_t g = i >> 1;
    const int h = (int)(i & 1);
    if (g >= n) return;
    float c1, c2;
    adam_step_bias(ah, c1, c2);
    const uint32_t o0 = offsets[g], o1r = offsets[g + 1];
    const uint32_t o1 = offsets[n] <= capacity ? o1r : o0;   // else the binning overflowed: zero gradient
    float4 gh = make_float4(0.f, 0.f, 0.f, 0.f);
    gather_half(part, o0, o1, h, gh);                     // this lane's 4 of the sums
    const float4 mine = p[2 * g + h];
    // the partner lane's halves: all the sums and params for the map
    const float4 oth = make_float4(__shfl_xor(gh.x, 1, 64), __shfl_xor(gh.y, 1, 64), __shfl_xor(gh.z, 1, 64),
                                   __shfl_xor(gh.w, 1, 64));
    const float4 op = make_float4(__shfl_xor(mine.x, 1, 64), __shfl_xor(mine.y, 1, 64), __shfl_xor(mine.z, 1, 64),
                                  __shfl_xor(mine.w, 1, 64));
    const float4 s0 = h ? oth : gh, s1 = h ? gh : oth;
    const float4 a = h ? op : mine, b = h ? mine : op;
    float4 r0 = make_float4(0.f, 0.f, 0.f, 0.f), r1 = r0;
    if (o1 > o0) {
        const CholRS c = rs_cholesky(a.z, a.w, b.x);
        const float3 r = conic_rows(c.l11, c.l21, c.l22);
        slot_grad_rs(a, b, 1.0f, 1.0f, r.x, r.y, r.z, s0, s1, r0, r1);
    }
    const float4 rg = h ? r1 : r0;
    float P[4] = {mine.x, mine.y, mine.z, mine.w};
    const float G[4] = {rg.x, rg.y, rg.z, rg.w};
    const float4 m4 = m[2 * g + h], v4 = v[2 * g + h];
    float M[4] = {m4.x, m4.y, m4.z, m4.w};
    float V[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) adam_update(P[k], G[k], M[k], V[k], ah.lr[4 * h + k], ah, c1, c2);
    p[2 * g + h] = make_float4(P[0], P[1], P[2], P[3]);
    m[2 * g + h] = make_float4(M[0], M[1], M[2], M[3]);
    v[2 * g + h] = make_float4(V[0], V[1], V[2], V[3]);
    if (chol) {                                           // the next step's Cholesky form
        const float4 np = make_float4(P[0], P[1], P[2], P[3]);
        const float4 qp = make_float4(__shfl_xor(np.x, 1, 64), __shfl_xor(np.y, 1, 64), __shfl_xor(np.z, 1, 64),
                                      __shfl_xor(np.w, 1, 64));
        const float4 A = h ? qp : np, B = h ? np : qp;
        const CholRS c = rs_cholesky(A.z, A.w, B.x);
        if (h == 0) chol[2 * g] = make_float4(A.x, A.y, c.l11, c.l21);
        else chol[2 * g + 1] = make_float4(c.l22, B.y, B.z, B.w);
    }
}

// dparams (+)= the gradient w.r.t. params of form `kind` from the pair slots: one thread per
// Gaussian, its slots added in emission order (as k_grad_gather), then the map of its form --
// the Cholesky form's (slot_grad_half, then the scaling by D) or the rotation-scale form's
// (slot_grad_rs) -- with the rows of the record the raster used.
__global__ __launch_bounds__(256) void k_grad_gather_params(int kind, int64_t n, const float4 *__restrict__ params,
                                                            float fx, float fy, const float4 *__restrict__ records,
                                                            const uint32_t *__restrict__ offsets, uint32_t capacity,
                                                            const float4 *__restrict__ part,
                                                            float4 *__restrict__ dparams) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= n || offsets[n] > capacity) return;          // overflow: nothing was rendered
    const uint32_t o0 = offsets[g], o1 = offsets[g + 1];
    if (o1 == o0) return;
    float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
    gather_slots(part, o0, o1, s0, s1);
    const float4 rp = records[2 * g], rq = records[2 * g + 1];
    float4 r0, r1;
    if (kind == 1) {
        slot_grad_rs(params[2 * g], params[2 * g + 1], fx, fy, rp.z, rp.w, rq.x, s0, s1, r0, r1);
    } else {
        const float4 d0 = slot_grad_half(0, rp.z, rp.w, rq.x, s0), d1 = slot_grad_half(1, rp.z, rp.w, rq.x, s1);
        r0 = make_float4(fx * d0.x, fy * d0.y, fx * d0.z, fy * d0.w);
        r1 = make_float4(fy * d1.x, d1.y, d1.z, d1.w);
    }
    float4 o = dparams[2 * g], q = dparams[2 * g + 1];
    o.x += r0.x; o.y += r0.y; o.z += r0.z; o.w += r0.w;
    q.x += r1.x; q.y += r1.y; q.z += r1.z; q.w += r1.w;
    dparams[2 * g] = o;
    dparams[2 * g + 1] = q;
}

hipError_t launch_params_to_cholesky(int kind, int64_t n, const float *in, float fx, float fy, float *out,
                                     hipStream_t s) {
    if (n == 0) return hipSuccess;
    k_params_to_cholesky<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
        kind, n, reinterpret_cast<const float4 *>(in), fx, fy, reinterpret_cast<float4 *>(out));
    return hipGetLastError();
}

hipError_t launch_grad_gather_params(int kind, int n, int W, int H, const float *params, float fx, float fy,
                                     const float *records, const uint32_t *offsets, int64_t capacity, const void *ws,
                                     float *dparams, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const BwdPlan pl = make_bwd_plan(W, H, capacity);
    k_grad_gather_params<<<(unsigned)(((int64_t)n + 255) / 256), 256, 0, s>>>(
        kind, n, reinterpret_cast<const float4 *>(params), fx, fy, reinterpret_cast<const float4 *>(records), offsets,
        (uint32_t)capacity, reinterpret_cast<const float4 *>(static_cast<const char *>(ws) + pl.off_part),
        reinterpret_cast<float4 *>(dparams));
    return hipGetLastError();
}

hipError_t launch_adam_pairs_rs(int n, int W, int H, const uint32_t *offsets, int64_t capacity, const void *ws,
                                float *p, float *m, float *v, const float *lr, double beta1, double beta2, double eps,
                                int step, const float *loss_partials, int64_t loss_count, float *d_loss, float *chol,
                                hipStream_t s) {
    const int nb = (int)((2 * (int64_t)n + 255) / 256) + (d_loss ? 1 : 0);
    if (nb == 0) return hipSuccess;
    const BwdPlan pl = make_bwd_plan(W, H, capacity);
    const AdamHP a = make_adam_hp(lr, beta1, beta2, eps, step, nullptr);
    const int ntiles = ((W + kTile - 1) / kTile) * ((H + kTile - 1) / kTile);
    k_adam_pairs_rs<<<nb, 256, 0, s>>>(
        n, offsets, (uint32_t)capacity, reinterpret_cast<const float4 *>(static_cast<const char *>(ws) + pl.off_part),
        reinterpret_cast<float4 *>(p), reinterpret_cast<float4 *>(m), reinterpret_cast<float4 *>(v), a,
        loss_partials, ntiles, loss_count > 0 ? 1.0 / (double)loss_count : 0.0, d_loss,
        reinterpret_cast<float4 *>(chol));
    return hipGetLastError();
}

hipError_t launch_params_to_cholesky_grad(int kind, int64_t n, const float *in, float fx, float fy,
                                          const float *dout, float *din, int accumulate, hipStream_t s) {
    if (n == 0) return hipSuccess;
    k_params_to_cholesky_grad<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
        kind, n, reinterpret_cast<const float4 *>(in), fx, fy, reinterpret_cast<const float4 *>(dout),
        reinterpret_cast<float4 *>(din), accumulate);
    return hipGetLastError();
}

}  // namespace gi
