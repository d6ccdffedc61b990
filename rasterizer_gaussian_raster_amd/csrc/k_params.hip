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
// Gaussian (a, b) scaled by (fx, fy).
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
            const float inv = 1.0f / c.l11;
            const float gl11 = g11 - (g21 * c.l21 + g22 * c.l22) * inv;
            const float gA = 0.5f * gl11 * inv, gB = g21 * inv, gP = g22 * inv;
            const float cc = c.cs * c.cs, ss = c.sn * c.sn, csn = c.cs * c.sn;
            const float dsq = (c.ax - c.ay) * (c.ax + c.ay);
            const float gax = 2.0f * c.ax * fmaf(gA, cc, gB * csn) + gP * c.ay;
            const float gay = 2.0f * c.ay * fmaf(gA, ss, -(gB * csn)) + gP * c.ax;
            const float gth = fmaf(-2.0f * (csn * dsq), gA, gB * ((cc - ss) * dsq));
            r0 = make_float4(gmx, gmy, copysignf(1.0f, a.z) * gax, copysignf(1.0f, a.w) * gay);
            r1 = make_float4(gth, d1.y, d1.z, d1.w);
        }
    } else {
        r0 = make_float4(gmx, gmy, g11, g21);
        r1 = make_float4(g22, d1.y, d1.z, d1.w);
    }
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

// Rotation-scale training: each Gaussian's per-pair gradient slots added in emission order (the
// Cholesky-form gradient, as k_grad_gather forms it), the chain rule, and the Adam update of the
// rotation-scale params; two lanes per Gaussian (four values each, swapped for the chain rule and
// the conversion).  The spare last workgroup reduces the loss.
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
    const int i = blockIdx.x * 256 + threadIdx.x;         // lane h = i & 1 of Gaussian i >> 1: params 4h .. 4h + 3
    const int g = i >> 1, h = i & 1;
    if (g >= n) return;
    float c1, c2;
    adam_step_bias(ah, c1, c2);
    const uint32_t o0 = offsets[g], o1r = offsets[g + 1];
    const uint32_t o1 = offsets[n] <= capacity ? o1r : o0;   // else the binning overflowed: zero gradient
    float4 gh = make_float4(0.f, 0.f, 0.f, 0.f);
    gather_half(part, o0, o1, h, gh);                     // this lane's 4 of the Cholesky-form gradient
    const float4 mine = p[2 * g + h];
    // the partner lane's halves: the whole gradient and params for the chain rule
    const float4 oth = make_float4(__shfl_xor(gh.x, 1, 64), __shfl_xor(gh.y, 1, 64), __shfl_xor(gh.z, 1, 64),
                                   __shfl_xor(gh.w, 1, 64));
    const float4 op = make_float4(__shfl_xor(mine.x, 1, 64), __shfl_xor(mine.y, 1, 64), __shfl_xor(mine.z, 1, 64),
                                  __shfl_xor(mine.w, 1, 64));
    const float4 d0 = h ? oth : gh, d1 = h ? gh : oth;
    const float4 a = h ? op : mine, b = h ? mine : op;
    float4 r0 = make_float4(0.f, 0.f, 0.f, 0.f), r1 = r0;
    if (o1 > o0) chol_chain(1, a, b, 1.0f, 1.0f, d0, d1, r0, r1);
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

// Moment-matching merge of Gaussian pairs: one thread per pair, in fp64 (the covariance sum and
// its factor cancel; the chip's fp64 rate is no concern for a per-pair op).  Masses
// w = |det L| sum |c|; mean and covariance of the weighted mixture; L = chol(Sigma) with a positive
// diagonal; colours keep each channel's integral.  An index outside [0, n) gives a NaN row.
__global__ __launch_bounds__(256) void k_merge_pairs(int64_t np, int64_t n, const float4 *__restrict__ params,
                                                    const int2 *__restrict__ pairs, float4 *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= np) return;
    const int2 pr = pairs[t];
    if (pr.x < 0 || pr.y < 0 || pr.x >= n || pr.y >= n) {
        const float q = __int_as_float(0x7fc00000);
        out[2 * t] = make_float4(q, q, q, q);
        out[2 * t + 1] = make_float4(q, q, q, q);
        return;
    }
    const float4 a0 = params[2 * (int64_t)pr.x], a1 = params[2 * (int64_t)pr.x + 1];
    const float4 b0 = params[2 * (int64_t)pr.y], b1 = params[2 * (int64_t)pr.y + 1];
    const double da = fabs((double)a0.z * a1.x), db = fabs((double)b0.z * b1.x);
    const double wa = da * (fabs((double)a1.y) + fabs((double)a1.z) + fabs((double)a1.w));
    const double wb = db * (fabs((double)b1.y) + fabs((double)b1.z) + fabs((double)b1.w));
    const double W = wa + wb;
    const double fa = W > 0.0 ? wa / W : 0.5, fb = W > 0.0 ? wb / W : 0.5;
    const double mx = fa * a0.x + fb * b0.x, my = fa * a0.y + fb * b0.y;
    const double ax = a0.x - mx, ay = a0.y - my, bx = b0.x - mx, by = b0.y - my;
    const double al11 = a0.z, al21 = a0.w, al22 = a1.x, bl11 = b0.z, bl21 = b0.w, bl22 = b1.x;
    const double s11 = fa * (al11 * al11 + ax * ax) + fb * (bl11 * bl11 + bx * bx);
    const double s21 = fa * (al11 * al21 + ax * ay) + fb * (bl11 * bl21 + bx * by);
    const double s22 = fa * (al21 * al21 + al22 * al22 + ay * ay) + fb * (bl21 * bl21 + bl22 * bl22 + by * by);
    const double l11 = sqrt(s11), l21 = s21 / l11, l22 = sqrt(s22 - l21 * l21);
    const double dn = l11 * l22;
    out[2 * t] = make_float4((float)mx, (float)my, (float)l11, (float)l21);
    out[2 * t + 1] = make_float4((float)l22, (float)((da * a1.y + db * b1.y) / dn), (float)((da * a1.z + db * b1.z) / dn),
                                 (float)((da * a1.w + db * b1.w) / dn));
}

hipError_t launch_merge_pairs(int64_t np, int64_t n, const float *params, const int32_t *pairs, float *out,
                              hipStream_t s) {
    if (np == 0) return hipSuccess;
    k_merge_pairs<<<(unsigned)((np + 255) / 256), 256, 0, s>>>(np, n, reinterpret_cast<const float4 *>(params),
                                                              reinterpret_cast<const int2 *>(pairs),
                                                              reinterpret_cast<float4 *>(out));
    return hipGetLastError();
}

hipError_t launch_params_to_cholesky(int kind, int64_t n, const float *in, float fx, float fy, float *out,
                                     hipStream_t s) {
    if (n == 0) return hipSuccess;
    k_params_to_cholesky<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
        kind, n, reinterpret_cast<const float4 *>(in), fx, fy, reinterpret_cast<float4 *>(out));
    return hipGetLastError();
}

hipError_t launch_adam_pairs_rs(int n, int W, int H, const uint32_t *offsets, int64_t capacity, const void *ws,
                                float *p, float *m, float *v, const float *lr, double beta1, double beta2, double eps,
                                int step, const float *loss_partials, int64_t loss_count, float *d_loss, float *chol,
                                hipStream_t s) {
    const int nb = (2 * n + 255) / 256 + (d_loss ? 1 : 0);
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
