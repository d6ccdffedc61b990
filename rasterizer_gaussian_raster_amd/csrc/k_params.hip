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

__global__ __launch_bounds__(256) void k_params_to_cholesky_grad(int kind, int64_t n, const float4 *__restrict__ in,
                                                                float fx, float fy, const float4 *__restrict__ dout,
                                                                float4 *__restrict__ din, int accumulate) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= n) return;
    const float4 a = in[2 * g], b = in[2 * g + 1];
    const float4 d0 = dout[2 * g], d1 = dout[2 * g + 1];
    // gradients w.r.t. the unscaled Cholesky form
    const float gmx = fx * d0.x, gmy = fy * d0.y, g11 = fx * d0.z, g21 = fy * d0.w, g22 = fy * d1.x;
    float4 r0, r1;
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
    if (accumulate) {
        const float4 o0 = din[2 * g], o1 = din[2 * g + 1];
        r0 = make_float4(o0.x + r0.x, o0.y + r0.y, o0.z + r0.z, o0.w + r0.w);
        r1 = make_float4(o1.x + r1.x, o1.y + r1.y, o1.z + r1.z, o1.w + r1.w);
    }
    din[2 * g] = r0;
    din[2 * g + 1] = r1;
}

hipError_t launch_params_to_cholesky(int kind, int64_t n, const float *in, float fx, float fy, float *out,
                                     hipStream_t s) {
    if (n == 0) return hipSuccess;
    k_params_to_cholesky<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
        kind, n, reinterpret_cast<const float4 *>(in), fx, fy, reinterpret_cast<float4 *>(out));
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
