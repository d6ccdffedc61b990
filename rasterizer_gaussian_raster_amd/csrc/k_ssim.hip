// k_ssim.hip -- the SSIM pixel loss L = w1 mean|x - y| + w2 mean (x - y)^2 + ws (1 - SSIM) and dL/dx
// ("Drawing with Gaussians", 2D fitting: (1 - w) L1 + w (1 - SSIM); "FlashImgs", Commands:
// --loss l1+ssim / l2+ssim).  Per channel, local statistics under an 11x11 Gaussian window
// (sigma 1.5, normalised), zero outside the image:
//   SSIM(p) = (2 mx my + C1)(2 sxy + C2) / ((mx^2 + my^2 + C1)(sxx + syy + C2)).
// The gradient of the mean SSIM needs the window sums of three per-pixel derivatives of the map
// (with respect to mx, Exx = <x^2>, Exy = <x y>):
//   dSSIM/dx(q) = (1/3HW) sum_p G(q - p) [D0(p) + 2 x(q) D1(p) + y(q) D2(p)].
// Two stencil kernels, one 16x16 output tile per workgroup and channel, the window separable:
//   k_ssim_fwd  stages x, y of the tile and a 5-pixel halo in LDS, filters the five moments
//               (rows, then columns), writes D0..D2 and per-tile partial sums (SSIM, |e|, e^2);
//   k_ssim_bwd  stages D0..D2 with the halo, filters them, forms dL/dx; its spare last workgroup
//               adds up the partials (fp64, fixed order) into the loss.
// HBM-bound stencils: 8 B read + 12 B written per entry, then 20 B read + 4 B written.
#include <hip/hip_runtime.h>

#include <cmath>

#include "gi_launch.hpp"

namespace gi {

constexpr int kSsimT = 16, kSsimR = 5, kSsimS = kSsimT + 2 * kSsimR;   // 26 staged rows / columns
constexpr float kC1 = 0.0001f, kC2 = 0.0009f;

struct SsimWin { float g[11]; };

__device__ __forceinline__ float ssim_at(const float *a, int W, int H, int i, int j) {
    return (i >= 0 && i < H && j >= 0 && j < W) ? a[(size_t)i * W + j] : 0.0f;
}

__global__ __launch_bounds__(256) void k_ssim_fwd(int W, int H, const float *__restrict__ x,
                                                  const float *__restrict__ y, SsimWin win,
                                                  float *__restrict__ D, float *__restrict__ part) {
    __shared__ float sv[2][kSsimS][kSsimS + 1];           // x, y of the staged pixels
    __shared__ float hs[5][kSsimS][kSsimT + 1];
    __shared__ float red[3][4];
    const int tid = threadIdx.x, ch = blockIdx.z;
    const int x0 = blockIdx.x * kSsimT, y0 = blockIdx.y * kSsimT;
    const size_t plane = (size_t)W * H;
    const float *xc = x + ch * plane, *yc = y + ch * plane;
    // every load of the staging goes out before the first LDS store (one round of memory latency)
    constexpr int kRounds = (kSsimS * kSsimS + 255) / 256;
    float vx[kRounds], vy[kRounds];
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
        const int e = tid + 256 * q, r = e / kSsimS, c = e % kSsimS;
        const bool ok = e < kSsimS * kSsimS;
        vx[q] = ok ? ssim_at(xc, W, H, y0 - kSsimR + r, x0 - kSsimR + c) : 0.0f;
        vy[q] = ok ? ssim_at(yc, W, H, y0 - kSsimR + r, x0 - kSsimR + c) : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
        const int e = tid + 256 * q, r = e / kSsimS, c = e % kSsimS;
        if (e < kSsimS * kSsimS) {
            sv[0][r][c] = vx[q];
            sv[1][r][c] = vy[q];
        }
    }
    __syncthreads();
    // rows: every staged row, the tile's columns, two adjacent columns per thread (their 12 inputs
    // read once from LDS; the pass is bound by LDS reads)
    if (tid < kSsimS * kSsimT / 2) {
        const int r = tid >> 3, c = (tid & 7) * 2;
        float xv[12], yv[12];
#pragma unroll
        for (int b = 0; b < 12; ++b) {
            xv[b] = sv[0][r][c + b];
            yv[b] = sv[1][r][c + b];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, a4 = 0.f;
#pragma unroll
            for (int b = 0; b < 11; ++b) {
                const float g = win.g[b], u = xv[b + h], w = yv[b + h];
                a0 = fmaf(g, u, a0);
                a1 = fmaf(g, w, a1);
                a2 = fmaf(g, u * u, a2);
                a3 = fmaf(g, w * w, a3);
                a4 = fmaf(g, u * w, a4);
            }
            hs[0][r][c + h] = a0; hs[1][r][c + h] = a1; hs[2][r][c + h] = a2; hs[3][r][c + h] = a3;
            hs[4][r][c + h] = a4;
        }
    }
    __syncthreads();
    // columns: two vertically adjacent outputs per thread (threads < 128), the 12 rows they need
    // read once from LDS
    float f = 0.f, l1 = 0.f, l2 = 0.f;
    if (tid < kSsimT * kSsimT / 2) {
    const int tx = tid & 15, ty0 = (tid >> 4) * 2;
    float mm[2][5] = {{0.f, 0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        float hv[12];
#pragma unroll
        for (int a = 0; a < 12; ++a) hv[a] = hs[k][ty0 + a][tx];
#pragma unroll
        for (int a = 0; a < 11; ++a) {
            mm[0][k] = fmaf(win.g[a], hv[a], mm[0][k]);
            mm[1][k] = fmaf(win.g[a], hv[a + 1], mm[1][k]);
        }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
    const float *m = mm[r];
    const int ty = ty0 + r;
    const int i = y0 + ty, j = x0 + tx;
    if (i < H && j < W) {
        const float mx = m[0], my = m[1];
        const float sxx = m[2] - mx * mx, syy = m[3] - my * my, sxy = m[4] - mx * my;
        const float n1 = fmaf(2.0f * mx, my, kC1), n2 = fmaf(2.0f, sxy, kC2);
        const float d1 = mx * mx + my * my + kC1, d2 = sxx + syy + kC2;
        // hardware reciprocals (1 ulp): the divisions' rounding is far below the loss's tolerance
        const float rn1 = __builtin_amdgcn_rcpf(n1), rn2 = __builtin_amdgcn_rcpf(n2);
        const float rd1 = __builtin_amdgcn_rcpf(d1), rd2 = __builtin_amdgcn_rcpf(d2);
        const float fr = (n1 * n2) * (rd1 * rd2);
        f += fr;
        const float D0 = fr * (2.0f * my * (rn1 - rn2) + 2.0f * mx * (rd2 - rd1));
        const size_t o = ch * plane + (size_t)i * W + j;
        D[o] = D0;
        D[3 * plane + o] = -fr * rd2;
        D[6 * plane + o] = 2.0f * fr * rn2;
        const float e = sv[0][ty + kSsimR][tx + kSsimR] - sv[1][ty + kSsimR][tx + kSsimR];
        l1 += fabsf(e);
        l2 += e * e;
    }
    }
    }
    // tile partials, reduced in a fixed order
    float v[3] = {f, l1, l2};
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        float s = v[k];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
        if ((tid & 63) == 0) red[k][tid >> 6] = s;
    }
    __syncthreads();
    if (tid < 3) {
        const size_t t = ((size_t)ch * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
        part[3 * t + tid] = ((red[tid][0] + red[tid][1]) + red[tid][2]) + red[tid][3];
    }
}

__global__ __launch_bounds__(256) void k_ssim_bwd(int W, int H, const float *__restrict__ x,
                                                  const float *__restrict__ y, SsimWin win,
                                                  const float *__restrict__ D, float w1, float w2, float ws,
                                                  float *__restrict__ dL, const float *__restrict__ part,
                                                  int nparts, double w1d, double w2d, double wsd,
                                                  float *__restrict__ loss) {
    const size_t plane = (size_t)W * H;
    const double inv_n = 1.0 / (3.0 * (double)plane);
    if (blockIdx.z == 3) {                                // the spare workgroup: the loss
        if (blockIdx.x != 0 || blockIdx.y != 0) return;
        __shared__ double sred[3][4];
        double a[3] = {0.0, 0.0, 0.0};
        for (int t = threadIdx.x; t < nparts; t += 256)
#pragma unroll
            for (int k = 0; k < 3; ++k) a[k] += (double)part[3 * t + k];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) a[k] += __shfl_xor(a[k], d, 64);
            if ((threadIdx.x & 63) == 0) sred[k][threadIdx.x >> 6] = a[k];
        }
        __syncthreads();
        if (threadIdx.x == 0 && loss) {
            double t[3];
            for (int k = 0; k < 3; ++k) t[k] = ((sred[k][0] + sred[k][1]) + sred[k][2]) + sred[k][3];
            loss[0] = (float)(w1d * t[1] * inv_n + w2d * t[2] * inv_n + wsd * (1.0 - t[0] * inv_n));
        }
        return;
    }
    __shared__ float sd[3][kSsimS][kSsimS + 1];
    __shared__ float hs[3][kSsimS][kSsimT + 1];
    const int tid = threadIdx.x, ch = blockIdx.z;
    const int x0 = blockIdx.x * kSsimT, y0 = blockIdx.y * kSsimT;
    // two vertically adjacent outputs per thread (threads < 128); their inputs load with the staging
    const bool act = tid < kSsimT * kSsimT / 2;
    const int tx = tid & 15, ty0 = ((tid >> 4) & 7) * 2;
    float xv[2], yv[2];
    size_t oo[2];
    bool ins[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i = y0 + ty0 + r, j = x0 + tx;
        ins[r] = act && i < H && j < W;
        oo[r] = ch * plane + (size_t)(ins[r] ? i : 0) * W + (ins[r] ? j : 0);
        xv[r] = x[oo[r]];
        yv[r] = y[oo[r]];
    }
    constexpr int kRounds = (kSsimS * kSsimS + 255) / 256;
    float v[3][kRounds];
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
        const int e = tid + 256 * q, r = e / kSsimS, c = e % kSsimS;
        const bool ok = e < kSsimS * kSsimS;
#pragma unroll
        for (int k = 0; k < 3; ++k)
            v[k][q] = ok ? ssim_at(D + (3 * k + ch) * plane, W, H, y0 - kSsimR + r, x0 - kSsimR + c) : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
        const int e = tid + 256 * q, r = e / kSsimS, c = e % kSsimS;
        if (e < kSsimS * kSsimS)
#pragma unroll
            for (int k = 0; k < 3; ++k) sd[k][r][c] = v[k][q];
    }
    __syncthreads();
    if (tid < kSsimS * kSsimT / 2) {                      // rows, two adjacent columns per thread
        const int r = tid >> 3, c = (tid & 7) * 2;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            float dv[12];
#pragma unroll
            for (int b = 0; b < 12; ++b) dv[b] = sd[k][r][c + b];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float a = 0.f;
#pragma unroll
                for (int b = 0; b < 11; ++b) a = fmaf(win.g[b], dv[b + h], a);
                hs[k][r][c + h] = a;
            }
        }
    }
    __syncthreads();
    if (!act) return;
    float ss[2][3] = {{0.f, 0.f, 0.f}, {0.f, 0.f, 0.f}};
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        float hv[12];
#pragma unroll
        for (int a = 0; a < 12; ++a) hv[a] = hs[k][ty0 + a][tx];
#pragma unroll
        for (int a = 0; a < 11; ++a) {
            ss[0][k] = fmaf(win.g[a], hv[a], ss[0][k]);
            ss[1][k] = fmaf(win.g[a], hv[a + 1], ss[1][k]);
        }
    }
    const float n = (float)(3.0 * (double)plane);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (!ins[r]) continue;
        const float e = xv[r] - yv[r];
        const float dssim = fmaf(yv[r], ss[r][2], fmaf(2.0f * xv[r], ss[r][1], ss[r][0])) / n;
        const float sg = e > 0.0f ? 1.0f : (e < 0.0f ? -1.0f : 0.0f);
        dL[oo[r]] = fmaf(w1, sg / n, fmaf(w2, 2.0f * e / n, -(ws * dssim)));
    }
}

static SsimWin ssim_window() {
    SsimWin w;
    double g[11], s = 0.0;
    for (int k = 0; k < 11; ++k) {
        g[k] = std::exp(-((k - 5) * (k - 5)) / (2.0 * 1.5 * 1.5));
        s += g[k];
    }
    for (int k = 0; k < 11; ++k) w.g[k] = (float)(g[k] / s);
    return w;
}

size_t ssim_workspace_bytes(int W, int H) {
    const size_t plane = (size_t)W * H;
    const size_t tiles = (size_t)((W + kSsimT - 1) / kSsimT) * ((H + kSsimT - 1) / kSsimT) * 3;
    return ((9 * plane * sizeof(float) + 255) & ~(size_t)255) + 3 * tiles * sizeof(float);
}

hipError_t launch_loss_ssim(int W, int H, const float *x, const float *y, float w1, float w2, float ws, float *dL,
                            float *loss, void *ws_ptr, hipStream_t s) {
    const SsimWin win = ssim_window();
    const size_t plane = (size_t)W * H;
    float *D = static_cast<float *>(ws_ptr);
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws_ptr) +
                                            ((9 * plane * sizeof(float) + 255) & ~(size_t)255));
    const dim3 grid((W + kSsimT - 1) / kSsimT, (H + kSsimT - 1) / kSsimT, 3);
    const int nparts = (int)(grid.x * grid.y * 3);
    k_ssim_fwd<<<grid, 256, 0, s>>>(W, H, x, y, win, D, part);
    const dim3 grid_b(grid.x, grid.y, 4);                  // z = 3: the loss workgroup (0, 0, 3)
    k_ssim_bwd<<<grid_b, 256, 0, s>>>(W, H, x, y, win, D, w1, w2, ws, dL, part, nparts, (double)w1, (double)w2,
                                      (double)ws, loss);
    return hipGetLastError();
}

}  // namespace gi
