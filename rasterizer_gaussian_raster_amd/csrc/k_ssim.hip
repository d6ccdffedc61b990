// k_ssim.hip -- the SSIM pixel loss L = w1 mean|x - y| + w2 mean (x - y)^2 + ws (1 - SSIM) and dL/dx
// ("Drawing with Gaussians", 2D fitting: (1 - w) L1 + w (1 - SSIM); "FlashImgs", Commands:
// --loss l1+ssim / l2+ssim).  Per channel, local statistics under an 11x11 Gaussian window
// (sigma 1.5, normalised), zero outside the image:
//   SSIM(p) = (2 mx my + C1)(2 sxy + C2) / ((mx^2 + my^2 + C1)(sxx + syy + C2)).
// The gradient of the mean SSIM needs the window sums of three per-pixel derivatives of the map
// (with respect to mx, Exx = <x^2>, Exy = <x y>):
//   dSSIM/dx(q) = (1/3HW) sum_p G(q - p) [D0(p) + 2 x(q) D1(p) + y(q) D2(p)].
// Two stencil kernels over 32x32 output tiles, one workgroup per tile and channel, the window
// separable (rows, then columns):
//   k_ssim_fwd  stages x, y of the tile and a 5-pixel halo in LDS; the row pass gives each thread
//               four adjacent outputs of a staged row (14 inputs, their products formed once, read
//               as float4 runs), the column pass four vertically adjacent outputs of a column; it
//               writes D0..D2 and per-tile partial sums (SSIM, |e|, e^2);
//   k_ssim_bwd  stages D0..D2 with the halo, filters them the same way and forms dL/dx; its spare
//               last workgroup adds up the partials (fp64, fixed order) into the loss.
// Both are FP32-VALU bound: 5 (then 3) maps x 11 taps per pass and output, the row pass over
// 42 staged rows per 32 output rows.  HBM: 8 B read + 12 B written per entry, then 20 B read +
// 4 B written.
#include <hip/hip_runtime.h>

#include <cmath>

#include "gi_launch.hpp"

namespace gi {

constexpr int kSsimR = 5;                                   // window radius
constexpr int kSsimTW = 32, kSsimTH = 32;                   // output tile
constexpr int kSsimSW = kSsimTW + 2 * kSsimR;               // staged columns (42)
constexpr int kSsimSH = kSsimTH + 2 * kSsimR;               // staged rows (42)
constexpr int kSsimSP = (kSsimSW + 2 + 3) & ~3;             // staged row stride: 16-byte rows, room for
                                                            // the last group's 14-wide read (44)
constexpr int kSsimNG = kSsimTW / 4;                        // 4-column groups per row (8)
constexpr int kSsimStageRounds = (kSsimSH + 3) / 4;         // staging: 4 rows x 64 columns per round
static_assert(kSsimSW <= 64, "a staged row is one wave wide");
constexpr float kC1 = 0.0001f, kC2 = 0.0009f;

struct SsimWin { float g[11]; };

// 14 consecutive floats of an LDS row from a 16-byte aligned start.
__device__ __forceinline__ void lds_run14(const float *p, float (&v)[14]) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4),
                 c = *reinterpret_cast<const float4 *>(p + 8);
    const float2 d = *reinterpret_cast<const float2 *>(p + 12);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    v[8] = c.x; v[9] = c.y; v[10] = c.z; v[11] = c.w;
    v[12] = d.x; v[13] = d.y;
}

// Stages NM planes (each W x H, `plane` apart) over the tile's rows and columns plus the halo into
// s[m][row][col] (zero outside the image).  Thread (tid / 64, tid % 64) takes column tid % 64 of
// rows tid / 64 + 4k: every row is one contiguous read; all loads go out before the first store.
template <int NM>
__device__ __forceinline__ void ssim_stage(const float *__restrict__ src, size_t plane, int W, int H, int x0, int y0,
                                           float (*s)[kSsimSH][kSsimSP]) {
    const int tid = threadIdx.x, c = tid & 63, r0 = tid >> 6;
    const int gx = x0 - kSsimR + c;
    const bool colok = c < kSsimSW && gx >= 0 && gx < W;
    float v[NM][kSsimStageRounds];
#pragma unroll
    for (int k = 0; k < kSsimStageRounds; ++k) {
        const int r = r0 + 4 * k, gy = y0 - kSsimR + r;
        const bool ok = colok && r < kSsimSH && gy >= 0 && gy < H;
        const size_t o = ok ? (size_t)gy * W + gx : 0;
#pragma unroll
        for (int m = 0; m < NM; ++m) v[m][k] = ok ? src[m * plane + o] : 0.0f;
    }
    if (c < kSsimSW) {
#pragma unroll
        for (int k = 0; k < kSsimStageRounds; ++k) {
            const int r = r0 + 4 * k;
            if (r < kSsimSH) {
#pragma unroll
                for (int m = 0; m < NM; ++m) s[m][r][c] = v[m][k];
            }
        }
    }
}

struct SsimFwdLds {
    alignas(16) float s[2][kSsimSH][kSsimSP];      // x, y of the staged pixels
    alignas(16) float h[3][kSsimSH][kSsimTW];      // row pass: (x, y), then (x^2, y^2, x y)
    float red[3][4];
};

// The maps a forward pass filters, by mode: kSsimFull filters x, y (first pass) and x^2, y^2, x y
// (second); kSsimPrepared takes the target's from the workspace and filters x, then x^2, x y;
// kSsimTarget filters the target's alone, y then y^2 (what kSsimPrepared reads).
enum SsimMode { kSsimFull = 0, kSsimPrepared = 1, kSsimTarget = 2 };
template <int MODE, bool SECOND>
struct SsimMaps {
    static constexpr int n = MODE == kSsimFull ? (SECOND ? 3 : 2) : MODE == kSsimPrepared ? (SECOND ? 2 : 1) : 1;
};

// Row pass for the task t (staged row t / NG, outputs 4 (t % NG) .. + 3) into h: the maps of
// SsimMaps, products formed once per input.  Every map takes the same operations in the same order
// in every mode, so a prepared target's statistics carry the bits of the full pass.
template <int MODE, bool SECOND>
__device__ __forceinline__ void ssim_fwd_rows(SsimFwdLds &L, int t, const SsimWin &win) {
    const int r = t / kSsimNG, c0 = (t % kSsimNG) * 4;
    constexpr int NM = SsimMaps<MODE, SECOND>::n;
    float in[NM][14];
    {
        float xv[14], yv[14];
        if (MODE != kSsimTarget) lds_run14(&L.s[0][r][c0], xv);
        if (MODE != kSsimPrepared || SECOND) lds_run14(&L.s[1][r][c0], yv);
#pragma unroll
        for (int b = 0; b < 14; ++b) {
            if (MODE == kSsimFull) {
                if (SECOND) {
                    in[0][b] = xv[b] * xv[b];
                    in[1][b] = yv[b] * yv[b];
                    in[2][b] = xv[b] * yv[b];
                } else {
                    in[0][b] = xv[b];
                    in[1][b] = yv[b];
                }
            } else if (MODE == kSsimPrepared) {
                if (SECOND) {
                    in[0][b] = xv[b] * xv[b];
                    in[NM - 1][b] = xv[b] * yv[b];
                } else {
                    in[0][b] = xv[b];
                }
            } else {
                in[0][b] = SECOND ? yv[b] * yv[b] : yv[b];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < NM; ++k) {
        float4 o;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            float a = 0.f;
#pragma unroll
            for (int b = 0; b < 11; ++b) a = fmaf(win.g[b], in[k][b + h], a);
            reinterpret_cast<float *>(&o)[h] = a;
        }
        *reinterpret_cast<float4 *>(&L.h[k][r][c0]) = o;
    }
}

// Column pass of NM maps of h: the four outputs (column tx, rows ty0 .. ty0 + 3) of each.
template <int NM>
__device__ __forceinline__ void ssim_cols(const float (*h)[kSsimSH][kSsimTW], int tx, int ty0, const SsimWin &win,
                                          float (&out)[4][NM]) {
#pragma unroll
    for (int k = 0; k < NM; ++k) {
        float hv[14];
#pragma unroll
        for (int a = 0; a < 14; ++a) hv[a] = h[k][ty0 + a][tx];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float m = 0.f;
#pragma unroll
            for (int a = 0; a < 11; ++a) m = fmaf(win.g[a], hv[a + q], m);
            out[q][k] = m;
        }
    }
}

constexpr int kSsimRowTasks = kSsimSH * kSsimNG;           // 336: one round of 256 threads + 80
static_assert(kSsimRowTasks <= 512, "at most two row tasks per thread");

// T: the target's window statistics, planes T[c] = mean of channel c, T[3 + c] = mean of its square
// (written by kSsimTarget, read by kSsimPrepared).
template <int MODE>
__global__ __launch_bounds__(256) void k_ssim_fwd(int W, int H, const float *__restrict__ x,
                                                  const float *__restrict__ y, SsimWin win,
                                                  float *__restrict__ D, float *__restrict__ part,
                                                  float *__restrict__ T) {
    __shared__ __align__(16) SsimFwdLds L;
    const int tid = threadIdx.x, ch = blockIdx.z;
    const int x0 = blockIdx.x * kSsimTW, y0 = blockIdx.y * kSsimTH;
    const size_t plane = (size_t)W * H;
    const int tx = tid & (kSsimTW - 1), ty0 = (tid / kSsimTW) * 4;   // this thread's four outputs
    const int j = x0 + tx;
    float ty_m[4], ty_e[4];                               // kSsimPrepared: the target's statistics
    if (MODE == kSsimPrepared) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = y0 + ty0 + q;
            const size_t o = (i < H && j < W) ? (size_t)i * W + j : 0;
            ty_m[q] = T[ch * plane + o];
            ty_e[q] = T[(3 + ch) * plane + o];
        }
    }
    {
        // x and y (separate arrays): the staging of ssim_stage, two sources
        const float *xc = MODE == kSsimTarget ? nullptr : x + ch * plane, *yc = y + ch * plane;
        const int c = tid & 63, r0 = tid >> 6;
        const int gx = x0 - kSsimR + c;
        const bool colok = c < kSsimSW && gx >= 0 && gx < W;
        float vx[kSsimStageRounds], vy[kSsimStageRounds];
#pragma unroll
        for (int k = 0; k < kSsimStageRounds; ++k) {
            const int r = r0 + 4 * k, gy = y0 - kSsimR + r;
            const bool ok = colok && r < kSsimSH && gy >= 0 && gy < H;
            const size_t o = ok ? (size_t)gy * W + gx : 0;
            if (MODE != kSsimTarget) vx[k] = ok ? xc[o] : 0.0f;
            vy[k] = ok ? yc[o] : 0.0f;
        }
        if (c < kSsimSW) {
#pragma unroll
            for (int k = 0; k < kSsimStageRounds; ++k) {
                const int r = r0 + 4 * k;
                if (r < kSsimSH) {
                    if (MODE != kSsimTarget) L.s[0][r][c] = vx[k];
                    L.s[1][r][c] = vy[k];
                }
            }
        }
    }
    __syncthreads();
    // the means
    constexpr int NA = SsimMaps<MODE, false>::n, NB = SsimMaps<MODE, true>::n;
    ssim_fwd_rows<MODE, false>(L, tid, win);
    if (tid + 256 < kSsimRowTasks) ssim_fwd_rows<MODE, false>(L, tid + 256, win);
    __syncthreads();
    float mu[4][NA];
    ssim_cols<NA>(L.h, tx, ty0, win, mu);
    __syncthreads();                                      // h is rewritten
    // the second moments
    ssim_fwd_rows<MODE, true>(L, tid, win);
    if (tid + 256 < kSsimRowTasks) ssim_fwd_rows<MODE, true>(L, tid + 256, win);
    __syncthreads();
    float m2[4][NB];
    ssim_cols<NB>(L.h, tx, ty0, win, m2);
    if (MODE == kSsimTarget) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = y0 + ty0 + q;
            if (i < H && j < W) {
                T[ch * plane + (size_t)i * W + j] = mu[q][0];
                T[(3 + ch) * plane + (size_t)i * W + j] = m2[q][0];
            }
        }
        return;
    }
    float f = 0.f, l1 = 0.f, l2 = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int ty = ty0 + q, i = y0 + ty;
        if (i < H && j < W) {
            const float mx = mu[q][0], my = MODE == kSsimFull ? mu[q][NA - 1] : ty_m[q];
            const float exx = m2[q][0], eyy = MODE == kSsimFull ? m2[q][1] : ty_e[q], exy = m2[q][NB - 1];
            const float sxx = exx - mx * mx, syy = eyy - my * my, sxy = exy - mx * my;
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
            const float e = L.s[0][ty + kSsimR][tx + kSsimR] - L.s[1][ty + kSsimR][tx + kSsimR];
            l1 += fabsf(e);
            l2 += e * e;
        }
    }
    // tile partials, reduced in a fixed order
    float v[3] = {f, l1, l2};
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        float s = v[k];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
        if ((tid & 63) == 0) L.red[k][tid >> 6] = s;
    }
    __syncthreads();
    if (tid < 3) {
        const size_t t = ((size_t)ch * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
        part[3 * t + tid] = ((L.red[tid][0] + L.red[tid][1]) + L.red[tid][2]) + L.red[tid][3];
    }
}

struct SsimBwdLds {
    union {                                         // the row pass overwrites the staged maps
        alignas(16) float s[3][kSsimSH][kSsimSP];  // D0, D1, D2 of the staged pixels
        alignas(16) float h[3][kSsimSH][kSsimTW];  // their row pass
    };
};

// Row pass of the three staged maps for the task t (staged row t / NG, outputs 4 (t % NG) .. + 3).
__device__ __forceinline__ void ssim_bwd_rows(const SsimBwdLds &L, int t, const SsimWin &win, float4 (&o)[3]) {
    const int r = t / kSsimNG, c0 = (t % kSsimNG) * 4;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        float dv[14];
        lds_run14(&L.s[k][r][c0], dv);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            float a = 0.f;
#pragma unroll
            for (int b = 0; b < 11; ++b) a = fmaf(win.g[b], dv[b + h], a);
            reinterpret_cast<float *>(&o[k])[h] = a;
        }
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
    // 1-D grid: the tiles (x fastest, then y, then channel), then one more workgroup for the loss
    const int gx = (W + kSsimTW - 1) / kSsimTW, gy = (H + kSsimTH - 1) / kSsimTH;
    const int bid = blockIdx.x, per_ch = gx * gy;
    if (bid == 3 * per_ch) {                              // the spare workgroup: the loss
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
    __shared__ __align__(16) SsimBwdLds L;
    const int tid = threadIdx.x, ch = bid / per_ch, rem = bid - ch * per_ch;
    const int x0 = (rem % gx) * kSsimTW, y0 = (rem / gx) * kSsimTH;
    // the four outputs' x and y load with the staging (column tid % 32, rows 4 (tid / 32) ..)
    const int tx = tid & (kSsimTW - 1), ty0 = (tid / kSsimTW) * 4;
    const int j = x0 + tx;
    float xv[4], yv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = y0 + ty0 + q;
        const bool in = i < H && j < W;
        const size_t o = ch * plane + (in ? (size_t)i * W + j : 0);
        xv[q] = x[o];
        yv[q] = y[o];
    }
    ssim_stage<3>(D + ch * plane, 3 * plane, W, H, x0, y0, L.s);
    __syncthreads();
    // rows: four adjacent outputs per task, held in registers until every thread has read the
    // staged maps (the results overwrite them)
    float4 o1[3], o2[3];
    ssim_bwd_rows(L, tid, win, o1);
    const bool two = tid + 256 < kSsimRowTasks;
    if (two) ssim_bwd_rows(L, tid + 256, win, o2);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        *reinterpret_cast<float4 *>(&L.h[k][tid / kSsimNG][(tid % kSsimNG) * 4]) = o1[k];
        if (two) *reinterpret_cast<float4 *>(&L.h[k][(tid + 256) / kSsimNG][((tid + 256) % kSsimNG) * 4]) = o2[k];
    }
    __syncthreads();
    float ss[4][3];
    ssim_cols<3>(L.h, tx, ty0, win, ss);
    // 1 / (3 H W) rounded once (the products below round like the divisions they replace, to 1 ulp)
    const float inv_nf = (float)inv_n;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = y0 + ty0 + q;
        if (i >= H || j >= W) continue;
        const float e = xv[q] - yv[q];
        const float dssim = fmaf(yv[q], ss[q][2], fmaf(2.0f * xv[q], ss[q][1], ss[q][0])) * inv_nf;
        const float sg = e > 0.0f ? 1.0f : (e < 0.0f ? -1.0f : 0.0f);
        dL[ch * plane + (size_t)i * W + j] = fmaf(w1, sg * inv_nf, fmaf(w2, 2.0f * e * inv_nf, -(ws * dssim)));
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

static size_t ssim_tiles(int W, int H) {
    return (size_t)((W + kSsimTW - 1) / kSsimTW) * ((H + kSsimTH - 1) / kSsimTH) * 3;
}

// Workspace: D (9 planes) | the target's statistics T (6 planes) | the tile partials.
struct SsimWs {
    float *D, *T, *part;
};
static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
static SsimWs ssim_ws(int W, int H, void *ws) {
    const size_t plane = (size_t)W * H;
    char *b = static_cast<char *>(ws);
    SsimWs w;
    w.D = reinterpret_cast<float *>(b);
    w.T = reinterpret_cast<float *>(b + align256(9 * plane * sizeof(float)));
    w.part = reinterpret_cast<float *>(b + align256(9 * plane * sizeof(float)) + align256(6 * plane * sizeof(float)));
    return w;
}

size_t ssim_workspace_bytes(int W, int H) {
    const size_t plane = (size_t)W * H;
    return align256(9 * plane * sizeof(float)) + align256(6 * plane * sizeof(float)) +
           3 * ssim_tiles(W, H) * sizeof(float);
}

hipError_t launch_ssim_target(int W, int H, const float *y, void *ws_ptr, hipStream_t s) {
    const SsimWs w = ssim_ws(W, H, ws_ptr);
    const dim3 grid((W + kSsimTW - 1) / kSsimTW, (H + kSsimTH - 1) / kSsimTH, 3);
    k_ssim_fwd<kSsimTarget><<<grid, 256, 0, s>>>(W, H, nullptr, y, ssim_window(), nullptr, nullptr, w.T);
    return hipGetLastError();
}

hipError_t launch_loss_ssim(int W, int H, const float *x, const float *y, float w1, float w2, float ws, float *dL,
                            float *loss, void *ws_ptr, bool target_prepared, hipStream_t s) {
    const SsimWin win = ssim_window();
    const SsimWs w = ssim_ws(W, H, ws_ptr);
    const dim3 grid((W + kSsimTW - 1) / kSsimTW, (H + kSsimTH - 1) / kSsimTH, 3);
    const int nparts = (int)ssim_tiles(W, H);
    if (target_prepared)
        k_ssim_fwd<kSsimPrepared><<<grid, 256, 0, s>>>(W, H, x, y, win, w.D, w.part, w.T);
    else
        k_ssim_fwd<kSsimFull><<<grid, 256, 0, s>>>(W, H, x, y, win, w.D, w.part, nullptr);
    k_ssim_bwd<<<nparts + 1, 256, 0, s>>>(W, H, x, y, win, w.D, w1, w2, ws, dL, w.part, nparts, (double)w1,
                                          (double)w2, (double)ws, loss);
    return hipGetLastError();
}

}  // namespace gi
