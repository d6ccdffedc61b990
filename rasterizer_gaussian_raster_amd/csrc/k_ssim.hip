// k_ssim.hip -- the SSIM pixel loss L = w1 mean|x - y| + w2 mean (x - y)^2 + ws (1 - SSIM) and dL/dx
// ("Drawing with Gaussians", 2D fitting: (1 - w) L1 + w (1 - SSIM); "FlashImgs", Commands:
// --loss l1+ssim / l2+ssim).  Per channel, local statistics under an 11x11 Gaussian window
// (sigma 1.5, normalised), zero outside the image:
//   SSIM(p) = (2 mx my + C1)(2 sxy + C2) / ((mx^2 + my^2 + C1)(sxx + syy + C2)).
// The gradient of the mean SSIM needs the window sums of three per-pixel derivatives of the map
// (with respect to mx, Exx = <x^2>, Exy = <x y>):
//   dSSIM/dx(q) = (1/3HW) sum_p G(q - p) [D0(p) + 2 x(q) D1(p) + y(q) D2(p)].
// The window is separable: every filtering below is a row pass then a column pass.
//   k_ssim_target  the target's half of the statistics (my, Eyy per pixel), the same for every
//                  image of a fit: formed once into the workspace as float2 planes;
//   k_ssim_loss    the rest in one pass per 48x32 output tile and channel: it stages x, y over the
//                  tile and a 10-pixel border (float4 loads), filters x, x^2, x y over the tile and
//                  a 5-pixel border, forms D0..D2 there, filters those in turn and writes dL/dx of
//                  the tile with the tile's partial sums (SSIM, |e|, e^2); the workgroup that
//                  finishes last adds up the partials (fp64, fixed order) into the loss.
// No per-pixel map goes through memory between the passes: HBM sees x, y, (my, Eyy) and dL/dx once
// (20 B per entry).  The work is FP32 VALU: per tile and map 52 x 60 row-pass outputs and 42 x 58
// statistics, then 42 x 48 and 32 x 48 for D, 11 taps each.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>

#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

constexpr int kSsimR = 5;                                   // window radius
constexpr int kSsimT = 32;                                  // output tile (32 x 32)
constexpr float kC1 = 0.0001f, kC2 = 0.0009f;
constexpr int kTicketGroups = 16;                           // first-level ticket counters of the loss
constexpr int kTicketStride = 64;                           // unsigned: one counter per 256 bytes

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

// 18 consecutive floats of an LDS row from a 16-byte aligned start.
__device__ __forceinline__ void lds_run18(const float *p, float (&v)[18]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float4 a = *reinterpret_cast<const float4 *>(p + 4 * k);
        v[4 * k] = a.x; v[4 * k + 1] = a.y; v[4 * k + 2] = a.z; v[4 * k + 3] = a.w;
    }
    const float2 d = *reinterpret_cast<const float2 *>(p + 16);
    v[16] = d.x; v[17] = d.y;
}

// The window over 14 consecutive inputs: four adjacent outputs (taps in a fixed order).
__device__ __forceinline__ float4 win4(const float (&v)[14], const SsimWin &w) {
    float o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        float a = 0.f;
#pragma unroll
        for (int b = 0; b < 11; ++b) a = fmaf(w.g[b], v[b + h], a);
        o[h] = a;
    }
    return make_float4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------------------------------------
// k_ssim_target: (my, Eyy) of every pixel of channel blockIdx.z, one 32x32 tile per workgroup.

constexpr int kTgSW = kSsimT + 2 * kSsimR;                  // staged columns and rows (42)
constexpr int kTgSP = 44;                                   // staged row stride (16-byte rows)
constexpr int kTgRounds = (kTgSW + 3) / 4;                  // staging: 4 rows x 64 columns per round
constexpr int kTgRowTasks = kTgSW * (kSsimT / 4);           // 336
static_assert(kTgSW <= 64 && kTgRowTasks <= 512, "one staged row per wave, two row tasks per thread");

struct SsimTargetLds {
    alignas(16) float s[kTgSW][kTgSP];                      // y of the staged pixels
    alignas(16) float h[2][kTgSW][kSsimT];                  // row pass of y, y^2
};

__global__ __launch_bounds__(256) void k_ssim_target(int W, int H, const float *__restrict__ y, SsimWin win,
                                                     float2 *__restrict__ T, unsigned *__restrict__ done) {
    __shared__ __align__(16) SsimTargetLds L;
    const int tid = threadIdx.x, ch = blockIdx.z;
    const int x0 = blockIdx.x * kSsimT, y0 = blockIdx.y * kSsimT;
    const size_t plane = (size_t)W * H;
    const float *yc = y + ch * plane;
    if (done && (blockIdx.x | blockIdx.y | blockIdx.z) == 0 && tid <= kTicketGroups)   // the loss's ticket counts
        done[kTicketStride * tid] = 0;
    {
        // thread (tid / 64, tid % 64) stages column tid % 64 of rows tid / 64 + 4k
        const int c = tid & 63, r0 = tid >> 6, gx = x0 - kSsimR + c;
        const bool colok = c < kTgSW && gx >= 0 && gx < W;
        float v[kTgRounds];
#pragma unroll
        for (int k = 0; k < kTgRounds; ++k) {
            const int r = r0 + 4 * k, gy = y0 - kSsimR + r;
            const bool ok = colok && r < kTgSW && gy >= 0 && gy < H;
            v[k] = ok ? yc[(size_t)gy * W + gx] : 0.0f;
        }
        if (c < kTgSW) {
#pragma unroll
            for (int k = 0; k < kTgRounds; ++k)
                if (r0 + 4 * k < kTgSW) L.s[r0 + 4 * k][c] = v[k];
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int t = tid + 256 * u;
        if (t < kTgRowTasks) {
            const int r = t / (kSsimT / 4), c0 = (t % (kSsimT / 4)) * 4;
            float v[14], v2[14];
            lds_run14(&L.s[r][c0], v);
#pragma unroll
            for (int b = 0; b < 14; ++b) v2[b] = v[b] * v[b];
            *reinterpret_cast<float4 *>(&L.h[0][r][c0]) = win4(v, win);
            *reinterpret_cast<float4 *>(&L.h[1][r][c0]) = win4(v2, win);
        }
    }
    __syncthreads();
    const int tx = tid & (kSsimT - 1), ty0 = (tid / kSsimT) * 4, j = x0 + tx;
    float hv[2][14];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int a = 0; a < 14; ++a) hv[k][a] = L.h[k][ty0 + a][tx];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = y0 + ty0 + q;
        float m[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            float a = 0.f;
#pragma unroll
            for (int b = 0; b < 11; ++b) a = fmaf(win.g[b], hv[k][b + q], a);
            m[k] = a;
        }
        if (i < H && j < W) T[ch * plane + (size_t)i * W + j] = make_float2(m[0], m[1]);
    }
}

// ---------------------------------------------------------------------------------------------
// k_ssim_loss: one workgroup per 48x32 output tile and channel (a 768x512 image has 768 of them,
// three per CU of MI355X, in one round).  Regions, relative to the tile's origin (x0, y0):
//   staged      rows y0 - 10 .. y0 + 41 (52), columns x0 - 10 .. x0 + 57 (68);
//   statistics  rows y0 - 5 .. y0 + 36 (42), columns x0 - 5 .. x0 + 52 (58; the row pass forms 60
//               in groups of four, the last two unused);
//   D           the statistics region.
// LDS holds the staged maps, ONE map's row pass at a time (x, then x^2, then x y; later D0, D1, D2
// in turn) and one of D0..D2, about 51 KB.  Every row stride is an odd multiple of 4 floats, and
// the tasks that read or write float4 runs give a wave's lanes consecutive rows of one column group,
// so each 8 lanes' float4 accesses cover the 32 banks once.
constexpr int kLossNT = 512;                                // threads per workgroup (8 waves)
constexpr int kLossWaves = kLossNT / 64;
constexpr int kTW = 48, kTH = 32;                           // output tile
constexpr int kSR = kTH + 4 * kSsimR;                       // 52 staged rows
constexpr int kSC = kTW + 4 * kSsimR;                       // 68 staged columns
constexpr int kSP = 68;                                     // staged row stride (4 mod 32)
constexpr int kSV = (kTW + 24) / 4;                         // float4 loads per staged row (from x0 - 12)
constexpr int kSN4 = kSR * kSV;                             // 936 per map
constexpr int kMR = kTH + 2 * kSsimR;                       // 42 statistics rows
constexpr int kMC = kTW + 2 * kSsimR;                       // 58 statistics columns
constexpr int kMG = (kMC + 7) / 8;                          // 8 row-pass column groups of 8 outputs
constexpr int kHP = 68;                                     // row-pass stride (4 mod 32; >= 8 kMG)
constexpr int kRowTasks = kSR * kMG;                        // 416: one round
constexpr int kColRows = 6;                                 // outputs per column task
constexpr int kColGroups = kMR / kColRows;                  // 7
constexpr int kColTasks = kMC * kColGroups;                 // 406: one round
constexpr int kDP = 60;                                     // D stride (28 mod 32)
constexpr int kBG = kTW / 4;                                // 12 D row-pass column groups
constexpr int kBRowTasks = kMR * kBG;                       // 504
constexpr int kBP = 52;                                     // D row-pass stride (20 mod 32)
constexpr int kOutTasks = kTW * (kTH / 4);                  // 384 tasks of four outputs
constexpr int rounds(int n) { return (n + kLossNT - 1) / kLossNT; }
static_assert(kSP >= kSC && kHP >= 8 * kMG && kDP >= kMC && kBP >= kTW, "strides");
static_assert(8 * (kMG - 1) + 18 <= kSP + 6 && 4 * (kBG - 1) + 14 <= kMC, "row-pass reads");
static_assert(kColGroups * kColRows == kMR && kRowTasks <= kLossNT && kColTasks <= kLossNT, "one round");

struct SsimLossLds {
    alignas(16) float s[2][kSR][kSP];                       // x, y staged (kept to the end)
    alignas(16) float d[kMR][kDP];                          // one of D0..D2 over the statistics region
    union {
        alignas(16) float h[kSR][kHP];                      // row pass of one of x, x^2, x y
        alignas(16) float hb[kMR][kBP];                     // row pass of one of D0..D2
    };
    float red[3][kLossWaves];
    double dred[3][kLossWaves];
    int last;
};
// the row pass's last column group reads six floats past the end of its row (for the six unused
// outputs): the next row's, or for the last row of y the first six of d, which follows s
static_assert(offsetof(SsimLossLds, d) == sizeof(float) * 2 * kSR * kSP, "d follows s");

// Stages x and y (one channel each) over the staged region into s (zero outside the image), in two
// halves so that other loads can be issued between them: ssim_stage_load issues this thread's loads,
// ssim_stage_store writes them.  Loads are float4s from x0 - 12 (VEC: W a multiple of 4 and 16-byte
// aligned planes, so each float4 of a row lies wholly inside or wholly outside the image; else
// element by element), stored as two float2 halves two columns to the left (the halves outside the
// staged columns are dropped).
constexpr int kStageRounds = rounds(kSN4);                  // 2
template <bool VEC>
__device__ __forceinline__ void ssim_stage_load(const float *__restrict__ x, const float *__restrict__ y, int W,
                                                int H, int x0, int y0, float4 (&vx)[kStageRounds],
                                                float4 (&vy)[kStageRounds]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < kStageRounds; ++k) {
        const int f = tid + kLossNT * k, r = f / kSV, c = (f - r * kSV) * 4;
        const int gy = y0 - 2 * kSsimR + r, gx = x0 - 12 + c;
        const bool rowok = f < kSN4 && gy >= 0 && gy < H;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (VEC) {
            if (rowok && gx >= 0 && gx < W) {
                const size_t o = (size_t)gy * W + gx;
                a = *reinterpret_cast<const float4 *>(x + o);
                b = *reinterpret_cast<const float4 *>(y + o);
            }
        } else if (rowok) {
            const size_t row = (size_t)gy * W;
            float *pa = reinterpret_cast<float *>(&a), *pb = reinterpret_cast<float *>(&b);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (gx + e >= 0 && gx + e < W) {
                    pa[e] = x[row + gx + e];
                    pb[e] = y[row + gx + e];
                }
        }
        vx[k] = a;
        vy[k] = b;
    }
}
__device__ __forceinline__ void ssim_stage_store(const float4 (&vx)[kStageRounds], const float4 (&vy)[kStageRounds],
                                                 float (*s)[kSR][kSP]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < kStageRounds; ++k) {
        const int f = tid + kLossNT * k, r = f / kSV, c = (f - r * kSV) * 4 - 2;
        if (f < kSN4) {
            if (c >= 0) {
                *reinterpret_cast<float2 *>(&s[0][r][c]) = make_float2(vx[k].x, vx[k].y);
                *reinterpret_cast<float2 *>(&s[1][r][c]) = make_float2(vy[k].x, vy[k].y);
            }
            if (c + 2 < kSC) {
                *reinterpret_cast<float2 *>(&s[0][r][c + 2]) = make_float2(vx[k].z, vx[k].w);
                *reinterpret_cast<float2 *>(&s[1][r][c + 2]) = make_float2(vy[k].z, vy[k].w);
            }
        }
    }
}

// Row pass task t of map MAP (0: x, 1: x^2, 2: x y): staged row t % 52, statistics columns
// 8 (t / 52) .. + 7 from 18 consecutive staged values.
template <int MAP>
__device__ __forceinline__ void ssim_loss_rows(SsimLossLds &L, int t, const SsimWin &win) {
    const int g = t / kSR, r = t - g * kSR, c0 = 8 * g;
    float v[18];
    lds_run18(&L.s[0][r][c0], v);
    if (MAP == 1) {
#pragma unroll
        for (int b = 0; b < 18; ++b) v[b] = v[b] * v[b];
    } else if (MAP == 2) {
        float w[18];
        lds_run18(&L.s[1][r][c0], w);
#pragma unroll
        for (int b = 0; b < 18; ++b) v[b] = v[b] * w[b];
    }
    float o[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) {
        float a = 0.f;
#pragma unroll
        for (int b = 0; b < 11; ++b) a = fmaf(win.g[b], v[b + h], a);
        o[h] = a;
    }
    *reinterpret_cast<float4 *>(&L.h[r][c0]) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4 *>(&L.h[r][c0 + 4]) = make_float4(o[4], o[5], o[6], o[7]);
}

// Column task u: statistics column u % 58, rows 6 (u / 58) .. + 5.
__device__ __forceinline__ void ssim_col_task(int u, int &jj, int &i0) {
    const int g = u / kMC;
    jj = u - g * kMC;
    i0 = kColRows * g;
}

// The 11-tap window down a column of an LDS map (row stride P) from its first row: N vertically
// adjacent outputs.
template <int P, int N>
__device__ __forceinline__ void ssim_col(const float *col, const SsimWin &win, float (&o)[N]) {
    float hv[N + 10];
#pragma unroll
    for (int a = 0; a < N + 10; ++a) hv[a] = col[a * P];
#pragma unroll
    for (int q = 0; q < N; ++q) {
        float a = 0.f;
#pragma unroll
        for (int b = 0; b < 11; ++b) a = fmaf(win.g[b], hv[b + q], a);
        o[q] = a;
    }
}

// One statistics map: its row pass into h, then the column pass of this thread's column task.
template <int MAP>
__device__ __forceinline__ void ssim_loss_map(SsimLossLds &L, const SsimWin &win, bool coltask, int jj, int i0,
                                              float (&m)[kColRows]) {
    const int tid = threadIdx.x;
    if (tid < kRowTasks) ssim_loss_rows<MAP>(L, tid, win);
    __syncthreads();
    if (coltask) ssim_col<kHP, kColRows>(&L.h[i0][jj], win, m);
    __syncthreads();                                        // h is rewritten next
}

// three workgroups (24 waves) per CU: at most 80 VGPRs
template <bool VEC>
__global__ __launch_bounds__(kLossNT) __attribute__((amdgpu_waves_per_eu(6))) void k_ssim_loss(
    int W, int H, const float *__restrict__ x, const float *__restrict__ y, const float2 *__restrict__ T, SsimWin win,
    float w1, float w2, float ws, float *__restrict__ dL, float *__restrict__ part, int ntiles, int nblk, double w1d,
    double w2d, double wsd, float *__restrict__ loss, unsigned *__restrict__ done) {
    __shared__ __align__(16) SsimLossLds L;
    const int tile = xcd_remap(blockIdx.x, nblk);           // an XCD takes neighbouring tiles
    if (tile >= ntiles) return;
    const int gx = (W + kTW - 1) / kTW, gy = (H + kTH - 1) / kTH, per_ch = gx * gy;
    const int ch = tile / per_ch, rem = tile - ch * per_ch;
    const int x0 = (rem % gx) * kTW, y0 = (rem / gx) * kTH;
    const size_t plane = (size_t)W * H;
    const int tid = threadIdx.x;
    // the staged maps' loads first, then the target's statistics at this thread's column tasks
    // (needed later; pixel 0 of the plane stands in outside the image, where they are not used)
    float4 vx[kStageRounds], vy[kStageRounds];
    ssim_stage_load<VEC>(x + ch * plane, y + ch * plane, W, H, x0, y0, vx, vy);
    // this thread's column task: statistics column jj, rows i0 .. i0 + 5
    const bool coltask = tid < kColTasks;
    int jj, i0;
    ssim_col_task(tid, jj, i0);
    const int px = x0 - kSsimR + jj;
    float2 tq[kColRows];
#pragma unroll
    for (int q = 0; q < kColRows; ++q) {
        const int py = y0 - kSsimR + i0 + q;
        const bool ok = coltask && px >= 0 && px < W && py >= 0 && py < H;
        tq[q] = T[ch * plane + (ok ? (size_t)py * W + px : 0)];
    }
    ssim_stage_store(vx, vy, L.s);
    __syncthreads();
    // the statistics: mx, Exx, Exy at the column task's pixels
    float mx[kColRows], exx[kColRows], exy[kColRows];
    ssim_loss_map<0>(L, win, coltask, jj, i0, mx);
    ssim_loss_map<1>(L, win, coltask, jj, i0, exx);
    ssim_loss_map<2>(L, win, coltask, jj, i0, exy);
    // the map and D0..D2 there (zero outside the image)
    float f = 0.f, D[3][kColRows];
    {
        const bool colin = coltask && px >= 0 && px < W;
        const bool colown = jj >= kSsimR && jj < kSsimR + kTW;
#pragma unroll
        for (int q = 0; q < kColRows; ++q) {
            const int i = i0 + q, py = y0 - kSsimR + i;
            D[0][q] = D[1][q] = D[2][q] = 0.f;
            if (colin && py >= 0 && py < H) {
                const float a = mx[q], my = tq[q].x, eyy = tq[q].y;
                const float xx = a * a, yy = my * my;
                const float sxx = exx[q] - xx, syy = eyy - yy, sxy = exy[q] - a * my;
                const float n1 = fmaf(2.0f * a, my, kC1), n2 = fmaf(2.0f, sxy, kC2);
                const float d1 = (xx + yy) + kC1, d2 = (sxx + syy) + kC2;
                // one hardware reciprocal (1 ulp) of d1 d2 (>= C1 C2) serves every quotient:
                //   SSIM = n1 n2 r,  dSSIM/dmx = 2 r (my (n2 - n1) + mx SSIM (d1 - d2)),
                //   dSSIM/dExx = -SSIM d1 r,  dSSIM/dExy = 2 n1 r,  r = 1 / (d1 d2)
                const float r = __builtin_amdgcn_rcpf(d1 * d2);
                const float fr = (n1 * n2) * r;
                if (colown && i >= kSsimR && i < kSsimR + kTH) f += fr;   // the tile's own pixels
                D[0][q] = (2.0f * r) * fmaf(a * fr, d1 - d2, my * (n2 - n1));
                D[1][q] = -(fr * d1) * r;
                D[2][q] = (2.0f * n1) * r;
            }
        }
    }
    // this thread's four outputs (tasks below 384): column tx, rows ty0 .. ty0 + 3 of the tile
    const bool outtask = tid < kOutTasks;
    const int tx = tid % kTW, ty0 = 4 * (tid / kTW) % kTH, j = x0 + tx;
    // the tile's partial sums (SSIM over its pixels, |e| and e^2 at them), reduced in a fixed order
    // now, so that the loss's ticket is taken while D is filtered
    {
        float l1 = 0.f, l2 = 0.f;
        if (outtask) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (y0 + ty0 + q >= H || j >= W) continue;
                const int r = ty0 + q + 2 * kSsimR, c = tx + 2 * kSsimR;
                const float e = L.s[0][r][c] - L.s[1][r][c];
                l1 += fabsf(e);
                l2 += e * e;
            }
        }
        float v[3] = {f, l1, l2};
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            float sm = v[k];
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) sm += __shfl_xor(sm, d, 64);
            if ((tid & 63) == 0) L.red[k][tid >> 6] = sm;   // read after the next barrier
        }
    }
    // The partials go out as device-scope stores (written through to the device's coherent level);
    // once they have completed, the first wave takes a ticket of its group of tiles (one D map later,
    // so neither wait holds the workgroup up); a group's last tile takes a ticket of the groups one
    // map later again.  The workgroup with the last of those reads every partial back with
    // device-scope loads at its end.  Nothing else is published, so no cache write-back is needed.
    // Sixteen group counters on their own 256-byte lines keep the atomics on one address few.
    const int gsize = (ntiles + kTicketGroups - 1) / kTicketGroups, grp = tile / gsize;
    const int members = min(gsize, ntiles - grp * gsize), ngroups = (ntiles + gsize - 1) / gsize;
    unsigned *cg = done + kTicketStride * grp, *ct = done + kTicketStride * kTicketGroups;
    unsigned gticket = 0, tticket = 0;
    // the window sums of D0, D1, D2 at the four outputs, one map at a time
    float ss[3][4];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        if (coltask) {
#pragma unroll
            for (int q = 0; q < kColRows; ++q) L.d[i0 + q][jj] = D[k][q];
        }
        __syncthreads();
        if (k == 0 && loss && tid < 3) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < kLossWaves; ++w) t += L.red[tid][w];
            __hip_atomic_store(&part[3 * tile + tid], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int u = 0; u < rounds(kBRowTasks); ++u) {
            const int t = tid + kLossNT * u;
            if (t < kBRowTasks) {                           // lanes: consecutive rows of a column group
                const int g = t / kMR, i = t - g * kMR, c0 = 4 * g;
                float dv[14];
                lds_run14(&L.d[i][c0], dv);
                *reinterpret_cast<float4 *>(&L.hb[i][c0]) = win4(dv, win);
            }
        }
        __syncthreads();
        if (outtask) ssim_col<kBP, 4>(&L.hb[ty0][tx], win, ss[k]);
        if (k == 0 && loss && tid < 64) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);                  // the partials' stores have completed
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (tid == 0) gticket = __hip_atomic_fetch_add(cg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (k == 1 && loss && tid == 0 && gticket == (unsigned)(members - 1)) {
            __hip_atomic_store(cg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
            tticket = __hip_atomic_fetch_add(ct, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
        }
        if (k < 2) __syncthreads();                         // d and hb are rewritten next
    }
    const double inv_n = 1.0 / (3.0 * (double)plane);
    // 1 / (3 H W) rounded once (the products below round like the divisions they replace, to 1 ulp)
    const float inv_nf = (float)inv_n;
    if (outtask) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = y0 + ty0 + q;
            if (i >= H || j >= W) continue;
            const int r = ty0 + q + 2 * kSsimR, c = tx + 2 * kSsimR;
            const float xo = L.s[0][r][c], yo = L.s[1][r][c];
            const float e = xo - yo;
            const float dssim = fmaf(yo, ss[2][q], fmaf(2.0f * xo, ss[1][q], ss[0][q])) * inv_nf;
            const float sg = e > 0.0f ? 1.0f : (e < 0.0f ? -1.0f : 0.0f);
            dL[ch * plane + (size_t)i * W + j] = fmaf(w1, sg * inv_nf, fmaf(w2, 2.0f * e * inv_nf, -(ws * dssim)));
        }
    }
    if (!loss) return;
    if (tid == 0) L.last = tticket == (unsigned)ngroups;    // 0 unless this is a group's last tile
    __syncthreads();
    if (!L.last) return;
    // the last workgroup: every tile's partials, in tile order per thread, then a fixed tree
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    double a[3] = {0.0, 0.0, 0.0};
    for (int t = tid; t < ntiles; t += kLossNT)
#pragma unroll
        for (int k = 0; k < 3; ++k)
            a[k] += (double)__hip_atomic_load(&part[3 * t + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) a[k] += __shfl_xor(a[k], d, 64);
        if ((tid & 63) == 0) L.dred[k][tid >> 6] = a[k];
    }
    __syncthreads();
    if (tid == 0) {
        double s[3];
        for (int k = 0; k < 3; ++k) {
            s[k] = 0.0;
            for (int w = 0; w < kLossWaves; ++w) s[k] += L.dred[k][w];
        }
        loss[0] = (float)(w1d * s[1] * inv_n + w2d * s[2] * inv_n + wsd * (1.0 - s[0] * inv_n));
        __hip_atomic_store(ct, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);      // ready for the next call
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

static int ssim_tiles(int W, int H) { return ((W + kTW - 1) / kTW) * ((H + kTH - 1) / kTH) * 3; }

// Workspace: the target's statistics T (3 planes of float2) | the tile partials | the ticket counts
// (zeroed by k_ssim_target, left at zero by every loss call).
struct SsimWs {
    float2 *T;
    float *part;
    unsigned *done;
};
static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
static SsimWs ssim_ws(int W, int H, void *ws) {
    const size_t plane = (size_t)W * H;
    char *b = static_cast<char *>(ws);
    const size_t tb = align256(3 * plane * sizeof(float2));
    const size_t pb = align256(3 * (size_t)ssim_tiles(W, H) * sizeof(float));
    SsimWs w;
    w.T = reinterpret_cast<float2 *>(b);
    w.part = reinterpret_cast<float *>(b + tb);
    w.done = reinterpret_cast<unsigned *>(b + tb + pb);
    return w;
}

size_t ssim_workspace_bytes(int W, int H) {
    const size_t plane = (size_t)W * H;
    return align256(3 * plane * sizeof(float2)) + align256(3 * (size_t)ssim_tiles(W, H) * sizeof(float)) +
           (kTicketGroups + 1) * kTicketStride * sizeof(unsigned);
}

hipError_t launch_ssim_target(int W, int H, const float *y, void *ws_ptr, hipStream_t s) {
    const SsimWs w = ssim_ws(W, H, ws_ptr);
    const dim3 grid((W + kSsimT - 1) / kSsimT, (H + kSsimT - 1) / kSsimT, 3);
    k_ssim_target<<<grid, 256, 0, s>>>(W, H, y, ssim_window(), w.T, w.done);
    return hipGetLastError();
}

hipError_t launch_loss_ssim(int W, int H, const float *x, const float *y, float w1, float w2, float ws, float *dL,
                            float *loss, void *ws_ptr, bool target_prepared, hipStream_t s) {
    if (!target_prepared) {
        const hipError_t e = launch_ssim_target(W, H, y, ws_ptr, s);
        if (e != hipSuccess) return e;
    }
    const SsimWin win = ssim_window();
    const SsimWs w = ssim_ws(W, H, ws_ptr);
    const int ntiles = ssim_tiles(W, H), nblk = (ntiles + 7) & ~7;
    const bool vec = W % 4 == 0 && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15) == 0;
    if (vec)
        k_ssim_loss<true><<<nblk, kLossNT, 0, s>>>(W, H, x, y, w.T, win, w1, w2, ws, dL, w.part, ntiles, nblk,
                                                   (double)w1, (double)w2, (double)ws, loss, w.done);
    else
        k_ssim_loss<false><<<nblk, kLossNT, 0, s>>>(W, H, x, y, w.T, win, w1, w2, ws, dL, w.part, ntiles, nblk,
                                                (double)w1, (double)w2, (double)ws, loss, w.done);
    return hipGetLastError();
}

}  // namespace gi
