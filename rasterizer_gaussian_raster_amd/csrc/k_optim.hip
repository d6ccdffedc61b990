// k_optim.hip -- L2 loss with its image gradient ("FlashImgs", train --loss l2)
// and the fused Adam step (fvdb GaussianSplatOptimizer: Adam; "Drawing with
// Gaussians": fused optimizer kernels).  Both are HBM-bound streaming kernels:
//   loss: 8 B read + 4 B written per image entry;
//   Adam: 16 B read (p, g, m, v) + 12 B written (p, m, v) per scalar, +4 B when
//         the gradient is cleared for the next step.
#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

constexpr int kLossThreads = 256;
constexpr int kLossBlocks = 1024;

__global__ __launch_bounds__(kLossThreads) void k_loss_partial(int64_t count, const float *__restrict__ img,
                                                               const float *__restrict__ tgt,
                                                               float *__restrict__ grad, float scale,
                                                               double *__restrict__ part) {
    __shared__ double sm[kLossThreads / 64];
    double s = 0.0;
    const int64_t stride = (int64_t)gridDim.x * kLossThreads;
    for (int64_t i = (int64_t)blockIdx.x * kLossThreads + threadIdx.x; i < count; i += stride) {
        const float d = img[i] - tgt[i];
        if (grad) grad[i] = scale * d;
        s += (double)d * (double)d;
    }
    // fixed-order reduction: lanes (xor tree), then waves in index order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double b = 0.0;
        for (int w = 0; w < kLossThreads / 64; ++w) b += sm[w];
        part[blockIdx.x] = b;
    }
}

__global__ __launch_bounds__(64) void k_loss_final(int nparts, int64_t count, const double *__restrict__ part,
                                                   float *__restrict__ loss) {
    double s = 0.0;
    for (int i = threadIdx.x; i < nparts; i += 64) s += part[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (threadIdx.x == 0) *loss = (float)(s / (double)count);
}

static int loss_blocks(int64_t count) {
    const int64_t b = (count + kLossThreads * 4 - 1) / (kLossThreads * 4);
    return (int)(b < 1 ? 1 : (b > kLossBlocks ? kLossBlocks : b));
}

size_t loss_workspace_bytes(int64_t count) { return sizeof(double) * (size_t)loss_blocks(count); }

hipError_t launch_loss_l2(int64_t count, const float *image, const float *target, float *dL_dimage, float *d_loss,
                          void *ws, hipStream_t s) {
    const int nb = loss_blocks(count);
    const float scale = (float)(2.0 / (double)count);
    k_loss_partial<<<nb, kLossThreads, 0, s>>>(count, image, target, dL_dimage, scale, static_cast<double *>(ws));
    if (d_loss) k_loss_final<<<1, 64, 0, s>>>(nb, count, static_cast<const double *>(ws), d_loss);
    return hipGetLastError();
}

struct AdamArgs {
    float lr[16];
    float b1, omb1, b2, omb2, eps;   // omb = 1 - beta, formed in double
    double b1d, b2d;                 // for the bias corrections
    int step;
    int row_len;
};

struct AdamBias {
    float inv_bc1, inv_sqrt_bc2;
};

__device__ __forceinline__ void adam_one(float &p, float &g, float &m, float &v, float lr, const AdamArgs &a,
                                         const AdamBias &c) {
    AdamHP h{};
    h.b1 = a.b1;
    h.omb1 = a.omb1;
    h.b2 = a.b2;
    h.omb2 = a.omb2;
    h.eps = a.eps;
    adam_update(p, g, m, v, lr, h, c.inv_bc1, c.inv_sqrt_bc2);
}

// 4 consecutive scalars per thread (row_len divisible by 4, 16-byte aligned arrays).
__global__ __launch_bounds__(256) void k_adam4(int64_t n4, float4 *__restrict__ p, float4 *__restrict__ g,
                                               float4 *__restrict__ m, float4 *__restrict__ v, AdamArgs a,
                                               int zero_grad) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    float4 P = p[i], G = g[i], Mm = m[i], V = v[i];
    AdamBias c;
    adam_bias(a.b1d, a.b2d, a.step, c.inv_bc1, c.inv_sqrt_bc2);
    const int s0 = (int)((i * 4) % a.row_len);
    adam_one(P.x, G.x, Mm.x, V.x, a.lr[s0 + 0], a, c);
    adam_one(P.y, G.y, Mm.y, V.y, a.lr[s0 + 1], a, c);
    adam_one(P.z, G.z, Mm.z, V.z, a.lr[s0 + 2], a, c);
    adam_one(P.w, G.w, Mm.w, V.w, a.lr[s0 + 3], a, c);
    p[i] = P;
    m[i] = Mm;
    v[i] = V;
    if (zero_grad) g[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(256) void k_adam1(int64_t n, float *__restrict__ p, float *__restrict__ g,
                                               float *__restrict__ m, float *__restrict__ v, AdamArgs a,
                                               int zero_grad) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float P = p[i], G = g[i], Mm = m[i], V = v[i];
    AdamBias c;
    adam_bias(a.b1d, a.b2d, a.step, c.inv_bc1, c.inv_sqrt_bc2);
    adam_one(P, G, Mm, V, a.lr[i % a.row_len], a, c);
    p[i] = P;
    m[i] = Mm;
    v[i] = V;
    if (zero_grad) g[i] = 0.0f;
}

hipError_t launch_adam(int64_t rows, int row_len, float *p, float *g, float *m, float *v, const float *lr,
                       double beta1, double beta2, double eps, int step, int zero_grad, hipStream_t s) {
    AdamArgs a{};
    for (int i = 0; i < row_len; ++i) a.lr[i] = lr[i];
    a.b1 = (float)beta1;
    a.omb1 = (float)(1.0 - beta1);
    a.b2 = (float)beta2;
    a.omb2 = (float)(1.0 - beta2);
    a.eps = (float)eps;
    a.b1d = beta1;
    a.b2d = beta2;
    a.step = step;
    a.row_len = row_len;
    const int64_t n = rows * row_len;
    if (n == 0) return hipSuccess;
    if (row_len % 4 == 0) {
        const int64_t n4 = n / 4;
        k_adam4<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(n4, reinterpret_cast<float4 *>(p),
                                                              reinterpret_cast<float4 *>(g),
                                                              reinterpret_cast<float4 *>(m),
                                                              reinterpret_cast<float4 *>(v), a, zero_grad);
    } else {
        k_adam1<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(n, p, g, m, v, a, zero_grad);
    }
    return hipGetLastError();
}

}  // namespace gi
