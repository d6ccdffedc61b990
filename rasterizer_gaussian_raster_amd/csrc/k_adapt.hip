// k_adapt.hip -- changing the set of Gaussians between fitting steps: merging it
// down to a target count ("FlashImgs", merge: an overcomplete set merged down by
// moment matching, 80K -> 50K) and adaptive density control ("FlashImgs",
// Training features: dead, out-of-bounds and bloated Gaussians relocated to
// high-error pixels).  The rules (readings; the pages state none):
//
// Merge round.  Cost of merging i and j = Runnalls' bound on the increase of the
// KL divergence when two mixture components are replaced by their moment-matched
// merge ("Kullback-Leibler approach to Gaussian mixture reduction", IEEE Trans.
// AES 2007):  B = 1/2 [W log det S_m - w_i log det S_i - w_j log det S_j], with the
// masses w = |det L| sum|c| and the merged covariance S_m of gi_merge_pairs,
// in fp64 in the order written below, the smaller index first.  Candidates: the
// other mergeable Gaussians whose mean lies in the same or a neighbouring 16x16
// cell (the cell of the clamped mean pixel).  Each Gaussian picks its cheapest
// candidate (ties: smaller index); pairs that pick each other are merged -- all,
// or the cheapest by (fp32 cost, smaller index) when more than asked for.
//
// Density control.  Flags: dead (a non-finite parameter, l11 or l22 zero, or
// max|c| < 1/255), out of bounds (mean outside [0,W) x [0,H)), bloated (largest
// eigenvalue of Sigma above (max(W,H)/16)^2, decided by the rational test below).
// The K = min(#flagged, W H) pixels of largest fp32 error e = |target - image|^2
// (ties: smaller index), in pixel order, go to the flagged Gaussians in index
// order: mean at the pixel centre, L = s0 I, colour = the residual there.
//
// Both reduce to "the K smallest of m distinct 64-bit keys" (a radix select: 8
// passes of an LDS histogram per byte) and order-preserving compaction (block
// counts, one scan block, block-local scans): every choice is deterministic and
// the outputs keep index order.
#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

typedef unsigned long long u64;

// ---------------------------------------------------------------------------
// the K smallest of m distinct keys
// ---------------------------------------------------------------------------
struct SelState {
    u64 prefix, mask;          // the bytes of the threshold decided so far
    uint32_t remaining;        // rank still to reach within the keys matching prefix
    uint32_t all, none;        // K >= m: every key; K == 0: none
    uint32_t pad;
    uint32_t hist[256];
};

// K = min(k, m), m = *d_m (or m_host when d_m is NULL), k = *d_k (or k_host).  One block of 256.
__global__ __launch_bounds__(256) void k_sel_init(SelState *st, const uint32_t *d_m, uint32_t m_host,
                                                  const uint32_t *d_k, uint32_t k_host) {
    const uint32_t m = d_m ? *d_m : m_host;
    const uint32_t K = min(d_k ? *d_k : k_host, m);
    if (threadIdx.x == 0) {
        st->prefix = 0ull;
        st->mask = 0ull;
        st->remaining = K;
        st->all = K >= m ? 1u : 0u;
        st->none = K == 0u ? 1u : 0u;
    }
    st->hist[threadIdx.x] = 0u;
}

__global__ __launch_bounds__(256) void k_sel_hist(const u64 *__restrict__ keys, const uint32_t *d_m, uint32_t m_host,
                                                  SelState *st, int shift) {
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0u;
    __syncthreads();
    if (st->all || st->none) return;                      // uniform
    const uint32_t m = d_m ? *d_m : m_host;
    const u64 mask = st->mask, prefix = st->prefix;
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < m; i += gridDim.x * 256u) {
        const u64 key = keys[i];
        if ((key & mask) == prefix) atomicAdd(&h[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (h[threadIdx.x]) atomicAdd(&st->hist[threadIdx.x], h[threadIdx.x]);
}

// The digit of this byte: the first d where the keys below it reach `remaining`.
__global__ __launch_bounds__(256) void k_sel_pick(SelState *st, int shift) {
    __shared__ uint32_t h[256];
    if (st->all || st->none) return;
    h[threadIdx.x] = st->hist[threadIdx.x];
    st->hist[threadIdx.x] = 0u;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t r = st->remaining;
        uint32_t cum = 0u;
        int d = 0;
        for (; d < 255; ++d) {
            if (cum + h[d] >= r) break;
            cum += h[d];
        }
        st->remaining = r - cum;
        st->prefix |= (u64)d << shift;
        st->mask |= (u64)255 << shift;
    }
}

__device__ __forceinline__ bool sel_taken(const SelState &st, u64 key) {
    return st.all || (!st.none && key <= st.prefix);
}

// The threshold of the min(k, m) smallest keys into st (m, k from the device when d_m, d_k are
// given; m_max bounds m).
hipError_t launch_select(const u64 *keys, const uint32_t *d_m, uint32_t m_max, const uint32_t *d_k, uint32_t k_host,
                         SelState *st, hipStream_t s) {
    k_sel_init<<<1, 256, 0, s>>>(st, d_m, m_max, d_k, k_host);
    const int nb = (int)min((m_max + 255u) / 256u, 1024u);
    for (int shift = 56; shift >= 0; shift -= 8) {
        k_sel_hist<<<nb > 0 ? nb : 1, 256, 0, s>>>(keys, d_m, m_max, st, shift);
        k_sel_pick<<<1, 256, 0, s>>>(st, shift);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// order-preserving compaction of the elements i < m with pred(i): emit(i, position)
// ---------------------------------------------------------------------------
constexpr int kCmpPer = 4;                      // elements per thread
constexpr uint32_t kCmpBlock = 256u * kCmpPer;  // elements per block

template <class Pred>
__global__ __launch_bounds__(256) void k_cmp_count(Pred pred, const uint32_t *d_m, uint32_t m_host,
                                                   uint32_t *__restrict__ bcount) {
    __shared__ uint32_t ws[4];
    const uint32_t m = d_m ? *d_m : m_host;
    const uint32_t base = blockIdx.x * kCmpBlock + threadIdx.x * kCmpPer;
    uint32_t c = 0u;
#pragma unroll
    for (int k = 0; k < kCmpPer; ++k) c += (base + k < m && pred(base + k)) ? 1u : 0u;
    const uint32_t inc = wave_scan_incl(c);
    if ((threadIdx.x & 63) == 63) ws[threadIdx.x >> 6] = inc;
    __syncthreads();
    if (threadIdx.x == 0) bcount[blockIdx.x] = ((ws[0] + ws[1]) + ws[2]) + ws[3];
}

// One block of 1024: exclusive scan of nb block counts in place; the total to *total.
__global__ __launch_bounds__(1024) void k_cmp_scan(uint32_t *__restrict__ b, uint32_t nb, uint32_t *__restrict__ total) {
    __shared__ uint32_t ws[16];
    const uint32_t per = (nb + 1023u) / 1024u;
    const uint32_t beg = threadIdx.x * per;
    uint32_t s = 0u;
    for (uint32_t i = 0; i < per; ++i)
        if (beg + i < nb) s += b[beg + i];
    const uint32_t inc = wave_scan_incl(s);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 63) ws[wave] = inc;
    __syncthreads();
    uint32_t off = 0u, tot = 0u;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        off += w < wave ? ws[w] : 0u;
        tot += ws[w];
    }
    uint32_t run = off + inc - s;
    for (uint32_t i = 0; i < per; ++i)
        if (beg + i < nb) {
            const uint32_t v = b[beg + i];
            b[beg + i] = run;
            run += v;
        }
    if (threadIdx.x == 0) *total = tot;
}

template <class Pred, class Emit>
__global__ __launch_bounds__(256) void k_cmp_write(Pred pred, Emit emit, const uint32_t *d_m, uint32_t m_host,
                                                   const uint32_t *__restrict__ bbase) {
    __shared__ uint32_t ws[4];
    const uint32_t m = d_m ? *d_m : m_host;
    const uint32_t base = blockIdx.x * kCmpBlock + threadIdx.x * kCmpPer;
    bool f[kCmpPer];
    uint32_t c = 0u;
#pragma unroll
    for (int k = 0; k < kCmpPer; ++k) {
        f[k] = base + k < m && pred(base + k);
        c += f[k] ? 1u : 0u;
    }
    const uint32_t inc = wave_scan_incl(c);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 63) ws[wave] = inc;
    __syncthreads();
    uint32_t pos = bbase[blockIdx.x] + inc - c;
    for (int w = 0; w < wave; ++w) pos += ws[w];
#pragma unroll
    for (int k = 0; k < kCmpPer; ++k)
        if (f[k]) emit(base + k, pos++);
}

inline uint32_t cmp_blocks(uint32_t m) { return (m + kCmpBlock - 1u) / kCmpBlock; }

// scratch: cmp_blocks(m_max) + 1 u32; *count = the number emitted
template <class Pred, class Emit>
hipError_t launch_compact(Pred pred, Emit emit, const uint32_t *d_m, uint32_t m_max, uint32_t *scratch,
                          uint32_t *count, hipStream_t s) {
    const uint32_t nb = cmp_blocks(m_max);
    if (nb == 0u) {
        k_cmp_scan<<<1, 1024, 0, s>>>(scratch, 0u, count);          // writes a zero count
        return hipGetLastError();
    }
    k_cmp_count<Pred><<<nb, 256, 0, s>>>(pred, d_m, m_max, scratch);
    k_cmp_scan<<<1, 1024, 0, s>>>(scratch, nb, count);
    k_cmp_write<Pred, Emit><<<nb, 256, 0, s>>>(pred, emit, d_m, m_max, scratch);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// merge rounds
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool merge_ok(float4 a, float4 b) {
    return isfinite(a.x) && isfinite(a.y) && isfinite(a.z) && isfinite(a.w) && isfinite(b.x) && isfinite(b.y) &&
           isfinite(b.z) && isfinite(b.w) && a.z != 0.0f && b.x != 0.0f;
}

// Each mergeable Gaussian as a one-pixel box at its clamped mean pixel (its cell is that pixel's
// tile); others empty.  The tile binning then lists every cell's Gaussians in index order.
__global__ __launch_bounds__(256) void k_merge_cells(int n, int W, int H, const float4 *__restrict__ p,
                                                     uint2 *__restrict__ box, uint32_t *__restrict__ cnt) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float4 a = p[2 * (size_t)i], b = p[2 * (size_t)i + 1];
    if (!merge_ok(a, b)) {
        box[i] = make_uint2(1u | (1u << 16), 0u);
        cnt[i] = 0u;
        return;
    }
    const float x = fminf(fmaxf(floorf(a.x), 0.0f), (float)(W - 1));
    const float y = fminf(fmaxf(floorf(a.y), 0.0f), (float)(H - 1));
    const uint32_t px = (uint32_t)x, py = (uint32_t)y;
    box[i] = make_uint2(px | (py << 16), px | (py << 16));
    cnt[i] = 1u;
}

// The merge cost of a (the smaller index) and b, in the order of the oracle's definition.
__device__ __forceinline__ double merge_cost(float4 a0, float4 a1, float4 b0, float4 b1) {
    const double a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const double b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    const double da = fabs(a[2] * a[4]), db = fabs(b[2] * b[4]);
    const double wa = da * ((fabs(a[5]) + fabs(a[6])) + fabs(a[7]));
    const double wb = db * ((fabs(b[5]) + fabs(b[6])) + fabs(b[7]));
    const double W = wa + wb;
    const double fa = W > 0 ? wa / W : 0.5, fb = W > 0 ? wb / W : 0.5;
    const double mx = fa * a[0] + fb * b[0], my = fa * a[1] + fb * b[1];
    const double ax = a[0] - mx, ay = a[1] - my, bx = b[0] - mx, by = b[1] - my;
    const double s11 = fa * (a[2] * a[2] + ax * ax) + fb * (b[2] * b[2] + bx * bx);
    const double s21 = fa * (a[2] * a[3] + ax * ay) + fb * (b[2] * b[3] + bx * by);
    const double s22 = fa * ((a[3] * a[3] + a[4] * a[4]) + ay * ay) + fb * ((b[3] * b[3] + b[4] * b[4]) + by * by);
    const double dm = s11 * s22 - s21 * s21;
    if (!(dm > 0.0)) return __longlong_as_double(0x7ff0000000000000ll);   // +inf
    if (W == 0.0) return 0.0;
    return 0.5 * (W * log(dm) - wa * log(da * da) - wb * log(db * db));
}

// Thread t takes the t-th binned Gaussian (cell order: neighbouring threads share their cells)
// and picks its cheapest candidate in the 3x3 cells around its own.
__global__ __launch_bounds__(256) void k_merge_best(int n, int W, int H, int tiles_x, int tiles_y,
                                                    const float4 *__restrict__ p, const uint32_t *__restrict__ vals,
                                                    const uint2 *__restrict__ ranges,
                                                    const uint32_t *__restrict__ d_num, int32_t *__restrict__ best,
                                                    double *__restrict__ cost) {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    if (t >= *d_num) return;
    const uint32_t i = vals[t];
    const float4 a0 = p[2 * (size_t)i], a1 = p[2 * (size_t)i + 1];
    // the cell of the clamped mean pixel, as k_merge_cells binned it
    const int cx = (int)fminf(fmaxf(floorf(a0.x), 0.0f), (float)(W - 1)) >> 4;
    const int cy = (int)fminf(fmaxf(floorf(a0.y), 0.0f), (float)(H - 1)) >> 4;
    int32_t bj = -1;
    double bc = 0.0;
    for (int yy = max(cy - 1, 0); yy <= min(cy + 1, tiles_y - 1); ++yy)
        for (int xx = max(cx - 1, 0); xx <= min(cx + 1, tiles_x - 1); ++xx) {
            const uint2 rg = ranges[yy * tiles_x + xx];
            for (uint32_t e = rg.x; e < rg.y; ++e) {
                const uint32_t j = vals[e];
                if (j == i) continue;
                const float4 b0 = p[2 * (size_t)j], b1 = p[2 * (size_t)j + 1];
                const double c = i < j ? merge_cost(a0, a1, b0, b1) : merge_cost(b0, b1, a0, a1);
                if (bj < 0 || c < bc || (c == bc && (int32_t)j < bj)) {
                    bj = (int32_t)j;
                    bc = c;
                }
            }
        }
    best[i] = bj;
    cost[i] = bc;
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t *__restrict__ a, int n, int32_t v) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) a[i] = v;
}

struct MutualPred {
    const int32_t *best;
    const double *cost;
    __device__ bool operator()(uint32_t i) const {
        const int32_t j = best[i];
        return j > (int32_t)i && best[j] == (int32_t)i && isfinite(cost[i]);
    }
};

// An order-preserving 32-bit image of a float (-0 taken as +0, as a float comparison does).
__device__ __forceinline__ uint32_t float_order(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct MutualEmit {
    const int32_t *best;
    const double *cost;
    int2 *pairs;
    u64 *keys;
    __device__ void operator()(uint32_t i, uint32_t pos) const {
        pairs[pos] = make_int2((int)i, best[i]);
        keys[pos] = ((u64)float_order((float)cost[i]) << 32) | i;
    }
};

struct KeyPred {
    const u64 *keys;
    const SelState *st;
    __device__ bool operator()(uint32_t t) const { return sel_taken(*st, keys[t]); }
};

struct PairEmit {
    const int2 *src;
    int2 *dst;
    __device__ void operator()(uint32_t t, uint32_t pos) const { dst[pos] = src[t]; }
};

__global__ __launch_bounds__(256) void k_merge_partners(const int2 *__restrict__ pairs, int64_t np,
                                                        int32_t *__restrict__ partner) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= np) return;
    const int2 pr = pairs[t];
    partner[pr.x] = pr.y;
    partner[pr.y] = pr.x;
}

struct KeepPred {
    const int32_t *partner;
    __device__ bool operator()(uint32_t i) const { return partner[i] < 0 || partner[i] > (int32_t)i; }
};

// Moment-matching merge of Gaussians a and b (Cholesky form) in fp64: masses w = |det L| sum |c|;
// mean and covariance of the w-weighted mixture; L = chol(Sigma) with a positive diagonal;
// colours keep each channel's integral (2 pi |det L| c).
__device__ __forceinline__ void merge_two(float4 a0, float4 a1, float4 b0, float4 b1, float4 &o0, float4 &o1) {
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
    o0 = make_float4((float)mx, (float)my, (float)l11, (float)l21);
    o1 = make_float4((float)l22, (float)((da * a1.y + db * b1.y) / dn), (float)((da * a1.z + db * b1.z) / dn),
                     (float)((da * a1.w + db * b1.w) / dn));
}

// The merged Gaussian of each given pair: one thread per pair.  An index outside [0, n) gives a
// NaN row.
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
    float4 o0, o1;
    merge_two(params[2 * (int64_t)pr.x], params[2 * (int64_t)pr.x + 1], params[2 * (int64_t)pr.y],
              params[2 * (int64_t)pr.y + 1], o0, o1);
    out[2 * t] = o0;
    out[2 * t + 1] = o1;
}

hipError_t launch_merge_pairs(int64_t np, int64_t n, const float *params, const int32_t *pairs, float *out,
                              hipStream_t s) {
    if (np == 0) return hipSuccess;
    k_merge_pairs<<<(unsigned)((np + 255) / 256), 256, 0, s>>>(np, n, reinterpret_cast<const float4 *>(params),
                                                              reinterpret_cast<const int2 *>(pairs),
                                                              reinterpret_cast<float4 *>(out));
    return hipGetLastError();
}

struct KeepEmit {
    const int32_t *partner;
    const float4 *p;
    float4 *out;
    __device__ void operator()(uint32_t i, uint32_t pos) const {
        const float4 a0 = p[2 * (size_t)i], a1 = p[2 * (size_t)i + 1];
        const int32_t j = partner[i];
        if (j < 0) {
            out[2 * (size_t)pos] = a0;
            out[2 * (size_t)pos + 1] = a1;
            return;
        }
        float4 o0, o1;
        merge_two(a0, a1, p[2 * (size_t)j], p[2 * (size_t)j + 1], o0, o1);
        out[2 * (size_t)pos] = o0;
        out[2 * (size_t)pos + 1] = o1;
    }
};

// Merge workspace: the cell binning's buffers, the picks and costs, the pairs and their keys,
// the select state and compaction scratch, the partner array and a second params buffer.
struct MergePlan {
    BinPlan bin;
    size_t off_box, off_cnt, off_off, off_keys, off_vals, off_ranges, off_num, off_binws, off_best, off_cost,
        off_pairs, off_pkeys, off_pairs2, off_sel, off_scan, off_count, off_partner, off_tmp, bytes;
};

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

MergePlan make_merge_plan(int W, int H, int64_t n) {
    MergePlan m{};
    const size_t nn = (size_t)(n > 0 ? n : 1), half = nn / 2 + 1;
    m.bin = make_bin_plan((int)n, W, H, n > 0 ? n : 1);
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = a256(o + bytes); return at; };
    m.off_box = take(8 * nn);
    m.off_cnt = take(4 * nn);
    m.off_off = take(4 * (nn + 1));
    m.off_keys = take(4 * nn);
    m.off_vals = take(4 * nn);
    m.off_ranges = take(8 * (size_t)m.bin.ntiles);
    m.off_num = take(8);
    m.off_binws = take(m.bin.bytes);
    m.off_best = take(4 * nn);
    m.off_cost = take(8 * nn);
    m.off_pairs = take(8 * half);
    m.off_pkeys = take(8 * half);
    m.off_pairs2 = take(8 * half);
    m.off_sel = take(sizeof(SelState));
    m.off_scan = take(4 * ((size_t)cmp_blocks((uint32_t)nn) + 1));
    m.off_count = take(16);
    m.off_partner = take(4 * nn);
    m.off_tmp = take(32 * nn);
    m.bytes = o;
    return m;
}

size_t merge_workspace_bytes(int W, int H, int64_t n) { return make_merge_plan(W, H, n).bytes; }

// One round on params [n][8]: the picks, the mutual pairs (all, or the max_pairs cheapest), in
// ascending smaller index at pairs_out; the count to d_count.  ws is laid out for n_cap >= n
// Gaussians (the cell binning itself is planned for n).
hipError_t launch_merge_round(int W, int H, int n_cap, int n, const float *params, uint32_t max_pairs,
                              int32_t *pairs_out, uint32_t *d_count, void *ws, hipStream_t s) {
    const MergePlan m = make_merge_plan(W, H, n_cap);
    const BinPlan bin = make_bin_plan(n, W, H, n > 0 ? n : 1);
    if (n > n_cap || bin.bytes > m.bin.bytes) return hipErrorInvalidValue;
    char *w = static_cast<char *>(ws);
    uint2 *box = reinterpret_cast<uint2 *>(w + m.off_box);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(w + m.off_cnt);
    uint32_t *offs = reinterpret_cast<uint32_t *>(w + m.off_off);
    uint32_t *keys = reinterpret_cast<uint32_t *>(w + m.off_keys);
    uint32_t *vals = reinterpret_cast<uint32_t *>(w + m.off_vals);
    uint32_t *ranges = reinterpret_cast<uint32_t *>(w + m.off_ranges);
    uint32_t *num = reinterpret_cast<uint32_t *>(w + m.off_num);
    int32_t *best = reinterpret_cast<int32_t *>(w + m.off_best);
    double *cost = reinterpret_cast<double *>(w + m.off_cost);
    int2 *pairs = reinterpret_cast<int2 *>(w + m.off_pairs);
    u64 *pkeys = reinterpret_cast<u64 *>(w + m.off_pkeys);
    SelState *st = reinterpret_cast<SelState *>(w + m.off_sel);
    uint32_t *scan = reinterpret_cast<uint32_t *>(w + m.off_scan);
    uint32_t *npair = reinterpret_cast<uint32_t *>(w + m.off_count);
    const float4 *p = reinterpret_cast<const float4 *>(params);
    const int nb = (n + 255) / 256;
    if (n > 0) {
        k_merge_cells<<<nb, 256, 0, s>>>(n, W, H, p, box, cnt);
        k_fill_i32<<<nb, 256, 0, s>>>(best, n, -1);
    }
    hipError_t e = launch_bin_sort(bin, reinterpret_cast<const uint16_t *>(box), cnt, offs, keys, vals, ranges,
                                   nullptr, num, w + m.off_binws, s);
    if (e != hipSuccess) return e;
    if (n > 0)
        k_merge_best<<<nb, 256, 0, s>>>(n, W, H, bin.tiles_x, bin.ntiles / bin.tiles_x, p, vals,
                                        reinterpret_cast<const uint2 *>(ranges), num, best, cost);
    e = launch_compact(MutualPred{best, cost}, MutualEmit{best, cost, pairs, pkeys}, nullptr, (uint32_t)n, scan,
                       npair, s);
    if (e != hipSuccess) return e;
    const uint32_t half = (uint32_t)(n / 2 + 1);
    e = launch_select(pkeys, npair, half, nullptr, max_pairs, st, s);
    if (e != hipSuccess) return e;
    return launch_compact(KeyPred{pkeys, st}, PairEmit{pairs, reinterpret_cast<int2 *>(pairs_out)}, npair, half,
                          scan, d_count, s);
}

// params [n][8] with the given disjoint pairs merged: out [n - np][8] (index order kept); ws laid
// out for n_cap >= n Gaussians.
hipError_t launch_merge_apply(int n_cap, int n, const float *params, int64_t np, const int32_t *pairs, float *out,
                              void *ws, int W, int H, hipStream_t s) {
    if (n > n_cap) return hipErrorInvalidValue;
    const MergePlan m = make_merge_plan(W, H, n_cap);
    char *w = static_cast<char *>(ws);
    int32_t *partner = reinterpret_cast<int32_t *>(w + m.off_partner);
    uint32_t *scan = reinterpret_cast<uint32_t *>(w + m.off_scan);
    uint32_t *kept = reinterpret_cast<uint32_t *>(w + m.off_count) + 1;
    if (n == 0) return hipSuccess;
    k_fill_i32<<<(n + 255) / 256, 256, 0, s>>>(partner, n, -1);
    if (np > 0)
        k_merge_partners<<<(unsigned)((np + 255) / 256), 256, 0, s>>>(reinterpret_cast<const int2 *>(pairs), np,
                                                                       partner);
    return launch_compact(KeepPred{partner},
                          KeepEmit{partner, reinterpret_cast<const float4 *>(params), reinterpret_cast<float4 *>(out)},
                          nullptr, (uint32_t)n, scan, kept, s);
}

float *merge_tmp_params(void *ws, int W, int H, int64_t n) {
    return reinterpret_cast<float *>(static_cast<char *>(ws) + make_merge_plan(W, H, n).off_tmp);
}

int32_t *merge_pairs_buffer(void *ws, int W, int H, int64_t n) {
    return reinterpret_cast<int32_t *>(static_cast<char *>(ws) + make_merge_plan(W, H, n).off_pairs2);
}

uint32_t *merge_count_ptr(void *ws, int W, int H, int64_t n) {
    return reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + make_merge_plan(W, H, n).off_count) + 2;
}

// ---------------------------------------------------------------------------
// adaptive density control
// ---------------------------------------------------------------------------
// 1 dead, 2 out of bounds, 4 bloated (fp64 decisions in the stated order).
__device__ __forceinline__ int32_t adc_flag(float4 a, float4 b, int W, int H) {
    if (!(isfinite(a.x) && isfinite(a.y) && isfinite(a.z) && isfinite(a.w) && isfinite(b.x) && isfinite(b.y) &&
          isfinite(b.z) && isfinite(b.w)))
        return 1;
    if (a.z == 0.0f || b.x == 0.0f) return 1;
    int32_t f = 0;
    const double cm = fmax(fabs((double)b.y), fmax(fabs((double)b.z), fabs((double)b.w)));
    if (cm < 1.0 / 255.0) f |= 1;
    if (!(a.x >= 0.0f && a.x < (float)W && a.y >= 0.0f && a.y < (float)H)) f |= 2;
    const double l11 = a.z, l21 = a.w, l22 = b.x;
    const double s11 = l11 * l11, s21 = l11 * l21, s22 = l21 * l21 + l22 * l22;
    const double side = (double)(W > H ? W : H) / 16.0, t = side * side;
    if (!(s11 <= t && s22 <= t && (t - s11) * (t - s22) >= s21 * s21)) f |= 4;
    return f;
}

__global__ __launch_bounds__(256) void k_adc_flags(int n, int W, int H, const float4 *__restrict__ p,
                                                   int32_t *__restrict__ flags) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) flags[i] = adc_flag(p[2 * (size_t)i], p[2 * (size_t)i + 1], W, H);
}

// Key of pixel q: the larger error first, then the smaller index.
__global__ __launch_bounds__(256) void k_adc_keys(int64_t npix, const float *__restrict__ image,
                                                  const float *__restrict__ target, u64 *__restrict__ keys) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= npix) return;
    const float r0 = target[q] - image[q], r1 = target[npix + q] - image[npix + q];
    const float r2 = target[2 * npix + q] - image[2 * npix + q];
    float e = fmaf(r2, r2, fmaf(r1, r1, r0 * r0));
    if (!(e >= 0.0f)) e = 0.0f;                           // a NaN error counts as none
    keys[q] = ((u64)(~__float_as_uint(e)) << 32) | (uint32_t)q;
}

struct FlagPred {
    const int32_t *flags;
    __device__ bool operator()(uint32_t i) const { return flags[i] != 0; }
};

struct IndexEmit {
    uint32_t *list;
    __device__ void operator()(uint32_t i, uint32_t pos) const { list[pos] = i; }
};

// The k-th flagged Gaussian (k < min(#flagged, #pixels)) to the k-th chosen pixel.
__global__ __launch_bounds__(256) void k_adc_move(int n, int W, int64_t npix, const uint32_t *__restrict__ glist,
                                                  const uint32_t *__restrict__ d_nf,
                                                  const uint32_t *__restrict__ plist, const float *__restrict__ image,
                                                  const float *__restrict__ target, float s0, float4 *__restrict__ p,
                                                  float4 *__restrict__ m, float4 *__restrict__ v,
                                                  uint32_t *__restrict__ d_moved) {
    const uint32_t K = (uint32_t)min((int64_t)*d_nf, npix);
    const uint32_t k = blockIdx.x * 256u + threadIdx.x;
    if (k == 0 && d_moved) *d_moved = K;
    if (k >= K || (int)k >= n) return;
    const uint32_t g = glist[k];
    const int64_t q = plist[k];
    const float r0 = target[q] - image[q], r1 = target[npix + q] - image[npix + q];
    const float r2 = target[2 * npix + q] - image[2 * npix + q];
    p[2 * (size_t)g] = make_float4((float)(q % W) + 0.5f, (float)(q / W) + 0.5f, s0, 0.0f);
    p[2 * (size_t)g + 1] = make_float4(s0, r0, r1, r2);
    if (m) {
        m[2 * (size_t)g] = make_float4(0.f, 0.f, 0.f, 0.f);
        m[2 * (size_t)g + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (v) {
        v[2 * (size_t)g] = make_float4(0.f, 0.f, 0.f, 0.f);
        v[2 * (size_t)g + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

struct AdcPlan {
    size_t off_flags, off_glist, off_pkeys, off_plist, off_sel, off_scan, off_count, bytes;
};

AdcPlan make_adc_plan(int W, int H, int64_t n) {
    AdcPlan a{};
    const size_t nn = (size_t)(n > 0 ? n : 1), npix = (size_t)W * (size_t)H;
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = a256(o + bytes); return at; };
    a.off_flags = take(4 * nn);
    a.off_glist = take(4 * nn);
    a.off_pkeys = take(8 * npix);
    a.off_plist = take(4 * (nn < npix ? nn : npix));
    a.off_sel = take(sizeof(SelState));
    a.off_scan = take(4 * ((size_t)cmp_blocks((uint32_t)(nn > npix ? nn : npix)) + 1));
    a.off_count = take(16);
    a.bytes = o;
    return a;
}

size_t adc_workspace_bytes(int W, int H, int64_t n) { return make_adc_plan(W, H, n).bytes; }

hipError_t launch_adc(int W, int H, int n, float *params, float *m, float *v, const float *image,
                      const float *target, float s0, int32_t *flags_out, uint32_t *d_moved, void *ws, hipStream_t s) {
    const AdcPlan a = make_adc_plan(W, H, n);
    char *w = static_cast<char *>(ws);
    int32_t *flags = flags_out ? flags_out : reinterpret_cast<int32_t *>(w + a.off_flags);
    uint32_t *glist = reinterpret_cast<uint32_t *>(w + a.off_glist);
    u64 *pkeys = reinterpret_cast<u64 *>(w + a.off_pkeys);
    uint32_t *plist = reinterpret_cast<uint32_t *>(w + a.off_plist);
    SelState *st = reinterpret_cast<SelState *>(w + a.off_sel);
    uint32_t *scan = reinterpret_cast<uint32_t *>(w + a.off_scan);
    uint32_t *nf = reinterpret_cast<uint32_t *>(w + a.off_count);
    uint32_t *np_sel = nf + 1;
    const int64_t npix = (int64_t)W * H;
    if (n > 0) k_adc_flags<<<(n + 255) / 256, 256, 0, s>>>(n, W, H, reinterpret_cast<const float4 *>(params), flags);
    hipError_t e = launch_compact(FlagPred{flags}, IndexEmit{glist}, nullptr, (uint32_t)n, scan, nf, s);
    if (e != hipSuccess) return e;
    k_adc_keys<<<(unsigned)((npix + 255) / 256), 256, 0, s>>>(npix, image, target, pkeys);
    // the min(#flagged, npix) smallest pixel keys: K comes from the device count
    e = launch_select(pkeys, nullptr, (uint32_t)npix, nf, (uint32_t)npix, st, s);
    if (e != hipSuccess) return e;
    e = launch_compact(KeyPred{pkeys, st}, IndexEmit{plist}, nullptr, (uint32_t)npix, scan, np_sel, s);
    if (e != hipSuccess) return e;
    if (n > 0)
        k_adc_move<<<(n + 255) / 256, 256, 0, s>>>(n, W, npix, glist, nf, plist, image, target, s0,
                                                  reinterpret_cast<float4 *>(params), reinterpret_cast<float4 *>(m),
                                                  reinterpret_cast<float4 *>(v), d_moved);
    else if (d_moved)
        k_adc_move<<<1, 256, 0, s>>>(0, W, npix, glist, nf, plist, image, target, s0, nullptr, nullptr, nullptr,
                                     d_moved);
    return hipGetLastError();
}

}  // namespace gi
