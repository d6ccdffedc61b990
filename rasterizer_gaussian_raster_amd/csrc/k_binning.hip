// k_binning.hip -- tile lists from per-Gaussian pixel boxes.
//
//   1. k_group_sums   : per 256-Gaussian group, sum of tile counts (u64); clears
//                       the tile ranges.
//   2. k_group_scan   : one workgroup scans the group sums -> group bases, M
//                       (only for more than 2048 groups; below that each emit
//                       workgroup adds up the sums before it itself).
//   3. k_emit         : per group, offsets[] and one (tile id, index) pair per
//                       covered tile, emitted in (index, tile row, tile column)
//                       order; the group's pairs are spread evenly over its
//                       256 lanes by a binary search in LDS (no lane walks a
//                       large Gaussian alone).
//   4. LSD radix sort on the tile id, 1..8-bit digits per pass (as many passes
//      as the id needs), each pass = digit counts per 4096-key block ->
//      exclusive scan of the digit-major count table -> stable scatter, where
//      each key's rank among equal digits is found with wave ballots in key
//      order, so the sort is stable and each tile list ends up in ascending
//      Gaussian index.
//   5. k_ranges       : one thread per sorted pair marks where each tile's run
//                       starts and ends.
//
// Binning is the tile-binned scheme of the FlashImgs viewer ("Web viewer":
// tile-binned compute) with fvdb's 16-pixel tiles (tile_size).  All steps are
// HBM/latency bound: ~20 B per pair per sort pass, 12 B per Gaussian to emit.
#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

constexpr int kSortThreads = 256;
constexpr int kSortIters = 4;
constexpr int kMaxRedundantGroups = 2048;              // emit sums the group totals itself up to this
constexpr int kMaxRawTable = 0;                        // scatter forms its digit offsets itself up to this (off: slower)
constexpr int kSortChunk = kSortThreads * kSortIters;   // keys per sort block
constexpr int kScanItems = 16;
constexpr int kScanChunk = 256 * kScanItems;           // table entries per scan block

struct BinHeader {
    unsigned long long total;   // M, 64-bit
    uint32_t m_eff;             // M if M <= capacity, else 0 (nothing emitted or sorted)
    uint32_t pad[13];
};

// ---------------------------------------------------------------------------
// block-wide exclusive scan (NT threads, wave64)
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T wave_scan_any(T x) {
    const int lane = threadIdx.x & 63;
    T inc = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        T y = __shfl_up(inc, d, 64);
        if (lane >= d) inc += y;
    }
    return inc;
}
template <>
__device__ __forceinline__ uint32_t wave_scan_any<uint32_t>(uint32_t x) { return wave_scan_incl(x); }

template <typename T, int NT>
__device__ __forceinline__ T block_exclusive_scan(T x, T *smem /*[NT/64]*/, T *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const T inc = wave_scan_any<T>(x);
    if (lane == 63) smem[wave] = inc;
    __syncthreads();
    T off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const T sw = smem[w];
        off += (w < wave) ? sw : T(0);
        tot += sw;
    }
    __syncthreads();
    *total = tot;
    return off + inc - x;
}

// ---------------------------------------------------------------------------
// 1-3: counts -> offsets -> emitted pairs
// ---------------------------------------------------------------------------
// Also clears the tile ranges (tiles that receive no pair keep (0, 0)).
__global__ __launch_bounds__(256) void k_group_sums(int n, const uint32_t *__restrict__ counts,
                                                    unsigned long long *__restrict__ part, int ntiles,
                                                    uint2 *__restrict__ ranges) {
    __shared__ unsigned long long sm[4];
    for (int t = blockIdx.x * 256 + threadIdx.x; t < ntiles; t += gridDim.x * 256) ranges[t] = make_uint2(0u, 0u);
    if (n == 0) return;
    const int g = blockIdx.x * 256 + threadIdx.x;
    unsigned long long c = g < n ? counts[g] : 0ull;
    unsigned long long tot;
    block_exclusive_scan<unsigned long long, 256>(c, sm, &tot);
    if (threadIdx.x == 0) part[blockIdx.x] = tot;
}

// One workgroup of 1024: exclusive scan of the group sums in place; publishes M.
__global__ __launch_bounds__(1024) void k_group_scan(int ngroups, int n, long long capacity,
                                                     unsigned long long *__restrict__ part,
                                                     BinHeader *__restrict__ hdr, uint32_t *__restrict__ offsets,
                                                     uint32_t *__restrict__ d_num) {
    __shared__ unsigned long long sm[16];
    const int per = (ngroups + 1023) / 1024;
    const int beg = threadIdx.x * per;
    unsigned long long s = 0;
    for (int i = 0; i < per; ++i)
        if (beg + i < ngroups) s += part[beg + i];
    unsigned long long tot;
    unsigned long long run = block_exclusive_scan<unsigned long long, 1024>(s, sm, &tot);
    for (int i = 0; i < per; ++i)
        if (beg + i < ngroups) {
            const unsigned long long v = part[beg + i];
            part[beg + i] = run;
            run += v;
        }
    if (threadIdx.x == 0) {
        hdr->total = tot;
        hdr->m_eff = (tot <= (unsigned long long)capacity) ? (uint32_t)tot : 0u;
        const uint32_t sat = tot > 0xffffffffull ? 0xffffffffu : (uint32_t)tot;
        *d_num = sat;
        offsets[n] = sat;
    }
}

// part[] holds either the exclusive group bases (scanned by k_group_scan) or, when
// `redundant`, the raw group sums: then every block adds up the sums before it
// (and all of them for M) itself, and block 0 publishes M -- one launch fewer.
__global__ __launch_bounds__(256) void k_emit(int n, int ngroups, int redundant, long long capacity, int tiles_x,
                                              const uint32_t *__restrict__ counts,
                                              const uint2 *__restrict__ pixbox,
                                              const unsigned long long *__restrict__ part,
                                              BinHeader *__restrict__ hdr, uint32_t *__restrict__ offsets,
                                              uint32_t *__restrict__ d_num,
                                              uint32_t *__restrict__ keys, uint32_t *__restrict__ vals) {
    __shared__ uint32_t excl[257];
    __shared__ uint2 box[256];
    __shared__ uint32_t sm[4];
    __shared__ unsigned long long sm64[8];
    const int tid = threadIdx.x;
    const int g = blockIdx.x * 256 + tid;
    const uint32_t c = g < n ? counts[g] : 0u;
    uint32_t tot;
    const uint32_t local = block_exclusive_scan<uint32_t, 256>(c, sm, &tot);
    unsigned long long base, total;
    if (redundant) {
        unsigned long long before = 0, all = 0;
        for (int i = tid; i < ngroups; i += 256) {
            const unsigned long long v = part[i];
            all += v;
            before += i < (int)blockIdx.x ? v : 0ull;
        }
        unsigned long long tb, ta;
        block_exclusive_scan<unsigned long long, 256>(before, sm64, &tb);
        block_exclusive_scan<unsigned long long, 256>(all, sm64 + 4, &ta);
        base = tb;
        total = ta;
        if (blockIdx.x == 0 && tid == 0) {
            hdr->total = total;
            hdr->m_eff = (total <= (unsigned long long)capacity) ? (uint32_t)total : 0u;
            const uint32_t sat = total > 0xffffffffull ? 0xffffffffu : (uint32_t)total;
            *d_num = sat;
            offsets[n] = sat;
        }
    } else {
        base = part[blockIdx.x];
        total = hdr->total;
    }
    if (g < n) {
        const unsigned long long o = base + local;
        offsets[g] = o > 0xffffffffull ? 0xffffffffu : (uint32_t)o;
    }
    if (total > (unsigned long long)capacity || tot == 0) return;   // overflow (or nothing to emit): uniform
    excl[tid] = local;
    if (tid == 0) excl[256] = tot;
    box[tid] = g < n ? pixbox[g] : make_uint2(0u, 0u);
    __syncthreads();
    const uint32_t b32 = (uint32_t)base;
    for (uint32_t idx = tid; idx < tot; idx += 256) {
        int lo = 0, hi = 256;                 // excl[lo] <= idx < excl[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (excl[mid] <= idx) lo = mid; else hi = mid;
        }
        const uint32_t r = idx - excl[lo];
        const uint2 bx = box[lo];
        const uint32_t tx0 = (bx.x & 0xffffu) >> 4, ty0 = (bx.x >> 16) >> 4;
        const uint32_t tx1 = (bx.y & 0xffffu) >> 4;
        const uint32_t wt = tx1 - tx0 + 1;
        const uint32_t q = r / wt, rem = r - q * wt;
        keys[b32 + idx] = (ty0 + q) * (uint32_t)tiles_x + tx0 + rem;
        vals[b32 + idx] = (uint32_t)(blockIdx.x * 256 + lo);
    }
}

// ---------------------------------------------------------------------------
// 4: stable LSD radix sort pass
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSortThreads) void k_sort_count(const uint32_t *__restrict__ keys,
                                                             const BinHeader *__restrict__ hdr, int shift,
                                                             int bits, uint32_t *__restrict__ table, int nbs) {
    __shared__ uint32_t h[256];
    const int radix = 1 << bits;
    const int tid = threadIdx.x;
    if (tid < radix) h[tid] = 0;
    __syncthreads();
    const uint32_t M = hdr->m_eff;
    const uint32_t base = blockIdx.x * (uint32_t)kSortChunk;
    for (int it = 0; it < kSortIters; ++it) {
        const uint32_t idx = base + it * kSortThreads + tid;
        if (idx < M) atomicAdd(&h[(keys[idx] >> shift) & (radix - 1)], 1u);
    }
    __syncthreads();
    if (tid < radix) table[(size_t)tid * nbs + blockIdx.x] = h[tid];
}

// `counts_raw`: the table holds the digit counts themselves (no scan pass ran);
// each block then forms its own offsets: thread d adds digit d's counts over the
// blocks in use (those before this one, and all of them for the digit total),
// and a block scan over the digit totals gives each digit's start.
__global__ __launch_bounds__(kSortThreads) void k_sort_scatter(const uint32_t *__restrict__ kin,
                                                               const uint32_t *__restrict__ vin,
                                                               uint32_t *__restrict__ kout,
                                                               uint32_t *__restrict__ vout,
                                                               const BinHeader *__restrict__ hdr, int shift,
                                                               int bits, const uint32_t *__restrict__ table,
                                                               int nbs, int counts_raw) {
    __shared__ uint32_t run[256];          // next output slot per digit
    __shared__ uint32_t wcnt[4][256];      // per wave: keys of each digit in this round
    __shared__ uint32_t sm[4];
    const uint32_t M = hdr->m_eff;
    const uint32_t base = blockIdx.x * (uint32_t)kSortChunk;
    if (base >= M) return;
    const int radix = 1 << bits;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (counts_raw) {
        const int used = (int)((M + kSortChunk - 1) / kSortChunk);
        uint32_t before = 0, total = 0;
        if (tid < radix) {
            const uint32_t *row = table + (size_t)tid * nbs;
            for (int b = 0; b < used; ++b) {
                const uint32_t c = row[b];
                total += c;
                before += b < (int)blockIdx.x ? c : 0u;
            }
        }
        uint32_t all;
        const uint32_t start = block_exclusive_scan<uint32_t, kSortThreads>(total, sm, &all);
        if (tid < radix) run[tid] = start + before;
    } else if (tid < radix) {
        run[tid] = table[(size_t)tid * nbs + blockIdx.x];
    }
    for (int i = tid; i < 4 * 256; i += kSortThreads) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const uint64_t below = lanes_below();
    for (int it = 0; it < kSortIters; ++it) {
        const uint32_t rbase = base + it * kSortThreads;
        if (rbase >= M) break;                                  // uniform
        const uint32_t idx = rbase + tid;
        const bool valid = idx < M;
        const uint32_t key = valid ? kin[idx] : 0u;
        const uint32_t val = valid ? vin[idx] : 0u;
        const uint32_t d = (key >> shift) & (uint32_t)(radix - 1);
        uint64_t peers = __ballot(valid);
        for (int bit = 0; bit < bits; ++bit) {
            const bool on = (d >> bit) & 1u;
            const uint64_t m = __ballot(on);
            peers &= on ? m : ~m;
        }
        const uint32_t rank = (uint32_t)__popcll(peers & below);
        const bool leader = valid && (peers >> lane) == 1ull;   // highest lane of the digit group
        if (leader) wcnt[wave][d] = (uint32_t)__popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t pos = run[d] + rank;
            for (int w = 0; w < wave; ++w) pos += wcnt[w][d];
            kout[pos] = key;
            vout[pos] = val;
        }
        __syncthreads();
        if (tid < radix) {
            run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
            wcnt[0][tid] = 0; wcnt[1][tid] = 0; wcnt[2][tid] = 0; wcnt[3][tid] = 0;
        }
        __syncthreads();
    }
}

// exclusive scan of a u32 array in place: one workgroup when it is short,
// otherwise reduce -> scan of block sums -> rescan with offsets.
// count <= 1024 * kScanSingleItems.  Element r * 1024 + i lives in thread i's
// register v[r] (coalesced loads, all issued together); its exclusive prefix is
// the totals of rows before r, plus the row-r totals of waves before thread i's
// wave, plus the DPP wave scan within the wave.
constexpr int kScanSingleItems = 32;
__global__ __launch_bounds__(1024) void k_scan_single(uint32_t *__restrict__ a, int count) {
    __shared__ uint32_t wsum[16][kScanSingleItems];     // [wave][row] totals -> exclusive over waves
    __shared__ uint32_t rowpre[kScanSingleItems];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rows = (count + 1023) / 1024;
    uint32_t v[kScanSingleItems], inc[kScanSingleItems];
#pragma unroll
    for (int r = 0; r < kScanSingleItems; ++r) {
        const int e = r * 1024 + tid;
        v[r] = (r < rows && e < count) ? a[e] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kScanSingleItems; ++r) {
        if (r >= rows) break;
        inc[r] = wave_scan_incl(v[r]);
        if (lane == 63) wsum[wave][r] = inc[r];
    }
    __syncthreads();
    if (tid < rows) {                     // one thread per row: exclusive over waves, row total
        uint32_t run = 0;
        for (int w = 0; w < 16; ++w) {
            const uint32_t x = wsum[w][tid];
            wsum[w][tid] = run;
            run += x;
        }
        rowpre[tid] = run;
    }
    __syncthreads();
    if (tid < 64) {                       // one wave: exclusive over rows
        const uint32_t tot = tid < rows ? rowpre[tid] : 0u;
        const uint32_t x = wave_scan_incl(tot);
        if (tid < rows) rowpre[tid] = x - tot;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kScanSingleItems; ++r) {
        if (r >= rows) break;
        const int e = r * 1024 + tid;
        if (e < count) a[e] = rowpre[r] + wsum[wave][r] + inc[r] - v[r];
    }
}

__global__ __launch_bounds__(256) void k_scan_reduce(const uint32_t *__restrict__ a, int count,
                                                     uint32_t *__restrict__ sums) {
    __shared__ uint32_t sm[4];
    const int beg = blockIdx.x * kScanChunk + threadIdx.x * kScanItems;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i)
        if (beg + i < count) s += a[beg + i];
    uint32_t tot;
    block_exclusive_scan<uint32_t, 256>(s, sm, &tot);
    if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

__global__ __launch_bounds__(256) void k_scan_down(uint32_t *__restrict__ a, int count,
                                                   const uint32_t *__restrict__ sums) {
    __shared__ uint32_t sm[4];
    const int beg = blockIdx.x * kScanChunk + threadIdx.x * kScanItems;
    uint32_t v[kScanItems];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        v[i] = (beg + i < count) ? a[beg + i] : 0u;
        s += v[i];
    }
    uint32_t tot;
    uint32_t run = block_exclusive_scan<uint32_t, 256>(s, sm, &tot) + sums[blockIdx.x];
#pragma unroll
    for (int i = 0; i < kScanItems; ++i)
        if (beg + i < count) {
            a[beg + i] = run;
            run += v[i];
        }
}

static hipError_t scan_u32(uint32_t *a, int count, uint32_t *sums, hipStream_t s) {
    if (count <= 1024 * kScanSingleItems) {
        k_scan_single<<<1, 1024, 0, s>>>(a, count);
        return hipGetLastError();
    }
    const int nb = (count + kScanChunk - 1) / kScanChunk;
    k_scan_reduce<<<nb, 256, 0, s>>>(a, count, sums);
    k_scan_single<<<1, 1024, 0, s>>>(sums, nb);
    k_scan_down<<<nb, 256, 0, s>>>(a, count, sums);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 5: tile ranges
// ---------------------------------------------------------------------------
// One thread per sorted pair: the first and last pair of each tile's run write
// its start and end (the ranges were cleared by k_group_sums).
__global__ __launch_bounds__(256) void k_ranges(const uint32_t *__restrict__ keys, const BinHeader *__restrict__ hdr,
                                                uint32_t *__restrict__ ranges) {
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    const uint32_t M = hdr->m_eff;
    if (i >= M) return;
    const uint32_t k = keys[i];
    if (i == 0 || keys[i - 1] != k) ranges[2 * k] = i;
    if (i + 1 == M || keys[i + 1] != k) ranges[2 * k + 1] = i + 1;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

BinPlan make_bin_plan(int n, int W, int H, int64_t capacity) {
    BinPlan p{};
    p.n = n; p.W = W; p.H = H;
    p.tiles_x = (W + kTile - 1) / kTile;
    const int tiles_y = (H + kTile - 1) / kTile;
    p.ntiles = p.tiles_x * tiles_y;
    p.capacity = capacity;
    int B = 0;
    while ((1ll << B) < (long long)p.ntiles) ++B;          // key bits: ids in [0, ntiles)
    p.passes = (B + 7) / 8;
    for (int i = 0; i < 4; ++i) p.bits[i] = 0;
    if (p.passes > 0) {
        const int w = (B + p.passes - 1) / p.passes;
        int left = B;
        for (int i = 0; i < p.passes; ++i) { p.bits[i] = left < w ? left : w; left -= p.bits[i]; }
    }
    p.nb_g = (n + 255) / 256;
    p.nbs = (int)((capacity + kSortChunk - 1) / kSortChunk);
    size_t off = align256(sizeof(BinHeader));
    p.off_part = off; off = align256(off + sizeof(unsigned long long) * (size_t)(p.nb_g > 0 ? p.nb_g : 1));
    p.off_kalt = off; off = align256(off + sizeof(uint32_t) * (size_t)(capacity > 0 ? capacity : 1));
    p.off_valt = off; off = align256(off + sizeof(uint32_t) * (size_t)(capacity > 0 ? capacity : 1));
    const size_t table = (size_t)256 * (size_t)(p.nbs > 0 ? p.nbs : 1);
    p.off_table = off; off = align256(off + sizeof(uint32_t) * table);
    p.off_tsp = off; off = align256(off + sizeof(uint32_t) * ((table + kScanChunk - 1) / kScanChunk + 1));
    p.bytes = off;
    return p;
}

const void *bin_total_ptr(const void *ws) { return &static_cast<const BinHeader *>(ws)->total; }

hipError_t launch_bin_sort(const BinPlan &p, const uint16_t *pixbox, const uint32_t *counts, uint32_t *offsets,
                           uint32_t *keys, uint32_t *vals, uint32_t *ranges, uint32_t *d_num, void *ws,
                           hipStream_t s) {
    char *w = static_cast<char *>(ws);
    BinHeader *hdr = reinterpret_cast<BinHeader *>(w);
    unsigned long long *part = reinterpret_cast<unsigned long long *>(w + p.off_part);
    uint32_t *kalt = reinterpret_cast<uint32_t *>(w + p.off_kalt);
    uint32_t *valt = reinterpret_cast<uint32_t *>(w + p.off_valt);
    uint32_t *table = reinterpret_cast<uint32_t *>(w + p.off_table);
    uint32_t *tsp = reinterpret_cast<uint32_t *>(w + p.off_tsp);

    k_group_sums<<<p.nb_g > 0 ? p.nb_g : 1, 256, 0, s>>>(p.n, counts, part, p.ntiles,
                                                         reinterpret_cast<uint2 *>(ranges));
    const int redundant = p.nb_g > 0 && p.nb_g <= kMaxRedundantGroups;
    if (!redundant) k_group_scan<<<1, 1024, 0, s>>>(p.nb_g, p.n, (long long)p.capacity, part, hdr, offsets, d_num);
    // Emit into the buffer that the last pass reads from, so the result lands in keys/vals.
    uint32_t *ek = (p.passes & 1) ? kalt : keys;
    uint32_t *ev = (p.passes & 1) ? valt : vals;
    if (p.nb_g > 0)
        k_emit<<<p.nb_g, 256, 0, s>>>(p.n, p.nb_g, redundant, (long long)p.capacity, p.tiles_x, counts,
                                      reinterpret_cast<const uint2 *>(pixbox), part, hdr, offsets, d_num, ek, ev);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint32_t *srck = ek, *srcv = ev;
    uint32_t *dstk = (srck == keys) ? kalt : keys, *dstv = (srcv == vals) ? valt : vals;
    int shift = 0;
    for (int pass = 0; pass < p.passes && p.nbs > 0; ++pass) {
        const int bits = p.bits[pass];
        k_sort_count<<<p.nbs, kSortThreads, 0, s>>>(srck, hdr, shift, bits, table, p.nbs);
        const int raw = (1 << bits) * p.nbs <= kMaxRawTable;
        if (!raw) {
            e = scan_u32(table, (1 << bits) * p.nbs, tsp, s);
            if (e != hipSuccess) return e;
        }
        k_sort_scatter<<<p.nbs, kSortThreads, 0, s>>>(srck, srcv, dstk, dstv, hdr, shift, bits, table, p.nbs, raw);
        shift += bits;
        uint32_t *tk = srck, *tv = srcv;
        srck = dstk; srcv = dstv; dstk = tk; dstv = tv;
    }
    if (p.capacity > 0)
        k_ranges<<<(unsigned)((p.capacity + 255) / 256), 256, 0, s>>>(keys, hdr, ranges);
    return hipGetLastError();
}

}  // namespace gi
