// k_binning.hip -- tile lists from per-Gaussian pixel boxes.
//
// Every Gaussian g covers a rectangle of tiles; its pairs (tile id, g) are
// numbered in (index, tile row, tile column) order, pair m of g sitting at
// emission slot offsets[g] + m.  A stable radix sort on the tile id then leaves
// each tile's list in ascending Gaussian index.
//
//   1. k_group_sums : per 256-Gaussian group, the sum of tile counts (u64);
//                     clears the tile ranges.  Up to 2048 groups it also
//                     writes the group's first-digit histogram (as the
//                     preprocess kernels do when they form the counts), and
//                     steps 2-3 do not run.
//   2. k_group_scan : one workgroup scans the group sums (more than 2048 groups).
//   3. k_count0     : per segment of 4 groups: offsets[], M, and the histogram
//                     of the first digit over the segment's pairs.
//   4. k_scatter0w  : (up to 2048 groups) first sort pass, one group per block:
//                     each block adds up the group sums and the histograms
//                     before it itself, writes its offsets[] and scatters.
//      k_scatter0   : (more groups) first sort pass over segments of 4 groups.
//                     The pairs are never written in emission order: they are
//                     regenerated from the pixel boxes wherever they are needed
//                     (each thread walks its own Gaussian's tiles; when some
//                     Gaussian of the segment covers more than 64 tiles, a
//                     binary search in LDS spreads the pairs over the lanes).
//   Then, by the number B of key bits and the size of the pair buffer:
//     B <= 8         : that pass sorted the whole key; its workgroup 0 writes
//                      the tile ranges from the digit starts.
//     B <= 16, small : the first pass took the high digit; k_bucket_sort, one
//                      workgroup per high digit, sorts its bucket by the low
//                      digit and writes the bucket's tile ranges from its counts.
//     otherwise      : LSD -- the first pass took the low digit, k_count /
//                      k_scatter take the next ones over blocks of 1024-4096
//                      keys, and k_ranges marks where each run starts and ends.
//   5. k_tile_order : (optional) the order in which the raster kernels should
//                     take the tiles: sorted by decreasing list length and dealt
//                     to the CUs in serpentine layers, which balances the CUs
//                     when the whole grid is resident at once.
//
// Each scatter ranks up to 4096 keys at a time: every wave takes a contiguous
// span of the chunk and finds the rank of each key among the equal digits of
// its span with wave ballots (in key order, hence stable); the chunk is then
// reordered by digit in LDS and written out in runs, so consecutive lanes store
// to consecutive addresses.  Digit tables of up to 32K entries are never
// scanned by a kernel of their own: each scatter block adds up the entries it
// needs itself.
//
// Binning is the tile-binned scheme of the FlashImgs viewer ("Web viewer":
// tile-binned compute) with fvdb's 16-pixel tiles (tile_size).  All steps are
// HBM or latency bound: ~20 B per pair per sort pass after the first.
#include "gi_device.hpp"
#include "gi_launch.hpp"

namespace gi {

constexpr int kBT = 256;                       // threads per binning block
constexpr int kPerLane = 16;                   // keys per lane per chunk (at most)
constexpr int kChunk = kBT * kPerLane;         // keys per first-pass chunk
constexpr int kMaxRedundantGroups = 2048;      // count0 adds up the group sums itself up to this
constexpr int kMaxRedundantTable = 32768;      // digit tables up to this are not scanned ...
constexpr int64_t kMaxRedundantReads = 8 << 20;// ... when all blocks together read at most this many entries
constexpr int kScanItems = 16;
constexpr int kScanChunk = 256 * kScanItems;   // table entries per scan block
constexpr uint32_t kDirectMax = 64;            // a thread emits its Gaussian's pairs itself up to this many tiles
constexpr int64_t kMaxBucketCapacity = 1ll << 26; // bucket pass for pair buffers up to this (larger: LSD passes)
constexpr bool kDirectScatter = true;          // one-chunk buckets store keys without an LDS reorder (the
                                               // segmented first pass keeps the reorder)

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

// One barrier: the workgroup sums of x and y (u64) and the exclusive scan of c
// (with its total), over NT threads.  sm64 [2 NT/64] and sm32 [NT/64] must not
// be reused without a barrier.
template <int NT>
__device__ __forceinline__ void block_sums2_scan(unsigned long long x, unsigned long long y, uint32_t c,
                                                 unsigned long long &sx, unsigned long long &sy, uint32_t &excl,
                                                 uint32_t &ctot, unsigned long long *sm64, uint32_t *sm32) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        x += __shfl_xor(x, o, 64);
        y += __shfl_xor(y, o, 64);
    }
    const uint32_t inc = wave_scan_incl(c);
    if (lane == 63) {
        sm64[wave] = x;
        sm64[NW + wave] = y;
        sm32[wave] = inc;
    }
    __syncthreads();
    unsigned long long ax = 0, ay = 0;
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        ax += sm64[w];
        ay += sm64[NW + w];
        const uint32_t v = sm32[w];
        off += w < wave ? v : 0u;
        tot += v;
    }
    sx = ax;
    sy = ay;
    excl = off + inc - c;
    ctot = tot;
}

__device__ __forceinline__ uint32_t sat32(unsigned long long x) { return x > 0xffffffffull ? 0xffffffffu : (uint32_t)x; }

// ---------------------------------------------------------------------------
// pair regeneration: a segment's exclusive scan of tile counts and its boxes in LDS
// ---------------------------------------------------------------------------
template <int S>
struct SegLds {
    uint32_t excl[S + 1];
    uint2 box[S];
};

// Pair `idx` (< excl[ns]) of a segment of ns Gaussians: its tile id and the
// segment-local index of its Gaussian (the last l with excl[l] <= idx, which
// never names a Gaussian without tiles).  The search has no branch: a probe
// past the segment reads excl[ns] (> idx), so several searches of one thread
// interleave their LDS reads.
template <int S>
__device__ __forceinline__ void regen_pair(const SegLds<S> &G, int ns, uint32_t idx, int tiles_x, uint32_t &key,
                                           int &lo) {
    int l = 0;
#pragma unroll
    for (int step = S >> 1; step > 0; step >>= 1) {
        const int c = l + step;
        l = G.excl[c < ns ? c : ns] <= idx ? c : l;
    }
    const uint32_t r = idx - G.excl[l];
    const uint2 bx = G.box[l];
    const uint32_t tx0 = (bx.x & 0xffffu) >> 4, ty0 = (bx.x >> 16) >> 4;
    const uint32_t tx1 = (bx.y & 0xffffu) >> 4;
    const uint32_t wt = tx1 - tx0 + 1;
    const uint32_t q = r / wt, rem = r - q * wt;
    key = (ty0 + q) * (uint32_t)tiles_x + tx0 + rem;
    lo = l;
}

// The lanes among `peers` whose digit equals this lane's d (digits of at most 8 bits: a bit above
// the digit's width is clear in every lane and leaves the set as it is).  Per bit: its ballot m,
// kept where this lane's bit is set and inverted where it is clear (~(m ^ spread bit)), in
// straight-line code.
__device__ __forceinline__ uint64_t match_digit(uint32_t d, uint64_t peers) {
    uint32_t lo = (uint32_t)peers, hi = (uint32_t)(peers >> 32);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const uint32_t sp = (uint32_t)((int32_t)(d << (31 - b)) >> 31);   // bit b spread over the word
        const uint64_t m = __ballot(sp != 0u);
        lo &= ~((uint32_t)m ^ sp);                        // lanes whose bit equals this lane's
        hi &= ~((uint32_t)(m >> 32) ^ sp);
    }
    return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// digit bases of one sort block
// ---------------------------------------------------------------------------
// Table layouts: "redundant" = [column][radix] raw counts (radix >= 4), read
// by every block; "scanned" = [radix][ncols_cap], exclusive-scanned in place
// beforehand.  Every column up to ncols_cap is written (zeros past M).
struct BaseLds {
    uint4 part_b[kBT], part_t[kBT];
    uint32_t sm[4];
};

// Per-thread partial sums of the table entries this block needs, loaded in one
// round (split from digit_finish so the loads overlap the caller's own).
struct DigitAcc {
    uint4 b, t;      // redundant: sums over the thread's columns (before `me`, all) of 4 digits
    uint32_t x;      // scanned: the block's base of digit tid
};

template <int NB = 16, int NT = kBT>
__device__ __forceinline__ DigitAcc digit_load(const uint32_t *__restrict__ table, int redundant, int ncols_cap,
                                               int me, int bits) {
    const int tid = threadIdx.x;
    DigitAcc a;
    a.b = make_uint4(0u, 0u, 0u, 0u);
    a.t = a.b;
    a.x = 0u;
    if (!redundant) {
        if (tid < (1 << bits)) a.x = table[(size_t)tid * ncols_cap + me];
        return a;
    }
    // uint4 q of column c holds digits 4*(q mod Q) .. +3, Q = radix/4 (divides 256):
    // thread t always reads the same 4 digits, from columns t/Q, t/Q + NT/Q, ...
    const int lq = bits - 2;
    const int g4 = tid & ((1 << lq) - 1);
    const int cstep = NT >> lq;
    const uint4 *t4 = reinterpret_cast<const uint4 *>(table);
    // batches of NB loads, all in flight together (one batch when NB * NT * 4
    // >= kMaxRedundantTable, the most a redundant table holds)
    // (unconditional loads with 32-bit offsets: columns past the end read entry 0 and are dropped)
    if (NB * NT * 4 >= kMaxRedundantTable) {            // one batch covers every redundant table: no loop
        const int c0 = tid >> lq;                       // (a loop would first wait for every load in flight)
        uint4 v[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int c = c0 + k * cstep;
            v[k] = t4[c < ncols_cap ? ((uint32_t)c << lq) + (uint32_t)g4 : 0u];
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int c = c0 + k * cstep;
            if (c >= ncols_cap) v[k] = make_uint4(0u, 0u, 0u, 0u);
            a.t.x += v[k].x; a.t.y += v[k].y; a.t.z += v[k].z; a.t.w += v[k].w;
            if (c < me) { a.b.x += v[k].x; a.b.y += v[k].y; a.b.z += v[k].z; a.b.w += v[k].w; }
        }
        return a;
    }
    for (int c0 = tid >> lq; c0 < ncols_cap; c0 += NB * cstep) {
        uint4 v[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int c = c0 + k * cstep;
            v[k] = t4[c < ncols_cap ? ((uint32_t)c << lq) + (uint32_t)g4 : 0u];
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int c = c0 + k * cstep;
            if (c >= ncols_cap) v[k] = make_uint4(0u, 0u, 0u, 0u);
            a.t.x += v[k].x; a.t.y += v[k].y; a.t.z += v[k].z; a.t.w += v[k].w;
            if (c < me) { a.b.x += v[k].x; a.b.y += v[k].y; a.b.z += v[k].z; a.b.w += v[k].w; }
        }
    }
    return a;
}

// gbase[d] = first output position of this block's keys of digit d.
__device__ __forceinline__ void digit_finish(const DigitAcc &a, int redundant, int bits, uint32_t *gbase,
                                             BaseLds &B) {
    const int tid = threadIdx.x, radix = 1 << bits;
    if (!redundant) {
        if (tid < radix) gbase[tid] = a.x;
        __syncthreads();
        return;
    }
    const int q = radix >> 2;
    B.part_b[tid] = a.b;
    B.part_t[tid] = a.t;
    __syncthreads();
    uint32_t b = 0, t = 0;
    if (q >= 16) {                                     // digit d: add the kBT / q threads that hold it
        if (tid < radix) {
            const uint32_t *pb = reinterpret_cast<const uint32_t *>(B.part_b);
            const uint32_t *pt = reinterpret_cast<const uint32_t *>(B.part_t);
            const int g4 = tid >> 2, comp = tid & 3;
            for (int k = 0; k < kBT / q; ++k) {
                b += pb[(g4 + k * q) * 4 + comp];
                t += pt[(g4 + k * q) * 4 + comp];
            }
        }
    } else {
        for (int s = kBT >> 1; s >= q; s >>= 1) {      // fold threads with equal tid mod q
            if (tid < s) {
                const uint4 ob = B.part_b[tid + s], ot = B.part_t[tid + s];
                uint4 &mb = B.part_b[tid], &mt = B.part_t[tid];
                mb.x += ob.x; mb.y += ob.y; mb.z += ob.z; mb.w += ob.w;
                mt.x += ot.x; mt.y += ot.y; mt.z += ot.z; mt.w += ot.w;
            }
            __syncthreads();
        }
        if (tid < radix) {
            b = reinterpret_cast<const uint32_t *>(B.part_b)[tid];    // uint4 (d>>2), component (d&3)
            t = reinterpret_cast<const uint32_t *>(B.part_t)[tid];
        }
    }
    uint32_t all;
    const uint32_t start = block_exclusive_scan<uint32_t, kBT>(t, B.sm, &all);
    if (tid < radix) gbase[tid] = start + b;
    __syncthreads();
}

// ---------------------------------------------------------------------------
// one chunk of a stable scatter
// ---------------------------------------------------------------------------
template <int PL>
struct ChunkLds {
    uint32_t cnt[4][256];     // per wave: keys of each digit so far -> wave's first local slot
    uint32_t dstart[256];     // chunk-local first slot of each digit
    uint32_t gbase[256];      // global position of the block's next key of each digit
    uint32_t sk[kBT * PL], sv[kBT * PL];
    uint32_t sm[4];
};

// Scatters the chunk's `cc` keys to kout/vout at gbase[digit] + (rank of the
// key among the chunk's keys of its digit), then, unless it is the block's last
// chunk, advances gbase past the chunk.  L.dstart[d] keeps the chunk-local
// first slot of digit d afterwards.  With flat_base, key j of the chunk's
// digit order goes to flat_base + j (gbase is ignored): the chunk is a whole
// bucket sorted in place of its input range.
// Key i sits in lane i % 64 of wave i / span, register (i % span) / 64, for
// the `span` (a multiple of 64, span * 4 >= cc) the caller loaded with.
// Entered and left by all threads with LDS in a settled state.
// With DIRECT, each key is stored straight from its register to its final
// position (no LDS reorder; stores of a wave scatter over the digits' runs):
// fewer barriers for the small chunks of the first pass and of the buckets.
template <int PL, bool DIRECT = false>
__device__ __forceinline__ void scatter_chunk(ChunkLds<PL> &L, int cc, int span, int shift, int bits,
                                              const uint32_t (&key)[PL], const uint32_t (&val)[PL],
                                              uint32_t *__restrict__ kout, uint32_t *__restrict__ vout,
                                              uint32_t cap, bool last, uint32_t flat_base = 0xffffffffu) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int radix = 1 << bits;
    const uint32_t dmask = (uint32_t)(radix - 1);
    if (tid < radix) { L.cnt[0][tid] = 0u; L.cnt[1][tid] = 0u; L.cnt[2][tid] = 0u; L.cnt[3][tid] = 0u; }
    __syncthreads();
    const int iters = span >> 6;                          // <= PL; guards on `it` are uniform
    const uint64_t below = lanes_below();
    uint32_t rk[PL];
#pragma unroll
    for (int it = 0; it < PL; ++it) {
        if (it >= iters) continue;
        const int idx = wave * span + it * 64 + lane;
        const bool valid = idx < cc;
        const uint32_t d = (key[it] >> shift) & dmask;
        const uint64_t peers = match_digit(d, __ballot(valid));
        const uint32_t before = valid ? L.cnt[wave][d] : 0u;
        rk[it] = before + (uint32_t)__popcll(peers & below);
        if (valid && (peers >> lane) == 1ull) L.cnt[wave][d] = before + (uint32_t)__popcll(peers);
    }
    __syncthreads();
    uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
    if (tid < radix) { c0 = L.cnt[0][tid]; c1 = L.cnt[1][tid]; c2 = L.cnt[2][tid]; c3 = L.cnt[3][tid]; }
    const uint32_t tot = c0 + c1 + c2 + c3;
    uint32_t all;
    const uint32_t ds = block_exclusive_scan<uint32_t, kBT>(tot, L.sm, &all);
    if (tid < radix) {
        L.dstart[tid] = ds;
        if (flat_base != 0xffffffffu) L.gbase[tid] = flat_base + ds;
        L.cnt[0][tid] = ds;
        L.cnt[1][tid] = ds + c0;
        L.cnt[2][tid] = ds + c0 + c1;
        L.cnt[3][tid] = ds + c0 + c1 + c2;
    }
    __syncthreads();
    if (DIRECT) {
#pragma unroll
        for (int it = 0; it < PL; ++it) {
            if (it >= iters) continue;
            const int idx = wave * span + it * 64 + lane;
            if (idx < cc) {
                const uint32_t d = (key[it] >> shift) & dmask;
                const uint32_t pos = L.gbase[d] + (L.cnt[wave][d] + rk[it]) - L.dstart[d];
                if (pos < cap) {                          // holds by construction; keeps a bad table in bounds
                    kout[pos] = key[it];
                    vout[pos] = val[it];
                }
            }
        }
        if (last) return;                                 // uniform
        __syncthreads();
        if (tid < radix) L.gbase[tid] += tot;
        __syncthreads();
        return;
    }
#pragma unroll
    for (int it = 0; it < PL; ++it) {
        if (it >= iters) continue;
        const int idx = wave * span + it * 64 + lane;
        if (idx < cc) {
            const uint32_t lp = L.cnt[wave][(key[it] >> shift) & dmask] + rk[it];
            if (lp < (uint32_t)(kBT * PL)) {
                L.sk[lp] = key[it];
                L.sv[lp] = val[it];
            }
        }
    }
    __syncthreads();
    for (int j = tid; j < cc; j += kBT) {
        const uint32_t k = L.sk[j];
        const uint32_t d = (k >> shift) & dmask;
        const uint32_t pos = L.gbase[d] + (uint32_t)j - L.dstart[d];
        if (pos < cap) {                                  // holds by construction; keeps a bad table in bounds
            kout[pos] = k;
            vout[pos] = L.sv[j];
        }
    }
    if (last) return;                                     // uniform
    __syncthreads();
    if (tid < radix) L.gbase[tid] += tot;
    __syncthreads();
}

// ---------------------------------------------------------------------------
// 1-2: group sums
// ---------------------------------------------------------------------------
// Also clears the tile ranges (tiles that receive no pair keep (0, 0)); with
// n == 0 it publishes M = 0 itself.  With hist.table set it also writes the
// group's first-pass digit histogram (no count kernel runs then).
__global__ __launch_bounds__(kBT) void k_group_sums(int n, const uint32_t *__restrict__ counts,
                                                    const uint2 *__restrict__ pixbox,
                                                    unsigned long long *__restrict__ part, int ntiles,
                                                    uint2 *__restrict__ ranges, BinHeader *__restrict__ hdr,
                                                    uint32_t *__restrict__ offsets, uint32_t *__restrict__ d_num,
                                                    BinHist hist, uint32_t *__restrict__ d_max) {
    __shared__ unsigned long long sm[4];
    __shared__ uint32_t h[256];
    const int tid = threadIdx.x;
    for (int t = blockIdx.x * kBT + tid; t < ntiles; t += gridDim.x * kBT) ranges[t] = make_uint2(0u, 0u);
    if (n == 0) {
        if (blockIdx.x == 0 && tid == 0) {
            hdr->total = 0ull;
            hdr->m_eff = 0u;
            *d_num = 0u;
            offsets[0] = 0u;
        }
        return;
    }
    const int radix = 1 << hist.bits;
    if (hist.table && tid < radix) h[tid] = 0u;
    const int g = blockIdx.x * kBT + tid;
    const uint32_t c = g < n ? counts[g] : 0u;
    const uint2 bx = (hist.table && g < n) ? pixbox[g] : make_uint2(0u, 0u);
    unsigned long long tot;
    block_exclusive_scan<unsigned long long, kBT>((unsigned long long)c, sm, &tot);   // barriers publish h
    if (tid == 0) part[blockIdx.x] = tot;
    if (hist.table) {                                     // uniform
        hist_add_pairs(h, c, bx, hist.tiles_x, hist.shift, (uint32_t)(radix - 1));
        __syncthreads();
        if (tid < radix) {
            if (hist.redundant) hist.table[(size_t)blockIdx.x * radix + tid] = h[tid];
            else hist.table[(size_t)tid * hist.ncols_cap + blockIdx.x] = h[tid];
        }
    }
}

// d_max (or NULL): the caller's running maximum of M, raised to this M.
__device__ __forceinline__ void publish_total(unsigned long long tot, long long capacity, int n,
                                              BinHeader *hdr, uint32_t *offsets, uint32_t *d_num,
                                              uint32_t *d_max) {
    hdr->total = tot;
    hdr->m_eff = (tot <= (unsigned long long)capacity) ? (uint32_t)tot : 0u;
    *d_num = sat32(tot);
    if (d_max) *d_max = max(*d_max, sat32(tot));
    offsets[n] = sat32(tot);
}

// One workgroup of 1024: exclusive scan of the group sums in place; publishes M.
__global__ __launch_bounds__(1024) void k_group_scan(int ngroups, int n, long long capacity,
                                                     unsigned long long *__restrict__ part,
                                                     BinHeader *__restrict__ hdr, uint32_t *__restrict__ offsets,
                                                     uint32_t *__restrict__ d_num, uint32_t *__restrict__ d_max) {
    __shared__ unsigned long long sm[16];
    constexpr int U = 8;                                  // sums held in registers (ngroups <= 8192: one round)
    const int per = (ngroups + 1023) / 1024;
    const int beg = threadIdx.x * per;
    unsigned long long s = 0;
    unsigned long long v[U];
    // rounds of U loads issued together (a load per loop trip would wait for each in turn)
    for (int i0 = 0; i0 < per; i0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = beg + i0 + u;
            v[u] = (i0 + u < per && i < ngroups) ? part[i] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) s += v[u];
    }
    unsigned long long tot;
    unsigned long long run = block_exclusive_scan<unsigned long long, 1024>(s, sm, &tot);
    if (per <= U) {                                       // uniform: the sums are still in v
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = beg + u;
            if (u < per && i < ngroups) {
                part[i] = run;
                run += v[u];
            }
        }
    } else {
        for (int i0 = 0; i0 < per; i0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = beg + i0 + u;
                v[u] = (i0 + u < per && i < ngroups) ? part[i] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = beg + i0 + u;
                if (i0 + u < per && i < ngroups) {
                    part[i] = run;
                    run += v[u];
                }
            }
        }
    }
    if (threadIdx.x == 0) publish_total(tot, capacity, n, hdr, offsets, d_num, d_max);
}

// ---------------------------------------------------------------------------
// 3: offsets + first-digit histogram per segment
// ---------------------------------------------------------------------------
// part[] holds the raw group sums when `redundant` (then block b adds up the
// sums before its first group, and all of them for M, itself; block 0
// publishes M), else the exclusive group bases from k_group_scan.
__global__ __launch_bounds__(kBT) void k_count0(int n, int ngroups, int seg_groups, int redundant,
                                                long long capacity, int tiles_x, int shift, int bits,
                                                int table_redundant,
                                                int ncols_cap, const uint32_t *__restrict__ counts,
                                                const uint2 *__restrict__ pixbox,
                                                const unsigned long long *__restrict__ part,
                                                BinHeader *__restrict__ hdr, uint32_t *__restrict__ offsets,
                                                uint32_t *__restrict__ d_num, uint32_t *__restrict__ table,
                                                uint32_t *__restrict__ d_max) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sm[4];
    __shared__ unsigned long long sm64[8];
    const int tid = threadIdx.x;
    const int radix = 1 << bits;
    const uint32_t dmask = (uint32_t)(radix - 1);
    if (tid < radix) hist[tid] = 0u;
    const int g0 = blockIdx.x * seg_groups;
    const int g1 = min(g0 + seg_groups, ngroups);
    // the first group's inputs, loaded together with the group sums
    int gid = g0 * kBT + tid;
    uint32_t c = gid < n ? counts[gid] : 0u;
    uint2 bx = gid < n ? pixbox[gid] : make_uint2(0u, 0u);
    unsigned long long base, total;
    if (redundant) {
        unsigned long long before = 0, all = 0;
        unsigned long long v[kMaxRedundantGroups / kBT];
#pragma unroll
        for (int k = 0; k < kMaxRedundantGroups / kBT; ++k) {
            const int i = tid + k * kBT;
            v[k] = i < ngroups ? part[i] : 0ull;
        }
#pragma unroll
        for (int k = 0; k < kMaxRedundantGroups / kBT; ++k) {
            all += v[k];
            before += tid + k * kBT < g0 ? v[k] : 0ull;
        }
        unsigned long long tb, ta;
        block_exclusive_scan<unsigned long long, kBT>(before, sm64, &tb);
        block_exclusive_scan<unsigned long long, kBT>(all, sm64 + 4, &ta);
        base = tb;
        total = ta;
        if (blockIdx.x == 0 && tid == 0) publish_total(total, capacity, n, hdr, offsets, d_num, d_max);
    } else {
        base = part[g0];
        total = hdr->total;
    }
    const bool emit = total <= (unsigned long long)capacity;
    for (int g = g0; g < g1; ++g) {
        if (g > g0) {
            gid = g * kBT + tid;
            c = gid < n ? counts[gid] : 0u;
            bx = gid < n ? pixbox[gid] : make_uint2(0u, 0u);
        }
        uint32_t tot;
        const uint32_t local = block_exclusive_scan<uint32_t, kBT>(c, sm, &tot);
        if (gid < n) offsets[gid] = sat32(base + local);
        if (emit) hist_add_pairs(hist, c, bx, tiles_x, shift, dmask);
        base += tot;
    }
    __syncthreads();
    if (tid < radix) {
        if (table_redundant) table[(size_t)blockIdx.x * radix + tid] = hist[tid];
        else table[(size_t)tid * ncols_cap + blockIdx.x] = hist[tid];
    }
}

// ---------------------------------------------------------------------------
// 4: first sort pass from the regenerated pairs (segments of 256 * SG Gaussians)
// ---------------------------------------------------------------------------
// Segments of SG groups, offsets[] and M from k_count0 (more than
// kMaxRedundantGroups groups; fewer take k_scatter0w below).  Workgroup 0 also
// publishes where each digit's run starts (bucket_start[d], d <= radix, the
// last one M) for the bucket pass, and, when this pass sorts the whole key
// (ranges != NULL), the tile ranges themselves.
template <int SG>
__global__ __launch_bounds__(kBT) void k_scatter0(int n, int tiles_x, int shift, int bits, int table_redundant,
                                                  int ncols_cap, const uint2 *__restrict__ pixbox,
                                                  const uint32_t *__restrict__ offsets,
                                                  const BinHeader *__restrict__ hdr,
                                                  const uint32_t *__restrict__ table, uint32_t *__restrict__ kout,
                                                  uint32_t *__restrict__ vout, uint32_t *__restrict__ bucket_start,
                                                  uint2 *__restrict__ ranges, int ntiles) {
    constexpr int S = kBT * SG;
    __shared__ SegLds<S> G;
    __shared__ ChunkLds<kPerLane> L;
    __shared__ BaseLds B;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int first = blockIdx.x * S;
    const int ns = min(S, n - first);
    // One round of loads: the segment's offsets and boxes, M, the digit table.
    uint32_t o[SG], o1[SG];
    uint2 bx[SG];
#pragma unroll
    for (int r = 0; r < SG; ++r) {
        const int i = r * kBT + tid;
        o[r] = i < ns ? offsets[first + i] : 0u;
        o1[r] = i < ns ? offsets[first + i + 1] : 0u;
        bx[r] = i < ns ? pixbox[first + i] : make_uint2(0u, 0u);
    }
    const uint32_t o0 = offsets[first];
    const uint32_t oend = offsets[first + ns];        // the next segment's first slot, or M
    const uint32_t M = hdr->m_eff;
    const DigitAcc acc = digit_load(table, table_redundant, ncols_cap, blockIdx.x, bits);
    if (M == 0u) return;                              // overflow or no pair (then offsets may saturate): uniform
#pragma unroll
    for (int r = 0; r < SG; ++r) {
        const int i = r * kBT + tid;
        if (i < ns) {
            G.excl[i] = o[r] - o0;
            G.box[i] = bx[r];
        }
    }
    if (tid == 0) G.excl[ns] = oend - o0;
    uint32_t cmax = 0;
#pragma unroll
    for (int r = 0; r < SG; ++r) cmax = max(cmax, o1[r] - o[r]);
    const bool big = __syncthreads_or(cmax > kDirectMax);   // else each thread emits its own pairs
    digit_finish(acc, table_redundant, bits, L.gbase, B);   // its barriers publish G
    if (blockIdx.x == 0) {
        const int radix = 1 << bits;
        if (tid < radix) bucket_start[tid] = L.gbase[tid];
        if (tid == 0) bucket_start[radix] = M;
        if (ranges && tid < radix && tid < ntiles) {
            const uint32_t a = L.gbase[tid], e = tid + 1 < radix ? L.gbase[tid + 1] : M;
            ranges[tid] = e > a ? make_uint2(a, e) : make_uint2(0u, 0u);
        }
    }
    const uint32_t tot = oend - o0;
    for (uint32_t cs = 0; cs < tot; cs += kChunk) {
        const int cc = (int)min((uint32_t)kChunk, tot - cs);
        const int span = ((cc + kBT - 1) / kBT) * 64;
        const int iters = span >> 6;
        uint32_t key[kPerLane], val[kPerLane];
        if (!big) {                                               // uniform
            // each thread writes its Gaussians' pairs of this chunk into the staging arrays
#pragma unroll
            for (int r = 0; r < SG; ++r) {
                const int i = r * kBT + tid;
                if (i >= ns) continue;
                const uint32_t e0 = o[r] - o0, e1 = o1[r] - o0;
                const uint32_t lo = max(e0, cs), hi = min(e1, cs + (uint32_t)cc);
                if (lo >= hi) continue;
                const uint32_t tx0 = (bx[r].x & 0xffffu) >> 4, ty0 = (bx[r].x >> 16) >> 4;
                const uint32_t wt = ((bx[r].y & 0xffffu) >> 4) - tx0 + 1;
                uint32_t q = (lo - e0) / wt, col = (lo - e0) - q * wt;
                uint32_t row = (ty0 + q) * (uint32_t)tiles_x + tx0;
                for (uint32_t x = lo; x < hi; ++x) {
                    L.sk[x - cs] = row + col;
                    L.sv[x - cs] = (uint32_t)(first + i);
                    if (++col == wt) { col = 0; row += (uint32_t)tiles_x; }
                }
            }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < kPerLane; ++it) {
                if (it < iters) {                                 // uniform
                    const int idx = wave * span + it * 64 + lane;
                    const int q = idx < cc ? idx : cc - 1;
                    key[it] = L.sk[q];
                    val[it] = L.sv[q];
                }
            }
        } else {
#pragma unroll
            for (int it = 0; it < kPerLane; ++it) {
                if (it < iters) {                                 // uniform
                    const int idx = wave * span + it * 64 + lane;
                    int lo;
                    regen_pair<S>(G, ns, cs + (uint32_t)(idx < cc ? idx : cc - 1), tiles_x, key[it], lo);
                    val[it] = (uint32_t)(first + lo);
                }
            }
        }
        scatter_chunk<kPerLane>(L, cc, span, shift, bits, key, val, kout, vout, M, cs + (uint32_t)kChunk >= tot);
    }
}

// ---------------------------------------------------------------------------
// 4w: the first pass for one-group segments, 512 threads per group
// ---------------------------------------------------------------------------
// With one group (256 Gaussians) per block the first pass runs about one block
// per CU and is bound by latency -- of the loads that feed it and of each
// wave's instruction stream -- not by memory bandwidth.  Threads 0..255 own the
// group's Gaussians.  One round of loads goes out at the start: the group's
// tile counts and boxes first, then the raw group sums and digit table (no
// count kernel ran).  The keys need only the counts and boxes: the group's
// emission scan is formed and the first chunk's keys are regenerated from it
// (binary search in LDS) and ranked while the sums and the table are still in
// flight; then each block forms its Gaussians' emission offsets, writes
// offsets[], and workgroup 0 publishes M and the bucket starts.  Each key is
// stored straight from its register: position = the block's next slot of the
// digit + the chunk's keys of the digit in earlier waves (those two summed once
// per wave and digit) + its rank among its wave's keys of the digit (ballots,
// in key order), so the pass is stable.
// (1024 threads per group measured slower: one such block per CU leaves a tail
// once the groups outnumber the CUs.)
constexpr int kWPL = 4;                        // keys per lane per chunk (at most)
constexpr int kWideThreads = 512;             // threads per group: 8 waves (two blocks fit a CU)

template <int NT>
struct WideLds {
    static constexpr int NW = NT / 64;
    SegLds<kBT> G;                             // the group's emission scan and boxes
    uint32_t cnt[NW][256];                     // per wave and digit: the chunk's keys of the digit in the wave,
                                               // then the wave's first output slot of the digit
    uint32_t gbase[256];                       // the block's first output slot of each digit
    uint4 fb[NW][64], ft[NW][64];              // per wave: digit-quad sums of the table (before, all)
    unsigned long long sm64[2 * NW];           // per wave: group sums before this group, all
    uint32_t sm32[NW];                         // per wave: its Gaussians' tile counts
    uint32_t dsum[4];                          // per wave of digits: their total keys
};

// Keys [cs, cs + cc) of the group (cc = min(CH, tot - cs)): each regenerated from the emission scan in
// L.G and ranked among its wave's keys of the same digit (wave-local counts in L.cnt[wave]; no barrier).
template <int NT>
__device__ __forceinline__ void wide_chunk_keys(WideLds<NT> &L, int ns, int first, uint32_t cs, int cc, int span,
                                                int tiles_x, int shift, int bits, uint32_t (&key)[kWPL],
                                                uint32_t (&val)[kWPL], uint32_t (&rk)[kWPL]) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int radix = 1 << bits, iters = span >> 6;
    const uint32_t dmask = (uint32_t)(radix - 1);
    // every slot's search runs (slots past the span repeat the last key; they are not ranked), so the
    // searches' LDS reads overlap instead of waiting on a branch per slot
#pragma unroll
    for (int it = 0; it < kWPL; ++it) {
        const int idx = wave * span + it * 64 + lane;
        int lo;
        regen_pair<kBT>(L.G, ns, cs + (uint32_t)(idx < cc ? idx : cc - 1), tiles_x, key[it], lo);
        val[it] = (uint32_t)(first + lo);
    }
    for (int d = lane; d < radix; d += 64) L.cnt[wave][d] = 0u;
    const uint64_t below = lanes_below();
#pragma unroll
    for (int it = 0; it < kWPL; ++it) {
        if (it >= iters) continue;                        // uniform
        const int idx = wave * span + it * 64 + lane;
        const bool valid = idx < cc;
        const uint32_t d = (key[it] >> shift) & dmask;
        const uint64_t peers = match_digit(d, __ballot(valid));
        const uint32_t before_w = valid ? L.cnt[wave][d] : 0u;
        rk[it] = before_w + (uint32_t)__popcll(peers & below);
        if (valid && (peers >> lane) == 1ull) L.cnt[wave][d] = before_w + (uint32_t)__popcll(peers);
    }
}

// Thread d < radix: each wave's key count of digit d in the chunk (L.cnt[w][d]) replaced by that
// wave's first slot of the digit, from nb (the block's next slot of d), which moves past the chunk.
template <int NT>
__device__ __forceinline__ void wave_starts(WideLds<NT> &L, uint32_t &nb) {
    constexpr int NW = NT / 64;
    const int d = threadIdx.x;
    uint32_t c[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) c[w] = L.cnt[w][d];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        L.cnt[w][d] = nb;
        nb += c[w];
    }
}

template <int NT, int NB>   // NB: table loads per thread, NB * NT * 4 >= the redundant table's entries
__global__ __launch_bounds__(NT, 2048 / NT) void k_scatter0w(int n, int tiles_x, int shift, int bits, int table_redundant,
                                                   int ncols_cap, const uint2 *__restrict__ pixbox,
                                                   uint32_t *__restrict__ offsets, BinHeader *__restrict__ hdr,
                                                   const uint32_t *__restrict__ table, uint32_t *__restrict__ kout,
                                                   uint32_t *__restrict__ vout, uint32_t *__restrict__ bucket_start,
                                                   uint2 *__restrict__ ranges, int ntiles,
                                                   const uint32_t *__restrict__ counts,
                                                   const unsigned long long *__restrict__ part, int ngroups,
                                                   long long capacity, uint32_t *__restrict__ d_num,
                                                   uint32_t *__restrict__ d_max) {
    constexpr int NW = NT / 64, CH = NT * kWPL;
    constexpr int NG = kMaxRedundantGroups / NT;          // group-sum loads per thread
    __shared__ WideLds<NT> L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int radix = 1 << bits;
    const uint32_t dmask = (uint32_t)(radix - 1);
    const int first = blockIdx.x * kBT;
    const int ns = min(kBT, n - first);
    const bool own = tid < ns;
    // one round of loads: counts and boxes first, then the group sums and the table, consumed only
    // after the first chunk's keys are ranked.  Every load is issued unconditionally (in-range index,
    // unused values dropped): with no branch among them, the wait for the counts leaves the rest in
    // flight.
    const int gi = first + (own ? tid : 0);
    const uint32_t c0 = counts[gi];
    const uint2 bx0 = pixbox[gi];
    unsigned long long v[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int i = tid + k * NT;
        v[k] = part[i < ngroups ? i : 0];
    }
    // redundant table: uint4 q of column c holds digits 4 (q mod Q) .. +3, Q = radix / 4; thread t
    // always reads the same 4 digits, from columns t / Q, t / Q + NT / Q, ...; scanned table: the
    // block's base of digit tid
    const int lq = table_redundant ? bits - 2 : 0;
    const int g4 = tid & ((1 << lq) - 1), cstep = NT >> lq, cfirst = tid >> lq;
    const uint4 *t4 = reinterpret_cast<const uint4 *>(table);
    uint4 tv[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        const int col = cfirst + k * cstep;
        tv[k] = t4[table_redundant && col < ncols_cap ? ((uint32_t)col << lq) + (uint32_t)g4 : 0u];
    }
    const uint32_t tx = table[!table_redundant && tid < radix ? (size_t)tid * ncols_cap + blockIdx.x : 0u];
    const uint32_t c = own ? c0 : 0u;
    const uint2 bx = own ? bx0 : make_uint2(0u, 0u);
    // the group's emission scan
    const uint32_t cinc = wave_scan_incl(c);
    if (lane == 63) L.sm32[wave] = cinc;
    __syncthreads();                                      // 1: wave totals of the tile counts
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t x = L.sm32[w];
        off += w < wave ? x : 0u;
        tot += x;
    }
    const uint32_t local = off + cinc - c;
    if (own) {
        L.G.excl[tid] = local;
        L.G.box[tid] = bx;
    }
    if (tid == 0) L.G.excl[ns] = tot;
    __syncthreads();                                      // 2: the emission scan
    // the first chunk's keys, regenerated and ranked (wave-local) while the loads above complete
    uint32_t key[kWPL], val[kWPL], rk[kWPL];
    int cc = (int)min((uint32_t)CH, tot);
    int span = ((cc + NT - 1) / NT) * 64;                 // keys per wave: a multiple of 64, NW * span >= cc
    if (tot > 0u) wide_chunk_keys<NT>(L, ns, first, 0u, cc, span, tiles_x, shift, bits, key, val, rk);
    // the group sums (before this group, all) and the table's digit partials, reduced per wave.  Each
    // sum is split into its low 16 bits and the rest (capped at 2^20: a larger group sum overflows
    // any pair buffer, and the capped total still does); over at most 2048 groups both parts stay
    // within 32 bits, so four DPP wave sums replace 64-bit shuffles.
    const int g = (int)blockIdx.x;
    uint32_t blo = 0, bhi = 0, alo = 0, ahi = 0;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int i = tid + k * NT;
        const unsigned long long x = i < ngroups ? v[k] : 0ull;
        const uint32_t lo = (uint32_t)x & 0xffffu;
        const uint32_t hi = (uint32_t)min(x >> 16, 1ull << 20);
        alo += lo;
        ahi += hi;
        blo += i < g ? lo : 0u;
        bhi += i < g ? hi : 0u;
    }
    blo = wave_scan_incl(blo);
    bhi = wave_scan_incl(bhi);
    alo = wave_scan_incl(alo);
    ahi = wave_scan_incl(ahi);
    if (lane == 63) {
        L.sm64[wave] = ((unsigned long long)bhi << 16) + blo;
        L.sm64[NW + wave] = ((unsigned long long)ahi << 16) + alo;
    }
    const int Q = radix >> 2;                             // digit quads (redundant tables: radix >= 4)
    if (table_redundant) {                                // uniform
        // load k of this wave covers columns [cw0, cw1] + k cstep (cw1 - cw0 < cstep): rounds within
        // the table and before this group are added whole (wave-uniform tests); the columns before
        // this group are a prefix of the rounds, so their sum is the running total taken once, at
        // the first round that reaches the group, plus that round's lanes before it
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        const int cw0 = (wv * 64) >> lq, cw1 = (wv * 64 + 63) >> lq;
        uint4 fb = make_uint4(0u, 0u, 0u, 0u), ft = fb;
        bool taken = false;                               // wave-uniform: fb is final
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int a0 = cw0 + k * cstep, a1 = cw1 + k * cstep, col = cfirst + k * cstep;
            if (a0 >= ncols_cap) break;                   // uniform
            uint4 x = tv[k];
            if (a1 >= ncols_cap) {                        // uniform: the round that crosses the table's end
                const bool in = col < ncols_cap;
                x.x = in ? x.x : 0u; x.y = in ? x.y : 0u; x.z = in ? x.z : 0u; x.w = in ? x.w : 0u;
            }
            if (!taken && a1 >= g) {                      // uniform: the first round that reaches this group
                fb = ft;
                if (a0 < g) {
                    const bool bf = col < g;
                    fb.x += bf ? x.x : 0u; fb.y += bf ? x.y : 0u; fb.z += bf ? x.z : 0u; fb.w += bf ? x.w : 0u;
                }
                taken = true;
            }
            ft.x += x.x; ft.y += x.y; ft.z += x.z; ft.w += x.w;
        }
        if (!taken) fb = ft;                              // every column of the wave is before this group
        // lanes with equal lane mod Q hold the same digits
        for (int o = Q; o < 64; o <<= 1) {
            fb.x += __shfl_xor(fb.x, o, 64); fb.y += __shfl_xor(fb.y, o, 64);
            fb.z += __shfl_xor(fb.z, o, 64); fb.w += __shfl_xor(fb.w, o, 64);
            ft.x += __shfl_xor(ft.x, o, 64); ft.y += __shfl_xor(ft.y, o, 64);
            ft.z += __shfl_xor(ft.z, o, 64); ft.w += __shfl_xor(ft.w, o, 64);
        }
        if (lane < Q) {
            L.fb[wave][lane] = fb;
            L.ft[wave][lane] = ft;
        }
    }
    __syncthreads();                                      // 3: sums, table partials and the waves' key counts
    unsigned long long tb = 0, ta = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        tb += L.sm64[w];
        ta += L.sm64[NW + w];
    }
    if (own) offsets[first + tid] = sat32(tb + local);
    if (blockIdx.x == 0 && tid == 0) publish_total(ta, capacity, n, hdr, offsets, d_num, d_max);
    const uint32_t M = ta <= (unsigned long long)capacity ? (uint32_t)ta : 0u;   // else nothing is emitted
    if (M == 0u) return;                                  // overflow or no pair: uniform
    // digit bases: gbase[d] = (keys of smaller digits, all groups) + (keys of d in earlier groups);
    // nb: (thread d < radix) the block's next slot of digit d
    uint32_t nb = 0u;
    if (table_redundant) {                                // uniform
        uint32_t sb = 0, st = 0;
        if (tid < radix) {
            const uint32_t *pb = reinterpret_cast<const uint32_t *>(&L.fb[0][0]);
            const uint32_t *pt = reinterpret_cast<const uint32_t *>(&L.ft[0][0]);
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                sb += pb[(w * 64 + (tid >> 2)) * 4 + (tid & 3)];
                st += pt[(w * 64 + (tid >> 2)) * 4 + (tid & 3)];
            }
        }
        const uint32_t dinc = wave_scan_incl(st);         // digits tid (< 256) sit in waves 0..3
        if (wave < 4 && lane == 63) L.dsum[wave] = dinc;
        __syncthreads();                                  // 4: digit totals per wave
        if (tid < radix) {
            uint32_t dbase = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) dbase += w < wave ? L.dsum[w] : 0u;
            nb = dbase + dinc - st + sb;
        }
    } else {
        nb = tx;                                          // the scanned table holds the bases
    }
    if (tid < radix) {
        L.gbase[tid] = nb;
        wave_starts<NT>(L, nb);
    }
    __syncthreads();                                      // 5: gbase and the waves' first slots
    if (blockIdx.x == 0) {
        if (tid < radix) bucket_start[tid] = L.gbase[tid];
        if (tid == 0) bucket_start[radix] = M;
        if (ranges && tid < radix && tid < ntiles) {
            const uint32_t a = L.gbase[tid], e = tid + 1 < radix ? L.gbase[tid + 1] : M;
            ranges[tid] = e > a ? make_uint2(a, e) : make_uint2(0u, 0u);
        }
    }
    for (uint32_t cs = 0; cs < tot;) {                    // the chunk's keys are ranked and the counts published
        const int iters = span >> 6;
        // position = the wave's first slot of the digit + the rank
#pragma unroll
        for (int it = 0; it < kWPL; ++it) {
            if (it >= iters) continue;                    // uniform
            const int idx = wave * span + it * 64 + lane;
            if (idx < cc) {
                const uint32_t d = (key[it] >> shift) & dmask;
                const uint32_t pos = L.cnt[wave][d] + rk[it];
                if (pos < M) {                            // holds by construction; keeps a bad table in bounds
                    kout[pos] = key[it];
                    vout[pos] = val[it];
                }
            }
        }
        cs += (uint32_t)CH;
        if (cs >= tot) break;                             // uniform: the last chunk
        __syncthreads();                                  // every wave has its positions: the rows are free
        cc = (int)min((uint32_t)CH, tot - cs);
        span = ((cc + NT - 1) / NT) * 64;
        wide_chunk_keys<NT>(L, ns, first, cs, cc, span, tiles_x, shift, bits, key, val, rk);
        __syncthreads();                                  // the waves' counts
        if (tid < radix) wave_starts<NT>(L, nb);
        __syncthreads();                                  // the waves' first slots
    }
}

// ---------------------------------------------------------------------------
// 5b: the bucket pass with 16 waves per bucket
// ---------------------------------------------------------------------------
// One block of 1024 threads per high digit: buckets are few (64 at 1020x678)
// and each holds thousands of keys, so a 4-wave block per bucket leaves most
// CUs idle and walks its keys in several rounds.  Keys sit 8 per lane (8192 per
// chunk); each wave ranks its span of the chunk by the low digit with ballots
// (in key order), and key position = the digit's next slot in the bucket + the
// chunk's keys of the digit in earlier waves + the rank: stable, stored straight
// from the registers.  The digit totals of the bucket are its tiles' ranges.
constexpr int kBWT = 1024, kBWW = kBWT / 64, kBWPL = 8;
struct BucketWLds {
    uint32_t cnt[kBWW][256];      // per wave and digit: the chunk's keys of the digit in the wave, then
                                  // in earlier waves (exclusive prefix over the waves)
    uint32_t gbase[256];          // next output slot of each digit
    uint32_t hist[256];           // the bucket's keys per digit (buckets of several chunks)
    uint32_t dsum[4];             // per wave of digits: their total
    uint32_t ldo[256];            // buckets of several chunks: each digit's first slot in the chunk's reorder
    uint32_t sk[kBWT * kBWPL], sv[kBWT * kBWPL];   // ... and the reordered chunk (digit-major, stable)
};

// Ranks of a chunk's keys (wave-local counts into L.cnt); ends with the barrier that publishes them.
__device__ __forceinline__ void bucketw_rank(BucketWLds &L, int cc, int span, int iters, int lo_bits,
                                             const uint32_t (&key)[kBWPL], uint32_t (&rk)[kBWPL]) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int radix = 1 << lo_bits;
    const uint32_t dmask = (uint32_t)(radix - 1);
    const uint64_t below = lanes_below();
    for (int d = lane; d < radix; d += 64) L.cnt[wave][d] = 0u;
#pragma unroll
    for (int it = 0; it < kBWPL; ++it) {
        if (it >= iters) continue;                        // uniform
        const int idx = wave * span + it * 64 + lane;
        const bool valid = idx < cc;
        const uint32_t d = key[it] & dmask;
        const uint64_t peers = match_digit(d, __ballot(valid));
        const uint32_t before = valid ? L.cnt[wave][d] : 0u;
        rk[it] = before + (uint32_t)__popcll(peers & below);
        if (valid && (peers >> lane) == 1ull) L.cnt[wave][d] = before + (uint32_t)__popcll(peers);
    }
    __syncthreads();
}

// gbase[d] = s0 + exclusive scan of tot over the digits (threads < radix hold tot), and the tiles'
// ranges.  Two barriers; gbase is published on return.
__device__ __forceinline__ void bucketw_bases(BucketWLds &L, uint32_t tot, uint32_t s0, int lo_bits, int ntiles,
                                              uint2 *__restrict__ ranges) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int radix = 1 << lo_bits;
    const uint32_t inc = wave_scan_incl(tot);             // digits (< 256) sit in waves 0..3
    if (wave < 4 && lane == 63) L.dsum[wave] = inc;
    __syncthreads();
    if (tid < radix) {
        uint32_t ex = inc - tot;
#pragma unroll
        for (int w = 0; w < 4; ++w) ex += w < wave ? L.dsum[w] : 0u;
        L.gbase[tid] = s0 + ex;
        const int t = (blockIdx.x << lo_bits) + tid;
        if (t < ntiles) ranges[t] = tot ? make_uint2(s0 + ex, s0 + ex + tot) : make_uint2(0u, 0u);
    }
    __syncthreads();
}

__global__ __launch_bounds__(kBWT) void k_bucket_sortw(const uint32_t *__restrict__ kin, const uint32_t *__restrict__ vin,
                                                       uint32_t *__restrict__ kout, uint32_t *__restrict__ vout,
                                                       const BinHeader *__restrict__ hdr,
                                                       const uint32_t *__restrict__ bucket_start, int lo_bits,
                                                       int ntiles, uint2 *__restrict__ ranges) {
    constexpr uint32_t CH = (uint32_t)kBWT * kBWPL;
    __shared__ BucketWLds L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int radix = 1 << lo_bits;
    const uint32_t dmask = (uint32_t)(radix - 1);
    const uint32_t M = hdr->m_eff;
    const uint32_t s0 = M ? bucket_start[blockIdx.x] : 0u, s1 = M ? bucket_start[blockIdx.x + 1] : 0u;
    if (s1 == s0) return;                                 // uniform: its tiles keep the cleared (0, 0)
    const bool one = s1 - s0 <= CH;                       // uniform
    if (!one) {                                           // the bucket's digit totals first
        if (tid < radix) L.hist[tid] = 0u;
        __syncthreads();
        for (uint32_t base = s0; base < s1; base += CH) {
            uint32_t k[kBWPL];
#pragma unroll
            for (int it = 0; it < kBWPL; ++it) {
                const uint32_t idx = base + it * kBWT + tid;
                k[it] = kin[idx < s1 ? idx : s1 - 1];
            }
#pragma unroll
            for (int it = 0; it < kBWPL; ++it)
                if (base + it * kBWT + tid < s1) atomicAdd(&L.hist[k[it] & dmask], 1u);
        }
        __syncthreads();
        bucketw_bases(L, tid < radix ? L.hist[tid] : 0u, s0, lo_bits, ntiles, ranges);
    }
    for (uint32_t base = s0; base < s1; base += CH) {    // uniform
        const int cc = (int)min(CH, s1 - base);
        const int span = ((cc + kBWT - 1) / kBWT) * 64;   // keys per wave: a multiple of 64, 16 * span >= cc
        const int iters = span >> 6;
        uint32_t key[kBWPL], val[kBWPL], rk[kBWPL];
#pragma unroll
        for (int it = 0; it < kBWPL; ++it) {
            if (it < iters) {                             // uniform
                const int idx = wave * span + it * 64 + lane;
                const uint32_t q = base + (uint32_t)(idx < cc ? idx : cc - 1);
                key[it] = kin[q];
                val[it] = vin[q];
            }
        }
        bucketw_rank(L, cc, span, iters, lo_bits, key, rk);
        // per digit, the chunk's keys in earlier waves: an exclusive prefix over the waves, in place
        uint32_t tot = 0;
        if (tid < radix)
#pragma unroll
            for (int w = 0; w < kBWW; ++w) {
                const uint32_t c = L.cnt[w][tid];
                L.cnt[w][tid] = tot;
                tot += c;
            }
        if (one) {                                        // the chunk is the bucket: its counts give the bases
            bucketw_bases(L, tot, s0, lo_bits, ntiles, ranges);   // (its barriers publish the prefix)
            // reordered in LDS (digit-major, stable), then the bucket goes out as one run
#pragma unroll
            for (int it = 0; it < kBWPL; ++it) {
                if (it >= iters) continue;                // uniform
                const int idx = wave * span + it * 64 + lane;
                if (idx < cc) {
                    const uint32_t d = key[it] & dmask;
                    const uint32_t loc = L.gbase[d] - s0 + L.cnt[wave][d] + rk[it];   // < cc by construction
                    L.sk[loc] = key[it];
                    L.sv[loc] = val[it];
                }
            }
            __syncthreads();
            for (int i = tid; i < cc; i += kBWT) {
                kout[s0 + (uint32_t)i] = L.sk[i];
                vout[s0 + (uint32_t)i] = L.sv[i];
            }
        } else {
            // a chunk of a big bucket is reordered in LDS (digit-major, stable) and written out as
            // runs: consecutive threads store consecutive slots
            const uint32_t inc = wave_scan_incl(tot);     // digits (< 256) sit in waves 0..3
            if (wave < 4 && lane == 63) L.dsum[wave] = inc;
            __syncthreads();
            if (tid < radix) {
                uint32_t ex = inc - tot;
#pragma unroll
                for (int w = 0; w < 4; ++w) ex += w < wave ? L.dsum[w] : 0u;
                L.ldo[tid] = ex;
            }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < kBWPL; ++it) {
                if (it >= iters) continue;                // uniform
                const int idx = wave * span + it * 64 + lane;
                if (idx < cc) {
                    const uint32_t d = key[it] & dmask;
                    const uint32_t loc = L.ldo[d] + L.cnt[wave][d] + rk[it];   // < cc by construction
                    L.sk[loc] = key[it];
                    L.sv[loc] = val[it];
                }
            }
            __syncthreads();
            for (int i = tid; i < cc; i += kBWT) {
                const uint32_t k = L.sk[i], d = k & dmask;
                const uint32_t pos = L.gbase[d] + ((uint32_t)i - L.ldo[d]);
                if (pos < s1) {
                    kout[pos] = k;
                    vout[pos] = L.sv[i];
                }
            }
        }
        if (base + CH >= s1) break;                       // uniform: the last chunk
        __syncthreads();                                  // every wave has its positions
        if (tid < radix) L.gbase[tid] += tot;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// 5: further passes over blocks of 256 * PL keys
// ---------------------------------------------------------------------------
template <int PL>
__global__ __launch_bounds__(kBT) void k_count(const uint32_t *__restrict__ keys, const BinHeader *__restrict__ hdr,
                                               int shift, int bits, int table_redundant, int ncols_cap,
                                               uint32_t *__restrict__ table) {
    constexpr int CH = kBT * PL;
    __shared__ uint32_t h[256];
    const int radix = 1 << bits;
    const int tid = threadIdx.x;
    if (tid < radix) h[tid] = 0u;
    __syncthreads();
    const uint32_t M = hdr->m_eff;
    const uint32_t base = blockIdx.x * (uint32_t)CH;
    if (base < M) {                                               // uniform
        uint32_t k[PL];
#pragma unroll
        for (int it = 0; it < PL; ++it) {
            const uint32_t idx = base + it * kBT + tid;
            k[it] = keys[idx < M ? idx : M - 1];
        }
#pragma unroll
        for (int it = 0; it < PL; ++it)
            if (base + it * kBT + tid < M) atomicAdd(&h[(k[it] >> shift) & (radix - 1)], 1u);
    }
    __syncthreads();
    if (tid < radix) {                                            // zero columns past M too
        if (table_redundant) table[(size_t)blockIdx.x * radix + tid] = h[tid];
        else table[(size_t)tid * ncols_cap + blockIdx.x] = h[tid];
    }
}

template <int PL>
__global__ __launch_bounds__(kBT) void k_scatter(const uint32_t *__restrict__ kin, const uint32_t *__restrict__ vin,
                                                 uint32_t *__restrict__ kout, uint32_t *__restrict__ vout,
                                                 const BinHeader *__restrict__ hdr, int shift, int bits,
                                                 int table_redundant, int ncols_cap,
                                                 const uint32_t *__restrict__ table) {
    constexpr int CH = kBT * PL, SPAN = PL * 64;
    __shared__ ChunkLds<PL> L;
    __shared__ BaseLds B;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint32_t base = blockIdx.x * (uint32_t)CH;
    const uint32_t M = hdr->m_eff;
    if (base >= M) return;                                        // uniform
    // the block's keys and the digit table in one round of loads
    uint32_t key[PL], val[PL];
#pragma unroll
    for (int it = 0; it < PL; ++it) {
        const uint32_t idx = base + wave * SPAN + it * 64 + lane;
        const uint32_t ii = idx < M ? idx : M - 1;
        key[it] = kin[ii];
        val[it] = vin[ii];
    }
    const DigitAcc acc = digit_load(table, table_redundant, ncols_cap, blockIdx.x, bits);
    digit_finish(acc, table_redundant, bits, L.gbase, B);
    const int cc = (int)min((uint32_t)CH, M - base);
    scatter_chunk(L, cc, SPAN, shift, bits, key, val, kout, vout, M, true);
}

// ---------------------------------------------------------------------------
// 5': second pass of the most-significant-digit order (keys up to 16 bits)
// ---------------------------------------------------------------------------
// One workgroup per bucket (pairs whose tile ids share the high digit, in
// emission order after the first pass): it counts the low digits, writes the
// ranges of the bucket's 2^lo tiles straight from those counts, and scatters
// the bucket stably by the low digit, 256 * PL pairs at a time.
template <int PL>
__global__ __launch_bounds__(kBT) void k_bucket_sort(const uint32_t *__restrict__ kin, const uint32_t *__restrict__ vin,
                                                     uint32_t *__restrict__ kout, uint32_t *__restrict__ vout,
                                                     const BinHeader *__restrict__ hdr,
                                                     const uint32_t *__restrict__ bucket_start, int lo_bits,
                                                     int ntiles, uint2 *__restrict__ ranges) {
    constexpr int CH = kBT * PL;
    __shared__ ChunkLds<PL> L;
    __shared__ uint32_t hist[256];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int radix = 1 << lo_bits;
    const uint32_t M = hdr->m_eff;
    const uint32_t s0 = M ? bucket_start[blockIdx.x] : 0u, s1 = M ? bucket_start[blockIdx.x + 1] : 0u;
    if (s1 - s0 <= (uint32_t)CH) {                                // uniform: the bucket is one chunk
        if (s1 == s0) return;                                     // its tiles keep the cleared (0, 0)
        const int cc = (int)(s1 - s0);
        const int span = ((cc + kBT - 1) / kBT) * 64;
        const int iters = span >> 6;
        uint32_t key[PL], val[PL];
#pragma unroll
        for (int it = 0; it < PL; ++it) {
            if (it < iters) {
                const int idx = wave * span + it * 64 + lane;
                const uint32_t q = s0 + (uint32_t)(idx < cc ? idx : cc - 1);
                key[it] = kin[q];
                val[it] = vin[q];
            }
        }
        scatter_chunk<PL, kDirectScatter>(L, cc, span, 0, lo_bits, key, val, kout, vout, M, true, s0);
        if (tid < radix) {                                        // the digit starts are the tile ranges
            const int t = (blockIdx.x << lo_bits) + tid;
            const uint32_t a = L.dstart[tid], e = tid + 1 < radix ? L.dstart[tid + 1] : (uint32_t)cc;
            if (t < ntiles) ranges[t] = e > a ? make_uint2(s0 + a, s0 + e) : make_uint2(0u, 0u);
        }
        return;
    }
    if (tid < radix) hist[tid] = 0u;
    __syncthreads();
    for (uint32_t base = s0; base < s1; base += CH) {            // uniform
        uint32_t k[PL];
#pragma unroll
        for (int it = 0; it < PL; ++it) {
            const uint32_t idx = base + it * kBT + tid;
            k[it] = kin[idx < s1 ? idx : s1 - 1];
        }
#pragma unroll
        for (int it = 0; it < PL; ++it)
            if (base + it * kBT + tid < s1) atomicAdd(&hist[k[it] & (uint32_t)(radix - 1)], 1u);
    }
    __syncthreads();
    const uint32_t c = tid < radix ? hist[tid] : 0u;
    uint32_t all;
    const uint32_t ex = block_exclusive_scan<uint32_t, kBT>(c, L.sm, &all);
    if (tid < radix) {
        const int t = (blockIdx.x << lo_bits) + tid;
        if (t < ntiles) ranges[t] = c ? make_uint2(s0 + ex, s0 + ex + c) : make_uint2(0u, 0u);
        L.gbase[tid] = s0 + ex;
    }
    __syncthreads();
    for (uint32_t base = s0; base < s1; base += CH) {            // uniform
        const int cc = (int)min((uint32_t)CH, s1 - base);
        const int span = ((cc + kBT - 1) / kBT) * 64;
        const int iters = span >> 6;
        uint32_t key[PL], val[PL];
#pragma unroll
        for (int it = 0; it < PL; ++it) {
            if (it < iters) {
                const int idx = wave * span + it * 64 + lane;
                const uint32_t q = base + (uint32_t)(idx < cc ? idx : cc - 1);
                key[it] = kin[q];
                val[it] = vin[q];
            }
        }
        scatter_chunk(L, cc, span, 0, lo_bits, key, val, kout, vout, M, base + (uint32_t)CH >= s1);
    }
}

// ---------------------------------------------------------------------------
// exclusive scan of a u32 array in place (large digit tables): one workgroup
// when it is short, otherwise block totals -> rescan, each rescan block adding
// up the totals before it (a scan of the totals in between only past
// kScanDownSums blocks).
// count <= 1024 * kScanSingleItems for the single form.  Element r * 1024 + i
// lives in thread i's register v[r] (coalesced loads, all issued together).
// ---------------------------------------------------------------------------
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
        if (r < rows) {                   // uniform over the block
            inc[r] = wave_scan_incl(v[r]);
            if (lane == 63) wsum[wave][r] = inc[r];
        }
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
        const int e = r * 1024 + tid;
        if (r < rows && e < count) a[e] = rowpre[r] + wsum[wave][r] + inc[r] - v[r];
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

// RAW: sums[] holds the raw block totals of k_scan_reduce and each block adds up those before it
// itself (at most kScanDownSums of them; no scan of the totals runs in between); else sums[] is
// their exclusive scan.
constexpr int kScanDownSums = 4 * 256;
template <bool RAW>
__global__ __launch_bounds__(256) void k_scan_down(uint32_t *__restrict__ a, int count,
                                                   const uint32_t *__restrict__ sums) {
    __shared__ uint32_t sm[4], pre[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int beg = blockIdx.x * kScanChunk + threadIdx.x * kScanItems;
    uint32_t b = 0;                                       // RAW: totals of the blocks before this one
    if (RAW) {
#pragma unroll
        for (int k = 0; k < kScanDownSums / 256; ++k) {
            const int j = threadIdx.x + k * 256;
            b += j < (int)blockIdx.x ? sums[j] : 0u;
        }
    }
    uint32_t v[kScanItems];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        v[i] = (beg + i < count) ? a[beg + i] : 0u;
        s += v[i];
    }
    // one barrier: the wave totals of s (for the scan) and of b (for the block's base)
    const uint32_t sinc = wave_scan_incl(s);
    const uint32_t binc = RAW ? wave_scan_incl(b) : 0u;
    if (lane == 63) {
        sm[wave] = sinc;
        pre[wave] = binc;
    }
    __syncthreads();
    uint32_t run = sinc - s;
#pragma unroll
    for (int w = 0; w < 4; ++w) run += (w < wave ? sm[w] : 0u) + (RAW ? pre[w] : 0u);
    if (!RAW) run += sums[blockIdx.x];
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
    if (nb > kScanDownSums) {                             // (beyond 4M entries) scan the block totals first
        k_scan_single<<<1, 1024, 0, s>>>(sums, nb);
        k_scan_down<false><<<nb, 256, 0, s>>>(a, count, sums);
        return hipGetLastError();
    }
    k_scan_down<true><<<nb, 256, 0, s>>>(a, count, sums);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 6: tile ranges
// ---------------------------------------------------------------------------
// Four sorted pairs per thread: a key that differs from its predecessor opens
// its tile's run and closes the predecessor's (the ranges were cleared by
// k_group_sums).
__global__ __launch_bounds__(256) void k_ranges(const uint32_t *__restrict__ keys, const BinHeader *__restrict__ hdr,
                                                uint32_t ntiles, uint32_t *__restrict__ ranges) {
    const uint32_t i0 = (blockIdx.x * 256u + threadIdx.x) * 4u;
    const uint32_t M = hdr->m_eff;
    if (i0 >= M) return;
    uint32_t k[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = min(keys[i0 + j < M ? i0 + j : M - 1], ntiles - 1);   // ids are < ntiles
    uint32_t prev = i0 > 0 ? min(keys[i0 - 1], ntiles - 1) : 0xffffffffu;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t i = i0 + j;
        if (i < M) {
            if (k[j] != prev) {
                ranges[2 * k[j]] = i;
                if (i > 0) ranges[2 * prev + 1] = i;
            }
            if (i + 1 == M) ranges[2 * k[j] + 1] = M;
            prev = k[j];
        }
    }
}

// ---------------------------------------------------------------------------
// 7: tile order (longest list first)
// ---------------------------------------------------------------------------
// A counting sort of the tiles by list length, one workgroup of 1024: lengths
// of 1023 or more share the first bucket, and tiles of equal bucket land in no
// particular order (the order only schedules work: every tile's results are
// its own, whatever the order).
// Launch position of the tile of sorted rank p: ranks are dealt in layers of
// `period` positions (the CU count: the hardware deals consecutive workgroups
// round-robin over the CUs), reversed in every odd layer, so that each CU's
// workgroups mix long and short lists when the whole grid is resident.
__device__ __forceinline__ uint32_t serpentine(uint32_t p, uint32_t period, uint32_t n) {
    const uint32_t layer = p / period, c = p - layer * period;
    const uint32_t base = layer * period, width = min(period, n - base);
    return base + ((layer & 1u) ? width - 1u - c : c);
}

__global__ __launch_bounds__(1024) void k_tile_order(const uint2 *__restrict__ ranges, int ntiles, int period,
                                                     uint32_t *__restrict__ order) {
    __shared__ uint32_t hist[1024];
    __shared__ uint32_t sm[16];
    const int tid = threadIdx.x;
    hist[tid] = 0u;
    __syncthreads();
    for (int t = tid; t < ntiles; t += 1024) {
        const uint2 r = ranges[t];
        const uint32_t len = r.y > r.x ? r.y - r.x : 0u;
        atomicAdd(&hist[1023u - min(len, 1023u)], 1u);
    }
    __syncthreads();
    const uint32_t h = hist[tid];
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<uint32_t, 1024>(h, sm, &tot);
    hist[tid] = ex;
    __syncthreads();
    for (int t = tid; t < ntiles; t += 1024) {
        const uint2 r = ranges[t];
        const uint32_t len = r.y > r.x ? r.y - r.x : 0u;
        const uint32_t rank = atomicAdd(&hist[1023u - min(len, 1023u)], 1u);
        order[serpentine(rank, (uint32_t)period, (uint32_t)ntiles)] = (uint32_t)t;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// CUs of the current device (cached per device; 256 if the query fails).
static int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

BinPlan make_bin_plan(int n, int W, int H, int64_t capacity) {
    BinPlan p{};
    p.n = n; p.W = W; p.H = H;
    p.tiles_x = (W + kTile - 1) / kTile;
    const int tiles_y = (H + kTile - 1) / kTile;
    p.ntiles = p.tiles_x * tiles_y;
    p.capacity = capacity;
    int B = 0;
    while ((1ll << B) < (long long)p.ntiles) ++B;          // key bits: ids in [0, ntiles)
    p.nb_g = (n + 255) / 256;
    p.redundant_groups = p.nb_g > 0 && p.nb_g <= kMaxRedundantGroups;
    p.seg_groups = p.nb_g <= kMaxRedundantGroups ? 1 : 4;
    p.nseg = (p.nb_g + p.seg_groups - 1) / p.seg_groups;
    auto redundant_ok = [&](int bits, int cols) {
        const size_t entries = ((size_t)1 << bits) * (size_t)(cols > 0 ? cols : 1);
        return bits >= 2 && entries <= (size_t)kMaxRedundantTable && (int64_t)entries * cols <= kMaxRedundantReads;
    };
    for (int i = 0; i < 4; ++i) p.bits[i] = 0;
    p.shift0 = 0;
    p.lo_bits = 0;
    if (B <= 8) {                            // one pass sorts the whole key
        p.order_kind = 0;
        p.passes = 1;
        p.bits[0] = B;
    } else if (B <= 16 && capacity <= kMaxBucketCapacity) {   // high digit first, then a workgroup per bucket
        p.order_kind = 1;
        p.passes = 1;
        const int lo_min = B - 8 > 1 ? B - 8 : 1;          // high digit <= 8 bits, low digit >= 1 bit
        int hi = B - 3 < 8 ? B - 3 : 8;
        if (hi < lo_min) hi = lo_min;
        // fewer buckets if that lets the first pass skip its scan kernels
        for (int h = hi; h >= lo_min && !redundant_ok(hi, p.nseg); --h)
            if (redundant_ok(h, p.nseg)) hi = h;
        p.bits[0] = hi;
        p.lo_bits = B - hi;
        p.shift0 = p.lo_bits;
        const int64_t per_bucket = capacity / 2 / ((int64_t)1 << hi);      // capacity holds ~2x slack
        p.bucket_lanes = per_bucket <= 1024 ? 4 : per_bucket <= 2048 ? 8 : 16;
    } else {                                 // LSD passes of <= 8 bits
        p.order_kind = 2;
        p.passes = (B + 7) / 8;
        const int w = (B + p.passes - 1) / p.passes;
        int left = B;
        for (int i = 0; i < p.passes; ++i) { p.bits[i] = left < w ? left : w; left -= p.bits[i]; }
    }
    // later LSD passes: smaller blocks when the pair buffer is small, so the launch still fills the chip
    p.pass_lanes = capacity <= (1ll << 19) ? 4 : capacity <= (1ll << 22) ? 8 : 16;
    const int64_t chunk = (int64_t)kBT * p.pass_lanes;
    p.nbs = (int)((capacity + chunk - 1) / chunk);
    size_t table = 1;
    for (int i = 0; i < p.passes; ++i) {
        const int cols = i == 0 ? p.nseg : p.nbs;
        p.ncols_cap[i] = cols;
        const size_t entries = ((size_t)1 << p.bits[i]) * (size_t)(cols > 0 ? cols : 1);
        p.table_redundant[i] = redundant_ok(p.bits[i], cols);
        if (entries > table) table = entries;
    }
    size_t off = align256(sizeof(BinHeader));
    p.off_part = off; off = align256(off + sizeof(unsigned long long) * (size_t)(p.nb_g > 0 ? p.nb_g : 1));
    p.off_kalt = off; off = align256(off + sizeof(uint32_t) * (size_t)(capacity > 0 ? capacity : 1));
    p.off_valt = off; off = align256(off + sizeof(uint32_t) * (size_t)(capacity > 0 ? capacity : 1));
    p.off_table = off; off = align256(off + sizeof(uint32_t) * table);
    p.off_tsp = off; off = align256(off + sizeof(uint32_t) * ((table + kScanChunk - 1) / kScanChunk + 1));
    p.off_bstart = off; off = align256(off + sizeof(uint32_t) * 260);
    p.bytes = off;
    return p;
}

const void *bin_total_ptr(const void *ws) { return &static_cast<const BinHeader *>(ws)->total; }

unsigned long long *bin_group_sums(const BinPlan &p, void *ws) {
    return reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + p.off_part);
}

BinHist bin_hist(const BinPlan &p, void *ws) {
    BinHist h{};
    if (p.n > 0 && p.seg_groups == 1 && p.redundant_groups) {
        h.table = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + p.off_table);
        h.tiles_x = p.tiles_x;
        h.shift = p.shift0;
        h.bits = p.bits[0];
        h.redundant = p.table_redundant[0];
        h.ncols_cap = p.ncols_cap[0];
    }
    return h;
}

bool bucket_list_mode(const BinPlan &p) { return p.n > 0 && p.order_kind == 1 && p.lo_bits <= 4; }

BucketList bin_bucket_list(const BinPlan &p, void *ws, uint32_t *keys, uint32_t *vals, uint32_t *ranges) {
    char *w = static_cast<char *>(ws);
    BucketList b{};
    b.kin = reinterpret_cast<const uint32_t *>(w + p.off_kalt);
    b.vin = reinterpret_cast<const uint32_t *>(w + p.off_valt);
    b.bstart = reinterpret_cast<const uint32_t *>(w + p.off_bstart);
    b.m_eff = &reinterpret_cast<const BinHeader *>(w)->m_eff;
    b.lo_bits = p.lo_bits;
    b.kout = keys;
    b.vout = vals;
    b.ranges = ranges;
    return b;
}

hipError_t launch_tile_order(const BinPlan &p, const uint32_t *ranges, uint32_t *tile_order, hipStream_t s) {
    k_tile_order<<<1, 1024, 0, s>>>(reinterpret_cast<const uint2 *>(ranges), p.ntiles, device_cus(), tile_order);
    return hipGetLastError();
}

// k_scatter0w with NT threads per group and the fewest table loads per thread that cover `entries`
// table entries.
template <int NT, typename... Args>
static void launch_scatter0w_nt(int64_t entries, int blocks, hipStream_t s, Args... args) {
    if (entries <= 4 * NT * 4) k_scatter0w<NT, 4><<<blocks, NT, 0, s>>>(args...);
    else if (entries <= 8 * NT * 4) k_scatter0w<NT, 8><<<blocks, NT, 0, s>>>(args...);
    else k_scatter0w<NT, (kMaxRedundantTable + 4 * NT - 1) / (4 * NT)><<<blocks, NT, 0, s>>>(args...);
}
template <typename... Args>
static void launch_scatter0w(int64_t entries, int blocks, hipStream_t s, Args... args) {
    launch_scatter0w_nt<kWideThreads>(entries, blocks, s, args...);
}

hipError_t launch_bin_sort(const BinPlan &p, const uint16_t *pixbox, const uint32_t *counts, uint32_t *offsets,
                           uint32_t *keys, uint32_t *vals, uint32_t *ranges, uint32_t *tile_order, uint32_t *d_num,
                           void *ws, hipStream_t s, bool groups_done, bool first_pass_only, uint32_t *d_max) {
    char *w = static_cast<char *>(ws);
    BinHeader *hdr = reinterpret_cast<BinHeader *>(w);
    unsigned long long *part = reinterpret_cast<unsigned long long *>(w + p.off_part);
    uint32_t *kalt = reinterpret_cast<uint32_t *>(w + p.off_kalt);
    uint32_t *valt = reinterpret_cast<uint32_t *>(w + p.off_valt);
    uint32_t *table = reinterpret_cast<uint32_t *>(w + p.off_table);
    uint32_t *tsp = reinterpret_cast<uint32_t *>(w + p.off_tsp);
    uint32_t *bstart = reinterpret_cast<uint32_t *>(w + p.off_bstart);
    const uint2 *box = reinterpret_cast<const uint2 *>(pixbox);
    uint2 *rg = reinterpret_cast<uint2 *>(ranges);
    const bool lsd = p.order_kind == 2;
    // the tile order when one is asked for (also for n == 0 or capacity == 0)
    auto finish = [&]() -> hipError_t {
        if (tile_order)
            k_tile_order<<<1, 1024, 0, s>>>(rg, p.ntiles, device_cus(), tile_order);
        return hipGetLastError();
    };

    // Segments of one group with the group sums read raw: the counting step is
    // folded into the kernel that forms the group sums (this one, or the
    // preprocess kernel) and the first scatter forms the offsets itself.
    const BinHist hist = bin_hist(p, ws);
    const bool folded = hist.table != nullptr;
    if (!groups_done || p.n == 0)
        k_group_sums<<<p.nb_g > 0 ? p.nb_g : 1, kBT, 0, s>>>(p.n, counts, box, part, p.ntiles, rg, hdr, offsets,
                                                            d_num, hist, d_max);
    if (p.n == 0) return finish();
    hipError_t e;
    if (!folded) {
        if (!p.redundant_groups)
            k_group_scan<<<1, 1024, 0, s>>>(p.nb_g, p.n, (long long)p.capacity, part, hdr, offsets, d_num, d_max);
        k_count0<<<p.nseg, kBT, 0, s>>>(p.n, p.nb_g, p.seg_groups, p.redundant_groups, (long long)p.capacity,
                                        p.tiles_x, p.shift0, p.bits[0], p.table_redundant[0], p.ncols_cap[0],
                                        counts, box, part, hdr, offsets, d_num, table, d_max);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p.capacity == 0) return finish();
    }
    if (!p.table_redundant[0]) {
        e = scan_u32(table, (1 << p.bits[0]) * p.ncols_cap[0], tsp, s);
        if (e != hipSuccess) return e;
    }
    // destination of the first pass: the final arrays unless another pass follows
    uint32_t *k0 = keys, *v0 = vals;
    if (p.order_kind == 1 || (lsd && (p.passes & 1) == 0)) { k0 = kalt; v0 = valt; }
    uint2 *rg0 = p.order_kind == 0 ? rg : nullptr;
    if (folded)             // also when capacity == 0: it publishes offsets and M
        launch_scatter0w(p.table_redundant[0] ? (int64_t)p.ncols_cap[0] << p.bits[0] : 0, p.nseg, s,
            p.n, p.tiles_x, p.shift0, p.bits[0], p.table_redundant[0], p.ncols_cap[0], box, offsets, hdr, table, k0,
            v0, bstart, rg0, p.ntiles, counts, part, p.nb_g, (long long)p.capacity, d_num, d_max);
    else                    // not folded: more than kMaxRedundantGroups groups, segments of 4
        k_scatter0<4><<<p.nseg, kBT, 0, s>>>(p.n, p.tiles_x, p.shift0, p.bits[0], p.table_redundant[0],
                                             p.ncols_cap[0], box, offsets, hdr, table, k0, v0, bstart, rg0,
                                             p.ntiles);
    if (p.capacity == 0) {
        e = hipGetLastError();
        return e != hipSuccess ? e : finish();
    }
    if (p.order_kind == 1 && first_pass_only) return hipGetLastError();
    if (p.order_kind == 1) {
        const int nbk = 1 << p.bits[0];
        if (p.bucket_lanes == 16)        // big buckets: 16 waves each
            k_bucket_sortw<<<nbk, kBWT, 0, s>>>(kalt, valt, keys, vals, hdr, bstart, p.lo_bits, p.ntiles, rg);
        else if (p.bucket_lanes == 4)
            k_bucket_sort<4><<<nbk, kBT, 0, s>>>(kalt, valt, keys, vals, hdr, bstart, p.lo_bits, p.ntiles, rg);
        else
            k_bucket_sort<8><<<nbk, kBT, 0, s>>>(kalt, valt, keys, vals, hdr, bstart, p.lo_bits, p.ntiles, rg);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return finish();
    }
    if (p.order_kind == 0) return finish();
    // LSD: further passes, then the ranges
    auto dst_k = [&](int i) { return ((p.passes - 1 - i) & 1) ? kalt : keys; };
    auto dst_v = [&](int i) { return ((p.passes - 1 - i) & 1) ? valt : vals; };
    int shift = p.bits[0];
    for (int i = 1; i < p.passes; ++i) {
        const uint32_t *sk = dst_k(i - 1), *sv = dst_v(i - 1);
        const int b = p.bits[i], tr = p.table_redundant[i], nc = p.ncols_cap[i];
        if (p.pass_lanes == 4) k_count<4><<<p.nbs, kBT, 0, s>>>(sk, hdr, shift, b, tr, nc, table);
        else if (p.pass_lanes == 8) k_count<8><<<p.nbs, kBT, 0, s>>>(sk, hdr, shift, b, tr, nc, table);
        else k_count<16><<<p.nbs, kBT, 0, s>>>(sk, hdr, shift, b, tr, nc, table);
        if (!tr) {
            e = scan_u32(table, (1 << b) * nc, tsp, s);
            if (e != hipSuccess) return e;
        }
        if (p.pass_lanes == 4)
            k_scatter<4><<<p.nbs, kBT, 0, s>>>(sk, sv, dst_k(i), dst_v(i), hdr, shift, b, tr, nc, table);
        else if (p.pass_lanes == 8)
            k_scatter<8><<<p.nbs, kBT, 0, s>>>(sk, sv, dst_k(i), dst_v(i), hdr, shift, b, tr, nc, table);
        else
            k_scatter<16><<<p.nbs, kBT, 0, s>>>(sk, sv, dst_k(i), dst_v(i), hdr, shift, b, tr, nc, table);
        shift += p.bits[i];
    }
    k_ranges<<<(unsigned)((p.capacity + 1023) / 1024), 256, 0, s>>>(keys, hdr, (uint32_t)p.ntiles, ranges);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return finish();
}

}  // namespace gi
