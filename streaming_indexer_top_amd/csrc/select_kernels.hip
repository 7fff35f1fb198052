// Partition-merge top-k of the CSA lightning indexer for gfx950.
//
// The page "StreamIndex: Memory-Bounded Compressed Sparse Attention via
// Streaming Top-k" (Abstract) makes a chunked partition-merge top-k driver
// its central component: keys are split into chunks, each query keeps its top
// keys per chunk and the partial lists are merged, so the full score tensor
// never exists.  This kernel is that step for one chunk: one workgroup per
// query row reads the row's chunk scores from the workspace once, keeps only
// those that can still enter the row's best k, sorts them, merges them with
// the row's running list and, after the last chunk, writes the row's outputs.
//
// Exactness: every (score, key) pair is mapped to a 64-bit orderable key
//     key = (orderable(score) << 32) | (0xFFFFFFFF - j)
// where orderable() is the monotone map of fp32 onto uint32 after -0 -> +0.
// A larger key means a better entry under (score desc, index asc), and keys
// are unique because j is, so the best k is a well-defined set whatever the
// chunking: top-k(A u B) = top-k(top-k(A) u top-k(B)).  Every decision below
// (which keys are kept, their order) is taken on these keys, so the outputs
// are bit-identical for every chunk size.
//
// Common path (scores with the score kernel's histogram summary): the
// summary names the bin b* (top 11 orderable bits) holding the chunk's k-th
// best key.  One streaming pass sorts each chunk key into "above b*" (all
// kept, fewer than k), "in b*" (the boundary) or dropped, and appends the kept
// ones to two LDS regions.  One bucket sort over both regions orders them;
// the first k are the chunk's best k.  The workgroup needs about 39 KB of LDS,
// so four rows share a CU.
#include <type_traits>

#include "csa_internal.h"

namespace csa {
namespace {

constexpr int NT = kSelectThreads;
constexpr int NWAVES = NT / 64;
constexpr int kSortMaxBucket = 64;    // larger buckets: bitonic sort instead

// Capacities of the kernel for k <= K (K = 2048 or 4096).  Region A holds
// the keys above the boundary bin (fewer than k), region B the keys in it
// (the running list, up to k keys, also goes there after the sort).
template <int K>
struct Caps {
    static constexpr int A = K;
    static constexpr int B = K;
    static constexpr int Cand = A + B;        // 64-bit key slots in LDS
    static constexpr int Buckets = Cand * 3 / 8;  // bucket sort: one 32-bit word per bucket
    static constexpr int PER = Cand / NT;     // keys per thread in the sort and radix select
    static constexpr int PT = K / NT;         // merged outputs per thread
    static_assert(kSelectPiece + K <= Cand, "fallback pieces must fit beside k keys");
    static_assert(Buckets % NT == 0 && Buckets >= 256, "bucket words double as a 256-bin histogram");
    static constexpr size_t lds_bytes = (size_t)Cand * 8 + (size_t)Buckets * 4;
};

__device__ inline float key_score(uint64_t key)
{
    uint32_t u = (uint32_t)(key >> 32);
    u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    return __uint_as_float(u);
}

__device__ inline int32_t key_index(uint64_t key)
{
    return (int32_t)(0xFFFFFFFFu - (uint32_t)key);
}

__device__ inline float score_of_orderable(uint32_t u)
{
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

__device__ inline uint32_t lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP: shifts within rows
// of 16 lanes, then the row totals broadcast to the rows above).
__device__ inline uint32_t wave_incl_sum(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false); // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false); // row_bcast:31
    return x;
}

__device__ inline uint32_t wave_min_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, off);
        v = o < v ? o : v;
    }
    return v;
}

__device__ inline uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, off);
        v = o > v ? o : v;
    }
    return v;
}

__device__ inline uint64_t wave_min_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(v, off);
        v = o < v ? o : v;
    }
    return v;
}

// Adds this lane's digit to a histogram.  Lanes of a wave that share a digit
// are counted together (a few rounds of "take the first pending lane's
// digit, ballot the lanes with the same digit, one atomic for all of them"),
// because score digits cluster and same-address LDS atomics serialise.
__device__ inline void hist_add(uint32_t *hist, bool in, uint32_t d, int lane)
{
    uint64_t pending = __ballot(in);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        if (pending == 0) return;
        const int leader = __builtin_ctzll(pending);
        const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
        const bool mine = ((pending >> lane) & 1ull) != 0;
        const uint64_t same = __ballot(mine && d == dl);
        if (lane == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(same));
        pending &= ~same;
    }
    if ((pending >> lane) & 1ull) atomicAdd(&hist[d], 1u);
}

struct SelectShared {
    uint64_t wmin[NWAVES];
    uint32_t wsum[NWAVES];
    uint32_t wred[NWAVES][4];
    uint32_t nA, nB;
    uint32_t count;
    uint32_t digit, above, bin;
};

// Minimum of cand[0..cnt) over the block (cnt > 0).
__device__ uint64_t block_min(const uint64_t *cand, int cnt, SelectShared &sh, int tid)
{
    uint64_t mn = ~0ull;
    for (int e = tid; e < cnt; e += NT) mn = cand[e] < mn ? cand[e] : mn;
    mn = wave_min_u64(mn);
    if ((tid & 63) == 0) sh.wmin[tid >> 6] = mn;
    __syncthreads();
    uint64_t r = sh.wmin[0];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) r = sh.wmin[w] < r ? sh.wmin[w] : r;
    __syncthreads();
    return r;
}

// Exclusive prefix sum of v over the block (thread order), and the total.
__device__ uint32_t block_exclusive_sum(uint32_t v, uint32_t &total, SelectShared &sh, int tid)
{
    const uint32_t x = wave_incl_sum(v);
    if ((tid & 63) == 63) sh.wsum[tid >> 6] = x;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
        const uint32_t s = sh.wsum[w];
        if (w < (tid >> 6)) before += s;
        total += s;
    }
    __syncthreads();
    return before + x - v;
}

// Of the 256 bins of hist, finds the one holding the need-th largest entry
// (bins in descending order): sh.digit = that bin, sh.above = entries in
// higher bins, sh.bin = entries in it.  Wave 0 works; the caller syncs.
__device__ inline void find_digit(const uint32_t *hist, uint32_t need, SelectShared &sh, int tid)
{
    if (tid >= 64) return;
    const int lane = tid;
    // Lane l owns bins 4l..4l+3; above(l) = entries in bins of higher lanes.
    uint32_t h[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) h[b] = hist[4 * lane + b];
    const uint32_t local = h[0] + h[1] + h[2] + h[3];
    uint32_t incl = local;  // sum over lanes >= this lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(incl, off);
        if (lane + off < 64) incl += y;
    }
    uint32_t above = incl - local;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
        if (above < need && need <= above + h[b]) {
            sh.digit = (uint32_t)(4 * lane + b);
            sh.above = above;
            sh.bin = h[b];
        }
        above += h[b];
    }
}

// Keeps the k largest of cand[0..cnt) (k < cnt <= Caps<K>::Cand) in cand[0..k), any
// order.  All entries must agree on the key bits above `first_shift + 8`;
// digits are 8 bits wide from there down (the last one clamped at bit 0).
// hist has 256 words.
template <int K>
__device__ void radix_select(uint64_t *cand, int cnt, int k, uint32_t *hist, SelectShared &sh,
                             int tid, int first_shift = 56)
{
    constexpr int PER_MAX = Caps<K>::PER;
    const int lane = tid & 63;
    uint32_t need = (uint32_t)k;
    uint64_t prefix = 0, mask = 0;
    for (int shift = first_shift;; shift -= 8) {
        if (shift < 0) shift = 0;
        hist[tid] = 0u;  // NT == 256 bins
        __syncthreads();
        const int rounds = (cnt + NT - 1) / NT;
        for (int rd = 0; rd < rounds; ++rd) {
            const int e = rd * NT + tid;
            uint64_t key = 0;
            bool in = false;
            if (e < cnt) {
                key = cand[e];
                in = (key & mask) == prefix;
            }
            hist_add(hist, in, (uint32_t)(key >> shift) & 255u, lane);
        }
        __syncthreads();
        find_digit(hist, need, sh, tid);
        __syncthreads();
        const uint32_t d = sh.digit;
        need -= sh.above;
        prefix |= (uint64_t)d << shift;
        mask |= 255ull << shift;
        const bool done = sh.bin == need || shift == 0;  // the whole bin is taken
        __syncthreads();
        if (done) break;
    }
    // Entries whose masked key is >= prefix are exactly the k best.
    uint64_t v[PER_MAX];
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < PER_MAX; ++i) {
        const int e = i * NT + tid;
        v[i] = e < cnt ? cand[e] : 0ull;
        if (e < cnt && (v[i] & mask) >= prefix) ++mine;
    }
    uint32_t total;
    uint32_t off = block_exclusive_sum(mine, total, sh, tid);  // barriers inside
#pragma unroll
    for (int i = 0; i < PER_MAX; ++i) {
        const int e = i * NT + tid;
        if (e < cnt && (v[i] & mask) >= prefix) cand[off++] = v[i];
    }
    __syncthreads();
}

// Sorts cand[0..n) descending; n <= the buffer size, which holds the next
// power of two.  Used for degenerate inputs (huge runs of equal scores).
__device__ void bitonic_desc(uint64_t *cand, int n, int tid)
{
    int p2 = 2;
    while (p2 < n) p2 <<= 1;
    for (int e = n + tid; e < p2; e += NT) cand[e] = 0ull;  // below every real key
    __syncthreads();
    for (int size = 2; size <= p2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (p2 >> 1); i += NT) {
                const int lo = ((i & ~(stride - 1)) << 1) | (i & (stride - 1));
                const int hi = lo | stride;
                const uint64_t x = cand[lo], y = cand[hi];
                const bool first_half_desc = (lo & size) == 0;
                if (first_half_desc ? (x < y) : (x > y)) {
                    cand[lo] = y;
                    cand[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

// Sorts the nA keys at cand[0..nA) and the nB keys at cand[A..A+nB)
// together, descending, into cand[0..nA+nB).  Every A key must be larger
// than every B key (A = above the boundary, B = in it; either may be empty).
//
// Bucket sort with the keys held in registers: each region's range
// [min, max] is cut into buckets of equal width (in the orderable integer
// when the region's scores share one sign, else in score value; B gets a
// share of the buckets proportional to its size, A the rest), which is
// monotone, so bucket order is key order.  One LDS atomic per key counts
// its bucket and gives its slot there; a prefix sum over the buckets (from the
// top) gives each bucket's first position; keys are scattered into bucket
// order, and each then finds its place inside its bucket by counting the
// larger keys there.  If a bucket holds more than kSortMaxBucket keys (many
// equal or clustered scores) a bitonic sort of the whole buffer takes over.
// bk: Caps<K>::Buckets words.
template <int K>
__device__ __forceinline__ void sort_keys(uint64_t *cand, int nA, int nB, uint32_t *bk, SelectShared &sh,
                          int tid)
{
    constexpr int kCapA = Caps<K>::A;
    constexpr int kCand = Caps<K>::Cand;
    constexpr int kBuckets = Caps<K>::Buckets;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    constexpr int PT = Caps<K>::PER;  // slots 0..PT/2-1 from A's region, the rest from B's
    constexpr int PH = PT / 2;
    static_assert(Caps<K>::A == Caps<K>::B, "equal regions: half the slots each");
    uint64_t key[PT];
    uint32_t loA = 0xFFFFFFFFu, hiA = 0u, loB = 0xFFFFFFFFu, hiB = 0u;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        const int e = (i % PH) * NT + tid;
        const bool inA = i < PH;
        const bool v = e < (inA ? nA : nB);
        key[i] = v ? cand[(inA ? 0 : kCapA) + e] : 0ull;
        const uint32_t u = (uint32_t)(key[i] >> 32);
        if (v && inA) {
            loA = u < loA ? u : loA;
            hiA = u > hiA ? u : hiA;
        }
        if (v && !inA) {
            loB = u < loB ? u : loB;
            hiB = u > hiB ? u : hiB;
        }
    }
    for (int e = tid; e < kBuckets; e += NT) bk[e] = 0u;
    loA = wave_min_u32(loA);
    hiA = wave_max_u32(hiA);
    loB = wave_min_u32(loB);
    hiB = wave_max_u32(hiB);
    if (lane == 0) {
        sh.wred[wave][0] = loA;
        sh.wred[wave][1] = hiA;
        sh.wred[wave][2] = loB;
        sh.wred[wave][3] = hiB;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
        loA = sh.wred[w][0] < loA ? sh.wred[w][0] : loA;
        hiA = sh.wred[w][1] > hiA ? sh.wred[w][1] : hiA;
        loB = sh.wred[w][2] < loB ? sh.wred[w][2] : loB;
        hiB = sh.wred[w][3] > hiB ? sh.wred[w][3] : hiB;
    }
    const int n = nA + nB;
    int nbB = 0;
    if (nB > 0) {
        nbB = nA == 0 ? kBuckets : (int)((int64_t)kBuckets * nB / n);
        nbB = nbB < 1 ? 1 : (nbB > kBuckets - 1 && nA > 0 ? kBuckets - 1 : nbB);
    }
    const int nbA = kBuckets - nbB;
    // Bucket of a key, monotone in it.  A region whose scores share one sign
    // is cut evenly in the orderable integer, which is close to a log scale
    // and gives the dense low end of a score tail finer buckets; a region
    // that crosses zero is cut evenly in score value (in the integer it
    // would spend most buckets on tiny magnitudes).  Either map is monotone,
    // so bucket order is key order; the clamps also catch inf and NaN.
    const bool intA = (loA ^ hiA) < 0x80000000u, intB = (loB ^ hiB) < 0x80000000u;
    const float fAlo = intA ? 0.0f : score_of_orderable(loA);
    const float fBlo = intB ? 0.0f : score_of_orderable(loB);
    const float wA = intA ? (float)(hiA - loA) : score_of_orderable(hiA) - fAlo;
    const float wB = intB ? (float)(hiB - loB) : score_of_orderable(hiB) - fBlo;
    const float scA = wA > 0.0f ? (float)nbA / wA : 0.0f;
    const float scB = wB > 0.0f ? (float)nbB / wB : 0.0f;
    const float topA = (float)(nbA - 1), topB = (float)(nbB - 1);
    auto bucket_of = [&](uint64_t kk, bool inA) -> uint32_t {
        const uint32_t u = (uint32_t)(kk >> 32);
        const bool in_int = inA ? intA : intB;
        const float x = in_int ? (float)(u - (inA ? loA : loB)) : score_of_orderable(u);
        float t = (x - (inA ? fAlo : fBlo)) * (inA ? scA : scB);
        t = fminf(fmaxf(t, 0.0f), inA ? topA : topB);
        return (uint32_t)(int)t + (inA ? (uint32_t)nbB : 0u);
    };
    uint32_t bkt[PT], slot[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        const int e = (i % PH) * NT + tid;
        const bool inA = i < PH;
        bkt[i] = 0u;
        slot[i] = 0u;
        if (e < (inA ? nA : nB)) {
            bkt[i] = bucket_of(key[i], inA);
            slot[i] = atomicAdd(&bk[bkt[i]], 1u);
        }
    }
    __syncthreads();
    // First position of every bucket, counted from the top bucket down;
    // thread t owns buckets kBuckets-1-(t*PB .. t*PB+PB-1).  The words become
    // (first position << 16) | size.
    constexpr int PB = kBuckets / NT;
    uint32_t c[PB];
    uint32_t mine = 0, big = 0;
#pragma unroll
    for (int j = 0; j < PB; ++j) {
        c[j] = bk[kBuckets - 1 - (tid * PB + j)];
        mine += c[j];
        big = c[j] > big ? c[j] : big;
    }
    big = wave_max_u32(big);
    if (lane == 0) sh.wred[wave][0] = big;
    uint32_t total;
    uint32_t run = block_exclusive_sum(mine, total, sh, tid);  // barriers inside
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) big = sh.wred[w][0] > big ? sh.wred[w][0] : big;
    if (big > (uint32_t)kSortMaxBucket) {
        // Degenerate: the whole buffer, with empty slots zeroed (below every
        // real key), through a bitonic sort.
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int e = (i % PH) * NT + tid;
            const bool inA = i < PH;
            if (e >= (inA ? nA : nB)) cand[(inA ? 0 : kCapA) + e] = 0ull;
        }
        __syncthreads();
        bitonic_desc(cand, kCand, tid);
        return;
    }
#pragma unroll
    for (int j = 0; j < PB; ++j) {
        bk[kBuckets - 1 - (tid * PB + j)] = (run << 16) | c[j];
        run += c[j];
    }
    __syncthreads();
    // Scatter into bucket order (every key is in registers).
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        const int e = (i % PH) * NT + tid;
        if (e < (i < PH ? nA : nB)) cand[(bk[bkt[i]] >> 16) + slot[i]] = key[i];
    }
    __syncthreads();
    // Place inside the bucket: count the larger keys there.
    uint32_t pos[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        const int e = (i % PH) * NT + tid;
        pos[i] = 0u;
        if (e < (i < PH ? nA : nB)) {
            const uint32_t wd = bk[bkt[i]];
            const int o = (int)(wd >> 16), m = (int)(wd & 0xFFFFu);
            int rk = 0;
            int q = o;
            // Four independent reads per round (the loop is bound by LDS
            // latency), then the rest one by one.
            for (; q + 3 < o + m; q += 4) {
                const uint64_t c0 = cand[q], c1 = cand[q + 1], c2 = cand[q + 2], c3 = cand[q + 3];
                rk += (c0 > key[i] ? 1 : 0) + (c1 > key[i] ? 1 : 0) + (c2 > key[i] ? 1 : 0) + (c3 > key[i] ? 1 : 0);
            }
            for (; q < o + m; ++q) rk += cand[q] > key[i] ? 1 : 0;
            pos[i] = (uint32_t)(o + rk);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        const int e = (i % PH) * NT + tid;
        if (e < (i < PH ? nA : nB)) cand[pos[i]] = key[i];
    }
    __syncthreads();
}

// Row context shared by the selection strategies below.
struct RowCtx {
    const uint32_t *src;  // the row's chunk scores as orderable() (a workspace row of clen)
    int64_t len;          // keys of this row in the chunk
    uint32_t c0;          // first key index of the chunk
    uint32_t u_lo;        // keys below this orderable score cannot enter the running best k
                          // (the list's k-th score + 1 when the list is full, else 0)
};

// Loads 16 consecutive orderable scores of a workspace row at `base`; at or
// past len it loads the row's first 16 instead (callers ignore positions >=
// len).  Unconditional, so that the compiler can count the loads in flight
// and wait only for the ones it needs.  Stays inside the row: base is a
// multiple of 16 below len <= row length, which is a multiple of 256.
__device__ inline void load16(const uint32_t *src, int64_t len, int64_t base, uint32_t (&v)[16])
{
    const uint32_t *p = src + (base < len ? base : 0);
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
        const uint4 x = *(const uint4 *)(p + i);
        v[i] = x.x;
        v[i + 1] = x.y;
        v[i + 2] = x.z;
        v[i + 3] = x.w;
    }
}

// One streaming pass over the row's chunk scores, 16 consecutive keys per
// thread per round, the next two rounds' loads in flight while this round is
// classified.  With eA >= eB >= r.u_lo: a key whose orderable score u has
// u >= eA goes to region A (cand[0..)), one with eB <= u < eA to region B
// (cand[A..)), any other is dropped.  Each wave reserves its slots with one
// LDS atomic per region per round; the order inside a region is arbitrary
// (the sort fixes it).  Returns the region sizes (clamped to the capacities,
// which the callers' counts never exceed).
template <int K>
__device__ __forceinline__ void collect(const RowCtx &r, uint32_t eA, uint32_t eB, uint64_t *cand,
                                        SelectShared &sh, int tid, int &nA, int &nB)
{
    constexpr int kCapA = Caps<K>::A;
    constexpr int kCapB = Caps<K>::B;
    constexpr int V = 16;
    constexpr int ROUND = NT * V;
    const int lane = tid & 63;
    if (tid == 0) {
        sh.nA = 0u;
        sh.nB = 0u;
    }
    __syncthreads();
    // Each lane's slot for the keys it drops: the bucket words behind the
    // candidate regions are unused until the sort, and one slot per lane keeps
    // the stores of a wave free of same-address conflicts.
    const uint32_t dummy = (uint32_t)Caps<K>::Cand + (uint32_t)tid;
    // FULL: every lane's 16 keys lie inside the row (all rounds but the
    // row's last), so no key needs a range test.
    auto process = [&](const uint32_t (&v)[V], int64_t base, auto full_t) {
        constexpr bool FULL = decltype(full_t)::value;
        const int rem = FULL ? V : (int)min((int64_t)V, max((int64_t)0, r.len - base));
        // Counts: keys >= eA (A) and keys >= eB (A and B), no branches.
        uint32_t ca = 0, cb = 0;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const bool in = FULL || i < rem;
            ca += (in && v[i] >= eA) ? 1u : 0u;
            cb += (in && v[i] >= eB) ? 1u : 0u;
        }
        const uint32_t cnt = ca | ((cb - ca) << 16);  // A low, B high
        const uint32_t incl = wave_incl_sum(cnt);
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        if (tot == 0u) return;  // wave-uniform
        // Lanes 0 and 1 reserve the wave's A and B slots with one LDS
        // atomic instruction (adding 0 is harmless).
        uint32_t bx = 0;
        if (lane < 2) bx = atomicAdd(lane ? &sh.nB : &sh.nA, lane ? (tot >> 16) : (tot & 0xFFFFu));
        const uint32_t ba = (uint32_t)__builtin_amdgcn_readlane((int)bx, 0);
        const uint32_t bb = (uint32_t)__builtin_amdgcn_readlane((int)bx, 1);
        const uint32_t excl = incl - cnt;
        uint32_t pa = ba + (excl & 0xFFFFu);
        uint32_t pb = (uint32_t)kCapA + bb + (excl >> 16);
        // The counts stay within the capacities on every path that calls
        // this; a wave whose slots would not fit stores only what fits.
        const bool fits = ba + (tot & 0xFFFFu) <= (uint32_t)kCapA &&
                          bb + (tot >> 16) <= (uint32_t)kCapB;  // wave-uniform
        const uint32_t capA = fits ? 0xFFFFFFFFu : (uint32_t)kCapA;
        const uint32_t capB = fits ? 0xFFFFFFFFu : (uint32_t)(kCapA + kCapB);
        // Every key is stored, a dropped one to this lane's spare slot.  The
        // low word of a key is 0xFFFFFFFF - j, j = c0 + base + i.
        const uint32_t nj0 = 0xFFFFFFFFu - (r.c0 + (uint32_t)base);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const bool in = FULL || i < rem;
            const bool isA = in && v[i] >= eA;
            const bool isAB = in && v[i] >= eB;
            const uint32_t slot = (isA & (pa < capA)) ? pa : ((isAB & !isA & (pb < capB)) ? pb : dummy);
            pa += isA ? 1u : 0u;
            pb += (isAB & !isA) ? 1u : 0u;
            cand[slot] = ((uint64_t)v[i] << 32) | (uint64_t)(nj0 - (uint32_t)i);
        }
    };
    // Three buffers rotate by name (the loop is unrolled by three): a copy
    // between buffers would wait for the load just issued into the source.
    uint32_t b0[V], b1[V], b2[V];
#pragma unroll
    for (int i = 0; i < V; ++i) b0[i] = b1[i] = b2[i] = 0u;
    const int64_t lane0 = (int64_t)tid * V;
    // Round starting at key rs: full rounds skip the range tests (uniform).
    auto round = [&](const uint32_t (&v)[V], int64_t rs) {
        if (rs + ROUND <= r.len) process(v, rs + lane0, std::true_type{});
        else process(v, rs + lane0, std::false_type{});
    };
    load16(r.src, r.len, lane0, b0);
    load16(r.src, r.len, ROUND + lane0, b1);
    for (int64_t e0 = 0; e0 < r.len; e0 += 3 * ROUND) {
        load16(r.src, r.len, e0 + 2 * ROUND + lane0, b2);
        round(b0, e0);
        if (e0 + ROUND >= r.len) break;  // uniform
        load16(r.src, r.len, e0 + 3 * ROUND + lane0, b0);
        round(b1, e0 + ROUND);
        if (e0 + 2 * ROUND >= r.len) break;
        load16(r.src, r.len, e0 + 4 * ROUND + lane0, b1);
        round(b2, e0 + 2 * ROUND);
    }
    __syncthreads();
    nA = __builtin_amdgcn_readfirstlane((int)min(sh.nA, (uint32_t)kCapA));
    nB = __builtin_amdgcn_readfirstlane((int)min(sh.nB, (uint32_t)kCapB));
    __syncthreads();
}

// Splits the boundary bin [lo_u, hi_u) (orderable values, width 2^shift;
// hi_u == 0: the bin reaches the top of the range) by its next 8 bits: a
// histogram over the chunk keys in the bin that beat the floor gives the
// sub-bin holding the need-th best of them.  Narrows [lo_u, hi_u) to it and
// returns the keys above it inside the old bin.
__device__ __forceinline__ uint32_t refine_bin(const RowCtx &r, uint32_t &lo_u, uint32_t &hi_u,
                                               int shift, uint32_t need, uint32_t *hist,
                                               SelectShared &sh, int tid)
{
    const int lane = tid & 63;
    hist[tid] = 0u;
    __syncthreads();
    const bool top = hi_u == 0u;
    const uint32_t lo = max(lo_u, r.u_lo);
    constexpr int V = 16;
    constexpr int ROUND = NT * V;
    auto count = [&](const uint32_t (&v)[V], int64_t base) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const uint32_t u = v[i];
            const bool in = base + i < r.len && u >= lo && (top || u < hi_u);
            hist_add(hist, in, (u >> (shift - 8)) & 255u, lane);
        }
    };
    // Two buffers rotating by name (unrolled by two), as in collect().
    uint32_t b0[V], b1[V];
#pragma unroll
    for (int i = 0; i < V; ++i) b0[i] = b1[i] = 0u;
    const int64_t lane0 = (int64_t)tid * V;
    load16(r.src, r.len, lane0, b0);
    for (int64_t e0 = 0; e0 < r.len; e0 += 2 * ROUND) {
        load16(r.src, r.len, e0 + ROUND + lane0, b1);
        count(b0, e0 + lane0);
        if (e0 + ROUND >= r.len) break;  // uniform
        load16(r.src, r.len, e0 + 2 * ROUND + lane0, b0);
        count(b1, e0 + ROUND + lane0);
    }
    __syncthreads();
    find_digit(hist, need, sh, tid);
    __syncthreads();
    const uint32_t above = sh.above;
    lo_u |= sh.digit << (shift - 8);
    hi_u = lo_u + (1u << (shift - 8));
    __syncthreads();
    return above;
}

// Q = the k best chunk keys that beat the floor, without a summary: the chunk
// is read in pieces, keys that cannot enter the current best k are dropped,
// and the candidates are cut back to k by radix select whenever they exceed k.
// Leaves them, unsorted, in cand[0..count) and returns the count.
template <int K>
__device__ __noinline__ int collect_pieces(uint64_t *cand, const RowCtx r, int k, uint32_t *hist,
                              SelectShared &sh, int tid)
{
    const int lane = tid & 63;
    int cnt = 0;
    bool full = false;
    uint64_t thr = 0;
    for (int64_t p0 = 0; p0 < r.len; p0 += kSelectPiece) {
        const int plen = (int)min((int64_t)kSelectPiece, r.len - p0);
        if (tid == 0) sh.count = 0u;
        __syncthreads();
        for (int e0 = 0; e0 < plen; e0 += NT) {
            const int e = e0 + tid;
            bool take = false;
            uint64_t key = 0;
            if (e < plen) {
                const uint32_t u = r.src[p0 + e];
                key = ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (r.c0 + (uint32_t)(p0 + e)));
                take = u >= r.u_lo && (!full || key > thr);
            }
            const uint64_t m = __ballot(take);
            if (m != 0) {  // wave-uniform
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(&sh.count, (uint32_t)__popcll(m));
                base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
                if (take) cand[cnt + base + lanes_below(m)] = key;
            }
        }
        __syncthreads();
        cnt += (int)sh.count;
        if (cnt > k) {
            radix_select<K>(cand, cnt, k, hist, sh, tid);
            cnt = k;
        }
        if (cnt >= k) {
            full = true;
            thr = block_min(cand, cnt, sh, tid);
        }
        __syncthreads();  // every thread has read sh.count before it is reset
    }
    return cnt;
}

// This thread's share of the merge of two descending lists L[0..nl) and
// Q[0..nq): the entries at positions p0..p0+PT-1 of the merged order, up to
// position `total`, in outv (merge-path split: a binary search for how many
// entries of L come before p0, then a sequential merge).  Returns how many
// it produced; kth receives the entry at position kpos if this thread has it.
template <int PT>
__device__ inline int merge_share(const uint64_t *L, int nl, const uint64_t *Q, int nq, int total,
                                  int p0, int kpos, uint64_t (&outv)[PT], uint64_t &kth)
{
    int nout = 0;
#pragma unroll
    for (int t = 0; t < PT; ++t) outv[t] = 0ull;
    if (p0 < total) {
        int lo = max(0, p0 - nq), hi = min(p0, nl);
        while (lo < hi) {  // i = entries taken from L before position p0
            const int mid = (lo + hi) >> 1;
            if (L[mid] > Q[p0 - 1 - mid]) lo = mid + 1;
            else hi = mid;
        }
        int i = lo, j = p0 - lo;
#pragma unroll
        for (int t = 0; t < PT; ++t) {
            if (p0 + t < total) {
                uint64_t v;
                if (j >= nq || (i < nl && L[i] > Q[j])) v = L[i++];
                else v = Q[j++];
                outv[t] = v;
                if (p0 + t == kpos) kth = v;
                ++nout;
            }
        }
    }
    return nout;
}

// Writes positions p0..p0+PT-1 (below k) of a row's outputs: the first nout
// from outv, then padding (idx -1, score -inf).  16-byte stores when aligned.
template <int PT>
__device__ inline void emit_share(int32_t *oi, float *os, int k, int p0, const uint64_t (&outv)[PT],
                                  int nout)
{
    int32_t vi[PT];
    float vs[PT];
#pragma unroll
    for (int t = 0; t < PT; ++t) {
        vi[t] = t < nout ? key_index(outv[t]) : -1;
        vs[t] = t < nout ? key_score(outv[t]) : -__builtin_inff();
    }
    const bool al16 = ((((uintptr_t)oi) | ((uintptr_t)os)) & 15u) == 0u;
    if (al16 && p0 + PT <= k) {  // 16-byte aligned, whole
#pragma unroll
        for (int t = 0; t < PT; t += 4) {
            *(int4 *)(oi + p0 + t) = make_int4(vi[t], vi[t + 1], vi[t + 2], vi[t + 3]);
            *(float4 *)(os + p0 + t) = make_float4(vs[t], vs[t + 1], vs[t + 2], vs[t + 3]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < PT; ++t) {
            if (p0 + t < k) {
                oi[p0 + t] = vi[t];
                os[p0 + t] = vs[t];
            }
        }
    }
}

// Writes this thread's share (positions p0.., nout entries) of a list of k
// slots; `whole`: all PT entries are real.
template <int PT>
__device__ inline void store_share(uint64_t *dst, int k, int p0, const uint64_t (&outv)[PT], int nout)
{
    if ((k & 1) == 0 && nout == PT) {  // 16-byte aligned, whole
#pragma unroll
        for (int t = 0; t < PT; t += 2) {
            ulonglong2 v2;
            v2.x = outv[t];
            v2.y = outv[t + 1];
            *(ulonglong2 *)(dst + p0 + t) = v2;
        }
    } else {
#pragma unroll
        for (int t = 0; t < PT; ++t)
            if (t < nout) dst[p0 + t] = outv[t];
    }
}

template <int K>
__global__ __launch_bounds__(NT, K <= 2048 ? 4 : 2) void select_kernel(SelectArgs a)
{
    constexpr int kCapA = Caps<K>::A;
    constexpr int kCapB = Caps<K>::B;
    extern __shared__ uint64_t smem[];
    __shared__ SelectShared sh;
    const int k = (int)a.k;
    uint64_t *cand = smem;                                 // Caps<K>::Cand keys
    uint32_t *bk = (uint32_t *)(smem + Caps<K>::Cand);    // bucket words (also a 256-bin histogram)
    const int tid = threadIdx.x;
    // Virtual row vr = split * rows + rl (split 0 and vr == rl without
    // splits); long rows first.
    const int64_t split = (int64_t)blockIdx.x / a.rows;
    const int64_t rl = a.rows - 1 - ((int64_t)blockIdx.x - split * a.rows);
    const int64_t vr = split * a.rows + rl;
    const int64_t row = a.row0 + rl;
    const int64_t n = n_usable(a.q_pos0 + row, a.T, a.m);
    const int64_t c0 = a.c0 + split * a.slen;  // first key of the split
    int64_t len = n - c0;
    len = len < 0 ? 0 : (len > a.slen ? a.slen : len);
    // Nothing to add and nothing to write: the running list stays as it is.
    // (The first chunk always runs so that every row's state is written.)
    if (!a.emit && !a.first && len == 0) return;

    int cnt_l = 0;
    uint64_t theta = 0;
    if (!a.first) {
        const RowState stt = a.state[vr];
        cnt_l = stt.count;
        theta = stt.theta;
    }

    RowCtx r;
    r.src = a.ws + rl * a.clen + split * a.slen;
    r.len = len;
    r.c0 = (uint32_t)c0;
    // A full running list admits only scores above its k-th (equal scores
    // lose to the list's lower indices).  Finite scores stay below
    // orderable(+inf) = 0xFF800000, so the +1 cannot wrap.
    r.u_lo = theta != 0 ? (uint32_t)(theta >> 32) + 1u : 0u;

    // Chunk-local best k (the partition step), sorted descending, in
    // cand[0..cnt_q).
    int cnt_q = 0;
    if (len > 0) {
        int nA = 0, nB = 0;
        bool done = false;
        if (a.meta) {
            const ChunkMeta mt = a.meta[vr];
            if (mt.total <= (uint32_t)k) {
                // Every key that beats the floor (at most k of them).
                collect<K>(r, r.u_lo, r.u_lo, cand, sh, tid, nA, nB);
                done = true;
            } else {
                constexpr int BIN_SHIFT = 32 - kHistBits;  // orderable bits below the bin
                uint32_t lo_u = mt.bin << BIN_SHIFT;        // boundary: orderable in [lo_u, hi_u)
                uint32_t hi_u = (mt.bin + 1u) << BIN_SHIFT;
                uint32_t in_bin = mt.in_bin;
                bool fits = true;
                if (in_bin > (uint32_t)kCapB) {
                    const uint32_t need = (uint32_t)k - mt.above;
                    const uint32_t up = refine_bin(r, lo_u, hi_u, BIN_SHIFT, need, bk, sh, tid);
                    in_bin = sh.bin;
                    fits = in_bin <= (uint32_t)kCapB;
                    (void)up;
                }
                if (fits) {
                    // Bin edges as orderable thresholds, raised to the floor.
                    // The top bin has no upper edge: 0xFFFFFFFF is above
                    // every finite score, so its keys all go to region B.
                    const uint32_t eA = max(hi_u == 0u ? 0xFFFFFFFFu : hi_u, r.u_lo);
                    const uint32_t eB = max(lo_u, r.u_lo);
                    collect<K>(r, eA, eB, cand, sh, tid, nA, nB);
                    done = true;
                }
            }
        }
        if (!done) {
            // No summary, or massively tied scores.
            nA = collect_pieces<K>(cand, r, k, bk, sh, tid);
            nB = 0;
        }
        if (nA + nB > 1) {
            sort_keys<K>(cand, nA, nB, bk, sh, tid);
        } else if (nB == 1) {
            // A single key (k = 1), found in region B: the sort would have
            // moved it to the front.
            if (tid == 0) cand[0] = cand[kCapA];
            __syncthreads();
        }
        cnt_q = min(k, nA + nB);
    }

    // Running list into the B region (free once the sort is done).
    uint64_t *lst = cand + kCapA;
    if (cnt_l > 0) {
        const uint64_t *src = a.lists + vr * a.k;
        for (int e = tid; e < cnt_l; e += NT) lst[e] = src[e];
    }
    __syncthreads();

    // Merge with the running list (both sorted descending) and keep the
    // first min(k, |L| + |Q|) entries: merge-path split, PT outputs per thread.
    const int total = min(k, cnt_l + cnt_q);
    constexpr int PT = Caps<K>::PT;  // outputs per thread (k <= K)
    const int p0 = tid * PT;
    uint64_t outv[PT];
    uint64_t kth = 0;  // the entry at position k-1, for the next chunk's floor
    const int nout = merge_share<PT>(lst, cnt_l, cand, cnt_q, total, p0, k - 1, outv, kth);
    if (a.emit) {
        // NT*PT = K >= k, so every position is written.
        emit_share<PT>(a.out_idx + row * a.k, a.out_score + row * a.k, k, p0, outv, nout);
    } else {
        store_share<PT>(a.lists + vr * a.k, k, p0, outv, nout);
        if (total == k && p0 <= k - 1 && k - 1 < p0 + nout) a.state[vr].theta = kth;
        if (tid == 0) {
            a.state[vr].count = total;
            if (total < k) a.state[vr].theta = 0;
        }
    }
}

// One merge round of split lists (see MergeArgs): workgroup (p, rl) merges
// the lists of virtual rows p*rows + rl and (p+half)*rows + rl.
template <int K>
__global__ __launch_bounds__(NT) void merge_kernel(MergeArgs a)
{
    extern __shared__ uint64_t smem[];
    const int tid = threadIdx.x;
    const int k = (int)a.k;
    const int64_t p = (int64_t)blockIdx.x / a.rows;
    const int64_t rl = a.rows - 1 - ((int64_t)blockIdx.x - p * a.rows);
    const int64_t va = p * a.rows + rl, vb = (p + a.half) * a.rows + rl;
    const int na = a.state[va].count, nb = a.state[vb].count;
    uint64_t *la = smem, *lb = smem + K;
    for (int e = tid; e < na; e += NT) la[e] = a.lists[va * a.k + e];
    for (int e = tid; e < nb; e += NT) lb[e] = a.lists[vb * a.k + e];
    __syncthreads();
    const int total = min(k, na + nb);
    constexpr int PT = Caps<K>::PT;
    const int p0 = tid * PT;
    uint64_t outv[PT];
    uint64_t kth = 0;
    const int nout = merge_share<PT>(la, na, lb, nb, total, p0, k - 1, outv, kth);
    if (a.emit) {
        const int64_t row = a.row0 + rl;
        emit_share<PT>(a.out_idx + row * a.k, a.out_score + row * a.k, k, p0, outv, nout);
    } else {
        store_share<PT>(a.lists + va * a.k, k, p0, outv, nout);
        if (tid == 0) a.state[va].count = total;
    }
}

// A four-way merge round (k <= 2048): workgroup (p, rl) merges the lists of
// virtual rows (p + j*quarter)*rows + rl, j = 0..3, into the first.  The best
// k of the union is the best k of (best k of lists 0,1) u (best k of 2,3).
__global__ __launch_bounds__(NT) void merge4_kernel(MergeArgs a)
{
    constexpr int K = 2048;
    extern __shared__ uint64_t smem[];
    const int tid = threadIdx.x;
    const int k = (int)a.k;
    const int64_t q4 = a.half;  // quarter: lists p, p+q4, p+2*q4, p+3*q4
    const int64_t p = (int64_t)blockIdx.x / a.rows;
    const int64_t rl = a.rows - 1 - ((int64_t)blockIdx.x - p * a.rows);
    int64_t v[4];
    int n[4];
    uint64_t *l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = (p + j * q4) * a.rows + rl;
        n[j] = a.state[v[j]].count;
        l[j] = smem + j * K;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        for (int e = tid; e < n[j]; e += NT) l[j][e] = a.lists[v[j] * a.k + e];
    __syncthreads();
    constexpr int PT = Caps<K>::PT;
    const int p0 = tid * PT;
    uint64_t ab[PT], cd[PT], kth = 0;
    const int nab = min(k, n[0] + n[1]), ncd = min(k, n[2] + n[3]);
    const int oab = merge_share<PT>(l[0], n[0], l[1], n[1], nab, p0, -1, ab, kth);
    const int ocd = merge_share<PT>(l[2], n[2], l[3], n[3], ncd, p0, -1, cd, kth);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < PT; ++t) {
        if (t < oab) l[0][p0 + t] = ab[t];
        if (t < ocd) l[2][p0 + t] = cd[t];
    }
    __syncthreads();
    const int total = min(k, nab + ncd);
    uint64_t outv[PT];
    const int nout = merge_share<PT>(l[0], nab, l[2], ncd, total, p0, -1, outv, kth);
    if (a.emit) {
        const int64_t row = a.row0 + rl;
        emit_share<PT>(a.out_idx + row * a.k, a.out_score + row * a.k, k, p0, outv, nout);
    } else {
        store_share<PT>(a.lists + v[0] * a.k, k, p0, outv, nout);
        if (tid == 0) a.state[v[0]].count = total;
    }
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream)
{
    if (a.rows <= 0 || a.half <= 0) return hipSuccess;
    const dim3 grid((unsigned)(a.rows * a.half));
    if (a.k <= 2048) {
        if (a.four) {
            static std::atomic<uint64_t> attr_done{0};
            const hipError_t e = set_dynamic_lds((const void *)merge4_kernel,
                                                 4 * 2048 * (int)sizeof(uint64_t), attr_done);
            if (e != hipSuccess) return e;
            merge4_kernel<<<grid, dim3(NT), 4 * 2048 * sizeof(uint64_t), stream>>>(a);
        } else {
            merge_kernel<2048><<<grid, dim3(NT), 2 * 2048 * sizeof(uint64_t), stream>>>(a);
        }
    } else {
        merge_kernel<4096><<<grid, dim3(NT), 2 * 4096 * sizeof(uint64_t), stream>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_select(const SelectArgs &a, hipStream_t stream)
{
    if (a.rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)(a.rows * a.nsplit));
    if (a.k <= 2048) {
        select_kernel<2048><<<grid, dim3(NT), Caps<2048>::lds_bytes, stream>>>(a);
    } else {
        static std::atomic<uint64_t> attr_done{0};
        const hipError_t e = set_dynamic_lds((const void *)select_kernel<4096>,
                                             (int)Caps<4096>::lds_bytes, attr_done);
        if (e != hipSuccess) return e;
        select_kernel<4096><<<grid, dim3(NT), Caps<4096>::lds_bytes, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace csa
