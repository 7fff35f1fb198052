// Partition-merge top-k of the CSA lightning indexer for gfx950.
//
// The page "StreamIndex: Memory-Bounded Compressed Sparse Attention via
// Streaming Top-k" (Abstract) makes a chunked partition-merge top-k driver
// its central component: keys are split into chunks, each query keeps its top
// keys per chunk and the partial lists are merged, so the full score tensor
// never exists.  This kernel is that step for one chunk: one workgroup per
// query row reads the row's chunk scores from the workspace, keeps only those
// that can still enter the row's running best-k list, and whenever the
// candidates exceed k selects the best k exactly.  After the last chunk it
// sorts the list and writes the row's outputs.
//
// Exactness: every (score, key) pair is mapped to a 64-bit orderable key
//     key = (orderable(score) << 32) | (0xFFFFFFFF - j)
// where orderable() is the monotone map of fp32 onto uint32 after -0 -> +0.
// A larger key means a better entry under (score desc, index asc), and keys
// are unique because j is, so the best k is a well-defined set whatever the
// chunking: top-k(A u B) = top-k(top-k(A) u top-k(B)).  Selection is a
// most-significant-digit radix select on these keys (8-bit digits, LDS
// histograms), so the outputs are bit-identical for every chunk size.
#include "csa_internal.h"

namespace csa {
namespace {

constexpr int NT = kSelectThreads;
constexpr int NWAVES = NT / 64;
constexpr int PER_MAX = (2048 + kSelectPiece + NT - 1) / NT;  // entries per thread, k <= 2048

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

__device__ inline uint64_t make_key(float sc, uint32_t j)
{
    return ((uint64_t)orderable(sc) << 32) | (uint64_t)(0xFFFFFFFFu - j);
}

__device__ inline uint32_t lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Adds this lane's digit to the histogram.  Lanes of a wave that share a
// digit are counted together (a few rounds of "take the first pending lane's
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
    uint32_t hist[256];
    uint64_t wmin[NWAVES];
    uint32_t wsum[NWAVES];
    uint32_t count, count2;
    uint32_t digit, above, bin;
};

__device__ inline uint64_t wave_min_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(v, off);
        v = o < v ? o : v;
    }
    return v;
}

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
    const int lane = tid & 63;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) sh.wsum[tid >> 6] = x;
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

// Keeps the k largest of cand[0..cnt) (cnt > k) in cand[0..k), any order.
// All entries must agree on the key bits above `first_shift + 8`; digits are
// 8 bits wide from there down (the last digit is clamped at bit 0).
__device__ void radix_select(uint64_t *cand, int cnt, int k, SelectShared &sh, int tid,
                             int first_shift = 56)
{
    const int lane = tid & 63;
    uint32_t need = (uint32_t)k;
    uint64_t prefix = 0, mask = 0;
    for (int shift = first_shift;; shift -= 8) {
        if (shift < 0) shift = 0;
        sh.hist[tid] = 0u;  // NT == 256 bins
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
            hist_add(sh.hist, in, (uint32_t)(key >> shift) & 255u, lane);
        }
        __syncthreads();
        if (tid < 64) {
            // Lane l owns bins 4l..4l+3.  above(l) = entries in bins of
            // higher lanes; scan runs from lane 63 downwards.
            uint32_t h[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) h[b] = sh.hist[4 * lane + b];
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
        __syncthreads();
        const uint32_t d = sh.digit;
        need -= sh.above;
        prefix |= (uint64_t)d << shift;
        mask |= 255ull << shift;
        if (sh.bin == need || shift == 0) break;  // the whole bin is taken: done
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

// Sorts cand[0..n) descending (the buffer must hold the next power of two).
__device__ void bitonic_desc(uint64_t *cand, int n, SelectShared &sh, int tid)
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

// Sorts cand[0..n) descending through a bucket pass.  Keys are binned by
// their score part into kSortBins buckets spread evenly over the row's
// [min, max] score range (monotone, so bucket order is key order), scattered
// into bucket order in tmp, and every key finds its place inside its bucket
// by counting the larger keys there.  Buckets are small for spread-out
// scores; if any bucket holds more than kSortMaxBucket keys (many equal or
// clustered scores) the bitonic sort takes over.  `bins` has 2*kSortBins
// words, `tmp` n entries (not overlapping cand).  Returns nothing; cand ends
// up sorted either way.
constexpr int kSortBins = 2048;
constexpr int kSortMaxBucket = 64;

__device__ void bucket_sort_desc(uint64_t *cand, uint64_t *tmp, int n, uint32_t *bins,
                                 SelectShared &sh, int tid)
{
    const int lane = tid & 63;
    uint32_t *cnt = bins;               // bucket sizes, then insertion cursors
    uint32_t *off = bins + kSortBins;   // first slot of each bucket (descending order)
    // Score range of the keys (orderable, then as fp32 values).
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int e = tid; e < n; e += NT) {
        const uint32_t u = (uint32_t)(cand[e] >> 32);
        lo = u < lo ? u : lo;
        hi = u > hi ? u : hi;
    }
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t a = (uint32_t)__shfl_xor((int)lo, o), b = (uint32_t)__shfl_xor((int)hi, o);
        lo = a < lo ? a : lo;
        hi = b > hi ? b : hi;
    }
    for (int e = tid; e < kSortBins; e += NT) cnt[e] = 0u;
    if (lane == 0) {
        sh.wsum[tid >> 6] = lo;
        sh.wmin[tid >> 6] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
        lo = sh.wsum[w] < lo ? sh.wsum[w] : lo;
        hi = (uint32_t)sh.wmin[w] > hi ? (uint32_t)sh.wmin[w] : hi;
    }
    // Buckets evenly spaced in score value: b = floor((s - lo) * scale), a
    // monotone function of s, clamped to the bucket range.
    const float flo = score_of_orderable(lo), fhi = score_of_orderable(hi);
    const float scale = fhi > flo ? (float)(kSortBins - 1) / (fhi - flo) : 0.0f;
    auto bucket = [&](uint64_t key) -> uint32_t {
        const float x = (score_of_orderable((uint32_t)(key >> 32)) - flo) * scale;
        const int b = (int)x;
        return (uint32_t)(b < 0 ? 0 : (b > kSortBins - 1 ? kSortBins - 1 : b));
    };
    // Histogram of the buckets.
    for (int e0 = 0; e0 < n; e0 += NT) {
        const int e = e0 + tid;
        uint32_t b = 0;
        if (e < n) b = bucket(cand[e]);
        hist_add(cnt, e < n, b, lane);
    }
    __syncthreads();
    // off[b] = keys in buckets above b; largest bucket.
    constexpr int PB = kSortBins / NT;
    uint32_t c[PB];
    uint32_t mine = 0, big = 0;
#pragma unroll
    for (int i = 0; i < PB; ++i) {
        c[i] = cnt[kSortBins - 1 - (tid * PB + i)];  // thread order = descending buckets
        mine += c[i];
        big = c[i] > big ? c[i] : big;
    }
    uint32_t total;
    uint32_t run = block_exclusive_sum(mine, total, sh, tid);
#pragma unroll
    for (int i = 0; i < PB; ++i) {
        off[kSortBins - 1 - (tid * PB + i)] = run;
        run += c[i];
    }
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t x = (uint32_t)__shfl_xor((int)big, o);
        big = x > big ? x : big;
    }
    if (lane == 0) sh.wsum[tid >> 6] = big;
    for (int e = tid; e < kSortBins; e += NT) cnt[e] = 0u;  // now insertion cursors
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) big = sh.wsum[w] > big ? sh.wsum[w] : big;
    __syncthreads();
    if (big > (uint32_t)kSortMaxBucket) {  // uniform
        bitonic_desc(cand, n, sh, tid);
        return;
    }
    // Scatter into bucket order.
    for (int e = tid; e < n; e += NT) {
        const uint64_t key = cand[e];
        const uint32_t b = bucket(key);
        tmp[off[b] + atomicAdd(&cnt[b], 1u)] = key;
    }
    __syncthreads();
    // Place each key: its bucket's start plus the number of larger keys in it.
    for (int e = tid; e < n; e += NT) {
        const uint64_t key = tmp[e];
        const uint32_t b = bucket(key);
        const int o = (int)off[b], m = (int)cnt[b];
        int rk = 0;
        for (int q = o; q < o + m; ++q) rk += tmp[q] > key ? 1 : 0;
        cand[o + rk] = key;
    }
    __syncthreads();
}

// Appends the keys for which `take` holds to buf[*count...] (wave ballot,
// one LDS atomic per wave).  `take` may differ per lane; every lane of the
// block must call it the same number of times.
__device__ inline void append(uint64_t *buf, uint32_t *count, bool take, uint64_t key, int lane)
{
    const uint64_t m = __ballot(take);
    if (m == 0) return;  // wave-uniform: nothing to add
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(count, (uint32_t)__popcll(m));
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
    if (take) buf[base + lanes_below(m)] = key;
}

// Row context shared by the selection strategies below.
struct RowCtx {
    const float *src;  // the row's chunk scores
    int64_t len;       // keys of this row in the chunk
    uint32_t c0;       // first key index of the chunk
    bool filt;         // keys must beat u_floor (the running list is full)
    uint32_t u_floor;
};

// Reads the row's chunk scores in rounds of NT*16 (16 consecutive keys per
// thread, vector loads), sorts each key into class 0 (dropped), 1 (-> bufa)
// or 2 (-> bufb) with classify(score), and appends the kept keys to their
// buffer in key-index order (a block-wide prefix sum per round gives every
// thread its write offsets).  Returns the counts in na, nb.
template <class F>
__device__ void collect2(const RowCtx &r, F classify, uint64_t *bufa, uint64_t *bufb, int &na,
                         int &nb, SelectShared &sh, int tid)
{
    constexpr int V = 16;
    na = 0;
    nb = 0;
    for (int64_t e0 = 0; e0 < r.len; e0 += (int64_t)NT * V) {
        const int64_t base = e0 + (int64_t)tid * V;
        float v[V];
        if (base + V <= r.len) {
#pragma unroll
            for (int i = 0; i < V; i += 4) {
                const float4 x = *(const float4 *)(r.src + base + i);
                v[i] = x.x;
                v[i + 1] = x.y;
                v[i + 2] = x.z;
                v[i + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) v[i] = base + i < r.len ? r.src[base + i] : 0.0f;
        }
        uint32_t cls = 0, cnt = 0;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const uint32_t c = base + i < r.len ? classify(v[i]) : 0u;
            cls |= c << (2 * i);
            cnt += c == 1u ? 1u : (c == 2u ? 0x10000u : 0u);
        }
        uint32_t total;
        const uint32_t off = block_exclusive_sum(cnt, total, sh, tid);
        int oa = na + (int)(off & 0xFFFFu), ob = nb + (int)(off >> 16);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const uint32_t c = (cls >> (2 * i)) & 3u;
            if (c != 0u) {
                const uint64_t key = make_key(v[i], r.c0 + (uint32_t)(base + i));
                if (c == 1u) bufa[oa++] = key;
                else bufb[ob++] = key;
            }
        }
        na += (int)(total & 0xFFFFu);
        nb += (int)(total >> 16);
    }
    __syncthreads();
}

// Q = every chunk key that beats the floor (there are at most k of them).
__device__ int collect_all(uint64_t *cand, const RowCtx &r, SelectShared &sh, int tid)
{
    const bool filt = r.filt;
    const float f_floor = score_of_orderable(r.u_floor);
    int na, nb;
    collect2(r, [&](float x) -> uint32_t { return (!filt || x > f_floor) ? 1u : 0u; }, cand,
             cand, na, nb, sh, tid);
    return na;
}

// Q = the k best chunk keys that beat the floor, using the score kernel's
// histogram summary: keys above bin b* are all in, keys in b* compete for the
// remaining places by an exact radix select on their remaining bits.  The
// bin edges are turned into fp32 thresholds (orderable() is monotone), so a
// key is classified by two float compares.  When bin b* holds more keys than
// the boundary buffer, one extra pass histograms the next 8 bits of the keys
// in b* and narrows the boundary to one sub-bin.  Returns -1 if even the
// sub-bin does not fit (massively tied scores); the caller falls back.
__device__ int collect_by_bin(uint64_t *cand, const RowCtx &r, const ChunkMeta &mt, int k,
                              SelectShared &sh, int tid)
{
    uint64_t *bnd = cand + k;  // boundary entries
    const bool filt = r.filt;
    const float f_floor = score_of_orderable(r.u_floor);
    constexpr int BIN_SHIFT = 32 - kHistBits;  // orderable bits below the bin
    uint32_t lo_u = mt.bin << BIN_SHIFT;        // boundary: orderable in [lo_u, hi_u)
    uint32_t hi_u = (mt.bin + 1u) << BIN_SHIFT;
    int need = k - (int)mt.above;
    int first_shift = 64 - kHistBits - 8;
    if (mt.in_bin > (uint32_t)kSelectPiece) {
        // Histogram of orderable bits [BIN_SHIFT-8, BIN_SHIFT) inside bin b*.
        sh.hist[tid] = 0u;
        __syncthreads();
        const float f_lo = mt.bin == 0u ? -__builtin_inff() : score_of_orderable(lo_u);
        const float f_hi = score_of_orderable(hi_u);
        const int lane = tid & 63;
        for (int64_t e0 = 0; e0 < r.len; e0 += NT) {
            const int64_t e = e0 + tid;
            bool in = false;
            uint32_t d = 0;
            if (e < r.len) {
                const float x = r.src[e];
                in = (!filt || x > f_floor) && x >= f_lo && !(x >= f_hi);
                d = (orderable(x) >> (BIN_SHIFT - 8)) & 255u;
            }
            hist_add(sh.hist, in, d, lane);
        }
        __syncthreads();
        if (tid < 64) {
            uint32_t h4[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) h4[b] = sh.hist[4 * tid + b];
            const uint32_t local = h4[0] + h4[1] + h4[2] + h4[3];
            uint32_t incl = local;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_down(incl, off);
                if (tid + off < 64) incl += y;
            }
            uint32_t above = incl - local;
#pragma unroll
            for (int b = 3; b >= 0; --b) {
                if (above < (uint32_t)need && (uint32_t)need <= above + h4[b]) {
                    sh.digit = (uint32_t)(4 * tid + b);
                    sh.above = above;
                    sh.bin = h4[b];
                }
                above += h4[b];
            }
        }
        __syncthreads();
        const uint32_t dsub = sh.digit;
        need -= (int)sh.above;
        const uint32_t sub_cnt = sh.bin;
        __syncthreads();
        if (sub_cnt > (uint32_t)kSelectPiece) return -1;
        lo_u |= dsub << (BIN_SHIFT - 8);
        hi_u = lo_u + (1u << (BIN_SHIFT - 8));
        first_shift -= 8;
    }
    // Boundary edges as fp32 thresholds (bin 0 starts at -inf).
    const float f_sure = score_of_orderable(hi_u);
    const float f_edge = lo_u == 0u ? -__builtin_inff() : score_of_orderable(lo_u);
    int above, in_bin;
    collect2(
        r,
        [&](float x) -> uint32_t {
            if (filt && !(x > f_floor)) return 0u;
            return x >= f_sure ? 1u : (x >= f_edge ? 2u : 0u);
        },
        cand, bnd, above, in_bin, sh, tid);
    need = k - above;
    if (in_bin > need) radix_select(bnd, in_bin, need, sh, tid, first_shift);
    for (int e = tid; e < need; e += NT) cand[above + e] = bnd[e];
    __syncthreads();
    return k;
}

// Q = the k best chunk keys that beat the floor, without a summary: the chunk
// is read in pieces, keys that cannot enter the current best k are dropped,
// and the candidates are cut back to k by radix select whenever they exceed k.
__device__ int collect_pieces(uint64_t *cand, const RowCtx &r, int k, SelectShared &sh, int tid)
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
                const uint32_t u = orderable(r.src[p0 + e]);
                key = ((uint64_t)u << 32) |
                      (uint64_t)(0xFFFFFFFFu - (r.c0 + (uint32_t)(p0 + e)));
                take = (!r.filt || u > r.u_floor) && (!full || key > thr);
            }
            append(cand + cnt, &sh.count, take, key, lane);
        }
        __syncthreads();
        cnt += (int)sh.count;
        if (cnt > k) {
            radix_select(cand, cnt, k, sh, tid);
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

__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a)
{
    extern __shared__ uint64_t smem[];
    __shared__ SelectShared sh;
    const int k = (int)a.k;
    uint64_t *cand = smem;                      // k + kSelectPiece entries
    uint64_t *lst = smem + k + kSelectPiece;    // k entries (running list)
    const int tid = threadIdx.x;
    const int64_t rl = a.rows - 1 - (int64_t)blockIdx.x;  // long rows first
    const int64_t row = a.row0 + rl;
    const int64_t n = n_usable(a.q_pos0 + row, a.T, a.m);
    int64_t len = n - a.c0;
    len = len < 0 ? 0 : (len > a.clen ? a.clen : len);
    // Nothing to add and nothing to write: the running list stays as it is.
    // (The first chunk always runs so that every row's state is written.)
    if (!a.emit && !a.first && len == 0) return;

    int cnt_l = 0;
    uint64_t theta = 0;
    if (!a.first) {
        const RowState stt = a.state[rl];
        cnt_l = stt.count;
        theta = stt.theta;
        const uint64_t *src = a.lists + rl * a.k;
        for (int e = tid; e < cnt_l; e += NT) lst[e] = src[e];
    }

    RowCtx r;
    r.src = a.ws + rl * a.clen;
    r.len = len;
    r.c0 = (uint32_t)a.c0;
    r.filt = theta != 0;
    r.u_floor = (uint32_t)(theta >> 32);

    // Chunk-local best k (the partition step), sorted descending.
    int cnt_q = 0;
    if (len > 0) {
        if (a.meta) {
            const ChunkMeta mt = a.meta[rl];
            if (mt.total <= (uint32_t)k) {
                cnt_q = collect_all(cand, r, sh, tid);
            } else {
                cnt_q = collect_by_bin(cand, r, mt, k, sh, tid);
                if (cnt_q < 0) cnt_q = collect_pieces(cand, r, k, sh, tid);
            }
        } else {
            cnt_q = collect_pieces(cand, r, k, sh, tid);
        }
    }
    __syncthreads();
    if (cnt_q > 1) {
        uint64_t *tmp = cand + k;  // free once Q sits in cand[0..k)
        uint32_t *bins = (uint32_t *)(smem + k + kSelectPiece + (a.first ? 0 : k));
        if (cnt_q > 64) bucket_sort_desc(cand, tmp, cnt_q, bins, sh, tid);
        else bitonic_desc(cand, cnt_q, sh, tid);
    }

    // Merge with the running list (both sorted descending) and write the
    // first min(k, |L| + |Q|) entries: merge-path split per thread.
    const int total = min(k, cnt_l + cnt_q);
    constexpr int PT = (2048 + NT - 1) / NT;  // outputs per thread (k <= 2048)
    const int p0 = tid * PT;
    uint64_t outv[PT];
    uint64_t kth = 0;  // the entry at position k-1, for the next chunk's floor
    int nout = 0;
    if (p0 < total) {
        int lo = max(0, p0 - cnt_q), hi = min(p0, cnt_l);
        while (lo < hi) {  // i = entries taken from L before position p0
            const int mid = (lo + hi) >> 1;
            if (lst[mid] > cand[p0 - 1 - mid]) lo = mid + 1;
            else hi = mid;
        }
        int i = lo, j = p0 - lo;
        for (int t = 0; t < PT; ++t) {
            if (p0 + t >= total) break;
            uint64_t v;
            if (j >= cnt_q || (i < cnt_l && lst[i] > cand[j])) v = lst[i++];
            else v = cand[j++];
            outv[t] = v;
            if (p0 + t == k - 1) kth = v;
            ++nout;
        }
    }
    if (a.emit) {
        int32_t *oi = a.out_idx + row * a.k;
        float *os = a.out_score + row * a.k;
        for (int t = 0; t < PT; ++t) {
            const int p = p0 + t;
            if (p >= k) break;
            if (t < nout) {
                oi[p] = key_index(outv[t]);
                os[p] = key_score(outv[t]);
            } else {
                oi[p] = -1;
                os[p] = -__builtin_inff();
            }
        }
        // Rows with k > 2048 do not exist (k <= CSA_MAX_K); positions beyond
        // NT*PT are covered because NT*PT >= k.
    } else {
        uint64_t *dst = a.lists + rl * a.k;
        for (int t = 0; t < nout; ++t) dst[p0 + t] = outv[t];
        if (total == k && p0 <= k - 1 && k - 1 < p0 + nout) a.state[rl].theta = kth;
        if (tid == 0) {
            a.state[rl].count = total;
            if (total < k) a.state[rl].theta = 0;
        }
    }
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t stream)
{
    if (a.rows <= 0) return hipSuccess;
    const size_t entries = (size_t)(a.k + kSelectPiece) + (a.first ? 0 : (size_t)a.k);
    const size_t lds = entries * sizeof(uint64_t) + 2 * kSortBins * sizeof(uint32_t);
    select_kernel<<<dim3((unsigned)a.rows), dim3(NT), lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace csa
