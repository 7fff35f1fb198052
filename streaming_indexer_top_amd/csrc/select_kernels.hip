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

__device__ inline uint64_t make_key(float s, uint32_t j)
{
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;  // -0 -> +0
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - j);
}

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
    uint32_t count;
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
__device__ void radix_select(uint64_t *cand, int cnt, int k, SelectShared &sh, int tid)
{
    const int lane = tid & 63;
    uint32_t need = (uint32_t)k;
    uint64_t prefix = 0, mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
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
        if (sh.bin == need) break;  // the whole bin is taken: done
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

// Sorts cand[0..n) descending (n <= cap, cap a power of two >= 2 available).
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

__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a)
{
    extern __shared__ uint64_t cand[];  // k + kSelectPiece entries
    __shared__ SelectShared sh;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t rl = a.rows - 1 - (int64_t)blockIdx.x;  // long rows first
    const int64_t row = a.row0 + rl;
    const int64_t n = n_usable(a.q_pos0 + row, a.T, a.m);
    int64_t len = n - a.c0;
    len = len < 0 ? 0 : (len > a.clen ? a.clen : len);
    const int k = (int)a.k;
    // Nothing to add and nothing to write: the running list stays as it is.
    // (The first chunk always runs so that every row's count is written.)
    if (!a.emit && !a.first && len == 0) return;

    int cnt = 0;
    if (!a.first) {
        cnt = a.counts[rl];
        const uint64_t *lst = a.lists + rl * a.k;
        for (int e = tid; e < cnt; e += NT) cand[e] = lst[e];
        __syncthreads();
    }
    bool full = cnt >= k;
    uint64_t thr = full ? block_min(cand, cnt, sh, tid) : 0ull;

    const float *src = a.ws + rl * a.clen;
    for (int64_t p0 = 0; p0 < len; p0 += kSelectPiece) {
        const int plen = (int)min((int64_t)kSelectPiece, len - p0);
        if (tid == 0) sh.count = 0u;
        __syncthreads();
        const int rounds = (plen + NT - 1) / NT;
        for (int rd = 0; rd < rounds; ++rd) {
            const int e = rd * NT + tid;
            bool take = false;
            uint64_t key = 0;
            if (e < plen) {
                key = make_key(src[p0 + e], (uint32_t)(a.c0 + p0 + e));
                take = !full || key > thr;
            }
            const uint64_t m = __ballot(take);
            uint32_t base = 0;
            if (lane == 0 && m) base = atomicAdd(&sh.count, (uint32_t)__popcll(m));
            base = (uint32_t)__shfl((int)base, 0);
            if (take) cand[cnt + base + lanes_below(m)] = key;
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

    if (a.emit) {
        if (cnt > 1) bitonic_desc(cand, cnt, sh, tid);
        int32_t *oi = a.out_idx + row * a.k;
        float *os = a.out_score + row * a.k;
        for (int t = tid; t < k; t += NT) {
            if (t < cnt) {
                const uint64_t key = cand[t];
                oi[t] = key_index(key);
                os[t] = key_score(key);
            } else {
                oi[t] = -1;
                os[t] = -__builtin_inff();
            }
        }
    } else {
        uint64_t *lst = a.lists + rl * a.k;
        for (int e = tid; e < cnt; e += NT) lst[e] = cand[e];
        if (tid == 0) a.counts[rl] = cnt;
    }
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t stream)
{
    if (a.rows <= 0) return hipSuccess;
    const size_t lds = (size_t)(a.k + kSelectPiece) * sizeof(uint64_t);
    select_kernel<<<dim3((unsigned)a.rows), dim3(NT), lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace csa
