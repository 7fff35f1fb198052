// Chunk scoring kernels of the CSA lightning indexer for gfx950.
//
// Operation (page "StreamIndex: Memory-Bounded Compressed Sparse Attention via
// Streaming Top-k", Abstract: the lightning indexer scores the compressed
// keys for every query with H_I heads): for each query row i of a batch and
// each usable key j of one key chunk
//
//     s(i,j) = sum_h w[i,h] * max(q[i,h,:] . kc[j,:], 0)
//
// and the result for the chunk goes to a workspace slice [rows][clen].  Only
// the head-reduced score leaves the kernel; the per-head logits live in
// registers, so the [S,H_I,T] tensor never exists.
//
// bf16 path: the contraction over the head dimension is a dense GEMM
// [H_I, D_I] x [D_I, N] per query, run on the MFMA units with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  A workgroup holds 8 query
// rows, one per wave; each wave keeps its query's q fragments (64 heads x 128
// dims = 64 VGPRs) and head weights resident and streams key tiles of NT keys
// that the whole workgroup stages, double-buffered, through LDS.  In the
// 32x32 accumulator layout a lane owns one key column and 16 head rows per
// 32-head block, so the ReLU and the weighted head sum run in registers with
// a single cross-half exchange at the end.
#include "csa_internal.h"

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float bf16_bits_to_float(uint16_t b)
{
    return __uint_as_float(((uint32_t)b) << 16);
}

// D: head dimension; HT: 32-head blocks (1 for H <= 32, else 2); NT: keys per
// LDS tile.  Block = 8 waves, one query row each.  Grid: x = query blocks of
// the batch (heaviest, i.e. latest, rows first), y = key spans of the chunk.
template <int D, int HT, int NT>
__global__ __launch_bounds__(512) void score_bf16_kernel(ScoreArgs a)
{
    constexpr int KSTEPS = D / 16;     // MFMA k-steps over the head dimension
    constexpr int CH = D / 8;          // 16-byte chunks per key row
    constexpr int ROWB = D * 2;        // bytes per key row
    constexpr int TILEB = NT * ROWB;   // bytes per LDS tile
    constexpr int NCHUNK = NT * CH;    // 16-byte chunks per tile
    constexpr int PER = (NCHUNK + 511) / 512;
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;   // which 8-wide k slice / which 4-row group
    const int col = lane & 31;    // key column (B, C) or head row (A)

    const int64_t nqb = (a.rows + kScoreWaves - 1) / kScoreWaves;
    const int64_t qb = nqb - 1 - (int64_t)blockIdx.x;
    const int64_t rl = qb * kScoreWaves + wave;       // row within the batch
    const bool active = rl < a.rows;
    const int64_t last = min(qb * kScoreWaves + kScoreWaves - 1, a.rows - 1);
    const int64_t n_hi = n_usable(a.q_pos0 + a.row0 + last, a.T, a.m);
    const int64_t kb0 = a.c0 + (int64_t)blockIdx.y * a.kspan;
    const int64_t kcap = min(a.c0 + a.clen, kb0 + a.kspan);
    const int64_t k_end = min(kcap, n_hi);
    if (kb0 >= k_end) return;  // uniform over the workgroup
    const int64_t my_end =
        active ? min(kcap, n_usable(a.q_pos0 + a.row0 + rl, a.T, a.m)) : kb0;
    const int ntiles = (int)((k_end - kb0 + NT - 1) / NT);

    // Resident A operand: q[row, ht*32 + col, ks*16 + half*8 .. +7].
    bf16x8 qf[HT][KSTEPS];
    float wv[HT][16];
    {
        const int64_t row = a.row0 + (active ? rl : 0);
        const __bf16 *qrow = (const __bf16 *)a.q + row * (int64_t)a.H * D;
        const uint16_t *wrow = (const uint16_t *)a.w + row * (int64_t)a.H;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int h = ht * 32 + col;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                bf16x8 v = {};
                if (active && h < a.H)
                    v = *(const bf16x8 *)(qrow + (int64_t)h * D + ks * 16 + half * 8);
                qf[ht][ks] = v;
            }
            // Head row held by accumulator register r of this lane.
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int hr = ht * 32 + ((r >> 2) << 3) + (half << 2) + (r & 3);
                wv[ht][r] = (active && hr < a.H) ? bf16_bits_to_float(wrow[hr]) : 0.0f;
            }
        }
    }

    // Key tile staging: tile t holds keys kb0 + t*NT .. +NT-1, row-major with
    // the 16-byte chunk index XOR-swizzled by the key so that the 32 lanes of
    // a B-fragment read fall in distinct bank groups.
    u32x4 st[PER];
    auto gload = [&](int t) {
        const int64_t base = kb0 + (int64_t)t * NT;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = p * 512 + tid;
            const int key = c / CH;
            const int ch = c % CH;
            const int64_t gk = base + key;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (c < NCHUNK && gk < k_end)
                v = *(const u32x4 *)((const uint16_t *)a.kc + gk * D + ch * 8);
            st[p] = v;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = p * 512 + tid;
            if (c < NCHUNK) {
                const int key = c / CH;
                const int ch = c % CH;
                *(u32x4 *)(lds + buf * TILEB + key * ROWB + ((ch ^ (key & (CH - 1))) << 4)) = st[p];
            }
        }
    };

    float *wsrow = a.ws + (active ? rl : 0) * a.clen - a.c0;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const bool more = t + 1 < ntiles;
        if (more) gload(t + 1);
        const int64_t base = kb0 + (int64_t)t * NT;
        if (active && base < my_end) {
            const unsigned char *tb = lds + (t & 1) * TILEB;
#pragma unroll
            for (int kb = 0; kb < NT / 32; ++kb) {
                const int key = kb * 32 + col;
                f32x16 acc[HT];
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    const int ch = 2 * ks + half;
                    const bf16x8 b =
                        *(const bf16x8 *)(tb + key * ROWB + ((ch ^ (key & (CH - 1))) << 4));
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht)
                        acc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ht][ks], b, acc[ht],
                                                                          0, 0, 0);
                }
                // ReLU and weighted head sum; this lane holds 16 of each
                // 32-head block's rows for key `key`, the other half-wave the
                // other 16.
                float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) s0 = fmaf(wv[0][r], fmaxf(acc[0][r], 0.0f), s0);
                if constexpr (HT == 2) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) s1 = fmaf(wv[1][r], fmaxf(acc[1][r], 0.0f), s1);
                }
                float s = s0 + s1;
                s = s + __shfl_xor(s, 32);
                const int64_t gk = base + key;
                if (half == 0 && gk < my_end) wsrow[gk] = s;
            }
        }
        if (more) lstore((t + 1) & 1);
        __syncthreads();
    }
}

// fp32 path: one workgroup per (row, 256-key block); one thread per key.
// The head dimension loop is plain fp32 FMA.
template <int D>
__global__ __launch_bounds__(256) void score_f32_kernel(ScoreArgs a)
{
    __shared__ float qs[64 * D];
    __shared__ float wsh[64];
    const int tid = threadIdx.x;
    const int64_t rl = (int64_t)blockIdx.x;
    const int64_t row = a.row0 + rl;
    const int64_t n = n_usable(a.q_pos0 + row, a.T, a.m);
    const int64_t kend = min(a.c0 + a.clen, n);
    const int64_t k0 = a.c0 + (int64_t)blockIdx.y * 256;
    if (k0 >= kend) return;
    const int H = a.H;
    const float *qrow = (const float *)a.q + row * (int64_t)H * D;
    for (int e = tid; e < H * D; e += 256) qs[e] = qrow[e];
    for (int e = tid; e < H; e += 256) wsh[e] = ((const float *)a.w)[row * H + e];
    __syncthreads();
    const int64_t gk = k0 + tid;
    if (gk >= kend) return;
    const float *key = (const float *)a.kc + gk * D;
    float kr[D];
#pragma unroll
    for (int d = 0; d < D; ++d) kr[d] = key[d];
    float s = 0.0f;
    for (int h = 0; h < H; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc = fmaf(qs[h * D + d], kr[d], acc);
        s = fmaf(wsh[h], fmaxf(acc, 0.0f), s);
    }
    a.ws[rl * a.clen + (gk - a.c0)] = s;
}

template <int D, int HT>
hipError_t launch_bf16_tile(const ScoreArgs &a, int32_t key_tile, dim3 grid, hipStream_t s)
{
    switch (key_tile) {
    case 64: score_bf16_kernel<D, HT, 64><<<grid, 512, 0, s>>>(a); break;
    case 128: score_bf16_kernel<D, HT, 128><<<grid, 512, 0, s>>>(a); break;
    case 256: score_bf16_kernel<D, HT, 256><<<grid, 512, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(const ScoreArgs &a, int32_t key_tile, dim3 grid, hipStream_t s)
{
    if (a.H <= 32) return launch_bf16_tile<D, 1>(a, key_tile, grid, s);
    return launch_bf16_tile<D, 2>(a, key_tile, grid, s);
}

}  // namespace

hipError_t launch_score(const ScoreArgs &a, int32_t dtype, int32_t D, int32_t key_tile,
                        int64_t ysplit, hipStream_t stream)
{
    if (a.rows <= 0) return hipSuccess;
    if (dtype == DT_BF16) {
        const int64_t nqb = (a.rows + kScoreWaves - 1) / kScoreWaves;
        dim3 grid((unsigned)nqb, (unsigned)ysplit);
        switch (D) {
        case 32: return launch_bf16_d<32>(a, key_tile, grid, stream);
        case 64: return launch_bf16_d<64>(a, key_tile, grid, stream);
        case 128: return launch_bf16_d<128>(a, key_tile, grid, stream);
        default: return hipErrorInvalidValue;
        }
    }
    dim3 grid((unsigned)a.rows, (unsigned)((a.clen + 255) / 256));
    switch (D) {
    case 32: score_f32_kernel<32><<<grid, 256, 0, stream>>>(a); break;
    case 64: score_f32_kernel<64><<<grid, 256, 0, stream>>>(a); break;
    case 128: score_f32_kernel<128><<<grid, 256, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace csa
