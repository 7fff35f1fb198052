// Chunk scoring kernels of the CSA lightning indexer for gfx950.
//
// Operation (page "StreamIndex: Memory-Bounded Compressed Sparse Attention via
// Streaming Top-k", Abstract: the lightning indexer scores the compressed
// keys for every query with H_I heads): for each query row i of a batch and
// each usable key j of one key chunk
//
//     s(i,j) = sum_h w[i,h] * max(q[i,h,:] . kc[j,:], 0)
//
// and the result for the chunk goes to a workspace slice [rows][clen], each
// score stored as its orderable() integer (the monotone fp32 -> u32 map that
// the selection compares).  Only the head-reduced score leaves the kernel;
// the per-head logits live in registers, so the [S,H_I,T] tensor never
// exists.
//
// bf16 path: the contraction over the head dimension is a dense GEMM
// [H_I, D_I] x [D_I, N] per query, run on the MFMA units with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  A workgroup holds 8 query
// rows, one per wave; each wave keeps its query's q fragments (64 heads x 128
// dims = 64 VGPRs) and head weights resident and streams key tiles of NT keys
// that the whole workgroup brings into LDS (by LDS DMA, double-buffered).  In
// the 32x32 accumulator layout a lane owns one key column and 16 rows of each
// 32-head block, so the ReLU and the weighted head sum run in registers, with
// one cross-half swap at the end.  A second grid dimension can split the
// chunk's keys (few query rows, e.g. decoding); the kernel details are at
// score_bf16_kernel below.
//
// fp32 path: the same contraction on v_mfma_f32_32x32x2_f32, with q resident
// in registers and 32-key tiles staged in LDS (score_f32_kernel below).
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

// Buffer resource of `bytes` bytes at `base` (raw, stride 0); accesses at
// or beyond `bytes` read 0 and write nothing.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// One 16-byte LDS DMA per lane: bytes [off, off+16) of the buffer land at
// dst + 16*lane (dst wave-uniform).  A plain device function: inside a
// lambda of the kernel template the host pass drops the kernel's stub.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, unsigned char *dst, int off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)dst, 16,
                                            off, 0, 0, 0);
}

// orderable() for scores that are never -0: every score here is a sum that
// starts at +0, and under round-to-nearest such a sum is never -0.
__device__ inline uint32_t orderable_nz(float s)
{
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ReLU on the bit pattern: a float with the sign bit set is a negative
// integer, so an integer max with 0 maps every negative score (and -0) to +0
// and leaves the rest unchanged, in one instruction and with no NaN quieting.
__device__ inline float relu_bits(float x)
{
    return __int_as_float(max(__float_as_int(x), 0));
}

// Chunk summary of one wave's row histogram h (kHistBins counts over the
// top bits of the orderable scores of the keys it counted): the bin b* that
// holds the need-th best counted key, the counts above b* and in it, and the
// total counted (with total <= need only the total matters).  One lane of
// the wave writes *dst.
__device__ __forceinline__ void write_chunk_summary(const uint32_t *h, int lane, uint32_t need,
                                                    ChunkMeta *dst)
{
    constexpr int PERL = kHistBins / 64;
    uint32_t mine = 0;
#pragma unroll 8
    for (int i = 0; i < PERL; ++i) mine += h[lane * PERL + i];
    uint32_t incl = mine;  // sum over lanes >= this lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(incl, off);
        if (lane + off < 64) incl += y;
    }
    const uint32_t total = __shfl(incl, 0);
    ChunkMeta m = {0u, 0u, 0u, total};
    if (total > need) {
        const uint32_t above_lane = incl - mine;
        const bool here = above_lane < need && need <= incl;
        const uint64_t who = __ballot(here);
        const int src = __builtin_ctzll(who);
        if (lane == src) {
            uint32_t above = above_lane;
            for (int i = PERL - 1; i >= 0; --i) {
                const uint32_t c = h[lane * PERL + i];
                if (above + c >= need) {
                    m.bin = (uint32_t)(lane * PERL + i);
                    m.above = above;
                    m.in_bin = c;
                    break;
                }
                above += c;
            }
            *dst = m;
        }
    } else if (lane == 0) {
        *dst = m;
    }
}

// D: head dimension; HT: 32-head blocks (ceil(H/32), at most 2); NT: keys
// per LDS tile; DB: double-buffered tiles.  Block = 8 waves, one query row
// each, covering the whole chunk for its rows.  Grid: query blocks of the
// batch, heaviest (latest) rows first.
//
// MFMA shape: v_mfma_f32_32x32x16_bf16 with A = q (32 heads x 16 dims, held
// in registers for the whole chunk) and B = kc (16 dims x 32 keys, read from
// LDS).  The 32x32 shape keeps eight issue slots of matrix work per MFMA
// instruction, which leaves the VALU room for the epilogue (MFMA and VALU
// instructions share the issue port).  In the accumulator layout lane l owns
// key column l%32 and 16 of each 32-head block's rows, so the ReLU and the
// weighted head sum run in registers.
//
// Pipeline per 32-key block kb, in half-block steps (4 of the 8 k-steps):
// the B fragments of the next step are read from LDS while the MFMAs of this
// step run, and the VALU epilogue of block kb-1 is spread over the two steps
// of block kb.  Blocks are finished in pairs: one 32-lane swap combines the
// two halves of each block's head sum and leaves lane l with the score of key
// 64*pair + l, so stores and histogram updates use all 64 lanes.
//
// Besides the scores, each wave builds an LDS histogram of its row's
// orderable scores (top 11 bits) over the chunk keys that beat the row's
// running k-th key theta, and at the end of the chunk reduces it to the bin
// b* that holds the k-th best of those keys (ChunkMeta).  The select kernel
// then only has to look at keys in bins >= b*.
template <int D, int HT, int NT, bool DB, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void score_bf16_kernel(ScoreArgs a)
{
    constexpr int THREADS = WAVES * 64;
    constexpr int KSTEPS = D / 16;     // MFMA k-steps over the head dimension
    constexpr int HALF = KSTEPS / 2;   // k-steps per pipeline step
    constexpr int CH = D / 8;          // 16-byte chunks per key row
    constexpr int ROWB = D * 2;        // bytes per key row
    constexpr int TILEB = NT * ROWB;   // bytes per LDS tile
    constexpr int NB = NT / 32;        // 32-key blocks per tile
    static_assert(NB % 2 == 0, "blocks are finished in pairs");
    // LDS: double-buffered key tiles are two static arrays (so that the
    // compiler can tell the tile being read from the tile being filled by
    // DMA); the row histograms, and the single-buffered tile, are dynamic.
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ __attribute__((aligned(16))) unsigned char tile_a[DB ? TILEB : 16];
    __shared__ __attribute__((aligned(16))) unsigned char tile_b[DB ? TILEB : 16];
    unsigned char *lds = smem;
    uint32_t *hist_all = (uint32_t *)(smem + (DB ? 0 : TILEB));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;   // which 8-dim k slice (A, B) / which 4-row group (C)
    const int col = lane & 31;    // key column (B, C) or head row (A)

    const int64_t nqb = (a.rows + WAVES - 1) / WAVES;
    const int64_t qb = nqb - 1 - (int64_t)blockIdx.x;
    const int64_t rl = qb * WAVES + wave;       // row within the batch
    const bool active = rl < a.rows;
    const int64_t last = min(qb * WAVES + WAVES - 1, a.rows - 1);
    const int64_t n_hi = n_usable(a.q_pos0 + a.row0 + last, a.T, a.m);
    // Keys of this workgroup: split blockIdx.y of the chunk.
    const int64_t split = (int64_t)blockIdx.y;
    const int64_t kb0 = a.c0 + split * a.slen;
    const int64_t kcap = min(a.c0 + a.clen, kb0 + a.slen);
    const int64_t k_end = min(kcap, n_hi);
    if (kb0 >= k_end) return;  // uniform: no row of this block has a key here
    const int64_t my_end =
        active ? min(kcap, n_usable(a.q_pos0 + a.row0 + rl, a.T, a.m)) : kb0;
    const int ntiles = (int)((k_end - kb0 + NT - 1) / NT);

    // Keys must beat the row's running k-th key to matter; chunk keys come
    // after every key already in the list, so on equal scores they lose and
    // the test is on the score part alone.
    uint32_t u_floor = 0;
    bool filt = false;
    if (active && a.state) {
        const uint64_t th = a.state[rl].theta;
        filt = th != 0;
        u_floor = (uint32_t)(th >> 32);
    }

    for (int e = tid; e < WAVES * kHistBins; e += THREADS) hist_all[e] = 0u;

    // Resident A operand: q[row, ht*32 + col, ks*16 + half*8 .. +7], and the
    // head weights of the accumulator rows this lane holds.  Every load is
    // unconditional (rows and heads clamped to valid ones, results zeroed
    // afterwards) so that all of them are in flight at once.
    bf16x8 qf[HT][KSTEPS];
    float wv[HT][16];
    {
        const int64_t row = a.row0 + (active ? rl : 0);
        const __bf16 *qrow = (const __bf16 *)a.q + row * (int64_t)a.H * D;
        const uint16_t *wrow = (const uint16_t *)a.w + row * (int64_t)a.H;
        uint16_t wraw[HT][16];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int h = min(ht * 32 + col, a.H - 1);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                qf[ht][ks] = *(const bf16x8 *)(qrow + (int64_t)h * D + ks * 16 + half * 8);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                wraw[ht][r] = wrow[min(ht * 32 + ((r >> 2) << 3) + (half << 2) + (r & 3), a.H - 1)];
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const bool hv = active && ht * 32 + col < a.H;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                if (!hv) qf[ht][ks] = bf16x8{};
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int hr = ht * 32 + ((r >> 2) << 3) + (half << 2) + (r & 3);
                wv[ht][r] = (active && hr < a.H) ? bf16_bits_to_float(wraw[ht][r]) : 0.0f;
            }
        }
    }

    // Key tile staging: tile t holds keys kb0 + t*NT .. +NT-1, row-major with
    // the 16-byte chunk slot of chunk ch of key `key` at ch ^ (key % CH), so
    // that the 16 lanes of each B-fragment read group fall in distinct bank
    // groups.  The next tile is loaded into registers while the current one
    // is computed and written to LDS after it.  (LDS DMA would save these
    // registers, but then every LDS histogram update would wait for all
    // outstanding global memory operations.)  Each tile is read through a
    // buffer resource that ends at the last usable key, so the per-thread
    // offsets are constants and keys past the end read as zeros (their
    // scores are never used).
    constexpr int NCHUNK = NT * CH;                // 16-byte chunks per tile
    constexpr int PER = (NCHUNK + THREADS - 1) / THREADS;      // chunks per thread
    u32x4 st[PER];
    auto gload = [&](int t) {
        const int64_t base = kb0 + (int64_t)t * NT;
        const int64_t nk = min((int64_t)NT, k_end - base);
        const __amdgpu_buffer_rsrc_t rs =
            buffer_rsrc((const uint16_t *)a.kc + base * D, (uint32_t)(nk * ROWB));
#pragma unroll
        for (int p = 0; p < PER; ++p)
            st[p] = __builtin_amdgcn_raw_buffer_load_b128(rs, (p * THREADS + tid) * 16, 0, 0);
    };
    // Double-buffered tiles are filled by LDS DMA: each wave moves 1 KiB
    // pieces, lane l of a piece landing at byte 16*l of it.  The lane loads
    // the global chunk that the swizzled layout puts there, so the tile in
    // LDS is the same as with register staging, without staging registers or
    // LDS writes.
    constexpr int NPIECE = TILEB / 1024;
    constexpr int PIECES_W = (NPIECE + WAVES - 1) / WAVES;  // pieces per wave
    int dma_off[PIECES_W];
#pragma unroll
    for (int j = 0; j < PIECES_W; ++j) {
        const int pos = (j * WAVES + wave) * 1024 + lane * 16;  // byte in the tile
        const int key = pos / ROWB;
        const int slot = (pos % ROWB) >> 4;
        dma_off[j] = key * ROWB + ((slot ^ (key & (CH - 1))) << 4);
    }
    auto dma = [&](unsigned char *dst, int t) {
        const int64_t base = kb0 + (int64_t)t * NT;
        const int64_t nk = min((int64_t)NT, k_end - base);
        const __amdgpu_buffer_rsrc_t rs =
            buffer_rsrc((const uint16_t *)a.kc + base * D, (uint32_t)(nk * ROWB));
#pragma unroll
        for (int j = 0; j < PIECES_W; ++j) {
            if (j * WAVES + wave < NPIECE)  // wave-uniform
                dma16(rs, dst + (j * WAVES + wave) * 1024, dma_off[j]);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = p * THREADS + tid;
            if (c < NCHUNK) {
                const int key = c / CH;
                const int ch = c % CH;
                *(u32x4 *)(lds + buf * TILEB + key * ROWB + ((ch ^ (key & (CH - 1))) << 4)) = st[p];
            }
        }
    };
    // Lane offsets of the B fragments inside a 32-key block: key col, chunk
    // 2*ks + half, swizzled by col % CH (block starts are multiples of 32
    // keys, so the swizzle does not depend on the block).
    int boff[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
        boff[ks] = col * ROWB + (((2 * ks + half) ^ (col & (CH - 1))) << 4);
    // B fragments of half-step hs (k-steps hs*HALF .. +HALF-1) of block kb.
    auto load_b = [&](const unsigned char *tb, int kb, int hs, bf16x8 (&b)[HALF]) {
#pragma unroll
        for (int j = 0; j < HALF; ++j)
            b[j] = *(const bf16x8 *)(tb + kb * 32 * ROWB + boff[hs * HALF + j]);
    };
    auto mfma_half = [&](const bf16x8 (&b)[HALF], int hs, f32x16 (&acc)[HT]) {
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                if (hs == 0 && j == 0)
                    acc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ht][0], b[0], f32x16{}, 0, 0, 0);
                else
                    acc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ht][hs * HALF + j], b[j],
                                                                      acc[ht], 0, 0, 0);
            }
        }
    };

    // Scores are stored and counted 64 keys at a time (2 blocks): chunk-
    // relative 32-bit key offsets, one lane per key.
    uint32_t *wsrow = a.ws + (active ? rl : 0) * a.clen + split * a.slen;
    const __amdgpu_buffer_rsrc_t ws_rs = buffer_rsrc(wsrow, (uint32_t)((kcap - kb0) * 4));
    const int my_len = (int)(my_end - kb0);  // keys of this row in the chunk
    uint32_t *h = hist_all + wave * kHistBins;

    // Per-lane share of one block, over register half rh (8 of the 16
    // accumulator rows of each 32-head block): ReLU and weighted sum, one
    // FMA chain in a fixed order (rows of half 0 of every head block, then
    // half 1).
    auto partial = [&](const f32x16 (&acc)[HT], int rh, float &sum) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
            for (int r = rh * 8; r < rh * 8 + 8; ++r)
                sum = fmaf(wv[ht][r], relu_bits(acc[ht][r]), sum);
        }
    };
    // Finishes blocks 2p and 2p+1 (pe, po: each lane's share of them).  The
    // 32-lane swap pairs the two half-waves, so lane l ends with the score of
    // key 64p + l, summed as (lanes 0-31 share) + (lanes 32-63 share).
    // Branch-free, so that the tile stays one scheduling region: lanes past
    // the row's last key store into unused slots of the row or, where a
    // 192-key tile runs past the end of the split (a multiple of 256 keys),
    // beyond the buffer range, where the store is dropped; they add 0 to the
    // histogram.
    auto finish2 = [&](float pe, float po, int rel0, bool real) {
        const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(pe), __float_as_uint(po),
                                                        false, false);
        const float sc = __uint_as_float(z[0]) + __uint_as_float(z[1]);
        const uint32_t u = orderable_nz(sc);
        const int rel = rel0 + lane;
        const bool valid = real && rel < my_len;
        __builtin_amdgcn_raw_buffer_store_b32(u, ws_rs, lane * 4, rel0 * 4, 0);
        const uint32_t inc = (valid && (!filt || u > u_floor)) ? 1u : 0u;
        // A plain LDS atomic here would make the compiler wait for every
        // tile DMA in flight; the add does not touch the tiles.
        const uint32_t hp = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t *)(
            h + (u >> (32 - kHistBits)));
        asm volatile("ds_add_u32 %0, %1" ::"v"(hp), "v"(inc));
    };

    // The last block of a tile is finished under the first block's MFMAs of
    // the wave's next tile (or flushed when there is none): acc[1] and the
    // pair state carry over the tile boundary.  On a wave's first tile the
    // carried slot holds zeros and its finish counts nothing; its store goes
    // to slots 0..63 of the row, which the tile's own first pair overwrites.
    f32x16 acc[2][HT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[i][ht] = f32x16{};
    float pe_c = 0.0f;  // even-block share of the carried pair
    int rel_c = 0;      // first key of the carried pair
    bool pend = false;  // a carried pair is waiting
    auto flush = [&]() {
        float pacc = 0.0f;
        partial(acc[1], 0, pacc);
        partial(acc[1], 1, pacc);
        finish2(pe_c, pacc, rel_c, true);
        pend = false;
    };

    // B fragments of two half-steps; with double-buffered tiles bb[0] holds
    // the next tile's first fragments when a tile starts (read early, see
    // the tile loop below).
    bf16x8 bb[2][HALF];
    // retire(): the barrier of a double-buffered tile and what follows it,
    // called by every wave once per tile; a wave with work in the tile calls
    // it before the tile's last step (whose B fragments are in registers by
    // then), so that the next tile's first LDS reads overlap that step's
    // MFMAs instead of stalling every wave after the barrier.
    auto compute_tile = [&](const unsigned char *tb, int t, auto &&retire) {
        const int rel_t = t * NT;  // tile start relative to the chunk
        if (active && rel_t < my_len) {
            float pacc = 0.0f;  // share of the block being finished
            float pe = 0.0f;    // share of the even block of the current pair
            const bool real_c = pend;
            if constexpr (!DB) load_b(tb, 0, 0, bb[0]);
#pragma unroll
            for (int step = 0; step < 2 * NB; ++step) {
                const int kb = step >> 1, hs = step & 1;
                if (step + 1 < 2 * NB)
                    load_b(tb, (step + 1) >> 1, (step + 1) & 1, bb[(step + 1) & 1]);
                if constexpr (DB) {
                    if (step == 2 * NB - 1) retire();
                }
                // Keep the prefetch here, one step ahead of its use.
                __builtin_amdgcn_sched_barrier(0);
                mfma_half(bb[step & 1], hs, acc[kb & 1]);
                // Half hs of the previous block's epilogue, under these MFMAs
                // (for kb == 0 the previous block is the carried one, acc[1]).
                if (hs == 0) pacc = 0.0f;
                partial(acc[(kb + 1) & 1], hs, pacc);
                if (hs == 1) {
                    if (kb == 0) finish2(pe_c, pacc, rel_c, real_c);
                    else if (((kb - 1) & 1) == 0) pe = pacc;
                    else finish2(pe, pacc, rel_t + (kb - 2) * 32, true);
                }
            }
            pe_c = pe;  // the tile's last pair (blocks NB-2, NB-1) is carried
            rel_c = rel_t + (NB - 2) * 32;
            pend = true;
        } else {
            if (pend) flush();
            if constexpr (DB) retire();
        }
    };
    auto no_retire = []() {};

    if constexpr (DB) {
        // Tile t+1 is DMA'd into the other buffer while tile t is computed.
        // The barrier that retires tile t (its fence waits for the DMA of
        // tile t+1) makes tile t+1 visible and frees tile t's buffer for
        // the DMA of tile t+2, which is issued right after it together with
        // the first B-fragment reads of tile t+1.  Unrolled by two so that
        // every access names its buffer at compile time.
        dma(tile_a, 0);
        __syncthreads();
        if (ntiles > 1) dma(tile_b, 1);
        if (active && my_len > 0) load_b(tile_a, 0, 0, bb[0]);
        for (int t = 0; t < ntiles; t += 2) {
            compute_tile(tile_a, t, [&]() {
                __syncthreads();
                if (t + 2 < ntiles) dma(tile_a, t + 2);
                if (t + 1 < ntiles && active && (t + 1) * NT < my_len) load_b(tile_b, 0, 0, bb[0]);
            });
            if (t + 1 >= ntiles) break;
            compute_tile(tile_b, t + 1, [&]() {
                __syncthreads();
                if (t + 3 < ntiles) dma(tile_b, t + 3);
                if (t + 2 < ntiles && active && (t + 2) * NT < my_len) load_b(tile_a, 0, 0, bb[0]);
            });
        }
    } else {
        gload(0);
        lstore(0);
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
            const bool more = t + 1 < ntiles;
            if (more) gload(t + 1);
            compute_tile(lds, t, no_retire);
            if (more) {
                __syncthreads();  // single buffer: all reads done
                lstore(0);
            }
            __syncthreads();
        }
    }
    if (pend) flush();

    // Chunk summary: locate the bin that holds the k-th best counted key.
    if (active && a.meta) write_chunk_summary(h, lane, (uint32_t)a.k, a.meta + split * a.rows + rl);
}

// fp32 path on the matrix cores: v_mfma_f32_32x32x2_f32 (the fp32 matrix
// rate equals the fp32 vector peak, and the products leave the VALU free).
// Workgroup: 8 waves, one query row each, over the keys of one chunk (or of
// one split of it, blockIdx.y), heaviest rows first, as in the bf16 kernel.
// A = q, 32 heads x 2 dims per MFMA, resident in registers for the whole
// workgroup; B = kc, 2 dims x 32 keys, from a 32-key LDS tile that all
// waves stage together, double-buffered behind one barrier per tile.
// k-step s covers dims 2s (lanes 0-31) and 2s+1 (lanes 32-63); each key's
// LDS row holds its even dims, then its odd dims, so one 16-byte read gives
// a lane four consecutive k-steps.  The accumulator layout is that of the
// bf16 kernel: lane l owns key l%32 and 16 of each 32-head block's rows, so
// ReLU and the weighted head sum run in registers and one 32-lane swap adds
// the two half-waves' shares.  Each wave also builds its row's histogram
// and chunk summary exactly as the bf16 kernel does.
template <int D, int HT>
__global__ __launch_bounds__(512) void score_f32_kernel(ScoreArgs a)
{
    constexpr int KS = D / 2;        // k-steps
    constexpr int ROW = D + 4;       // LDS floats per key row (padded against bank conflicts)
    constexpr int TILE = 32 * ROW;   // LDS floats per 32-key tile
    constexpr int F4 = 8 * D;        // 16-byte pieces of a tile in global memory
    constexpr int PER = (F4 + 511) / 512;
    __shared__ __attribute__((aligned(16))) float tile[2][TILE];
    __shared__ uint32_t hist_all[8 * kHistBins];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int c = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int64_t nqb = (a.rows + 7) / 8;
    const int64_t qb = nqb - 1 - (int64_t)blockIdx.x;
    const int64_t rl = qb * 8 + wave;
    const bool active = rl < a.rows;
    const int64_t last = min(qb * 8 + 7, a.rows - 1);
    const int64_t n_hi = n_usable(a.q_pos0 + a.row0 + last, a.T, a.m);
    const int64_t split = (int64_t)blockIdx.y;
    const int64_t kb0 = a.c0 + split * a.slen;
    const int64_t kcap = min(a.c0 + a.clen, kb0 + a.slen);
    const int64_t k_end = min(kcap, n_hi);
    if (kb0 >= k_end) return;  // uniform: no row of this block has a key here
    const int64_t my_end =
        active ? min(kcap, n_usable(a.q_pos0 + a.row0 + rl, a.T, a.m)) : kb0;

    // Keys must beat the row's running k-th key to be counted (chunk keys
    // come after every key already in the list, so equal scores lose).
    uint32_t u_floor = 0;
    bool filt = false;
    if (active && a.state) {
        const uint64_t th = a.state[rl].theta;
        filt = th != 0;
        u_floor = (uint32_t)(th >> 32);
    }
    for (int e = tid; e < 8 * kHistBins; e += 512) hist_all[e] = 0u;
    uint32_t *h = hist_all + wave * kHistBins;

    // Resident A operand and the weights of this lane's accumulator rows
    // (heads past H, and inactive rows, are zero).
    float qa[HT][KS];
    float wv[HT][16];
    {
        const int64_t row = a.row0 + (active ? rl : 0);
        const float *qrow = (const float *)a.q + row * (int64_t)a.H * D;
        const float *wrow = (const float *)a.w + row * (int64_t)a.H;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int hq = min(ht * 32 + c, a.H - 1);
            const bool hv = active && ht * 32 + c < a.H;
#pragma unroll
            for (int i = 0; i < D / 4; ++i) {
                const float4 x = *(const float4 *)(qrow + (int64_t)hq * D + 4 * i);
                qa[ht][2 * i] = hv ? (half ? x.y : x.x) : 0.0f;      // dim 4i + half
                qa[ht][2 * i + 1] = hv ? (half ? x.w : x.z) : 0.0f;  // dim 4i + 2 + half
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int hr = ht * 32 + ((r >> 2) << 3) + (half << 2) + (r & 3);
                wv[ht][r] = (active && hr < a.H) ? wrow[min(hr, a.H - 1)] : 0.0f;
            }
        }
    }

    // Tile staging: piece f = key * D/4 + i holds dims 4i..4i+3 of the key;
    // its even dims go to row positions 2i, 2i+1 and its odd dims to KS + 2i,
    // KS + 2i + 1.  Keys past k_end read the last usable key (never stored).
    float4 st[PER];
    auto gload = [&](int t) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int f = p * 512 + tid;
            if (f < F4) {
                const int64_t key = min(kb0 + (int64_t)t * 32 + f / (D / 4), k_end - 1);
                st[p] = *(const float4 *)((const float *)a.kc + key * D + 4 * (f % (D / 4)));
            }
        }
    };
    auto lstore = [&](float *dst) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int f = p * 512 + tid;
            if (f < F4) {
                float *r = dst + (f / (D / 4)) * ROW + 2 * (f % (D / 4));
                *(float2 *)r = make_float2(st[p].x, st[p].z);
                *(float2 *)(r + KS) = make_float2(st[p].y, st[p].w);
            }
        }
    };

    uint32_t *wsrow = a.ws + (active ? rl : 0) * a.clen;
    const int nblk = (int)((k_end - kb0 + 31) / 32);
    gload(0);
    lstore(tile[0]);
    __syncthreads();  // also orders the histogram clear before any count
    for (int blk = 0; blk < nblk; ++blk) {
        if (blk + 1 < nblk) gload(blk + 1);
        const float *tb = tile[blk & 1] + c * ROW + half * KS;
        f32x16 acc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x16{};
#pragma unroll
        for (int j = 0; j < KS / 4; ++j) {
            const float4 b = *(const float4 *)(tb + 4 * j);
            const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
                    acc[ht] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[ht][4 * j + t], bv[t], acc[ht],
                                                                   0, 0, 0);
        }
        // This lane's share of key c's score (its 16 rows of each head
        // block), then the other half-wave's share.
        float part = 0.0f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r) part = fmaf(wv[ht][r], fmaxf(acc[ht][r], 0.0f), part);
        const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                        false, false);
        const uint32_t u = orderable(__uint_as_float(z[0]) + __uint_as_float(z[1]));
        const int64_t key = kb0 + (int64_t)blk * 32 + c;
        if (half == 0 && key < my_end) {
            wsrow[key - a.c0] = u;
            if (!filt || u > u_floor) atomicAdd(&h[u >> (32 - kHistBits)], 1u);
        }
        if (blk + 1 < nblk) lstore(tile[(blk + 1) & 1]);
        __syncthreads();
    }

    // Chunk summary: locate the bin that holds the k-th best counted key.
    if (active && a.meta) write_chunk_summary(h, lane, (uint32_t)a.k, a.meta + split * a.rows + rl);
}

template <int D, int HT, int NT, bool DB, int WAVES>
hipError_t launch_bf16_cfg(const ScoreArgs &a, hipStream_t s)
{
    // Dynamic part: the histograms, plus the tile when single-buffered (the
    // double-buffered tiles are static arrays of the kernel).
    constexpr size_t lds = (DB ? 0 : (size_t)NT * D * 2) +
                           (size_t)WAVES * kHistBins * sizeof(uint32_t);
    static_assert(lds + (DB ? 2 * (size_t)NT * D * 2 : 0) <= 160 * 1024,
                  "LDS budget of a gfx950 workgroup");
    static std::atomic<uint64_t> attr_done{0};
    const hipError_t e =
        set_dynamic_lds((const void *)score_bf16_kernel<D, HT, NT, DB, WAVES>, (int)lds, attr_done);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((a.rows + WAVES - 1) / WAVES),
                    (unsigned)((a.clen + a.slen - 1) / a.slen));
    score_bf16_kernel<D, HT, NT, DB, WAVES><<<grid, WAVES * 64, lds, s>>>(a);
    return hipGetLastError();
}

template <int D, int HT, int NT, bool DB, int WAVES>
int blocks_per_cu_cfg()
{
    constexpr size_t lds = (DB ? 0 : (size_t)NT * D * 2) +
                           (size_t)WAVES * kHistBins * sizeof(uint32_t);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, (const void *)score_bf16_kernel<D, HT, NT, DB, WAVES>, WAVES * 64, lds) !=
        hipSuccess)
        return 0;
    return n;
}

template <int D, int HT>
int blocks_per_cu_tile(int32_t key_tile)
{
    switch (key_tile) {
    case 64: return blocks_per_cu_cfg<D, HT, 64, true, 8>();
    case 128: return blocks_per_cu_cfg<D, HT, 128, true, 8>();
    case 192: return blocks_per_cu_cfg<D, HT, 192, true, 8>();
    case 256: return blocks_per_cu_cfg<D, HT, 256, (D < 128), 8>();
    default: return 0;
    }
}

template <int D, int HT>
hipError_t launch_bf16_tile(const ScoreArgs &a, int32_t key_tile, hipStream_t s)
{
    // 8-row workgroups, one per CU; 256-key tiles of 128 dims are
    // single-buffered to stay within 160 KiB next to the 64 KiB of
    // histograms, while two 192-key tiles (2 x 48 KiB) fill it exactly: the
    // automatic choice, with a third fewer tile barriers than 128-key tiles.
    // (Two 4-row workgroups per CU were measured slower.)
    switch (key_tile) {
    case 64: return launch_bf16_cfg<D, HT, 64, true, 8>(a, s);
    case 128: return launch_bf16_cfg<D, HT, 128, true, 8>(a, s);
    case 192: return launch_bf16_cfg<D, HT, 192, true, 8>(a, s);
    case 256: return launch_bf16_cfg<D, HT, 256, (D < 128), 8>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_bf16_d(const ScoreArgs &a, int32_t key_tile, hipStream_t s)
{
    if (a.H <= 32) return launch_bf16_tile<D, 1>(a, key_tile, s);
    return launch_bf16_tile<D, 2>(a, key_tile, s);
}

template <int D, int HT>
int blocks_per_cu_f32()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void *)score_f32_kernel<D, HT>, 512,
                                                     0) != hipSuccess)
        return 0;
    return n;
}

}  // namespace

int score_blocks_per_cu(int32_t dtype, int32_t D, int32_t H, int32_t key_tile)
{
    const bool two = H > 32;
    if (dtype != DT_BF16) {
        switch (D) {
        case 32: return two ? blocks_per_cu_f32<32, 2>() : blocks_per_cu_f32<32, 1>();
        case 64: return two ? blocks_per_cu_f32<64, 2>() : blocks_per_cu_f32<64, 1>();
        case 128: return two ? blocks_per_cu_f32<128, 2>() : blocks_per_cu_f32<128, 1>();
        default: return 0;
        }
    }
    switch (D) {
    case 32: return two ? blocks_per_cu_tile<32, 2>(key_tile) : blocks_per_cu_tile<32, 1>(key_tile);
    case 64: return two ? blocks_per_cu_tile<64, 2>(key_tile) : blocks_per_cu_tile<64, 1>(key_tile);
    case 128:
        return two ? blocks_per_cu_tile<128, 2>(key_tile) : blocks_per_cu_tile<128, 1>(key_tile);
    default: return 0;
    }
}

hipError_t launch_score(const ScoreArgs &a, int32_t dtype, int32_t D, int32_t key_tile,
                        hipStream_t stream)
{
    if (a.rows <= 0) return hipSuccess;
    if (dtype == DT_BF16) {
        switch (D) {
        case 32: return launch_bf16_d<32>(a, key_tile, stream);
        case 64: return launch_bf16_d<64>(a, key_tile, stream);
        case 128: return launch_bf16_d<128>(a, key_tile, stream);
        default: return hipErrorInvalidValue;
        }
    }
    const dim3 grid((unsigned)((a.rows + 7) / 8), (unsigned)((a.clen + a.slen - 1) / a.slen));
    const bool two = a.H > 32;
    switch (D) {
    case 32:
        if (two) score_f32_kernel<32, 2><<<grid, 512, 0, stream>>>(a);
        else score_f32_kernel<32, 1><<<grid, 512, 0, stream>>>(a);
        break;
    case 64:
        if (two) score_f32_kernel<64, 2><<<grid, 512, 0, stream>>>(a);
        else score_f32_kernel<64, 1><<<grid, 512, 0, stream>>>(a);
        break;
    case 128:
        if (two) score_f32_kernel<128, 2><<<grid, 512, 0, stream>>>(a);
        else score_f32_kernel<128, 1><<<grid, 512, 0, stream>>>(a);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace csa
