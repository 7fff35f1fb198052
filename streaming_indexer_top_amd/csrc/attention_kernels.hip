// Sparse attention over the entries the lightning indexer selected, for gfx950.
//
// The page "StreamIndex: Memory-Bounded Compressed Sparse Attention via
// Streaming Top-k" (Abstract) ends the CSA pipeline with a sparse attention
// kernel that reads only the selected compressed entries.  It gives no
// formula or dimensions for it; this kernel computes the plain softmax
// attention of each query row over its selected entries in the shared-latent
// (multi-query) form: all H heads attend over the same entries, an entry's
// latent row is the key (dk dims) and its first dv dims are the value:
//
//   out[i,h,:] = sum_{e in sel(i)} p_{h,e} kv[e,:dv],
//   p_{h,e} = softmax over e of (scale * q[i,h,:] . kv[e,:])
//
// sel(i) = idx[i,:] without its -1 padding; an empty selection gives zeros.
//
// Two kernels, one workgroup per query row each.  For 64 heads,
// attention_split_kernel (further down) gives half of its 8 waves the logits
// and softmax and the other half P * V, one barrier per 32-entry tile.  For
// 32 heads, attention_kernel runs 4 waves per 32-head block.  Wave (hb, qq)
// keeps its heads' q for k-steps qq*KQ .. qq*KQ+KQ-1 resident (a quarter of
// dk), so every wave of a head block computes a partial 32x32 logit block per
// 32-entry tile with v_mfma_f32_32x32x16_bf16; the four partials meet in LDS.
// The selected latent rows are gathered by LDS DMA into the free one of
// three static tile buffers: each lane moves the 16 bytes its slot of the
// swizzled tile needs, straight from the row the index names (-1 reads
// zeros through the buffer range check).  The gather of tile t+2 starts at
// the beginning of tile step t and has until the end of that step.  The
// barriers inside the loop carry no memory fence (a fence would wait for
// every DMA in flight); the wait for a tile's DMAs is an explicit vmcnt
// before the barrier that publishes it.  Tile step t has
// two intervals between barriers:
//   1. wave qq of a head block finishes 8 of its 32 heads for tile t: sums
//      the four partial logit quarters in a fixed order, masks padding and
//      runs an online softmax in base 2 whose reference max moves only when
//      a head's max rises by more than 2^8 (the factor then rescales the
//      accumulators; otherwise they are left alone), and writes P (bf16,
//      transposed: one 8-byte store per lane) to LDS; under this vector
//      work the same waves' MFMAs compute the partial logits of tile t+1
//      (B fragments from the tile),
//   2. the partials of tile t+1 go to LDS, and P * V of tile t runs with
//      v_mfma_f32_32x32x16_bf16, wave qq owning a quarter of the dv output
//      dims: the V fragments (8 consecutive entries of one dim per lane)
//      come from the row-major tile by ds_read_b64_tr_b16, two transposing
//      8-byte reads per fragment.
// The softmax denominators are kept per lane and reduced once at the end.
#include "csa_internal.h"

#include <type_traits>

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;      // selected entries per tile
constexpr float kTau = 8.0f;   // a head's reference max moves when its max rises by more than this (log2 units)
constexpr int kPRow = 36;      // P^T row stride in bf16 elements (32 heads + padding against bank conflicts)

__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Tile swizzle: slot s of tile row r (16-byte slots, in groups of eight per
// 128 bytes) holds chunk s ^ sw8(r) of the row.  Rows are 1152 bytes apart,
// a multiple of 128, so without it every row would start on the same bank.
// The map sends row bits 0, 1, 2, 3 to slot bits 1, 2, 0, 1: the logit
// fragment read (eight or sixteen consecutive rows, one chunk each) and the
// transposing value read (four consecutive rows, four chunks each) then hit
// every bank once, whether the LDS serves 128 or 256 bytes a cycle.
__device__ inline int sw8(int r)
{
    return ((r >> 2) & 1) | (((r ^ (r >> 3)) & 1) << 1) | (((r >> 1) & 1) << 2);
}

// Transposing LDS read: within each 16-lane group, lane o receives element
// o%4 of the 8-byte rows that lanes o/4, o/4+4, o/4+8, o/4+12 point at.
__device__ inline i16x4 read_tr16(const unsigned char *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4 __attribute__((address_space(3))) *)(p));
}

// Max over the 32 lanes of each half-wave, returned to every lane of that
// half: DPP shifts within rows of 16 lanes, one row broadcast to the next
// row, then the last lane of each half read back.
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_f32(float v)
{
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

__device__ inline float half_max(float x)
{
    x = fmaxf(x, dpp_f32<0x111, 0xF>(x));  // row_shr:1
    x = fmaxf(x, dpp_f32<0x112, 0xF>(x));  // row_shr:2
    x = fmaxf(x, dpp_f32<0x114, 0xF>(x));  // row_shr:4
    x = fmaxf(x, dpp_f32<0x118, 0xF>(x));  // row_shr:8
    x = fmaxf(x, dpp_f32<0x142, 0xA>(x));  // row_bcast:15 into rows 1 and 3
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
    const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
    return (threadIdx.x & 32) ? hi : lo;
}

// Barrier without a memory fence: the compiler's fence would also wait for
// every LDS DMA in flight.  The wave's own LDS accesses are complete after
// lgkmcnt(0); the "memory" clobber keeps the compiler from moving memory
// accesses across it.
__device__ inline void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The head block's four rescale flags and both P fragments of a tile (four
// transposing 8-byte reads of P^T, as for the value fragments), read in one
// asm block with its own wait: as plain loads, the compiler's wait placement
// puts a wait for every DMA in flight before them, and one wait for all of
// them saves an LDS round trip before the P * V MFMAs.
__device__ inline uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ inline void lds_read_fp(const int *f, const __bf16 *p00, const __bf16 *p01, const __bf16 *p10,
                                   const __bf16 *p11, u32x4 &fl, i16x4 &t00, i16x4 &t01, i16x4 &t10, i16x4 &t11)
{
    asm volatile("ds_read_b128 %0, %5\n\tds_read_b64_tr_b16 %1, %6\n\tds_read_b64_tr_b16 %2, %7\n\t"
                 "ds_read_b64_tr_b16 %3, %8\n\tds_read_b64_tr_b16 %4, %9\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(fl), "=&v"(t00), "=&v"(t01), "=&v"(t10), "=&v"(t11)
                 : "v"(lds_addr(f)), "v"(lds_addr(p00)), "v"(lds_addr(p01)), "v"(lds_addr(p10)), "v"(lds_addr(p11))
                 : "memory");
}

// LDS stores of P and of the rescale factors, written as asm: the compiler
// cannot tell that they miss the tile a gather is filling, and as plain
// stores it would put a wait for every gather in flight before them.  The
// waits that order them are explicit (the barrier's lgkmcnt(0)).
__device__ inline void lds_store_b64(void *p, i16x4 v)
{
    asm volatile("ds_write_b64 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ inline void lds_store_b32(void *p, float v)
{
    asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}

// s_waitcnt vmcnt(N) (expcnt, lgkmcnt left alone), as the builtin so that
// the compiler's own wait placement knows about it.
template <int N>
__device__ inline void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One 16-byte LDS DMA per lane: bytes [off, off+16) of the buffer land at
// dst + 16*lane (dst wave-uniform).
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, unsigned char *dst, int off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)dst, 16,
                                            off, 0, 0, 0);
}

template <int DK, int DV, int HB>
__global__ __launch_bounds__(256 * HB) void attention_kernel(AttnArgs a)
{
    constexpr int WAVES = 4 * HB;
    constexpr int KQ = DK / 64;         // 16-dim k-steps per quarter of dk
    constexpr int NBW = DV / 128;       // 32-dim output blocks per wave
    constexpr int ROWB = DK * 2;        // bytes per latent row
    constexpr int TILEB = kTile * ROWB; // bytes per tile
    constexpr int NPIECE = TILEB / 1024;
    constexpr int PPW = (NPIECE + WAVES - 1) / WAVES;  // DMA pieces per wave
    static_assert(DK % 64 == 0 && DV % 128 == 0 && DV <= DK, "shape");
    static_assert(TILEB % 1024 == 0 && (DK / 8) % 8 == 0, "whole DMA pieces, 8-chunk swizzle");

    __shared__ __attribute__((aligned(16))) unsigned char tile0[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char tile1[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char tile2[TILEB];
    // part[w][r-1]: quad r (r = 1..3) of wave w's partial logits, for the
    // wave of its head block that finishes those heads.
    __shared__ __attribute__((aligned(16))) f32x4 part[WAVES][3][64];
    // P transposed: pT[hb][entry][head], read as the A fragments of P * V
    // by the same transposing loads as the value fragments.
    __shared__ __attribute__((aligned(16))) __bf16 pT[HB][kTile][kPRow];
    __shared__ __attribute__((aligned(16))) float alpha_s[HB * 32];
    __shared__ __attribute__((aligned(16))) float l_s[HB * 32];
    __shared__ __attribute__((aligned(16))) int flag_s[WAVES];
    __shared__ __attribute__((aligned(16))) unsigned char sink[1024];  // target of the spare DMAs

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hb = wave >> 2, qq = wave & 3;
    const int col = lane & 31, half = lane >> 5;
    const int64_t row = blockIdx.x;
    const int k = a.k;
    const int ntiles = (k + kTile - 1) / kTile;
    const int32_t *irow = a.idx + row * (int64_t)k;
    const int nkv = (int)a.T;  // an index outside [0, T) counts as padding

    // Resident q, heads rotated by 8*qq: A row r of this wave is head
    // hb*32 + (r + 8qq) % 32, so accumulator quad 0 (rows 4half .. 4half+3)
    // holds the heads this wave finishes (8qq + 4half + ii) and quad r the
    // heads of wave (qq + r) % 4.  Dims (qq*KQ + j)*16 + half*8 .. +7.
    bf16x8 qf[KQ];
    {
        const int head = hb * 32 + ((col + 8 * qq) & 31);
        const __bf16 *qh = (const __bf16 *)a.q + ((int64_t)row * a.H + head) * DK;
#pragma unroll
        for (int j = 0; j < KQ; ++j) qf[j] = *(const bf16x8 *)(qh + (qq * KQ + j) * 16 + half * 8);
    }
    // Wait for q here, ahead of the gather loads: otherwise the compiler
    // may place that wait in the tile loop, where it also waits for the
    // gather loads in flight.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // Entry index of tile row (lane % 32) of tile t; rows past k read the
    // last index (a valid address) and are masked where used.
    auto load_idx = [&](int t) -> int { return irow[min(t * kTile + col, k - 1)]; };
    // Gather of one tile: piece p of the tile is 1 KiB; its lane l holds
    // bytes [16l, 16l+16) of the piece, i.e. row r, slot s of the tile,
    // which is chunk s ^ sw8(r) of latent row idx[r] (the swizzle spreads a
    // B-fragment read over the banks).  Per piece the lane's row (as a
    // bpermute byte address) and chunk byte offset are fixed for the row.
    const __amdgpu_buffer_rsrc_t kv_rs = buffer_rsrc(a.kv, (uint32_t)(a.T * ROWB));
    int g_row[PPW], g_chunk[PPW];
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
        const int pos = (j * WAVES + wave) * 1024 + lane * 16;
        const int r = (pos / ROWB) & 31;  // pieces past the tile (p >= NPIECE) go to the sink
        g_row[j] = r * 4;
        // Spare pieces (the sink's) get an offset that is out of range for
        // any real row.
        g_chunk[j] = j * WAVES + wave < NPIECE ? (((pos % ROWB) >> 4) ^ sw8(r)) * 16 : (int)0x80000000;
    }
    // DMA gather of tile t into dst, rows from iv (idx of tile t).  Every
    // wave issues exactly PPW DMAs per call, whatever t: pieces past the
    // tile go to the sink, rows past k (all of them for t >= ntiles) read
    // zeros, so the count of memory ops in flight is the same on every
    // path and the waits can count on it.
    auto gdma = [&](unsigned char *dst, int iv, int t) {
        const int lim = k - t * kTile;  // rows r >= lim are past k
        // Byte offset of this lane's row (lane % 32); a negative index, or a
        // row past k, gets bit 31: out of the buffer's range, so the DMAs of
        // that row write zeros.
        const int eoff = (iv >= 0 && iv < nkv && col < lim) ? iv * ROWB : (int)0x80000000;
        int e[PPW];
#pragma unroll
        for (int j = 0; j < PPW; ++j) e[j] = __builtin_amdgcn_ds_bpermute(g_row[j], eoff);
#pragma unroll
        for (int j = 0; j < PPW; ++j) {
            const int p = j * WAVES + wave;
            dma16(kv_rs, p < NPIECE ? dst + p * 1024 : sink, e[j] + g_chunk[j]);
        }
    };
    f32x16 o[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) o[nb] = f32x16{};
    // Reference max, the threshold mref + kTau and the per-lane denominators
    // of heads 8qq + 4half + ii.
    float mref[4], thr[4], lsum[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        mref[ii] = -__builtin_inff();
        thr[ii] = -__builtin_inff();
        lsum[ii] = 0.0f;
    }
    const float c2 = a.scale_log2e;

    // Per-lane byte offsets inside a tile, fixed for the whole row.
    // Logit B fragments: entry col, chunk 2*(qq*KQ + j) + half, swizzled.
    int qk_off[KQ];
#pragma unroll
    for (int j = 0; j < KQ; ++j)
        qk_off[j] = col * ROWB + (((2 * (qq * KQ + j) + half) ^ sw8(col)) << 4);
    // Value fragments read by the transposing loads: this lane points at
    // entry kk*16 + eb + 4*s2 (s2: first or second half of its 8 entries),
    // dims dl..dl+3 of output block nb; inside a tile that is byte
    //   kk*16*ROWB + hi(nb) + tr_off[s2][parity(nb)]
    // where hi(nb) is the 128-byte group of the block's chunks and the
    // parity picks which half of that group, which the swizzle (sw8(entry))
    // permutes per lane.
    const int eb = ((lane >> 5) * 8) + ((lane & 15) >> 2);
    const int dl = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int cq = qq * (DV / 32);  // first output chunk of this wave
    int tr_off[2][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const int e = eb + 4 * s2;
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int bp = ((cq >> 2) + par) & 1;  // bit 2 of the block's first chunk
            tr_off[s2][par] = e * ROWB + (((bp * 4 + (dl >> 3)) ^ sw8(e)) << 4) + (dl & 7) * 2;
        }
    }

    // Logits of tile t+1 are computed during the softmax of tile t: the
    // MFMAs run while the same waves do the vector work.  acc holds them
    // from the first interval of a step to the second; own keeps this
    // wave's quarter of its own heads (quad 0) for the next softmax.
    f32x16 acc = {};
    f32x4 own = {};
    auto qk = [&](const unsigned char *tb) {
        acc = f32x16{};
#pragma unroll
        for (int j = 0; j < KQ; ++j) {
            const bf16x8 b = *(const bf16x8 *)(tb + qk_off[j]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[j], b, acc, 0, 0, 0);
        }
    };
    auto write_parts = [&]() {
        own = f32x4{acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
        for (int r4 = 1; r4 < 4; ++r4)  // quad 0 stays: this wave finishes those heads
            part[wave][r4 - 1][lane] = f32x4{acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
    };

    // Step t, two intervals.  First: the idx of tile t+3 and the gather of
    // tile t+2 (into the buffer tile t-1 left), this wave's logit sums of
    // tile t (own quarter, then waves qq+1, qq+2, qq+3: a fixed order), the
    // logit MFMAs of tile t+1, and the softmax of tile t (P, factors and
    // flag to LDS).  Second: the partial logits of tile t+1 to LDS, then
    // O = alpha * O + P V of tile t; the gather of tile t+2 is waited for
    // before the barrier that ends the step.  tb: tile t; tn: tile t+1;
    // dst: the buffer of tile t+2; ivc: idx of tile t, replaced by idx of
    // tile t+3; ivd: idx of tile t+2.
    auto step = [&](const unsigned char *tb, const unsigned char *tn, unsigned char *dst, int &ivc,
                    int ivd, int t) {
        const uint32_t vmask = (uint32_t)__ballot(ivc >= 0 && ivc < nkv && t * kTile + col < k);
        ivc = load_idx(t + 3);
        gdma(dst, ivd, t + 2);
        f32x4 s = own;
#pragma unroll
        for (int d = 1; d < 4; ++d) s += part[hb * 4 + ((qq + d) & 3)][3 - d][lane];
        if (t + 1 < ntiles) qk(tn);
        const bool valid = (vmask >> col) & 1u;
        float x[4];
        bool exceed = false;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            x[ii] = s[ii] * c2;
            exceed |= x[ii] > thr[ii];
        }
        exceed = exceed && valid;
        // A head's reference max moves only when some logit of the tile
        // exceeds it by more than kTau; usually none does, and the tile
        // maxima are not needed at all.
        const bool wave_need = __ballot(exceed) != 0;  // wave-uniform
        if (wave_need) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const float mx = half_max(valid ? x[ii] : -__builtin_inff());
                float alpha = 1.0f;
                if (mx > thr[ii]) {
                    alpha = __builtin_amdgcn_exp2f(mref[ii] - mx);
                    mref[ii] = mx;
                    thr[ii] = mx + kTau;
                    lsum[ii] *= alpha;
                }
                if (col == 0) alpha_s[hb * 32 + 8 * qq + 4 * half + ii] = alpha;
            }
        }
        i16x4 pw;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            // A present entry has a finite reference max (its logit set
            // one if none was); an absent one gets 0.
            const float p = valid ? __builtin_amdgcn_exp2f(x[ii] - mref[ii]) : 0.0f;
            lsum[ii] += p;
            pw[ii] = __builtin_bit_cast(short, (__bf16)p);
        }
        *(i16x4 *)&pT[hb][col][8 * qq + 4 * half] = pw;
        if (lane == 0) flag_s[wave] = wave_need ? 1 : 0;
        lds_barrier();
        if (t + 1 < ntiles) write_parts();
        // 3. O = alpha * O + P V for head block hb, dims qq*DV/4 .. +DV/4-1.
        u32x4 fl;
        i16x4 t00, t01, t10, t11;
        lds_read_fp(&flag_s[hb * 4], &pT[hb][eb][dl], &pT[hb][eb + 4][dl], &pT[hb][16 + eb][dl],
                    &pT[hb][16 + eb + 4][dl], fl, t00, t01, t10, t11);
        const i16x8 pa0 = {t00[0], t00[1], t00[2], t00[3], t01[0], t01[1], t01[2], t01[3]};
        const i16x8 pa1 = {t10[0], t10[1], t10[2], t10[3], t11[0], t11[1], t11[2], t11[3]};
        const bf16x8 pab[2] = {__builtin_bit_cast(bf16x8, pa0), __builtin_bit_cast(bf16x8, pa1)};
        const bool resc = __builtin_amdgcn_readfirstlane((int)(fl[0] | fl[1] | fl[2] | fl[3])) != 0;  // block-uniform
        if (resc) {
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                // A wave whose flag is clear wrote no factors this tile:
                // its heads keep 1.
                f32x4 al = *(const f32x4 *)&alpha_s[hb * 32 + 8 * j4 + 4 * half];
                if (fl[j4] == 0u) al = f32x4{1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) o[nb][4 * j4 + ii] *= al[ii];
            }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 pa = pab[kk];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int hi = ((cq + nb * 4) & ~7) * 16;  // wave-uniform
                const unsigned char *vb = tb + kk * 16 * ROWB + hi;
                const i16x4 v0 = read_tr16(vb + tr_off[0][nb & 1]);
                const i16x4 v1 = read_tr16(vb + tr_off[1][nb & 1]);
                const i16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, __builtin_bit_cast(bf16x8, vv),
                                                                o[nb], 0, 0, 0);
            }
        }
        vm_wait<0>();
        lds_barrier();
    };

    // Tiles rotate through the three buffers and three idx registers (the
    // loop is unrolled by three so that every access names its buffer).
    int iv0 = -1, iv1 = -1, iv2 = -1;
    if (ntiles > 0) {
        iv0 = load_idx(0);
        iv1 = load_idx(1);
        iv2 = load_idx(2);
        gdma(tile0, iv0, 0);
        gdma(tile1, iv1, 1);
        vm_wait<0>();
    }
    __syncthreads();
    if (ntiles > 0) {
        qk(tile0);
        write_parts();
    }
    __syncthreads();
    for (int t = 0; t < ntiles; t += 3) {
        step(tile0, tile1, tile2, iv0, iv2, t);
        if (t + 1 >= ntiles) break;
        step(tile1, tile2, tile0, iv1, iv0, t + 1);
        if (t + 2 >= ntiles) break;
        step(tile2, tile0, tile1, iv2, iv1, t + 2);
    }
    __syncthreads();

    // Denominators: sum the per-lane shares of each head over its 32 lanes.
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        float l = lsum[ii];
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) l += __shfl_xor(l, off);
        if (col == 0) l_s[hb * 32 + 8 * qq + 4 * half + ii] = l;
    }
    __syncthreads();
    __bf16 *orow = (__bf16 *)a.out + (int64_t)row * a.H * DV;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4 l4 = *(const f32x4 *)&l_s[hb * 32 + 8 * j4 + 4 * half];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int head = hb * 32 + 8 * j4 + 4 * half + ii;
            const float inv = l4[ii] > 0.0f ? 1.0f / l4[ii] : 0.0f;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int dim = qq * (DV / 4) + nb * 32 + col;
                orow[(int64_t)head * DV + dim] = (__bf16)(o[nb][4 * j4 + ii] * inv);
            }
        }
    }
}

// Role-split form for 64 heads: one workgroup of 8 waves per query row and
// one barrier per 32-entry tile step.  Waves w and w+4 of a workgroup share a
// SIMD, so every SIMD runs one logit wave and one output wave.
//   Logit waves 0..3: wave (hb, kh) keeps q of head block hb (32 heads) for
//   half kh of the dk k-steps and computes a partial 32x32 logit block per
//   tile (one MFMA chain).  Its A rows are rotated by 16*kh so that
//   accumulator quads 0 and 1 hold the 16 heads it finishes; quads 2 and 3
//   (its partner's heads) go to LDS.  In the next step it adds the partner's
//   half (a fixed order: own + partner), runs the online softmax in base 2
//   with a lazily moved reference max (as in attention_kernel), and writes P
//   (bf16, entry-major) and its rescale factors and flag.
//   Output waves 4..7: wave j owns dims j*dv/4 .. +dv/4-1 for all 64 heads
//   (128 accumulator registers at dv = 512).  In step s it rescales O when a
//   flag of tile s-1 is set and adds P(s-1) * V(s-1), V from registers, each
//   value fragment feeding both head blocks; then it loads V(s) from the
//   tile by transposing LDS reads.
// Step s: logits of tile s+1, softmax of tile s, P*V of tile s-1, gather of
// tile s+2 (into the buffer of tile s-1, free since step s-1).  The partial
// logits, P, factors and flags are double-buffered by step parity; the
// single barrier at the end of a step publishes them and the gathered tile.
// The logit MFMAs of a step are issued before its softmax: measured, that
// order is faster than the reverse.
template <int DK, int DV>
__global__ __launch_bounds__(512) void attention_split_kernel(AttnArgs a)
{
    constexpr int WAVES = 8;
    constexpr int KS = DK / 16;         // 16-dim k-steps over dk
    constexpr int KH = KS / 2;          // k-steps per logit wave
    constexpr int NBW = DV / 128;       // 32-dim output blocks per output wave
    constexpr int ROWB = DK * 2;
    constexpr int TILEB = kTile * ROWB;
    constexpr int NPIECE = TILEB / 1024;
    // 1 KiB gather pieces per wave: PO for an output wave, PL for a logit
    // wave (pieces 0 .. 4*PL-1 go to the logit waves, the rest to the output
    // waves), so that every DMA of a wave lands in the tile being gathered.
    constexpr int PO = NPIECE / 8;
    constexpr int PL = NPIECE / 4 - PO;
    static_assert(DK % 32 == 0 && DV % 128 == 0 && DV <= DK, "shape");
    static_assert(TILEB % 1024 == 0 && (DK / 8) % 8 == 0, "whole DMA pieces, 8-chunk swizzle");
    static_assert(NPIECE % 4 == 0 && 4 * PL + 4 * PO == NPIECE && PO >= 1, "pieces split by role");

    __shared__ __attribute__((aligned(16))) unsigned char tile0[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char tile1[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char tile2[TILEB];
    // part[parity][logit wave][quad 2, 3]: the partner's half of a partial logit block.
    __shared__ __attribute__((aligned(16))) f32x4 part[2][4][2][64];
    __shared__ __attribute__((aligned(16))) __bf16 pT[2][2][kTile][kPRow];
    __shared__ __attribute__((aligned(16))) float alpha_s[2][64];
    __shared__ __attribute__((aligned(16))) int flag_s[2][4];
    __shared__ __attribute__((aligned(16))) float l_s[64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool logit = wave < 4;  // wave-uniform role
    const int col = lane & 31, half = lane >> 5;
    const int64_t row = blockIdx.x;
    const int k = a.k;
    const int ntiles = (k + kTile - 1) / kTile;
    const int32_t *irow = a.idx + row * (int64_t)k;
    const int nkv = (int)a.T;

    // Logit wave: head block hb, k-step half kh.
    const int hb = (wave >> 1) & 1, kh = wave & 1;
    // Output wave: quarter dq of dv.
    const int dq = wave & 3;

    // The row's indices through a buffer resource that ends after its k
    // entries: entries past k (and every entry when k = 0) read 0, which the
    // gather's validity test masks by position.
    const __amdgpu_buffer_rsrc_t idx_rs = buffer_rsrc(irow, (uint32_t)k * 4u);
    auto load_idx = [&](int t) -> int {
        return (int)__builtin_amdgcn_raw_buffer_load_b32(idx_rs, col * 4, t * kTile * 4, 0);
    };
    // Steps 0 .. ntiles, none without entries (the same count in both roles).
    const int nsteps = ntiles > 0 ? ntiles + 1 : 0;
    const __amdgpu_buffer_rsrc_t kv_rs = buffer_rsrc(a.kv, (uint32_t)(a.T * ROWB));
    const int npw = logit ? PL : PO;  // this wave's pieces
    int g_row[PL], g_chunk[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) {
        const int p = logit ? j * 4 + wave : 4 * PL + j * 4 + (wave - 4);
        const int pos = p * 1024 + lane * 16;
        const int r = (pos / ROWB) & 31;
        g_row[j] = r * 4;
        g_chunk[j] = j < npw ? (((pos % ROWB) >> 4) ^ sw8(r)) * 16 : 0;
    }
    // The gather of tile t into dst: each wave issues its NP pieces (rows
    // past k and padding read zeros through the buffer range check).  Returns
    // the tile's mask of valid entries (bit e: entry e of the tile selects a
    // row of kv).
    auto gdma = [&](auto lg, unsigned char *dst, int iv, int t) -> uint32_t {
        constexpr bool LG = decltype(lg)::value;  // a logit wave's pieces
        constexpr int NP = LG ? PL : PO;
        const int lim = k - t * kTile;
        const bool valid = iv >= 0 && iv < nkv && col < lim;
        const int eoff = valid ? iv * ROWB : (int)0x80000000;
        int e[NP];
#pragma unroll
        for (int j = 0; j < NP; ++j) e[j] = __builtin_amdgcn_ds_bpermute(g_row[j], eoff);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int p = LG ? j * 4 + wave : 4 * PL + j * 4 + (wave - 4);
            dma16(kv_rs, dst + p * 1024, e[j] + g_chunk[j]);
        }
        return (uint32_t)__ballot(valid);
    };
    const std::true_type pl{};
    const std::false_type po{};
    // The two roles run separate loops (so that each wave holds only its
    // role's registers) with the same barriers: two before the loop, one per
    // step s = 0 .. ntiles (no step when there are no tiles), one after it.
    // Buffers rotate by three: tile s in buffer s % 3; step s reads tile s+1
    // (logits) and tile s (values) and gathers tile s+2.
    //   The logit loop is unrolled by three so that every LDS access names its
    // buffer: the compiler then sees that the tile being read is not the one
    // the gather is writing and does not wait for that gather.  The output
    // loop is not unrolled (unrolled, its 128 accumulators are shuffled
    // between copies and spill); its reads are P and a tile gathered steps
    // earlier, so it picks its buffers at run time.
    int iv0 = -1, iv1 = -1, iv2 = -1;  // idx of tiles 0, 1, 2
    if (ntiles > 0) {
        iv0 = load_idx(0);
        iv1 = load_idx(1);
        iv2 = load_idx(2);
    }
    if (logit) {
        // ---- logit wave (hb, kh) ----
        bf16x8 qf[KH];
        {
            const int head = hb * 32 + ((col + 16 * kh) & 31);
            const __bf16 *qh = (const __bf16 *)a.q + ((int64_t)row * 64 + head) * DK;
#pragma unroll
            for (int j = 0; j < KH; ++j) qf[j] = *(const bf16x8 *)(qh + (kh * KH + j) * 16 + half * 8);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): q before the gather loads
        // The softmax works on raw logits s with the scale c folded into the
        // exponent, exp2(s*c - m); a negative c is moved into q (an exact sign
        // flip) so that the running max of s is the max of s*c.
        const float c2 = fabsf(a.scale_log2e);
        const float tau_s = kTau / c2;  // the lazy-rescale margin in logit units (inf for c = 0)
        if (a.scale_log2e < 0.0f) {
#pragma unroll
            for (int j = 0; j < KH; ++j)
                qf[j] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qf[j]) ^ 0x80008000u);
        }
        // B fragment j (k-step kh*KH + j) of an entry row is chunk
        // c = 2*(kh*KH + j) + half, stored at chunk c ^ sw8(col); the swizzle
        // only touches the low three bits of c, so for j = 4m + r the offset
        // is qb[r] + 128*m, an immediate in the read.
        int qb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) qb[r] = col * ROWB + (((2 * (kh * KH + r) + half) ^ sw8(col)) << 4);
        f32x4 own0 = {}, own1 = {};  // quads 0, 1 of the next tile's partial logits
        float mref[8], thr[8], lsum[8];  // mref: scaled (s*c); thr: raw logit units
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
            mref[ii] = -__builtin_inff();
            thr[ii] = -__builtin_inff();
            lsum[ii] = 0.0f;
        }
        // Partial logits of a tile: one MFMA chain over the k-steps, the B
        // fragments read six k-steps ahead.
        auto qk = [&](const unsigned char *tb) {
            constexpr int G = 6;
            constexpr int NG = (KH + G - 1) / G;
            bf16x8 bA[G], bB[G];
            auto ld = [&](bf16x8 *bb, int g) {
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const int j = g * G + i;
                    if (j < KH) bb[i] = *(const bf16x8 *)(tb + qb[j & 3] + 128 * (j >> 2));
                }
            };
            f32x16 c = {};
            ld(bA, 0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                if (g + 1 < NG) ld((g & 1) ? bA : bB, g + 1);
                __builtin_amdgcn_sched_barrier(0);
                const bf16x8 *bb = (g & 1) ? bB : bA;
#pragma unroll
                for (int i = 0; i < G; ++i)
                    if (g * G + i < KH) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[g * G + i], bb[i], c, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            return c;
        };
        auto publish = [&](const f32x16 &acc, int par) {
            own0 = f32x4{acc[0], acc[1], acc[2], acc[3]};
            own1 = f32x4{acc[4], acc[5], acc[6], acc[7]};
            part[par][wave][0][lane] = f32x4{acc[8], acc[9], acc[10], acc[11]};
            part[par][wave][1][lane] = f32x4{acc[12], acc[13], acc[14], acc[15]};
        };
        // Softmax of a tile: own partial quads + the partner's, masked by
        // vmask; P, factors and flag to pT/alpha_s/flag_s[par].
        auto softmax = [&](int par, uint32_t vmask) {
            const f32x4 p0 = part[par][wave ^ 1][0][lane];
            const f32x4 p1 = part[par][wave ^ 1][1][lane];
            const f32x4 s0 = own0 + p0, s1 = own1 + p1;
            const bool valid = (vmask >> col) & 1u;
            float x[8];
            bool exceed = false;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                x[ii] = s0[ii];
                x[4 + ii] = s1[ii];
            }
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) exceed |= x[ii] > thr[ii];
            exceed = exceed && valid;
            const bool wave_need = __ballot(exceed) != 0;  // wave-uniform
            if (wave_need) {
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    const float mx = half_max(valid ? x[ii] : -__builtin_inff());
                    float alpha = 1.0f;
                    if (mx > thr[ii]) {
                        const float mc = mx * c2;
                        alpha = __builtin_amdgcn_exp2f(mref[ii] - mc);
                        mref[ii] = mc;
                        thr[ii] = mx + tau_s;
                        lsum[ii] *= alpha;
                    }
                    // accumulator row 8*(ii/4) + 4*half + ii%4 of the rotated
                    // block is head hb*32 + 16*kh + that row
                    if (col == 0)
                        lds_store_b32(&alpha_s[par][hb * 32 + 16 * kh + 8 * (ii >> 2) + 4 * half + (ii & 3)],
                                      alpha);
                }
            }
            i16x4 pw0, pw1;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
                const float pp = valid ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[ii], c2, -mref[ii])) : 0.0f;
                lsum[ii] += pp;
                if (ii < 4) pw0[ii] = __builtin_bit_cast(short, (__bf16)pp);
                else pw1[ii - 4] = __builtin_bit_cast(short, (__bf16)pp);
            }
            lds_store_b64(&pT[par][hb][col][16 * kh + 4 * half], pw0);
            lds_store_b64(&pT[par][hb][col][16 * kh + 8 + 4 * half], pw1);
            if (lane == 0) flag_s[par][wave] = wave_need ? 1 : 0;
        };
        // ivs: idx of tile s, replaced by idx of tile s+3; ivg: idx of tile
        // s+2; vmask: valid-entry mask of tile s; vnext receives that of tile
        // s+2 (the masks rotate through three slots, tile t in slot t % 3).
        auto step = [&](const unsigned char *tq, unsigned char *dst, int &ivs, int ivg, uint32_t vmask,
                        uint32_t &vnext, int st) {
            ivs = load_idx(st + 3);
            vnext = gdma(pl, dst, ivg, st + 2);
            if (st < ntiles) {
                const bool more = st + 1 < ntiles;
                f32x16 acc;  // written and read only when more
                if (more) acc = qk(tq);
                softmax(st & 1, vmask);
                if (more) publish(acc, (st + 1) & 1);
            }
            vm_wait<0>();
            lds_barrier();
        };
        uint32_t vm0 = 0, vm1 = 0, vm2 = 0;  // valid-entry masks of tiles 0, 1, 2 (mod 3)
        if (ntiles > 0) {
            vm0 = gdma(pl, tile0, iv0, 0);
            vm1 = gdma(pl, tile1, iv1, 1);
            vm_wait<0>();
        }
        __syncthreads();
        if (ntiles > 0) publish(qk(tile0), 0);
        __syncthreads();
        for (int st = 0; st < nsteps; st += 3) {
            step(tile1, tile2, iv0, iv2, vm0, vm2, st);
            if (st + 1 >= nsteps) break;
            step(tile2, tile0, iv1, iv0, vm1, vm0, st + 1);
            if (st + 2 >= nsteps) break;
            step(tile0, tile1, iv2, iv1, vm2, vm1, st + 2);
        }
        // Denominators: sum each head's per-lane shares over the 32 lanes of
        // a half.
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
            float l = lsum[ii];
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) l += __shfl_xor(l, off);
            if (col == 0) l_s[hb * 32 + 16 * kh + 8 * (ii >> 2) + 4 * half + (ii & 3)] = l;
        }
        __syncthreads();
    } else {
        // ---- output wave dq ----
        f32x16 o[2][NBW];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) o[h][nb] = f32x16{};
        const int eb = ((lane >> 5) * 8) + ((lane & 15) >> 2);
        const int dl = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int cq = dq * (DV / 32);
        int tr_off[2][2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int e = eb + 4 * s2;
#pragma unroll
            for (int par = 0; par < 2; ++par) {
                const int bp = ((cq >> 2) + par) & 1;
                tr_off[s2][par] = e * ROWB + (((bp * 4 + (dl >> 3)) ^ sw8(e)) << 4) + (dl & 7) * 2;
            }
        }
        bf16x8 vf[2][NBW];  // value fragments of the tile whose P*V comes next
        auto load_v = [&](const unsigned char *tb) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    const int hi = ((cq + nb * 4) & ~7) * 16;
                    const unsigned char *vb = tb + kk * 16 * ROWB + hi;
                    const i16x4 v0 = read_tr16(vb + tr_off[0][nb & 1]);
                    const i16x4 v1 = read_tr16(vb + tr_off[1][nb & 1]);
                    const i16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    vf[kk][nb] = __builtin_bit_cast(bf16x8, vv);
                }
        };
        // O = alpha * O + P V for the tile whose P sits in pT[par] and whose
        // V is in vf; P is read one head block at a time (8 registers).
        auto pv = [&](int par) {
            u32x4 fl;
            i16x4 t00, t01, t10, t11;
            lds_read_fp(&flag_s[par][0], &pT[par][0][eb][dl], &pT[par][0][eb + 4][dl],
                        &pT[par][0][16 + eb][dl], &pT[par][0][16 + eb + 4][dl], fl, t00, t01, t10, t11);
            const bool resc = __builtin_amdgcn_readfirstlane((int)(fl[0] | fl[1] | fl[2] | fl[3])) != 0;
            if (resc) {
                // Heads hb*32 + 16*kh .. +15 belong to logit wave 2*hb + kh;
                // a wave whose flag is clear wrote no factors: its heads keep 1.
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        f32x4 al = *(const f32x4 *)&alpha_s[par][h * 32 + 8 * j4 + 4 * half];
                        if (fl[2 * h + (j4 >> 1)] == 0u) al = f32x4{1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                            for (int ii = 0; ii < 4; ++ii) o[h][nb][4 * j4 + ii] *= al[ii];
                    }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h == 1)
                    lds_read_fp(&flag_s[par][0], &pT[par][1][eb][dl], &pT[par][1][eb + 4][dl],
                                &pT[par][1][16 + eb][dl], &pT[par][1][16 + eb + 4][dl], fl, t00, t01,
                                t10, t11);
                const bf16x8 pa0 = __builtin_bit_cast(
                    bf16x8, i16x8{t00[0], t00[1], t00[2], t00[3], t01[0], t01[1], t01[2], t01[3]});
                const bf16x8 pa1 = __builtin_bit_cast(
                    bf16x8, i16x8{t10[0], t10[1], t10[2], t10[3], t11[0], t11[1], t11[2], t11[3]});
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    o[h][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa0, vf[0][nb], o[h][nb], 0, 0, 0);
                    o[h][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa1, vf[1][nb], o[h][nb], 0, 0, 0);
                }
            }
        };
        auto buf = [&](int t) -> unsigned char * {
            const int b = t % 3;
            return b == 0 ? tile0 : (b == 1 ? tile1 : tile2);
        };
        if (ntiles > 0) {
            gdma(po, tile0, iv0, 0);
            gdma(po, tile1, iv1, 1);
            vm_wait<0>();
        }
        __syncthreads();
        __syncthreads();
        int ivg = iv2;  // idx of tile s+2
        for (int st = 0; st < nsteps; ++st) {
            const int nx = load_idx(st + 3);
            gdma(po, buf(st + 2), ivg, st + 2);
            ivg = nx;
            if (st >= 1) pv((st - 1) & 1);
            if (st < ntiles) load_v(buf(st));
            vm_wait<0>();
            lds_barrier();
        }
        __syncthreads();
        __bf16 *orow = (__bf16 *)a.out + (int64_t)row * 64 * DV;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const f32x4 l4 = *(const f32x4 *)&l_s[h * 32 + 8 * j4 + 4 * half];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int head = h * 32 + 8 * j4 + 4 * half + ii;
                    const float inv = l4[ii] > 0.0f ? 1.0f / l4[ii] : 0.0f;
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        const int dim = dq * (DV / 4) + nb * 32 + col;
                        orow[(int64_t)head * DV + dim] = (__bf16)(o[h][nb][4 * j4 + ii] * inv);
                    }
                }
            }
    }
}

template <int DK, int DV>
hipError_t launch_dims(const AttnArgs &a, hipStream_t s)
{
    if (a.H == 32) attention_kernel<DK, DV, 1><<<dim3((unsigned)a.S), 256, 0, s>>>(a);
    else if (a.H == 64) attention_split_kernel<DK, DV><<<dim3((unsigned)a.S), 512, 0, s>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

bool attention_shape_supported(int32_t H, int32_t dk, int32_t dv)
{
    return (H == 32 || H == 64) && ((dk == 576 && dv == 512) || (dk == 128 && dv == 128));
}

hipError_t launch_attention(const AttnArgs &a, int32_t dk, int32_t dv, hipStream_t stream)
{
    if (a.S <= 0) return hipSuccess;
    if (dk == 576 && dv == 512) return launch_dims<576, 512>(a, stream);
    if (dk == 128 && dv == 128) return launch_dims<128, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace csa
