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
// One workgroup of 8 waves per query row (attention_split_kernel below, for
// 32 and 64 heads).  Four logit waves compute the logits of a 32-entry tile
// with v_mfma_f32_32x32x16_bf16 (q resident in registers, each wave over a
// range of the dk k-steps), exchange partial logit blocks in LDS and run an
// online softmax in base 2 whose reference max moves only when a head's max
// rises by more than 2^8; four output waves accumulate P * V, each over a
// quarter of the dv output dims, with the V fragments taken from the
// row-major tile by transposing LDS reads (ds_read_b64_tr_b16).  The
// selected latent rows are gathered by LDS DMA into the free one of three
// static tile buffers: each lane moves the 16 bytes its slot of the swizzled
// tile needs, straight from the row the index names (padding and indices
// outside [0, T) read zeros through the buffer range check).  The barriers
// inside the loop carry no memory fence (a fence would wait for every DMA in
// flight); the wait for a tile's DMAs is an explicit vmcnt before the barrier
// that publishes it.  The softmax denominators are kept per lane and reduced
// once at the end.
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

// Role-split attention for HB head blocks of 32 heads (HB = 1 or 2): one
// workgroup of 8 waves per query row and one barrier per 32-entry tile step.
// Waves w and w+4 of a workgroup share a SIMD, so every SIMD runs one logit
// wave and one output wave.
//   Logit waves 0..3: wave (hb, ksp) keeps q of head block hb for k-step
//   range ksp (of NSPLIT = 4/HB ranges) and computes a partial 32x32 logit
//   block per tile (one MFMA chain).  Its A rows are rotated by 8*QPW*ksp
//   (QPW = 4/NSPLIT) so that accumulator quads 0 .. QPW-1 hold the 8*QPW
//   heads it finishes; its other quads go to LDS for the waves that finish
//   those heads.  In the next step it adds the other waves' partials to its
//   own (in a fixed order), runs the online softmax in base 2 with a lazily
//   moved reference max, and writes P (bf16, entry-major) and its rescale
//   factors and flag.
//   Output waves 4..7: wave j owns dims j*dv/4 .. +dv/4-1 for all heads
//   (64*HB accumulator registers at dv = 512).  In step s it rescales O when
//   a flag of tile s-1 is set and adds P(s-1) * V(s-1), V from registers,
//   each value fragment feeding every head block; then it loads V(s) from
//   the tile by transposing LDS reads.
// Step s: logits of tile s+1, softmax of tile s, P*V of tile s-1, gather of
// tile s+2 (into the buffer of tile s-1, free since step s-1).  The partial
// logits, P, factors and flags are double-buffered by step parity; the
// single barrier at the end of a step publishes them and the gathered tile.
// The logit MFMAs of a step are issued before its softmax: measured, that
// order is faster than the reverse.
template <int DK, int DV, int HB>
__global__ __launch_bounds__(512) void attention_split_kernel(AttnArgs a)
{
    constexpr int NH = 32 * HB;         // heads
    constexpr int NSPLIT = 4 / HB;      // logit waves per head block, one k-step range each
    constexpr int QPW = 4 / NSPLIT;     // accumulator quads (8 heads each) a logit wave finishes
    constexpr int NV = 4 * QPW;         // softmax values per lane of a logit wave
    constexpr int KS = DK / 16;         // 16-dim k-steps over dk
    constexpr int KH = KS / NSPLIT;     // k-steps per logit wave
    constexpr int NBW = DV / 128;       // 32-dim output blocks per output wave
    static_assert(HB == 1 || HB == 2, "32 or 64 heads");
    static_assert(KS % NSPLIT == 0, "whole k-step ranges");
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
    // part[parity][logit wave][quad QPW .. 3]: the quads of a partial logit
    // block whose heads other waves finish.
    __shared__ __attribute__((aligned(16))) f32x4 part[2][4][4 - QPW][64];
    __shared__ __attribute__((aligned(16))) __bf16 pT[2][HB][kTile][kPRow];
    __shared__ __attribute__((aligned(16))) float alpha_s[2][NH];
    __shared__ __attribute__((aligned(16))) int flag_s[2][4];
    __shared__ __attribute__((aligned(16))) float l_s[NH];

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

    // Logit wave: head block hb, k-step range ksp (of NSPLIT).
    const int hb = (wave & 3) / NSPLIT, ksp = (wave & 3) % NSPLIT;
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
    // loop is not unrolled (unrolled, its 64*HB accumulators are shuffled
    // between copies and spill); its reads are P and a tile gathered steps
    // earlier, so it picks its buffers at run time.
    int iv0 = -1, iv1 = -1, iv2 = -1;  // idx of tiles 0, 1, 2
    if (ntiles > 0) {
        iv0 = load_idx(0);
        iv1 = load_idx(1);
        iv2 = load_idx(2);
    }
    if (logit) {
        // ---- logit wave (hb, ksp) ----
        bf16x8 qf[KH];
        {
            const int head = hb * 32 + ((col + 8 * QPW * ksp) & 31);
            const __bf16 *qh = (const __bf16 *)a.q + ((int64_t)row * NH + head) * DK;
#pragma unroll
            for (int j = 0; j < KH; ++j) qf[j] = *(const bf16x8 *)(qh + (ksp * KH + j) * 16 + half * 8);
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
        // B fragment j (k-step ksp*KH + j) of an entry row is chunk
        // c = 2*(ksp*KH + j) + half, stored at chunk c ^ sw8(col); the swizzle
        // only touches the low three bits of c, so for j = 4m + r the offset
        // is qb[r] + 128*m, an immediate in the read.
        int qb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) qb[r] = col * ROWB + (((2 * (ksp * KH + r) + half) ^ sw8(col)) << 4);
        f32x4 own[QPW];  // quads 0 .. QPW-1 of the next tile's partial logits
#pragma unroll
        for (int oq = 0; oq < QPW; ++oq) own[oq] = f32x4{};
        float mref[NV], thr[NV], lsum[NV];  // mref: scaled (s*c); thr: raw logit units
#pragma unroll
        for (int ii = 0; ii < NV; ++ii) {
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
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
                if (q < QPW) own[q] = v;
                else part[par][wave][q - QPW][lane] = v;
            }
        };
        // Softmax of a tile: own partial quads + the other waves' of the head
        // block (in the fixed order ksp+1, ksp+2, ... mod NSPLIT), masked by
        // vmask; P, factors and flag to pT/alpha_s/flag_s[par].  Partner ks'
        // keeps the rows of own quad oq in its quad (QPW*(ksp - ks') + oq) mod 4.
        auto softmax = [&](int par, uint32_t vmask) {
            const bool valid = (vmask >> col) & 1u;
            float x[NV];
            bool exceed = false;
#pragma unroll
            for (int oq = 0; oq < QPW; ++oq) {
                f32x4 sq = own[oq];
#pragma unroll
                for (int d = 1; d < NSPLIT; ++d) {
                    const int ks2 = (ksp + d) % NSPLIT;
                    const int qp = (QPW * (ksp - ks2) + oq) & 3;
                    sq += part[par][hb * NSPLIT + ks2][qp - QPW][lane];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) x[4 * oq + i] = sq[i];
            }
#pragma unroll
            for (int ii = 0; ii < NV; ++ii) exceed |= x[ii] > thr[ii];
            exceed = exceed && valid;
            const bool wave_need = __ballot(exceed) != 0;  // wave-uniform
            if (wave_need) {
#pragma unroll
                for (int ii = 0; ii < NV; ++ii) {
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
                    // block is head hb*32 + 8*QPW*ksp + that row
                    if (col == 0)
                        lds_store_b32(&alpha_s[par][hb * 32 + 8 * QPW * ksp + 8 * (ii >> 2) + 4 * half + (ii & 3)],
                                      alpha);
                }
            }
            i16x4 pw[QPW];
#pragma unroll
            for (int ii = 0; ii < NV; ++ii) {
                const float pp = valid ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[ii], c2, -mref[ii])) : 0.0f;
                lsum[ii] += pp;
                pw[ii >> 2][ii & 3] = __builtin_bit_cast(short, (__bf16)pp);
            }
#pragma unroll
            for (int oq = 0; oq < QPW; ++oq)
                lds_store_b64(&pT[par][hb][col][8 * QPW * ksp + 8 * oq + 4 * half], pw[oq]);
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
        for (int ii = 0; ii < NV; ++ii) {
            float l = lsum[ii];
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) l += __shfl_xor(l, off);
            if (col == 0) l_s[hb * 32 + 8 * QPW * ksp + 8 * (ii >> 2) + 4 * half + (ii & 3)] = l;
        }
        __syncthreads();
    } else {
        // ---- output wave dq ----
        f32x16 o[HB][NBW];
#pragma unroll
        for (int h = 0; h < HB; ++h)
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
                // Heads h*32 + 8*QPW*ks .. +8*QPW-1 belong to logit wave
                // h*NSPLIT + ks; a wave whose flag is clear wrote no factors:
                // its heads keep 1.
#pragma unroll
                for (int h = 0; h < HB; ++h)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        f32x4 al = *(const f32x4 *)&alpha_s[par][h * 32 + 8 * j4 + 4 * half];
                        if (fl[h * NSPLIT + j4 / QPW] == 0u) al = f32x4{1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                            for (int ii = 0; ii < 4; ++ii) o[h][nb][4 * j4 + ii] *= al[ii];
                    }
            }
#pragma unroll
            for (int h = 0; h < HB; ++h) {
                if (h > 0)
                    lds_read_fp(&flag_s[par][0], &pT[par][h][eb][dl], &pT[par][h][eb + 4][dl],
                                &pT[par][h][16 + eb][dl], &pT[par][h][16 + eb + 4][dl], fl, t00, t01,
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
        __bf16 *orow = (__bf16 *)a.out + (int64_t)row * NH * DV;
#pragma unroll
        for (int h = 0; h < HB; ++h)
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
    if (a.H == 32) attention_split_kernel<DK, DV, 1><<<dim3((unsigned)a.S), 512, 0, s>>>(a);
    else if (a.H == 64) attention_split_kernel<DK, DV, 2><<<dim3((unsigned)a.S), 512, 0, s>>>(a);
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
