// C ABI and driver of libcsa_indexer.so: argument checks, workspace plan,
// and the launch sequence of the chunked partition-merge.
//
// Plan (page "StreamIndex: Memory-Bounded Compressed Sparse Attention via
// Streaming Top-k", Abstract: a chunked partition-merge top-k driver that
// never materialises the [B,S,H_I,T] score tensor; the page sweeps chunk size
// and key-tile size): the S query rows are processed in passes of R rows,
// R chosen so that one pass's scratch fits the workspace.  Within a pass the
// usable keys are cut into chunks of C keys.  For each chunk the score kernel
// writes the pass's [R, C] head-reduced scores, then the select kernel folds
// them into each row's running best-k list; the last chunk's select pass sorts
// the lists and writes idx/score.  Scratch is R*(4C + 16 [+ 8k + 16]) bytes,
// set by the workspace and never by S*T.  Problems with few query rows cut
// one chunk into G key splits instead, run in parallel, each with its own
// list, and merge the G lists in rounds of four (k <= 2048) or two
// (R*(4C + G*(16 + 8k + 16)) bytes).
#include <stdint.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/csa_indexer.h"

#include "csa_internal.h"

// Scratch of the allocation-free entry point: one fixed array per GPU, held
// from the library's first use there until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: the device
// address comes from hipGetSymbolAddress, once per device (scratch_on).
static __device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kDefaultBudget = int64_t(2) << 30;
constexpr int64_t kDefaultChunkCap = 65536;  // single chunk up to this many keys
constexpr int64_t kDefaultChunk = 65536;
constexpr int32_t kDefaultTile = 192;  // keys per LDS tile when the caller sets none
constexpr int64_t kMaxChunk = int64_t(1) << 24;  // keys; chunk offsets stay 32-bit in the kernels
constexpr int64_t kMaxRowsNoKeys = int64_t(1) << 20;  // rows per pass when no row has a key
constexpr size_t kAlign = 256;
// Key splits (automatic): used when a problem has fewer query blocks than
// this (a 256-CU part then has idle CUs), doubled until blocks x splits
// reaches twice it, capped by kMaxSplits and by kSplitMinKeys keys per split.
constexpr int64_t kSplitBlocks = 256;
constexpr int64_t kSplitMinKeys = 2048;
constexpr int32_t kMaxSplits = 128;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

static_assert(CSA_NOALLOC_SCRATCH_BYTES % kAlign == 0, "scratch size in whole alignment units");
std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;  // by device ordinal; null until looked up

// Device address of the current device's scratch (looked up on first use).
int scratch_on(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CSA_ERR_HIP;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return CSA_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CSA_OK;
}

struct Plan {
    int64_t n_max = 0;   // keys usable by the last row
    int64_t chunk = 0;   // keys per chunk (0: no row has a key)
    int64_t n_chunks = 0;
    int64_t splits = 1;  // key splits of the (single) chunk, scored and selected in parallel
    int64_t slen = 0;    // keys per split (== chunk without splits)
    int32_t tile = kDefaultTile;
    bool lists = false;  // several chunks or splits: lists live in the workspace
};

// Workspace layout of a pass of `rows` rows, in this order:
//   scores [rows][chunk] u32 (orderable fp32) | meta [splits*rows] ChunkMeta |
//   (several chunks or splits:) lists [splits*rows][k] u64 | state [splits*rows] RowState
struct PassLayout {
    size_t meta, lists, state, end;
};

PassLayout pass_layout(const Plan &p, int64_t rows, int64_t k)
{
    PassLayout l{0, 0, 0, 0};
    if (p.chunk == 0 || rows <= 0) return l;
    const size_t vrows = (size_t)rows * (size_t)p.splits;
    l.meta = align_up((size_t)rows * (size_t)p.chunk * sizeof(uint32_t));
    l.end = l.meta + align_up(vrows * sizeof(csa::ChunkMeta));
    if (p.lists) {
        l.lists = l.end;
        l.state = l.lists + align_up(vrows * (size_t)k * sizeof(uint64_t));
        l.end = l.state + align_up(vrows * sizeof(csa::RowState));
    }
    return l;
}

size_t pass_bytes(const Plan &p, int64_t rows, int64_t k) { return pass_layout(p, rows, k).end; }

int check_args(int64_t S, int64_t T, int32_t H, int32_t D, int32_t m, int64_t k,
               int64_t q_pos0, int32_t dtype, const csa_opts *opts)
{
    if (dtype != CSA_F32 && dtype != CSA_BF16) return CSA_ERR_BAD_DTYPE;
    if (S < 0 || T < 0 || m < 1 || k < 1 || q_pos0 < 0 || H < 1) return CSA_ERR_BAD_SHAPE;
    if (H > CSA_MAX_HEADS) return CSA_ERR_BAD_SHAPE;
    if (D != 32 && D != 64 && D != 128) return CSA_ERR_BAD_SHAPE;
    if (k > CSA_MAX_K) return CSA_ERR_UNSUPPORTED;
    if (T > (int64_t)INT32_MAX - 1) return CSA_ERR_UNSUPPORTED;
    if (S > ((int64_t)1 << 40) || q_pos0 > ((int64_t)1 << 40)) return CSA_ERR_UNSUPPORTED;
    if (opts) {
        if (opts->chunk_keys < 0 || (opts->chunk_keys % 256) != 0 || opts->chunk_keys > kMaxChunk)
            return CSA_ERR_BAD_OPTION;
        if (opts->key_tile != 0 && opts->key_tile != 64 && opts->key_tile != 128 &&
            opts->key_tile != 192 && opts->key_tile != 256)
            return CSA_ERR_BAD_OPTION;
        if (opts->workspace_budget < 0) return CSA_ERR_BAD_OPTION;
        const int32_t ks = opts->key_splits;
        if (ks < 0 || ks > kMaxSplits || (ks & (ks - 1)) != 0) return CSA_ERR_BAD_OPTION;
        for (int i = 0; i < 4; ++i)
            if (opts->reserved[i] != 0) return CSA_ERR_BAD_OPTION;
    }
    return CSA_OK;
}

int64_t budget_of(const csa_opts *opts)
{
    return (opts && opts->workspace_budget) ? opts->workspace_budget : kDefaultBudget;
}

// The plan: chunks of the usable keys, or, for problems with few query
// blocks (e.g. decoding a few new queries against a long key cache), one
// chunk cut into key splits that run in parallel.  Pure host arithmetic.
Plan make_plan(int64_t S, int64_t T, int32_t m, int64_t q_pos0, int64_t k, int32_t dtype,
               const csa_opts *opts)
{
    Plan p;
    p.n_max = S > 0 ? csa::n_usable(q_pos0 + S - 1, T, m) : 0;
    if (opts && opts->key_tile) p.tile = opts->key_tile;
    if (p.n_max == 0) return p;
    const int64_t n_round = (p.n_max + 255) / 256 * 256;
    const bool user_chunk = opts && opts->chunk_keys;
    const int32_t ks = opts ? opts->key_splits : 0;
    // Key splits: not with a chunk size the caller fixed.
    int64_t g = 1;
    if (!user_chunk && ks != 1) {
        if (ks >= 2) {
            g = ks;
        } else {
            const int64_t nqb = (S + csa::kScoreWaves - 1) / csa::kScoreWaves;
            if (nqb < kSplitBlocks) {
                g = 2;
                while (g < kMaxSplits && nqb * g < 2 * kSplitBlocks) g *= 2;
                while (g > 1 && p.n_max / g < kSplitMinKeys) g /= 2;
            }
        }
    }
    if (g > 1) {
        Plan q = p;
        q.splits = g;
        q.slen = ((p.n_max + g - 1) / g + 255) / 256 * 256;
        q.chunk = g * q.slen;
        q.n_chunks = 1;
        q.lists = true;
        // Automatic splits only where one pass holds every row; else chunks.
        if (ks >= 2 || pass_bytes(q, S, k) <= (size_t)budget_of(opts)) return q;
    }
    int64_t c = user_chunk ? opts->chunk_keys
                           : (n_round <= kDefaultChunkCap ? n_round : kDefaultChunk);
    if (c > n_round) c = n_round;
    p.chunk = c;
    p.slen = c;
    p.n_chunks = (p.n_max + c - 1) / c;
    p.lists = p.n_chunks > 1;
    return p;
}

// Rows per pass that fit `bytes` (0 if not even one query block fits).
int64_t rows_fitting(const Plan &p, int64_t S, int64_t k, size_t bytes)
{
    if (pass_bytes(p, S, k) <= bytes) return S;
    const size_t per_row = (size_t)p.chunk * 4 + (size_t)p.splits * sizeof(csa::ChunkMeta) +
                           (p.lists ? (size_t)p.splits * ((size_t)k * 8 + sizeof(csa::RowState))
                                    : 0);
    int64_t r = (int64_t)(bytes / per_row);
    r = r / csa::kScoreWaves * csa::kScoreWaves;
    while (r > 0 && pass_bytes(p, r, k) > bytes) r -= csa::kScoreWaves;
    return r;
}

// ---- optional per-kernel timing ----
struct ProfRecord {
    int kind;
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof_records;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event()
{
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

template <class F>
int launch_timed(int kind, hipStream_t s, F &&launch)
{
    ProfRecord rec{kind, nullptr, nullptr};
    const bool prof = g_prof_on;
    if (prof) {
        std::lock_guard<std::mutex> g(g_prof_mu);
        rec.start = prof_event();
        rec.stop = prof_event();
        if (rec.start) (void)hipEventRecord(rec.start, s);
    }
    hipError_t e = launch();
    if (prof) {
        std::lock_guard<std::mutex> g(g_prof_mu);
        if (rec.stop) (void)hipEventRecord(rec.stop, s);
        if (rec.start && rec.stop) g_prof_records.push_back(rec);
    }
    return e == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char *csa_status_str(int status)
{
    switch (status) {
    case CSA_OK: return "ok";
    case CSA_ERR_NULL_PTR: return "a required pointer is NULL";
    case CSA_ERR_BAD_SHAPE: return "bad shape: sizes must be >= 0, 1 <= H_I <= 64, D_I in {32,64,128}, m >= 1, k >= 1";
    case CSA_ERR_BAD_DTYPE: return "bad dtype: expected CSA_F32 or CSA_BF16";
    case CSA_ERR_MISALIGNED: return "misaligned pointer";
    case CSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small for one query block";
    case CSA_ERR_UNSUPPORTED: return "unsupported request: indexer k > 4096 or T >= 2^31; attention dtype, shape or size outside this build";
    case CSA_ERR_HIP: return "HIP call or kernel launch failed";
    case CSA_ERR_BAD_OPTION: return "bad option: chunk_keys must be a multiple of 256 up to 2^24, key_tile one of 64/128/192/256, key_splits 0 or a power of two up to 128, reserved fields 0";
    case CSA_ERR_SCRATCH_TOO_SMALL: return "allocation-free call: one query block needs more scratch than the library's fixed 256 MiB (use a smaller chunk_keys, or csa_indexer_topk with a workspace)";
    default: return "unknown status";
    }
}

int csa_indexer_topk_workspace_size(int64_t S, int64_t T, int32_t H_I, int32_t D_I, int32_t m,
                                    int64_t k, int64_t q_pos0, int32_t dtype,
                                    const csa_opts *opts, size_t *bytes_out)
{
    if (!bytes_out) return CSA_ERR_NULL_PTR;
    int st = check_args(S, T, H_I, D_I, m, k, q_pos0, dtype, opts);
    if (st != CSA_OK) return st;
    const Plan p = make_plan(S, T, m, q_pos0, k, dtype, opts);
    int64_t rows = rows_fitting(p, S, k, (size_t)budget_of(opts));
    const int64_t min_rows = S < csa::kScoreWaves ? S : csa::kScoreWaves;
    if (rows < min_rows) rows = min_rows;
    *bytes_out = pass_bytes(p, rows, k);
    return CSA_OK;
}

}  // extern "C"

namespace {

// Argument checks of one problem, before any HIP call; on success *rows_out
// is the pass size the workspace allows.
int check_call(const void *q, const void *w, const void *kc, int32_t dtype, int64_t S, int64_t T,
               int32_t H_I, int32_t D_I, int32_t m, int64_t k, int64_t q_pos0, int32_t *idx,
               float *score, void *workspace, size_t workspace_bytes, const csa_opts *opts,
               Plan *plan_out, int64_t *rows_out)
{
    int st = check_args(S, T, H_I, D_I, m, k, q_pos0, dtype, opts);
    if (st != CSA_OK) return st;
    const Plan p = make_plan(S, T, m, q_pos0, k, dtype, opts);
    *plan_out = p;
    *rows_out = 0;
    if (S == 0) return CSA_OK;
    if (!q || !w || !idx || !score) return CSA_ERR_NULL_PTR;
    if (p.n_max > 0 && !kc) return CSA_ERR_NULL_PTR;
    const size_t esz = dtype == CSA_BF16 ? 2 : 4;
    if (((uintptr_t)q & 15) || ((uintptr_t)kc & 15) || ((uintptr_t)w & (esz - 1)) ||
        ((uintptr_t)idx & 3) || ((uintptr_t)score & 3) || ((uintptr_t)workspace & (kAlign - 1)))
        return CSA_ERR_MISALIGNED;
    int64_t rows = S;
    if (p.chunk > 0) {
        if (!workspace) return CSA_ERR_NULL_PTR;
        rows = rows_fitting(p, S, k, workspace_bytes);
        if (rows <= 0) return CSA_ERR_WORKSPACE_TOO_SMALL;
    }
    *rows_out = rows;
    return CSA_OK;
}

// One problem, its arguments already checked: the pass plan and the launches.
int run_call(const void *q, const void *w, const void *kc, int32_t dtype, int64_t S, int64_t T,
             int32_t H_I, int32_t D_I, int32_t m, int64_t k, int64_t q_pos0, int32_t *idx,
             float *score, void *workspace, const Plan &p, int64_t rows, void *stream)
{
    int st = CSA_OK;
    if (S == 0) return CSA_OK;
    if (p.chunk == 0 && rows > kMaxRowsNoKeys) rows = kMaxRowsNoKeys;  // padding-only passes
    if (p.chunk > 0) {
        if (rows < S && p.splits == 1) {
            // Several passes.  Score workgroups of one pass run in rounds of
            // (CUs x workgroups per CU); a partial round leaves CUs idle for
            // a whole workgroup's time, so passes get whole rounds (only the
            // last pass has a partial one).  Without a round size (the
            // queries fail), rows are spread evenly over the passes so that
            // no pass is a handful of rows on a handful of CUs.
            int dev = 0, ncu = 0;
            int64_t round_rows = 0;
            if (hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) ==
                    hipSuccess) {
                const int bpc = csa::score_blocks_per_cu(dtype, D_I, H_I, p.tile);
                round_rows = (int64_t)ncu * bpc * csa::kScoreWaves;
            }
            if (round_rows <= 0) (void)hipGetLastError();  // a failed query is not a launch error
            if (round_rows > 0 && rows >= round_rows) {
                rows = rows / round_rows * round_rows;
            } else {
                const int64_t passes = (S + rows - 1) / rows;
                int64_t even = (S + passes - 1) / passes;
                even = (even + csa::kScoreWaves - 1) / csa::kScoreWaves * csa::kScoreWaves;
                if (even < rows) rows = even;
            }
        } else if (rows < S) {
            const int64_t passes = (S + rows - 1) / rows;
            int64_t even = (S + passes - 1) / passes;
            even = (even + csa::kScoreWaves - 1) / csa::kScoreWaves * csa::kScoreWaves;
            if (even < rows) rows = even;
        }
    }
    hipStream_t s = (hipStream_t)stream;

    char *wsb = (char *)workspace;
    for (int64_t r0 = 0; r0 < S; r0 += rows) {
        const int64_t nr = rows < S - r0 ? rows : S - r0;
        const int64_t n_hi = csa::n_usable(q_pos0 + r0 + nr - 1, T, m);
        const int64_t nch = (p.chunk > 0 && n_hi > 0) ? (n_hi + p.chunk - 1) / p.chunk : 1;
        const PassLayout lay = pass_layout(p, nr, k);
        uint32_t *ws_scores = (uint32_t *)wsb;
        csa::ChunkMeta *meta = p.chunk > 0 ? (csa::ChunkMeta *)(wsb + lay.meta) : nullptr;
        uint64_t *lists = p.lists ? (uint64_t *)(wsb + lay.lists) : nullptr;
        csa::RowState *state = p.lists ? (csa::RowState *)(wsb + lay.state) : nullptr;
        for (int64_t c = 0; c < nch; ++c) {
            const int64_t c0 = c * p.chunk;
            if (n_hi > c0) {
                csa::ScoreArgs sa;
                sa.q = q;
                sa.w = w;
                sa.kc = kc;
                sa.ws = ws_scores;
                sa.meta = meta;
                sa.state = c > 0 ? state : nullptr;
                sa.k = k;
                sa.row0 = r0;
                sa.rows = nr;
                sa.q_pos0 = q_pos0;
                sa.T = T;
                sa.c0 = c0;
                sa.clen = p.chunk;
                sa.slen = p.slen;
                sa.H = H_I;
                sa.m = m;
                st = launch_timed(CSA_KERNEL_SCORE, s, [&] {
                    return csa::launch_score(sa, dtype, D_I, p.tile, s);
                });
                if (st != CSA_OK) return st;
            }
            csa::SelectArgs se;
            se.ws = ws_scores;
            se.meta = meta;
            se.lists = lists;
            se.state = state;
            se.out_idx = idx;
            se.out_score = score;
            se.row0 = r0;
            se.rows = nr;
            se.q_pos0 = q_pos0;
            se.T = T;
            se.c0 = c0;
            se.clen = p.chunk;
            se.slen = p.slen;
            se.k = k;
            se.m = m;
            se.nsplit = (int32_t)p.splits;
            se.first = c == 0;
            // With splits every split's best k goes to its own list; the
            // merge rounds below combine them and write the outputs.
            se.emit = c == nch - 1 && p.splits == 1;
            st = launch_timed(CSA_KERNEL_SELECT, s, [&] { return csa::launch_select(se, s); });
            if (st != CSA_OK) return st;
            // Merge rounds: four lists into one while at least four are left
            // (k <= 2048), else two into one.
            for (int64_t left = p.splits; left > 1;) {
                const bool four = left >= 4 && k <= 2048;
                const int64_t next = four ? left / 4 : left / 2;
                csa::MergeArgs mg;
                mg.lists = lists;
                mg.state = state;
                mg.out_idx = idx;
                mg.out_score = score;
                mg.row0 = r0;
                mg.rows = nr;
                mg.k = k;
                mg.half = (int32_t)next;
                mg.four = four;
                mg.emit = next == 1;
                st = launch_timed(CSA_KERNEL_MERGE, s, [&] { return csa::launch_merge(mg, s); });
                if (st != CSA_OK) return st;
                left = next;
            }
        }
    }
    return CSA_OK;
}

}  // namespace

extern "C" {

int csa_indexer_topk(const void *q, const void *w, const void *kc, int32_t dtype, int64_t S,
                     int64_t T, int32_t H_I, int32_t D_I, int32_t m, int64_t k, int64_t q_pos0,
                     int32_t *idx, float *score, void *workspace, size_t workspace_bytes,
                     const csa_opts *opts, void *stream)
{
    Plan p;
    int64_t rows = 0;
    const int st = check_call(q, w, kc, dtype, S, T, H_I, D_I, m, k, q_pos0, idx, score,
                              workspace, workspace_bytes, opts, &p, &rows);
    if (st != CSA_OK) return st;
    return run_call(q, w, kc, dtype, S, T, H_I, D_I, m, k, q_pos0, idx, score, workspace, p, rows,
                    stream);
}

int csa_indexer_topk_noalloc(const void *q, const void *w, const void *kc, int32_t dtype,
                             int64_t S, int64_t T, int32_t H_I, int32_t D_I, int32_t m,
                             int64_t k, int64_t q_pos0, int32_t *idx, float *score,
                             const csa_opts *opts, void *stream)
{
    // The plan is made for the scratch size: a caller's budget can only
    // lower it.  The checks run on a stand-in workspace pointer (aligned,
    // never dereferenced) so that none of them needs a HIP call.
    csa_opts o{};
    if (opts) o = *opts;
    const int64_t cap = (int64_t)CSA_NOALLOC_SCRATCH_BYTES;
    if (o.workspace_budget >= 0 && (o.workspace_budget == 0 || o.workspace_budget > cap))
        o.workspace_budget = cap;
    Plan p;
    int64_t rows = 0;
    int st = check_call(q, w, kc, dtype, S, T, H_I, D_I, m, k, q_pos0, idx, score,
                        (void *)kAlign, CSA_NOALLOC_SCRATCH_BYTES, &o, &p, &rows);
    if (st == CSA_ERR_WORKSPACE_TOO_SMALL) return CSA_ERR_SCRATCH_TOO_SMALL;
    if (st != CSA_OK) return st;
    void *ws = nullptr;
    if (S > 0 && p.chunk > 0) {
        st = scratch_on(&ws);
        if (st != CSA_OK) return st;
    }
    return run_call(q, w, kc, dtype, S, T, H_I, D_I, m, k, q_pos0, idx, score, ws, p, rows,
                    stream);
}

int csa_indexer_topk_batched(const void *q, const void *w, const void *kc, int32_t dtype,
                             int64_t B, int64_t S, int64_t T, int32_t H_I, int32_t D_I,
                             int32_t m, int64_t k, int64_t q_pos0, int32_t *idx, float *score,
                             void *workspace, size_t workspace_bytes, const csa_opts *opts,
                             void *stream)
{
    if (B < 0) return CSA_ERR_BAD_SHAPE;
    Plan p;
    int64_t rows = 0;
    // Every problem has the same shape, so one check covers them all (slice
    // offsets keep the alignments: H_I*D_I and D_I elements are multiples of
    // 16 bytes, S*k outputs of 4).
    const int st = check_call(q, w, kc, dtype, S, T, H_I, D_I, m, k, q_pos0, idx, score,
                              workspace, workspace_bytes, opts, &p, &rows);
    if (st != CSA_OK || B == 0 || S == 0) return st;
    const size_t esz = dtype == CSA_BF16 ? 2 : 4;
    for (int64_t b = 0; b < B; ++b) {
        // The problems share the workspace: their launches are ordered on
        // the one stream.
        const int sb = run_call((const char *)q + (size_t)b * S * H_I * D_I * esz,
                                (const char *)w + (size_t)b * S * H_I * esz,
                                kc ? (const char *)kc + (size_t)b * T * D_I * esz : nullptr, dtype,
                                S, T, H_I, D_I, m, k, q_pos0, idx + (size_t)b * S * k,
                                score + (size_t)b * S * k, workspace, p, rows, stream);
        if (sb != CSA_OK) return sb;
    }
    return CSA_OK;
}

int csa_sparse_attention(const void *q, const void *kv, const int32_t *idx, void *out,
                         int32_t dtype, int64_t S, int64_t T, int32_t H, int32_t D_K,
                         int32_t D_V, int64_t k, float scale, void *stream)
{
    if (S < 0 || T < 0 || k < 0 || H <= 0 || D_K <= 0 || D_V <= 0) return CSA_ERR_BAD_SHAPE;
    if (dtype != CSA_BF16) return dtype == CSA_F32 ? CSA_ERR_UNSUPPORTED : CSA_ERR_BAD_DTYPE;
    // The kernel works with scale * log2(e); it must be finite too.
    const float scale_log2e = scale * 1.4426950408889634f;
    if (!std::isfinite(scale) || !std::isfinite(scale_log2e)) return CSA_ERR_BAD_SHAPE;
    if (!csa::attention_shape_supported(H, D_K, D_V)) return CSA_ERR_UNSUPPORTED;
    // T is bounded before the product, so that the product cannot overflow.
    if (k > ((int64_t)1 << 20) || S > INT32_MAX || T > INT32_MAX ||
        T * D_K * 2 >= ((int64_t)1 << 31))
        return CSA_ERR_UNSUPPORTED;
    if (S == 0) return CSA_OK;
    if (!q || !out || (k > 0 && !idx) || (T > 0 && !kv)) return CSA_ERR_NULL_PTR;
    if (((uintptr_t)q & 15) || ((uintptr_t)kv & 15) || ((uintptr_t)idx & 3) ||
        ((uintptr_t)out & 1))
        return CSA_ERR_MISALIGNED;
    csa::AttnArgs a;
    a.q = q;
    a.kv = kv;
    a.idx = idx;
    a.out = out;
    a.S = S;
    a.T = T;
    a.H = H;
    a.k = (int32_t)k;
    a.scale_log2e = scale_log2e;
    hipStream_t s = (hipStream_t)stream;
    return launch_timed(CSA_KERNEL_ATTENTION, s,
                        [&] { return csa::launch_attention(a, D_K, D_V, s); });
}

int csa_profile_enable(int enable)
{
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof_on = enable != 0;
    return CSA_OK;
}

int csa_profile_collect(double *ms_out, int64_t *launches_out, int32_t n_kinds)
{
    std::vector<ProfRecord> recs;
    {
        std::lock_guard<std::mutex> g(g_prof_mu);
        recs.swap(g_prof_records);
    }
    for (int i = 0; i < n_kinds; ++i) {
        if (ms_out) ms_out[i] = 0.0;
        if (launches_out) launches_out[i] = 0;
    }
    int st = CSA_OK;
    for (const ProfRecord &r : recs) {
        float ms = 0.0f;
        if (hipEventSynchronize(r.stop) != hipSuccess ||
            hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
            st = CSA_ERR_HIP;
        if (r.kind >= 0 && r.kind < n_kinds) {
            if (ms_out) ms_out[r.kind] += ms;
            if (launches_out) launches_out[r.kind] += 1;
        }
    }
    std::lock_guard<std::mutex> g(g_prof_mu);
    for (const ProfRecord &r : recs) {
        g_prof_pool.push_back(r.start);
        g_prof_pool.push_back(r.stop);
    }
    return st;
}

}  // extern "C"
