// Internal declarations shared by the driver and the kernel files of
// libcsa_indexer.so.  Not installed; the public interface is csa_indexer.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace csa {

// Keys usable by the query at absolute position `pos`: key j is usable iff
// (j+1)*m <= pos+1, capped by the T keys that exist.
__host__ __device__ inline int64_t n_usable(int64_t pos, int64_t T, int32_t m)
{
    int64_t n = (pos + 1) / m;
    if (n < 0) n = 0;
    return n < T ? n : T;
}

// Per-row state kept between chunk passes: the running list's k-th key
// (0 while the list holds fewer than k entries) and its length.
struct RowState {
    uint64_t theta;
    int32_t count;
    int32_t pad;
};

// Per-row summary of one chunk written by the score kernel: a histogram of
// the orderable scores (top 11 bits) of the chunk keys that beat the row's
// theta, reduced to the bin that holds the k-th best of them.
struct ChunkMeta {
    uint32_t bin;     // threshold bin b* (valid when total > k)
    uint32_t above;   // entries in bins above b*
    uint32_t in_bin;  // entries in bin b*
    uint32_t total;   // entries counted (keys beating theta)
};
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;

// Monotone map of an fp32 score onto uint32 (-0 taken as +0): a larger
// value means a larger score.
__host__ __device__ inline uint32_t orderable(float s)
{
    uint32_t u;
    __builtin_memcpy(&u, &s, 4);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One pass of the score kernel: a batch of query rows against one key chunk.
struct ScoreArgs {
    const void *q;    // [S][H][D], rows of this batch start at row0
    const void *w;    // [S][H]
    const void *kc;   // [T][D]
    uint32_t *ws;     // [rows][clen] head-reduced scores of this chunk, as orderable()
    ChunkMeta *meta;  // [rows] chunk summary (bf16 path only; may be null)
    const RowState *state;  // [rows] theta from earlier chunks, or null
    int64_t k;
    int64_t row0;     // first q row of the batch
    int64_t rows;     // rows in the batch
    int64_t q_pos0;   // absolute position of q row 0
    int64_t T;
    int64_t c0;       // first key of the chunk
    int64_t clen;     // chunk length in keys; also the ws row stride
    int64_t slen;     // keys per split (grid.y splits the chunk; slen == clen: no split)
    int32_t H;
    int32_t m;
};

// One pass of the select kernel over the same batch and chunk.
//
// With splits (nsplit > 1) every (split y, row r) pair is a virtual row
// y*rows + r that selects among the split's keys [c0 + y*slen, +slen) and
// leaves its sorted best k in lists / state at that index (first = 1,
// emit = 0); the merge kernel then combines the splits' lists.
struct SelectArgs {
    const uint32_t *ws;   // [rows][clen] orderable() scores written by the score pass
    const ChunkMeta *meta;  // [nsplit*rows] chunk summaries, or null (then no shortcut)
    uint64_t *lists;      // [nsplit*rows][k] running best-k lists, sorted descending
    RowState *state;      // [nsplit*rows] running list length and k-th key
    int32_t *out_idx;     // [S][k]
    float *out_score;     // [S][k]
    int64_t row0, rows, q_pos0, T;
    int64_t c0, clen;
    int64_t slen;         // keys per split (== clen without splits)
    int64_t k;
    int32_t m;
    int32_t nsplit;       // splits of the chunk (1: none)
    int32_t first;        // 1: no earlier chunk, the running lists start empty
    int32_t emit;         // 1: last chunk, sort the lists and write the outputs
};

// One round of the merge of split lists: for p < half, the lists of virtual
// rows p*rows + r and (p+half)*rows + r are merged into the first (with
// `four`, k <= 2048 only: the lists p + j*half, j = 0..3); with emit (the
// last round) the merged best k are written as the row's outputs.
struct MergeArgs {
    uint64_t *lists;      // [splits*rows][k]
    RowState *state;      // [splits*rows]
    int32_t *out_idx;     // [S][k]
    float *out_score;     // [S][k]
    int64_t row0, rows, k;
    int32_t half;
    int32_t emit;
    int32_t four;
};

// Dtype codes as in the public header.
enum { DT_F32 = 0, DT_BF16 = 1 };

// Raises a kernel's dynamic LDS limit on the current device, once per
// device: function attributes belong to a device, so `done` holds one bit
// per device ordinal (devices past 63 set it on every call, which is
// harmless).
inline hipError_t set_dynamic_lds(const void *fn, int bytes, std::atomic<uint64_t> &done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    if (bit) done.fetch_or(bit, std::memory_order_relaxed);
    return hipSuccess;
}

// Score kernel (either dtype): grid ceil(rows/8) x splits workgroups, each
// covering its split of the chunk for its 8 rows; the chunk summary of row r
// in split y goes to meta[y*rows + r].  key_tile applies to bf16 only.
hipError_t launch_score(const ScoreArgs &a, int32_t dtype, int32_t D, int32_t key_tile,
                        hipStream_t stream);

// Score workgroups that one CU runs at once (0 on error), for sizing passes
// in whole rounds of workgroups.
int score_blocks_per_cu(int32_t dtype, int32_t D, int32_t H, int32_t key_tile);

// Select kernel: one workgroup per (virtual) row of the batch.
hipError_t launch_select(const SelectArgs &a, hipStream_t stream);

// Merge kernel: one workgroup per (row, list pair) of a merge round.
hipError_t launch_merge(const MergeArgs &a, hipStream_t stream);

// Sparse attention over each query row's selected entries (one workgroup
// per row): q [S][H][dk] bf16, kv [T][dk] bf16 (the value of an entry is
// the first dv dims of its row), idx [S][k] int32 (-1 = none), out
// [S][H][dv] bf16.
struct AttnArgs {
    const void *q;
    const void *kv;
    const int32_t *idx;
    void *out;
    int64_t S, T;
    int32_t H, k;
    float scale_log2e;  // softmax scale times log2(e): the kernel uses exp2
};

// Supported shapes: H in {32, 64}; (dk, dv) in {(576, 512), (128, 128)}.
bool attention_shape_supported(int32_t H, int32_t dk, int32_t dv);
hipError_t launch_attention(const AttnArgs &a, int32_t dk, int32_t dv, hipStream_t stream);

// Keys of one chunk piece that the select kernel stages in LDS at a time.
constexpr int kSelectPiece = 2048;
constexpr int kSelectThreads = 256;
constexpr int kScoreWaves = 8;  // query rows per score workgroup (one per wave)

}  // namespace csa
