// Internal declarations shared by the driver and the kernel files of
// libcsa_indexer.so.  Not installed; the public interface is csa_indexer.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

// Keys usable by the query at absolute position `pos`: key j is usable iff
// (j+1)*m <= pos+1, capped by the T keys that exist.
__host__ __device__ inline int64_t n_usable(int64_t pos, int64_t T, int32_t m)
{
    int64_t n = (pos + 1) / m;
    if (n < 0) n = 0;
    return n < T ? n : T;
}

// One pass of the score kernel: a batch of query rows against one key chunk.
struct ScoreArgs {
    const void *q;    // [S][H][D], rows of this batch start at row0
    const void *w;    // [S][H]
    const void *kc;   // [T][D]
    float *ws;        // [rows][clen] head-reduced scores of this chunk
    int64_t row0;     // first q row of the batch
    int64_t rows;     // rows in the batch
    int64_t q_pos0;   // absolute position of q row 0
    int64_t T;
    int64_t c0;       // first key of the chunk
    int64_t clen;     // chunk length in keys; also the ws row stride
    int64_t kspan;    // keys handled by one workgroup along grid.y
    int32_t H;
    int32_t m;
};

// One pass of the select kernel over the same batch and chunk.
struct SelectArgs {
    const float *ws;      // [rows][clen] scores written by the score pass
    uint64_t *lists;      // [rows][k] running best-k lists (orderable keys)
    int32_t *counts;      // [rows] entries in each running list
    int32_t *out_idx;     // [S][k]
    float *out_score;     // [S][k]
    int64_t row0, rows, q_pos0, T;
    int64_t c0, clen;
    int64_t k;
    int32_t m;
    int32_t first;        // 1: no earlier chunk, the running lists start empty
    int32_t emit;         // 1: last chunk, sort the lists and write the outputs
};

// Dtype codes as in the public header.
enum { DT_F32 = 0, DT_BF16 = 1 };

// Score kernel: launches grid (ceil(rows/8) x ysplit) for bf16 or
// (rows x ceil(clen/256)) for fp32.  `ysplit` is ignored for fp32.
hipError_t launch_score(const ScoreArgs &a, int32_t dtype, int32_t D, int32_t key_tile,
                        int64_t ysplit, hipStream_t stream);

// Select kernel: one workgroup per row of the batch.
hipError_t launch_select(const SelectArgs &a, hipStream_t stream);

// Keys of one chunk piece that the select kernel stages in LDS at a time.
constexpr int kSelectPiece = 4096;
constexpr int kSelectThreads = 256;
constexpr int kScoreWaves = 8;  // query rows per score workgroup (one per wave)

}  // namespace csa
