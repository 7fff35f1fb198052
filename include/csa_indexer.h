/*
 * csa_indexer.h -- C ABI of libcsa_indexer.so, the MI355X (gfx950) library
 * for the Compressed Sparse Attention (CSA) lightning-indexer top-k.
 *
 * Operation (page "StreamIndex: Memory-Bounded Compressed Sparse Attention
 * via Streaming Top-k", Abstract): the lightning indexer, a learned scoring
 * projection over the compressed keys, scores every key for every query with
 * H_I indexer heads, and the top-k keys are kept per query.  The page's point
 * is that the public implementations build the whole [B,S,H_I,T] FP32 score
 * tensor before the top-k, while a chunked partition-merge top-k never does.
 * This library is such a partition-merge: it scores one chunk of keys for a
 * batch of queries at a time, keeps each query's best k per chunk and merges
 * them, so its scratch memory is bounded by the workspace the caller hands in
 * and never grows with S*T.
 *
 * The page prints no formula; the library computes
 *
 *   score(i,j) = sum_{h<H_I} w[i,h] * max(q[i,h,:] . kc[j,:], 0)
 *
 * for every key j usable by query row i: with p = q_pos0 + i its absolute
 * position, key j is usable iff (j+1)*m <= p+1, i.e. j < n(i) =
 * min(T, floor((p+1)/m)) (m is the compression ratio).  Row i of the output
 * holds its min(k, n(i)) best keys ordered by score descending, ties by key
 * index ascending, followed by padding idx = -1, score = -inf.  Scores are
 * fp32; a zero score is always +0.
 *
 * Memory: every pointer is a device pointer (HIP device memory of the current
 * device) owned by the caller.  Tensors are dense and row-major:
 *   q     [S][H_I][D_I]   dtype       (16-byte aligned)
 *   w     [S][H_I]        dtype       (aligned to the element size)
 *   kc    [T][D_I]        dtype       (16-byte aligned)
 *   idx   [S][k]          int32       (4-byte aligned)
 *   score [S][k]          float32     (4-byte aligned)
 *   workspace             bytes       (256-byte aligned)
 * Outputs are fully overwritten, padding included, and must not overlap the
 * inputs or the workspace.  The library allocates no device memory at call
 * time (csa_indexer_topk_noalloc works in a fixed array that is part of the
 * library's code object on each GPU) and keeps no state between calls that
 * affects results (apart from that, only the optional profiling counters
 * below).
 *
 * Asynchrony: all device work is enqueued on `stream` (a hipStream_t; NULL is
 * the default stream) and the call returns without waiting.  Results are
 * ready when the stream reaches that point.  Asynchronous device faults show
 * up at the caller's next synchronisation, not as a status here.  Host
 * threads may call the library concurrently, each with its own workspace
 * and outputs (the allocation-free form excepted, see there).
 *
 * Errors: functions return a csa status (0 = CSA_OK).  Every argument check
 * runs before any HIP call, so a call that fails a check enqueues nothing.
 * Inputs must be finite; NaN or Inf inputs are not detected and give
 * unspecified (but memory-safe) results.
 */
#ifndef CSA_INDEXER_H
#define CSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 4

/* Status codes. */
#define CSA_OK 0
#define CSA_ERR_NULL_PTR 1            /* a required pointer is NULL */
#define CSA_ERR_BAD_SHAPE 2           /* negative size, H_I/D_I/m/k out of range */
#define CSA_ERR_BAD_DTYPE 3           /* dtype is not CSA_F32 or CSA_BF16 */
#define CSA_ERR_MISALIGNED 4          /* a pointer breaks the alignment above */
#define CSA_ERR_WORKSPACE_TOO_SMALL 5 /* workspace_bytes below what one query block needs */
#define CSA_ERR_UNSUPPORTED 6         /* valid request outside what this build implements */
#define CSA_ERR_HIP 7                 /* a HIP call or kernel launch failed */
#define CSA_ERR_BAD_OPTION 8          /* a field of csa_opts is out of range */
#define CSA_ERR_SCRATCH_TOO_SMALL 9   /* allocation-free call: one query block needs more
                                         than CSA_NOALLOC_SCRATCH_BYTES */

/* Input dtypes (q, w and kc share one). */
#define CSA_F32 0  /* IEEE fp32 */
#define CSA_BF16 1 /* bfloat16; products are exact in fp32, sums are fp32 */

/* Supported ranges of this build. */
#define CSA_MAX_HEADS 64
#define CSA_MAX_K 4096

/*
 * Tuning options; a zero field (or a NULL pointer to the struct) means
 * "choose automatically".  Options change speed and workspace size only:
 * for a given input the outputs are bit-identical for every setting.
 */
typedef struct csa_opts {
    /* Keys per partition chunk: each query keeps its best k of every chunk
     * and merges them into a running list.  A multiple of 256 up to 2^24, or
     * 0. */
    int64_t chunk_keys;
    /* Keys staged in LDS per step of the bf16 score kernel: 64, 128, 192,
     * 256, or 0 (automatic: 192).  The fp32 path always stages 32 keys. */
    int32_t key_tile;
    /* Key splits (ignored when chunk_keys is set): the usable keys
     * form one chunk cut into this many splits that are scored and selected
     * in parallel, each split's best k going to its own list, and the lists
     * are merged in rounds that combine four lists (k <= 2048) or two.
     * For problems with few query rows (decoding a few new queries against
     * a long key cache), where chunks alone would leave most of the GPU
     * idle.  0 = automatic (used for fewer than 2048 rows
     * when one pass fits the workspace budget), 1 = never, or a power of two
     * up to 128. */
    int32_t key_splits;
    /* Upper bound, in bytes, on the workspace that
     * csa_indexer_topk_workspace_size plans for; 0 means 2 GiB.  A smaller
     * workspace only makes the library process fewer query rows per pass. */
    int64_t workspace_budget;
    int64_t reserved[4]; /* must be 0 */
} csa_opts;

/* CSA_ABI_VERSION of the built library. */
int csa_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *csa_status_str(int status);

/*
 * Workspace bytes that csa_indexer_topk needs to process all S rows in as few
 * passes as the budget allows.  Pure host arithmetic: no device access.
 * Arguments as for csa_indexer_topk (q_pos0 included, since it decides how
 * many keys the last row may use).  Writes the size to *bytes_out; the size is
 * 0 when no row has a usable key.
 */
int csa_indexer_topk_workspace_size(int64_t S, int64_t T, int32_t H_I, int32_t D_I,
                                    int32_t m, int64_t k, int64_t q_pos0, int32_t dtype,
                                    const csa_opts *opts, size_t *bytes_out);

/*
 * The indexer top-k (see the top of this file for the operation, layouts and
 * error behaviour).
 *   q, w, kc      inputs, dtype `dtype`
 *   S, T          query rows and compressed keys (>= 0; T < 2^31)
 *   H_I           indexer heads, 1..CSA_MAX_HEADS
 *   D_I           head dimension: 32, 64 or 128
 *   m             compression ratio (>= 1)
 *   k             keys kept per query, 1..CSA_MAX_K (k > T is fine: padding)
 *   q_pos0        absolute position of row 0 (>= 0): lets a caller process a
 *                 range of rows of a longer sequence
 *   idx, score    outputs [S][k]
 *   workspace     scratch device memory of workspace_bytes bytes; may be NULL
 *                 when the size query returns 0.  Any size at least one query
 *                 block's share works; larger ones need fewer passes.
 *   opts          tuning options or NULL
 *   stream        hipStream_t to enqueue on (NULL = default stream)
 */
int csa_indexer_topk(const void *q, const void *w, const void *kc, int32_t dtype,
                     int64_t S, int64_t T, int32_t H_I, int32_t D_I, int32_t m,
                     int64_t k, int64_t q_pos0, int32_t *idx, float *score,
                     void *workspace, size_t workspace_bytes, const csa_opts *opts,
                     void *stream);

/*
 * Allocation-free form of csa_indexer_topk, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same operation, arguments, layouts, options,
 * outputs and kernels, but no workspace argument.  Its scratch is a fixed
 * device array of CSA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held from the library's first use on that GPU until the process ends.
 * The call plans its passes for that size (opts->workspace_budget, if set,
 * can only lower it), so the outputs are bit-identical to csa_indexer_topk's
 * for the same inputs; with large problems it takes more passes.
 *
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (on different streams, or from different host threads without an
 * order between them) race and give undefined results.  Calls ordered on
 * one stream are fine.  Nothing in the scratch needs to start at zero; its
 * contents after a call are unspecified.
 *
 * Errors as for csa_indexer_topk, plus CSA_ERR_SCRATCH_TOO_SMALL when one
 * query block's share (8 rows x (4 x chunk keys + list and summary bytes))
 * exceeds the scratch, e.g. with a caller-fixed chunk_keys of 2^23 or more
 * keys.  Argument checks, that one included, run before any HIP call.  On its
 * first call on a GPU it looks up the scratch address there (no allocation);
 * a failed lookup gives CSA_ERR_HIP.  It allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine.
 */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int csa_indexer_topk_noalloc(const void *q, const void *w, const void *kc, int32_t dtype,
                             int64_t S, int64_t T, int32_t H_I, int32_t D_I, int32_t m,
                             int64_t k, int64_t q_pos0, int32_t *idx, float *score,
                             const csa_opts *opts, void *stream);

/*
 * Batched form (B=1 is the single call above): B independent problems of the
 * same shape, each with its own queries and its own compressed keys, e.g. the
 * sequences of a batch.  Layouts are the single call's with a leading batch
 * dimension, densely packed:
 *   q [B][S][H_I][D_I], w [B][S][H_I], kc [B][T][D_I], idx/score [B][S][k].
 * Problem b is exactly csa_indexer_topk on the b-th slices (same q_pos0 and
 * options), so its outputs are bit-identical to that call's.  The workspace
 * is sized for one problem (csa_indexer_topk_workspace_size with the same
 * S, T, ...) and is reused by the problems in turn, all enqueued on `stream`.
 * B = 0 is valid (no work); B < 0 is CSA_ERR_BAD_SHAPE.  All argument checks
 * run before any HIP call; a HIP failure while enqueueing problem b returns
 * CSA_ERR_HIP with problems 0..b-1 already enqueued.
 */
int csa_indexer_topk_batched(const void *q, const void *w, const void *kc, int32_t dtype,
                             int64_t B, int64_t S, int64_t T, int32_t H_I, int32_t D_I,
                             int32_t m, int64_t k, int64_t q_pos0, int32_t *idx, float *score,
                             void *workspace, size_t workspace_bytes, const csa_opts *opts,
                             void *stream);

/*
 * Kernel timing for benchmarks.  While enabled, every kernel launch made by
 * the library's entry points (the indexer calls, batched and allocation-free
 * forms included, and csa_sparse_attention) in this process is bracketed by
 * HIP events recorded on the launch's stream.  csa_profile_collect waits for those events, adds up the
 * elapsed milliseconds and the launch counts per kernel kind into
 * ms_out[kind] and launches_out[kind] for kind < n_kinds (either array may be
 * NULL), then forgets them.  Not thread-safe; meant for single-threaded
 * benchmark drivers.
 */
#define CSA_KERNEL_SCORE 0  /* chunk scoring: MFMA contraction + ReLU + head sum */
#define CSA_KERNEL_SELECT 1 /* chunk top-k, merge into running lists, emit */
#define CSA_KERNEL_MERGE 2  /* merge rounds of key-split lists, emit */
#define CSA_KERNEL_ATTENTION 3 /* sparse attention over the selected entries */
#define CSA_KERNEL_KINDS 4
int csa_profile_enable(int enable);
int csa_profile_collect(double *ms_out, int64_t *launches_out, int32_t n_kinds);

/*
 * Sparse attention over each query's selected entries: the consumer of the
 * indexer's output in the CSA pipeline.  The page ("StreamIndex: Memory-
 * Bounded Compressed Sparse Attention via Streaming Top-k", Abstract) says
 * that a sparse attention kernel reads only the selected compressed entries
 * and gives no formula or dimensions for it.  This function computes the
 * plain softmax attention of each query row over its selected entries in
 * the shared-latent (multi-query) form: all H heads attend over the same
 * entries; an entry's latent row kv[e, :] is the key and its first D_V
 * dims are the value:
 *
 *   out[i,h,:] = sum_{e in sel(i)} p_{h,e} kv[e, :D_V],
 *   p_{h,e}    = softmax over e of (scale * q[i,h,:] . kv[e,:])
 *
 * where sel(i) lists idx[i, :] without its -1 entries (an entry listed twice
 * counts twice).  A row with nothing selected gives zeros.
 *
 *   q    [S][H][D_K]   bf16   (16-byte aligned)
 *   kv   [T][D_K]      bf16   (16-byte aligned; may be NULL when T == 0)
 *   idx  [S][k]        int32  (4-byte aligned; may be NULL when k == 0)
 *   out  [S][H][D_V]   bf16   (2-byte aligned), fully overwritten
 *
 * idx entries are -1 or in [0, T) (what csa_indexer_topk writes); any
 * other value is treated like -1 (padding).
 * Logits and the softmax are fp32 (exp2 based, reference max moved lazily),
 * the weights are rounded to bf16 for the weighted sum, which accumulates in
 * fp32; out is rounded to bf16.
 *
 * dtype must be CSA_BF16 (CSA_F32 gives CSA_ERR_UNSUPPORTED).  This build
 * supports H in {32, 64} and (D_K, D_V) in {(576, 512), (128, 128)}; other
 * positive shapes give CSA_ERR_UNSUPPORTED, as do k > 2^20, S > 2^31 - 1 and
 * T * D_K * 2 >= 2^31.  scale must be finite, and so must scale * log2(e)
 * in fp32, i.e. |scale| below about 2.36e38 (else CSA_ERR_BAD_SHAPE).
 * Enqueued on `stream`; allocates nothing; needs no workspace.
 */
int csa_sparse_attention(const void *q, const void *kv, const int32_t *idx, void *out,
                         int32_t dtype, int64_t S, int64_t T, int32_t H, int32_t D_K,
                         int32_t D_V, int64_t k, float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_INDEXER_H */
