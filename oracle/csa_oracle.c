/*
 * csa_oracle.c -- plain CPU oracle for the Compressed Sparse Attention (CSA)
 * lightning-indexer step: score every causally valid compressed key for a
 * query, then keep that query's top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may build, load or call this file.  It shares
 * no code, header, table or helper with the GPU library, and the GPU library
 * never calls it.  It is deliberately slow and literal: one query row at a
 * time, every score in fp32 with a fixed summation order, then a full sort of
 * the row.  It is the "materialise then reduce" semantics that the page
 * "StreamIndex: Memory-Bounded Compressed Sparse Attention via Streaming
 * Top-k" (Abstract) uses as ground truth, computed row by row so that only one
 * row of scores ever exists.
 *
 * What it computes (the page names the pipeline -- a learned scoring
 * projection over compressed keys, then top-k per query -- but prints no
 * formula; the readings taken here are listed with the design notes):
 *
 *   n(i)      = min(T, floor((pos(i) + 1) / m))      key j usable iff (j+1)*m <= pos(i)+1
 *   a(i,h,j)  = sum_{d=0..D-1} q[i,h,d] * kc[j,d]     d ascending, from +0
 *   s(i,j)    = sum_{h=0..H-1} w[i,h] * max(a(i,h,j), 0)   h ascending, from +0
 *   row order : s descending, then j ascending (fp32 value compare, so -0 == +0)
 *   output    : the first min(k, n(i)) keys of that order, then idx -1 / score -inf
 *
 * Arithmetic: every product and every sum is a separate fp32 operation rounded
 * to nearest even.  Build with -ffp-contract=off and without fast-math so the
 * compiler neither fuses nor reorders them.
 *
 * Inputs must be finite; a non-finite input makes the call return
 * CSA_ORACLE_NONFINITE before any output is written.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CSA_ORACLE_OK 0
#define CSA_ORACLE_BAD_ARG (-1)
#define CSA_ORACLE_NONFINITE (-2)
#define CSA_ORACLE_NO_MEMORY (-3)

/* Number of keys query position `pos` may use (causal rule). */
static int64_t oracle_n_valid(int64_t pos, int64_t T, int32_t m)
{
    int64_t n = (pos + 1) / m;
    if (n < 0) n = 0;
    return n < T ? n : T;
}

/* One score s(i,j): nested sums in the fixed order stated above. */
static float oracle_score(const float *q_row, const float *w_row,
                          const float *key, int32_t H, int32_t D)
{
    float s = 0.0f;
    for (int32_t h = 0; h < H; ++h) {
        const float *qh = q_row + (int64_t)h * D;
        float a = 0.0f;
        for (int32_t d = 0; d < D; ++d) {
            float p = qh[d] * key[d];
            a = a + p;
        }
        float r = (a > 0.0f) ? a : 0.0f;
        float t = w_row[h] * r;
        s = s + t;
    }
    return s;
}

/* Scores of one query row for keys 0..n-1, written to out[0..n). */
int csa_oracle_row_scores(const float *q_row, const float *w_row,
                          const float *kc, int64_t n, int32_t H, int32_t D,
                          float *out)
{
    if (!q_row || !w_row || (n > 0 && (!kc || !out)) || H <= 0 || D <= 0 || n < 0)
        return CSA_ORACLE_BAD_ARG;
    for (int64_t j = 0; j < n; ++j)
        out[j] = oracle_score(q_row, w_row, kc + j * (int64_t)D, H, D);
    return CSA_ORACLE_OK;
}

/* Sort entry: a key index and its score. */
typedef struct {
    float s;
    int32_t j;
} oracle_entry;

/* Total order of the output: score descending, then key index ascending.
 * The comparison is on fp32 values, so -0 and +0 are equal and fall back to
 * the index. */
static int oracle_cmp(const void *pa, const void *pb)
{
    const oracle_entry *a = (const oracle_entry *)pa;
    const oracle_entry *b = (const oracle_entry *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    if (a->j < b->j) return -1;
    if (a->j > b->j) return 1;
    return 0;
}

typedef struct {
    const float *q, *w, *kc;
    const int64_t *pos;
    int64_t n_rows, T, k;
    int32_t H, D, m;
    int32_t *idx;
    float *score;
    int32_t tid, nthreads;
    int status;
} oracle_job;

static void *oracle_worker(void *arg)
{
    oracle_job *job = (oracle_job *)arg;
    oracle_entry *row = NULL;
    if (job->T > 0) {
        row = (oracle_entry *)malloc((size_t)job->T * sizeof(oracle_entry));
        if (!row) {
            job->status = CSA_ORACLE_NO_MEMORY;
            return NULL;
        }
    }
    /* Rows are dealt round-robin so that long (late) and short (early)
     * causal rows spread evenly over the threads. */
    for (int64_t r = job->tid; r < job->n_rows; r += job->nthreads) {
        const float *q_row = job->q + r * (int64_t)job->H * job->D;
        const float *w_row = job->w + r * (int64_t)job->H;
        int64_t n = oracle_n_valid(job->pos[r], job->T, job->m);
        for (int64_t j = 0; j < n; ++j) {
            row[j].s = oracle_score(q_row, w_row, job->kc + j * (int64_t)job->D,
                                    job->H, job->D);
            row[j].j = (int32_t)j;
        }
        if (n > 1) qsort(row, (size_t)n, sizeof(oracle_entry), oracle_cmp);
        int32_t *idx = job->idx + r * job->k;
        float *score = job->score + r * job->k;
        for (int64_t t = 0; t < job->k; ++t) {
            if (t < n) {
                idx[t] = row[t].j;
                score[t] = row[t].s;
            } else {
                idx[t] = -1;
                score[t] = -INFINITY;
            }
        }
    }
    free(row);
    job->status = CSA_ORACLE_OK;
    return NULL;
}

static int oracle_all_finite(const float *x, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

/*
 * Top-k for n_rows query rows.
 *   q     [n_rows][H][D] fp32   query rows (bf16 callers upcast exactly first)
 *   w     [n_rows][H]    fp32   per-query head weights
 *   kc    [T][D]         fp32   compressed keys, shared by every head
 *   pos   [n_rows]       int64  absolute position of each row (causality)
 *   idx   [n_rows][k]    int32  out: key indices, -1 padding
 *   score [n_rows][k]    fp32   out: scores, -inf padding
 * nthreads <= 0 means one thread.  Returns CSA_ORACLE_OK or a negative code.
 */
int csa_oracle_topk(const float *q, const float *w, const float *kc,
                    const int64_t *pos, int64_t n_rows, int64_t T, int32_t H,
                    int32_t D, int32_t m, int64_t k, int32_t *idx, float *score,
                    int32_t nthreads)
{
    if (n_rows < 0 || T < 0 || H <= 0 || D <= 0 || m <= 0 || k <= 0)
        return CSA_ORACLE_BAD_ARG;
    if (T > INT32_MAX) return CSA_ORACLE_BAD_ARG;
    if (n_rows == 0) return CSA_ORACLE_OK;
    if (!q || !w || !pos || !idx || !score || (T > 0 && !kc))
        return CSA_ORACLE_BAD_ARG;
    if (!oracle_all_finite(q, n_rows * (int64_t)H * D) ||
        !oracle_all_finite(w, n_rows * (int64_t)H) ||
        !oracle_all_finite(kc, T * (int64_t)D))
        return CSA_ORACLE_NONFINITE;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > n_rows) nthreads = (int32_t)n_rows;

    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *threads = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !threads) {
        free(jobs);
        free(threads);
        return CSA_ORACLE_NO_MEMORY;
    }
    int status = CSA_ORACLE_OK;
    int32_t started = 0;
    for (int32_t t = 0; t < nthreads; ++t) {
        jobs[t] = (oracle_job){q, w, kc, pos, n_rows, T, k, H, D, m,
                               idx, score, t, nthreads, CSA_ORACLE_OK};
        if (t == 0) continue; /* thread 0's share runs on the calling thread */
        if (pthread_create(&threads[t], NULL, oracle_worker, &jobs[t]) != 0) {
            status = CSA_ORACLE_NO_MEMORY;
            break;
        }
        started = t;
    }
    if (status == CSA_ORACLE_OK) oracle_worker(&jobs[0]);
    for (int32_t t = 1; t <= started; ++t) pthread_join(threads[t], NULL);
    if (status == CSA_ORACLE_OK)
        for (int32_t t = 0; t < nthreads; ++t)
            if (jobs[t].status != CSA_ORACLE_OK) status = jobs[t].status;
    free(jobs);
    free(threads);
    return status;
}
