/*
 * oracle.c -- plain fp64 CPU reference for chunked causal grouped-query
 * prefill attention over a KV cache.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never
 * links, calls or includes it, and it includes nothing from the GPU library.
 *
 * What is computed.  The definition is the one in the gnosis handoff page
 * "Prefill attention -> GPU: handoff", section "GPU design (the real fix)":
 *
 *   - the chunk's T query tokens are at sequence positions
 *     start_pos .. start_pos+T-1 and see L = start_pos + T cached keys;
 *   - grouped-query attention: num_kv_groups = num_heads / num_kv_heads and
 *     query head h uses kv head h / num_kv_groups;
 *   - scores are the dot product q.k multiplied by 1/sqrt(head_dim), the scale
 *     being applied before the row maximum and the softmax (Step 2);
 *   - key j is valid for query t only when j <= start_pos + t; masked keys
 *     contribute exactly nothing, as in the page's CPU loop, whose sum runs
 *     over keys 0..=pos only (Step 2, and "What already shipped": the per-(token, head)
 *     loop over the causal range 0..=pos);
 *   - row softmax, then the probability-weighted sum of the value rows
 *     (Step 3).
 *
 * The optional sliding window comes from the TensorSharp design page
 * "Design: closing the Gemma-4 long-prompt prefill gap", section 5, Option A:
 * each row's valid keys form one contiguous band [lo, hi] derived from
 * (start_pos, N, window).  The pages do not fix lo; this oracle takes the
 * band of the `window` most recent keys including the query's own position,
 * lo = max(0, pos - window + 1), which is also what a ring of `window` slots
 * written at pos % window holds (same page, requirement R4).  window <= 0
 * means no window.
 *
 * Layouts (gnosis page, "GPU design", Layout):
 *   q   element (t, h, d) at q[t*q_row_stride + h*head_dim + d]
 *   k,v element (kh, j, d) at k[kh*kv_head_stride + j*head_dim + d],
 *       i.e. one contiguous [L x head_dim] block per kv head, blocks
 *       kv_head_stride elements apart (a cache allocated for more than L
 *       positions has kv_head_stride = capacity*head_dim)
 *   out element (t, h, d) at out[(t*num_heads + h)*head_dim + d]
 *
 * Ring caches (the *_ring entry points).  Requirement R4 of the TensorSharp
 * page (section 4, "Requirements to enable replay") has sliding-window
 * layers write position pos into slot pos % (ring size) of a circular cache.
 * There key j of kv head kh is element (kh, j % ring_slots, d); nothing else
 * changes.  The ring must hold every key the chunk reads at the same time,
 * min(L, window + T - 1) slots (L for window 0); a shorter ring is an invalid
 * argument.
 *
 * Paged caches (the *_paged entry points; the FreeToken page "perf(spec):
 * capture the gemma4 assistant draft in cuda graphs" reads a sequence's
 * [0, cached_len) keys through its page table).  A pool of num_pages pages,
 * each holding page_size consecutive positions of every kv head: element
 * (pg, kh, r, d) at pool[((pg*num_kv_heads + kh)*page_size + r)*head_dim + d];
 * key j of kv head kh is row j % page_size of page page_table[j / page_size].
 * Every key a row reads must lie on a page of the pool (else invalid).
 *
 * Inputs are fp32 storage.  bf16 and fp16 values widen exactly to fp32, so
 * callers holding those types pass their fp32 images.  Every product and sum
 * is done in fp64 (the page's "independent f64 CPU recompute",
 * "Implementation status"), keys in ascending order, sums sequential.
 * Threads split the flat set of (t, h) rows; the arithmetic of a row does
 * not depend on the thread count (the page's argument for its rayon split,
 * "What already shipped").
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -pthread oracle.c -lm
 * (no -ffast-math: the order of the sums is part of the definition).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

struct problem {
    const float *q;
    const float *k;
    const float *v;
    int64_t q_row_stride;   /* elements between consecutive query tokens  */
    int64_t kv_head_stride; /* elements between consecutive kv heads      */
    int T, start_pos, num_heads, num_kv_heads, head_dim, window;
    int ring;               /* ring slots per kv head; 0: key j in row j */
    const int32_t *page_table; /* paged cache: page of each page_size keys, else NULL */
    int page_size, num_pages;
};

static int check_pages(const struct problem *P);
static int first_key(int pos, int window);

static int check_problem(const struct problem *P)
{
    if (!P->q || !P->k || !P->v) return -1;
    if (P->T < 1 || P->start_pos < 0) return -1;
    if (P->num_heads < 1 || P->num_kv_heads < 1 || P->head_dim < 1) return -1;
    if (P->num_heads % P->num_kv_heads != 0) return -1;
    if (P->window < 0) return -1;
    if (P->q_row_stride < (int64_t)P->num_heads * P->head_dim) return -1;
    if (P->ring < 0) return -1;
    if (P->page_table) return check_pages(P);
    const int64_t L = (int64_t)P->start_pos + P->T;
    if (P->ring > 0) {
        const int64_t need = P->window > 0 && (int64_t)P->window + P->T - 1 < L
                                 ? (int64_t)P->window + P->T - 1 : L;
        if (P->ring < need) return -1;
        if (P->kv_head_stride < (int64_t)P->ring * P->head_dim) return -1;
    } else if (P->kv_head_stride < L * P->head_dim) {
        return -1;
    }
    return 0;
}

/* Row of key j in its kv head's block: j, or its slot in a ring cache. */
static int64_t key_row(const struct problem *P, int j)
{
    return P->ring > 0 ? j % P->ring : j;
}

/* Element offset of key j of kv head kv_h from the start of k (or v). */
static int64_t key_offset(const struct problem *P, int kv_h, int j)
{
    if (P->page_table) {
        const int64_t page = P->page_table[j / P->page_size];
        return ((page * P->num_kv_heads + kv_h) * P->page_size + j % P->page_size) * P->head_dim;
    }
    return (int64_t)kv_h * P->kv_head_stride + key_row(P, j) * P->head_dim;
}

/* Paged cache: every key some row reads lies on a page of the pool. */
static int check_pages(const struct problem *P)
{
    if (P->page_size < 1 || P->num_pages < 1) return -1;
    for (int t = 0; t < P->T; ++t) {
        const int last = P->start_pos + t;
        const int lo = first_key(last, P->window);
        for (int j = lo; j < last + 1; ++j) {
            const int32_t pg = P->page_table[j / P->page_size];
            if (pg < 0 || pg >= P->num_pages) return -1;
        }
    }
    return 0;
}

/* First valid key of the query at absolute position pos. */
static int first_key(int pos, int window)
{
    if (window > 0 && pos - window + 1 > 0) return pos - window + 1;
    return 0;
}

/*
 * One output row: query token t, query head h.  `scores` has room for
 * start_pos + T doubles.  Writes head_dim doubles to out_row.
 */
static void attend_row(const struct problem *P, int t, int h, double *scores, double *out_row)
{
    const int D = P->head_dim;
    const int pos = P->start_pos + t;
    const int lo = first_key(pos, P->window);
    const int num_kv_groups = P->num_heads / P->num_kv_heads;
    const int kv_h = h / num_kv_groups;
    const float *q_row = P->q + (int64_t)t * P->q_row_stride + (int64_t)h * D;
    const double scale = 1.0 / sqrt((double)D);
    const int n = pos - lo + 1;

    /* scores over the valid keys lo..=pos, scaled before the softmax */
    for (int j = lo; j <= pos; ++j) {
        const float *k_row = P->k + key_offset(P, kv_h, j);
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += (double)q_row[d] * (double)k_row[d];
        scores[j - lo] = dot * scale;
    }

    /* row softmax: subtract the row maximum, exponentiate, normalise */
    double row_max = scores[0];
    for (int i = 1; i < n; ++i)
        if (scores[i] > row_max) row_max = scores[i];
    double total = 0.0;
    for (int i = 0; i < n; ++i) {
        scores[i] = exp(scores[i] - row_max);
        total += scores[i];
    }
    for (int i = 0; i < n; ++i)
        scores[i] = scores[i] / total;

    /* probability-weighted sum of the value rows, keys ascending */
    for (int d = 0; d < D; ++d)
        out_row[d] = 0.0;
    for (int j = lo; j <= pos; ++j) {
        const double p = scores[j - lo];
        const float *v_row = P->v + key_offset(P, kv_h, j);
        for (int d = 0; d < D; ++d)
            out_row[d] += p * (double)v_row[d];
    }
}

/* ---- threading over a list of (t, h) rows -------------------------------- */

struct row_job {
    const struct problem *P;
    const int32_t *row_t; /* NULL: all rows, row i = (i / num_heads, i % num_heads) */
    const int32_t *row_h;
    int64_t nrows;
    double *out;          /* nrows x head_dim */
    int worker, nworkers;
    int failed;
};

static void *row_worker(void *arg)
{
    struct row_job *J = (struct row_job *)arg;
    const struct problem *P = J->P;
    double *scores = (double *)malloc(sizeof(double) * (size_t)(P->start_pos + P->T));
    if (!scores) {
        J->failed = 1;
        return NULL;
    }
    for (int64_t i = J->worker; i < J->nrows; i += J->nworkers) {
        int t, h;
        if (J->row_t) {
            t = J->row_t[i];
            h = J->row_h[i];
        } else {
            t = (int)(i / P->num_heads);
            h = (int)(i % P->num_heads);
        }
        attend_row(P, t, h, scores, J->out + i * P->head_dim);
    }
    free(scores);
    return NULL;
}

static int run_rows(const struct problem *P, const int32_t *row_t, const int32_t *row_h,
                    int64_t nrows, double *out, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 1024) nthreads = 1024;
    if ((int64_t)nthreads > nrows) nthreads = (int)nrows;
    struct row_job *jobs = (struct row_job *)calloc((size_t)nthreads, sizeof(struct row_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -2;
    }
    int started = 0, rc = 0;
    for (int w = 0; w < nthreads; ++w) {
        jobs[w].P = P;
        jobs[w].row_t = row_t;
        jobs[w].row_h = row_h;
        jobs[w].nrows = nrows;
        jobs[w].out = out;
        jobs[w].worker = w;
        jobs[w].nworkers = nthreads;
    }
    for (int w = 1; w < nthreads; ++w) {
        if (pthread_create(&tids[w], NULL, row_worker, &jobs[w]) != 0) {
            /* the rows of a worker that could not start are taken by this thread */
            jobs[w].failed = 2;
            continue;
        }
        ++started;
    }
    row_worker(&jobs[0]);
    for (int w = 1; w < nthreads; ++w) {
        if (jobs[w].failed == 2) {
            jobs[w].failed = 0;
            row_worker(&jobs[w]);
        } else {
            pthread_join(tids[w], NULL);
        }
    }
    (void)started;
    for (int w = 0; w < nthreads; ++w)
        if (jobs[w].failed) rc = -2;
    free(jobs);
    free(tids);
    return rc;
}

/* ---- exported entry points ----------------------------------------------- */

/*
 * Whole chunk: out is [T][num_heads][head_dim] fp64.
 * Returns 0, -1 for invalid arguments, -2 when memory runs out.
 */
int oracle_prefill_attention(const float *q, int64_t q_row_stride,
                             const float *k_cache, const float *v_cache, int64_t kv_head_stride,
                             double *out, int T, int start_pos, int num_heads, int num_kv_heads,
                             int head_dim, int window, int nthreads)
{
    struct problem P = {q, k_cache, v_cache, q_row_stride, kv_head_stride,
                        T, start_pos, num_heads, num_kv_heads, head_dim, window, 0, NULL, 0, 0};
    if (check_problem(&P) || !out) return -1;
    return run_rows(&P, NULL, NULL, (int64_t)T * num_heads, out, nthreads);
}

/* Whole chunk over a ring cache of ring_slots slots per kv head. */
int oracle_prefill_attention_ring(const float *q, int64_t q_row_stride,
                                  const float *k_ring, const float *v_ring, int64_t kv_head_stride,
                                  int ring_slots, double *out, int T, int start_pos,
                                  int num_heads, int num_kv_heads, int head_dim, int window,
                                  int nthreads)
{
    struct problem P = {q, k_ring, v_ring, q_row_stride, kv_head_stride,
                        T, start_pos, num_heads, num_kv_heads, head_dim, window, ring_slots, NULL, 0, 0};
    if (ring_slots < 1 || check_problem(&P) || !out) return -1;
    return run_rows(&P, NULL, NULL, (int64_t)T * num_heads, out, nthreads);
}

int oracle_prefill_attention_rows_ring(const float *q, int64_t q_row_stride,
                                       const float *k_cache, const float *v_cache,
                                       int64_t kv_head_stride, int ring_slots,
                                       const int32_t *row_t, const int32_t *row_h, int64_t nrows,
                                       double *out, int T, int start_pos, int num_heads,
                                       int num_kv_heads, int head_dim, int window, int nthreads);

/*
 * Selected rows (row_t[i], row_h[i]) of the same chunk: out is [nrows][head_dim].
 */
int oracle_prefill_attention_rows(const float *q, int64_t q_row_stride,
                                  const float *k_cache, const float *v_cache, int64_t kv_head_stride,
                                  const int32_t *row_t, const int32_t *row_h, int64_t nrows,
                                  double *out, int T, int start_pos, int num_heads, int num_kv_heads,
                                  int head_dim, int window, int nthreads)
{
    return oracle_prefill_attention_rows_ring(q, q_row_stride, k_cache, v_cache, kv_head_stride, 0,
                                              row_t, row_h, nrows, out, T, start_pos, num_heads,
                                              num_kv_heads, head_dim, window, nthreads);
}

/* Selected rows over a ring cache (ring_slots 0: the linear layout). */
int oracle_prefill_attention_rows_ring(const float *q, int64_t q_row_stride,
                                       const float *k_cache, const float *v_cache,
                                       int64_t kv_head_stride, int ring_slots,
                                       const int32_t *row_t, const int32_t *row_h, int64_t nrows,
                                       double *out, int T, int start_pos, int num_heads,
                                       int num_kv_heads, int head_dim, int window, int nthreads)
{
    struct problem P = {q, k_cache, v_cache, q_row_stride, kv_head_stride,
                        T, start_pos, num_heads, num_kv_heads, head_dim, window, ring_slots, NULL, 0, 0};
    if (check_problem(&P) || !out || !row_t || !row_h || nrows < 1) return -1;
    for (int64_t i = 0; i < nrows; ++i)
        if (row_t[i] < 0 || row_t[i] >= T || row_h[i] < 0 || row_h[i] >= num_heads) return -1;
    return run_rows(&P, row_t, row_h, nrows, out, nthreads);
}

/*
 * The softmax probabilities of one row (t, h), for keys lo..=pos in order:
 * writes them to probs (room for start_pos + T doubles), stores lo in *first
 * and returns their count, or -1 for invalid arguments.
 */
int oracle_row_probabilities(const float *q, int64_t q_row_stride,
                             const float *k_cache, const float *v_cache, int64_t kv_head_stride,
                             int t, int h, double *probs, int *first,
                             int T, int start_pos, int num_heads, int num_kv_heads,
                             int head_dim, int window)
{
    struct problem P = {q, k_cache, v_cache, q_row_stride, kv_head_stride,
                        T, start_pos, num_heads, num_kv_heads, head_dim, window, 0, NULL, 0, 0};
    if (check_problem(&P) || !probs || !first) return -1;
    if (t < 0 || t >= T || h < 0 || h >= num_heads) return -1;
    double *out_row = (double *)malloc(sizeof(double) * (size_t)head_dim);
    if (!out_row) return -1;
    attend_row(&P, t, h, probs, out_row);
    free(out_row);
    const int pos = start_pos + t;
    *first = first_key(pos, window);
    return pos - *first + 1;
}

/*
 * KV cache write, the step before the attention: the gnosis page ("What
 * already shipped", Phase A) stores every token's K and V in the cache before
 * the attention runs; the TensorSharp page (section 4, requirement R4) puts
 * position pos at row pos of a global layer's cache and at slot
 * pos % (ring size) of a sliding-window layer's ring.  Tokens i = 0..T-1 are
 * written in order: K of token i, kv head kh, element d is read from
 * k_src[i*src_row_stride + kh*head_dim + d] (V alike) and stored at
 * k_cache[kh*kv_head_stride + row*head_dim + d] with row = start_pos + i, or
 * (start_pos + i) % ring_slots when ring_slots > 0.  Returns 0, or -1 for
 * invalid arguments.
 */
int oracle_kv_write(const float *k_src, const float *v_src, int64_t src_row_stride,
                    float *k_cache, float *v_cache, int64_t kv_head_stride, int ring_slots,
                    int T, int start_pos, int num_kv_heads, int head_dim)
{
    if (!k_src || !v_src || !k_cache || !v_cache) return -1;
    if (T < 1 || start_pos < 0 || num_kv_heads < 1 || head_dim < 1 || ring_slots < 0) return -1;
    if (src_row_stride < (int64_t)num_kv_heads * head_dim) return -1;
    const int64_t rows = ring_slots > 0 ? ring_slots : (int64_t)start_pos + T;
    if (kv_head_stride < rows * head_dim) return -1;
    for (int i = 0; i < T; ++i) {
        const int64_t pos = (int64_t)start_pos + i;
        const int64_t row = ring_slots > 0 ? pos % ring_slots : pos;
        for (int kh = 0; kh < num_kv_heads; ++kh) {
            const int64_t src = (int64_t)i * src_row_stride + (int64_t)kh * head_dim;
            const int64_t dst = (int64_t)kh * kv_head_stride + row * head_dim;
            for (int d = 0; d < head_dim; ++d) {
                k_cache[dst + d] = k_src[src + d];
                v_cache[dst + d] = v_src[src + d];
            }
        }
    }
    return 0;
}

/*
 * Selected rows (row_t[i], row_h[i]) over a paged cache (pools k_pool and
 * v_pool of num_pages pages of page_size positions): out is [nrows][head_dim].
 * Returns 0, -1 for invalid arguments (a key some row reads off the pool
 * included), -2 when memory runs out.
 */
int oracle_prefill_attention_rows_paged(const float *q, int64_t q_row_stride,
                                        const float *k_pool, const float *v_pool, int page_size,
                                        int num_pages, const int32_t *page_table,
                                        const int32_t *row_t, const int32_t *row_h, int64_t nrows,
                                        double *out, int T, int start_pos, int num_heads,
                                        int num_kv_heads, int head_dim, int window, int nthreads)
{
    struct problem P = {q, k_pool, v_pool, q_row_stride, 0,
                        T, start_pos, num_heads, num_kv_heads, head_dim, window, 0,
                        page_table, page_size, num_pages};
    if (!page_table || check_problem(&P) || !out || !row_t || !row_h || nrows < 1) return -1;
    for (int64_t i = 0; i < nrows; ++i)
        if (row_t[i] < 0 || row_t[i] >= T || row_h[i] < 0 || row_h[i] >= num_heads) return -1;
    return run_rows(&P, row_t, row_h, nrows, out, nthreads);
}

/* Whole chunk over a paged cache: out is [T][num_heads][head_dim]. */
int oracle_prefill_attention_paged(const float *q, int64_t q_row_stride,
                                   const float *k_pool, const float *v_pool, int page_size,
                                   int num_pages, const int32_t *page_table, double *out, int T,
                                   int start_pos, int num_heads, int num_kv_heads, int head_dim,
                                   int window, int nthreads)
{
    struct problem P = {q, k_pool, v_pool, q_row_stride, 0,
                        T, start_pos, num_heads, num_kv_heads, head_dim, window, 0,
                        page_table, page_size, num_pages};
    if (!page_table || check_problem(&P) || !out) return -1;
    return run_rows(&P, NULL, NULL, (int64_t)T * num_heads, out, nthreads);
}
