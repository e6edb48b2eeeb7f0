/*
 * Star Attention fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may load this file's library.  The GPU product path never calls it and
 * shares no code with it.
 *
 * Sources (pages, cited by title and section):
 *   [SUM]    "Star Attention: Efficient LLM Inference over Long Sequences",
 *            paper-graph-ui long-form summary of arXiv 2411.17116, section
 *            3.4 "Detailed, Sentence-Based Technical Breakdown".
 *   [README] "NVIDIA/Star-Attention" (shadowgraph.io mirror of the project
 *            README), section "Two Phases of Star Attention".
 *
 * Everything is computed in double precision from the exact input values
 * (bf16 or fp32 bit patterns widened to double).  Nothing is tiled, fused
 * or reordered: each output row is the textbook two-pass softmax over the
 * set of keys the method lets that row see.
 *
 * Conventions (readings of points the pages leave open):
 *   - layouts are head-major: q [Hq, rows, d], k/v [Hkv, tokens, d];
 *   - q head h reads kv head h / (Hq/Hkv)  (contiguous GQA groups);
 *   - scores are x_j = <q, k_j> / sqrt(d) unless the caller passes another
 *     scale; logs are natural logs;
 *   - the anchor is the first `anchor` context tokens, 0 <= anchor <= block.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* Widen one stored element to double.  bf16 is the top half of an IEEE
 * binary32, so the widening is exact.  F64 inputs carry values that are
 * not binary32 numbers (a dequantised cache: scale times a decoded code). */
static double load_elem(const void *base, int dtype, int64_t idx) {
    if (dtype == ORACLE_BF16) {
        uint16_t h = ((const uint16_t *)base)[idx];
        uint32_t w = ((uint32_t)h) << 16;
        float f;
        memcpy(&f, &w, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_F64) return ((const double *)base)[idx];
    return (double)((const float *)base)[idx];
}

/* ------------------------------------------------------------------ */
/* One row of attention over an explicit list of key indices.          */
/* x_j = scale * <q, k_j>;  M = max x_j;  l = sum exp(x_j - M);        */
/* out = sum exp(x_j - M) v_j / l;  returns (M, l).                    */
/* [SUM] 3.4, "The Attention Decomposition": the causal attention      */
/* formula with the 1/sqrt(d) scale; the two-pass max-subtracted form  */
/* is the same quantity written so that exp() cannot overflow.         */
/* ------------------------------------------------------------------ */
typedef struct {
    const void *q;      /* start of this row's query vector (element offset applied via q_off) */
    int64_t q_off;
    const void *k, *v;  /* kv base pointers                          */
    int64_t kv_off;     /* element offset of this kv head's token 0   */
    int dtype, d;
    double scale;
} row_ctx;

static void attend_row(const row_ctx *c, const int64_t *keys, int64_t n_keys,
                       double *xbuf, double *out, double *m_out, double *l_out) {
    int d = c->d;
    if (n_keys == 0) {                      /* empty partition: weight 0 */
        for (int e = 0; e < d; ++e) out[e] = 0.0;
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    double M = -INFINITY;
    for (int64_t t = 0; t < n_keys; ++t) {
        int64_t j = keys[t];
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += load_elem(c->q, c->dtype, c->q_off + e) *
                   load_elem(c->k, c->dtype, c->kv_off + j * d + e);
        xbuf[t] = c->scale * dot;
        if (xbuf[t] > M) M = xbuf[t];
    }
    double l = 0.0;
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    for (int64_t t = 0; t < n_keys; ++t) {
        double w = exp(xbuf[t] - M);
        l += w;
        int64_t j = keys[t];
        for (int e = 0; e < d; ++e)
            out[e] += w * load_elem(c->v, c->dtype, c->kv_off + j * d + e);
    }
    for (int e = 0; e < d; ++e) out[e] /= l;
    *m_out = M;
    *l_out = l;
}

/* ------------------------------------------------------------------ */
/* Phase 1: anchored blockwise-local context encoding.                 */
/*                                                                     */
/* [SUM] 3.4 Phase 1 Steps 1-5 and [README] "Phase 1 - Context         */
/* Encoding": the context is cut into contiguous blocks of `block`     */
/* tokens (the last one may be shorter); every block after the first   */
/* is prefixed with the anchor (the first block) and attended causally */
/* as a standalone sequence; block 1 is attended causally on its own.  */
/* Causal attention over [anchor ; own block] means a token at context */
/* position p in block i >= 1 sees every anchor token and the tokens   */
/* start_i .. p of its own block; a token of block 0 sees 0 .. p.      */
/* With anchor < block the anchor is the first `anchor` tokens.        */
/* ------------------------------------------------------------------ */
static int64_t phase1_visible(int64_t p, int64_t block, int64_t anchor, int64_t *keys) {
    int64_t i = p / block, start = i * block, n = 0;
    if (i >= 1)
        for (int64_t j = 0; j < anchor; ++j) keys[n++] = j;
    for (int64_t j = start; j <= p; ++j) keys[n++] = j;
    return n;
}

typedef struct {
    const void *q, *k, *v;
    int dtype;
    int64_t L, block, anchor, n_rows, q_rows;
    const int64_t *rows;   /* context positions to evaluate            */
    int hq, hkv, d;
    double scale;
    double *o, *lse;       /* [hq, n_rows, d], [hq, n_rows]             */
    int64_t next;          /* shared work counter                       */
    int q_rows_are_sampled;/* q holds only the sampled rows, in order  */
} p1_job;

static void *p1_worker(void *arg) {
    p1_job *J = (p1_job *)arg;
    int G = J->hq / J->hkv;
    int64_t max_keys = J->anchor + J->block;
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)max_keys);
    double *xbuf = (double *)malloc(sizeof(double) * (size_t)max_keys);
    for (;;) {
        int64_t w = __sync_fetch_and_add(&J->next, 1);
        if (w >= (int64_t)J->hq * J->n_rows) break;
        int h = (int)(w / J->n_rows);
        int64_t r = w % J->n_rows;
        int64_t p = J->rows[r];
        int64_t n = phase1_visible(p, J->block, J->anchor, keys);
        row_ctx c;
        c.q = J->q;
        c.q_off = ((int64_t)h * J->q_rows + (J->q_rows_are_sampled ? r : p)) * J->d;
        c.k = J->k; c.v = J->v;
        c.kv_off = (int64_t)(h / G) * J->L * J->d;
        c.dtype = J->dtype; c.d = J->d; c.scale = J->scale;
        double M, l;
        attend_row(&c, keys, n, xbuf, J->o + ((int64_t)h * J->n_rows + r) * J->d, &M, &l);
        J->lse[(int64_t)h * J->n_rows + r] = M + log(l);
    }
    free(keys);
    free(xbuf);
    return NULL;
}

static void run_threads(void *(*fn)(void *), void *job, int threads) {
    if (threads < 1) threads = 1;
    if (threads == 1) { fn(job); return; }
    pthread_t *t = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)threads);
    for (int i = 0; i < threads; ++i) pthread_create(&t[i], NULL, fn, job);
    for (int i = 0; i < threads; ++i) pthread_join(t[i], NULL);
    free(t);
}

/* Phase-1 outputs for the context positions rows[0..n_rows) of every q
 * head.  If q_sampled != 0, q holds only those rows ([hq, n_rows, d]);
 * otherwise q is the full [hq, L, d] tensor.  Returns 0, or -1 on bad
 * arguments. */
int star_oracle_phase1(const void *q, const void *k, const void *v, int dtype,
                       int64_t L, int64_t block, int64_t anchor,
                       int hq, int hkv, int d, double scale,
                       const int64_t *rows, int64_t n_rows, int q_sampled,
                       double *o, double *lse, int threads) {
    if (L < 1 || block < 1 || anchor < 0 || anchor > block || hkv < 1 || hq % hkv) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= L) return -1;
    p1_job J;
    J.q = q; J.k = k; J.v = v; J.dtype = dtype;
    J.L = L; J.block = block; J.anchor = anchor;
    J.rows = rows; J.n_rows = n_rows;
    J.q_rows = q_sampled ? n_rows : L;
    J.q_rows_are_sampled = q_sampled;
    J.hq = hq; J.hkv = hkv; J.d = d; J.scale = scale;
    J.o = o; J.lse = lse; J.next = 0;
    run_threads(p1_worker, &J, threads);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Phase 2 local attention of one partition (one "host").              */
/*                                                                     */
/* [SUM] 3.4 Phase 2 Step 3 and [README] "Phase 2": A_h is the softmax */
/* of the scaled scores over the partition's keys, normalised over     */
/* those keys only, applied to V_h; s_h is the sum of the exponentials */
/* over the partition.  It is returned as (m, l) with s_h = e^m * l so */
/* that no exponential of a raw score is ever formed.                  */
/*                                                                     */
/* The partition is tokens [lo, hi) of k/v (per-kv-head token stride   */
/* kv_tokens).  causal_offset < 0: every row sees every key; otherwise */
/* row i sees partition token t = j - lo only if t <= causal_offset+i  */
/* (the query host's own cache, where query and generated tokens are   */
/* causal among themselves).                                           */
/* ------------------------------------------------------------------ */
typedef struct {
    const void *q, *k, *v;
    int dtype;
    int64_t rows, kv_tokens, lo, hi, causal_offset;
    int hq, hkv, d;
    double scale;
    double *a, *m, *l;
    int64_t next;
} p2_job;

static void *p2_worker(void *arg) {
    p2_job *J = (p2_job *)arg;
    int G = J->hq / J->hkv;
    int64_t span = J->hi - J->lo;
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(span > 0 ? span : 1));
    double *xbuf = (double *)malloc(sizeof(double) * (size_t)(span > 0 ? span : 1));
    for (;;) {
        int64_t w = __sync_fetch_and_add(&J->next, 1);
        if (w >= (int64_t)J->hq * J->rows) break;
        int h = (int)(w / J->rows);
        int64_t i = w % J->rows;
        int64_t n = 0;
        for (int64_t j = J->lo; j < J->hi; ++j)
            if (J->causal_offset < 0 || (j - J->lo) <= J->causal_offset + i) keys[n++] = j;
        row_ctx c;
        c.q = J->q;
        c.q_off = ((int64_t)h * J->rows + i) * J->d;
        c.k = J->k; c.v = J->v;
        c.kv_off = (int64_t)(h / G) * J->kv_tokens * J->d;
        c.dtype = J->dtype; c.d = J->d; c.scale = J->scale;
        int64_t idx = (int64_t)h * J->rows + i;
        attend_row(&c, keys, n, xbuf, J->a + idx * J->d, &J->m[idx], &J->l[idx]);
    }
    free(keys);
    free(xbuf);
    return NULL;
}

int star_oracle_partial(const void *q, int64_t rows, const void *k, const void *v, int dtype,
                        int64_t kv_tokens, int64_t lo, int64_t hi, int64_t causal_offset,
                        int hq, int hkv, int d, double scale,
                        double *a, double *m, double *l, int threads) {
    if (hkv < 1 || hq % hkv || lo < 0 || hi < lo || hi > kv_tokens || rows < 0) return -1;
    p2_job J;
    J.q = q; J.k = k; J.v = v; J.dtype = dtype;
    J.rows = rows; J.kv_tokens = kv_tokens; J.lo = lo; J.hi = hi;
    J.causal_offset = causal_offset;
    J.hq = hq; J.hkv = hkv; J.d = d; J.scale = scale;
    J.a = a; J.m = m; J.l = l; J.next = 0;
    run_threads(p2_worker, &J, threads);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Global aggregation of P partitions.                                 */
/*                                                                     */
/* [README] "Phase 2": s_global = sum_h s_h and                        */
/* A_global = sum_h (s_h / s_global) A_h.  [SUM] 3.4 Phase 2 Step 5    */
/* asks for the same sum evaluated in log space; with s_h = e^{m_h}    */
/* l_h and M = max_h m_h, the common factor e^M cancels:               */
/*   w_h = l_h e^{m_h - M},  O = sum w_h A_h / sum w_h,                */
/*   LSE = log s_global = M + log sum w_h.                             */
/* Partitions with m = -inf weigh 0; if every partition is empty the   */
/* output is 0 and LSE = -inf.                                         */
/* ------------------------------------------------------------------ */
void star_oracle_merge(const double *a, const double *m, const double *l,
                       int n_parts, int64_t n_rows, int d,
                       double *o, double *lse) {
    for (int64_t r = 0; r < n_rows; ++r) {
        double M = -INFINITY;
        for (int p = 0; p < n_parts; ++p) {
            double mp = m[(int64_t)p * n_rows + r];
            if (mp > M) M = mp;
        }
        double *out = o + r * d;
        for (int e = 0; e < d; ++e) out[e] = 0.0;
        if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
        double W = 0.0;
        for (int p = 0; p < n_parts; ++p) {
            int64_t idx = (int64_t)p * n_rows + r;
            if (m[idx] == -INFINITY) continue;
            double w = l[idx] * exp(m[idx] - M);
            W += w;
            for (int e = 0; e < d; ++e) out[e] += w * a[idx * d + e];
        }
        for (int e = 0; e < d; ++e) out[e] /= W;
        lse[r] = M + log(W);
    }
}
