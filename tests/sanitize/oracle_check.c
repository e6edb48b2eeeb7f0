/*
 * The fp64 oracle (oracle/star_oracle.c) built with AddressSanitizer and
 * UndefinedBehaviorSanitizer and run over seeded random small shapes
 * (tests/test_sanitized_host.py).  Test infrastructure checking test
 * infrastructure: every buffer is allocated at the exact size the oracle's
 * documented layout needs, so a read or write past a row, a head or a
 * partition is reported by the sanitizer.  Covers every input type (fp32,
 * bf16 bit patterns, fp64), Phase 1 over all rows and over sampled rows,
 * partitions with and without a causal offset, empty partitions, merges with
 * empty partials, one to four threads, and the argument refusals.  Exit
 * status 0 and a final "ok" line mean no check failed and no sanitizer fired.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int star_oracle_phase1(const void *q, const void *k, const void *v, int dtype, int64_t L, int64_t block,
                       int64_t anchor, int hq, int hkv, int d, double scale, const int64_t *rows, int64_t n_rows,
                       int q_sampled, double *o, double *lse, int threads);
int star_oracle_partial(const void *q, int64_t rows, const void *k, const void *v, int dtype, int64_t kv_tokens,
                        int64_t lo, int64_t hi, int64_t causal_offset, int hq, int hkv, int d, double scale,
                        double *a, double *m, double *l, int threads);
void star_oracle_merge(const double *a, const double *m, const double *l, int n_parts, int64_t n_rows, int d,
                       double *o, double *lse);

#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #c);        \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

static uint64_t state = 20241126u;
static uint64_t next_u64(void) { /* splitmix64 */
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static int64_t uni(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1)); }
static double unit(void) { return (double)(next_u64() >> 11) / 9007199254740992.0 * 2.0 - 1.0; }

/* n elements of the given type (0 fp32, 1 bf16 bits, 2 fp64), uniform in [-2, 2). */
static void *random_elems(int dtype, int64_t n) {
    size_t sz = dtype == 0 ? 4 : (dtype == 1 ? 2 : 8);
    void *p = malloc((size_t)(n > 0 ? n : 1) * sz);
    for (int64_t i = 0; i < n; ++i) {
        double x = 2.0 * unit();
        if (dtype == 0) ((float *)p)[i] = (float)x;
        else if (dtype == 2) ((double *)p)[i] = x;
        else {
            float f = (float)x;
            uint32_t w;
            memcpy(&w, &f, 4);
            ((uint16_t *)p)[i] = (uint16_t)(w >> 16);
        }
    }
    return p;
}

static int all_finite(const double *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

int main(void) {
    int n1 = 0, n2 = 0, n3 = 0;
    for (int it = 0; it < 60; ++it) {
        int dtype = (int)uni(0, 2), hkv = (int)uni(1, 3), G = (int)uni(1, 4), d = (int)uni(1, 40);
        int hq = hkv * G;
        int64_t L = uni(1, 150), block = uni(1, L + 20), anchor = uni(0, block);
        int threads = (int)uni(1, 4);
        double scale = 1.0 / sqrt((double)d);
        void *k = random_elems(dtype, (int64_t)hkv * L * d), *v = random_elems(dtype, (int64_t)hkv * L * d);
        /* every row, full q */
        void *q = random_elems(dtype, (int64_t)hq * L * d);
        int64_t *rows = malloc(sizeof(int64_t) * (size_t)L);
        for (int64_t r = 0; r < L; ++r) rows[r] = r;
        double *o = malloc(sizeof(double) * (size_t)(hq * L * d)), *lse = malloc(sizeof(double) * (size_t)(hq * L));
        CHECK(star_oracle_phase1(q, k, v, dtype, L, block, anchor, hq, hkv, d, scale, rows, L, 0, o, lse, threads) == 0);
        CHECK(all_finite(o, (int64_t)hq * L * d) && all_finite(lse, (int64_t)hq * L));
        free(o);
        free(lse);
        /* sampled rows, sampled q */
        int64_t ns = uni(1, L);
        for (int64_t r = 0; r < ns; ++r) rows[r] = uni(0, L - 1);
        void *qs = random_elems(dtype, (int64_t)hq * ns * d);
        o = malloc(sizeof(double) * (size_t)(hq * ns * d));
        lse = malloc(sizeof(double) * (size_t)(hq * ns));
        CHECK(star_oracle_phase1(qs, k, v, dtype, L, block, anchor, hq, hkv, d, scale, rows, ns, 1, o, lse, threads) == 0);
        CHECK(all_finite(lse, (int64_t)hq * ns));
        /* refusals: anchor > block, a row past L, hq not a multiple of hkv */
        CHECK(star_oracle_phase1(qs, k, v, dtype, L, block, block + 1, hq, hkv, d, scale, rows, ns, 1, o, lse, 1) == -1);
        rows[0] = L;
        CHECK(star_oracle_phase1(qs, k, v, dtype, L, block, anchor, hq, hkv, d, scale, rows, ns, 1, o, lse, 1) == -1);
        if (hkv > 1) CHECK(star_oracle_phase1(qs, k, v, dtype, L, block, anchor, hq + 1, hkv, d, scale, rows, ns, 1, o,
                                              lse, 1) == -1);
        free(o);
        free(lse);
        free(qs);
        free(rows);
        free(q);
        n1 += 2;

        /* partitions of the context: plain, causal, empty; then their merge */
        int nr = (int)uni(1, 9), P = (int)uni(1, 5);
        void *qr = random_elems(dtype, (int64_t)hq * nr * d);
        double *a = malloc(sizeof(double) * (size_t)(P * hq * nr * d));
        double *m = malloc(sizeof(double) * (size_t)(P * hq * nr)), *l = malloc(sizeof(double) * (size_t)(P * hq * nr));
        for (int pi = 0; pi < P; ++pi) {
            int64_t lo = uni(0, L), hi = uni(lo, L);
            int64_t causal = uni(0, 2) == 0 ? -1 : uni(0, 5);
            size_t off = (size_t)pi * hq * nr;
            CHECK(star_oracle_partial(qr, nr, k, v, dtype, L, lo, hi, causal, hq, hkv, d, scale, a + off * d, m + off,
                                      l + off, threads) == 0);
            for (size_t i = 0; i < (size_t)(hq * nr); ++i) {
                if (hi == lo) CHECK(m[off + i] == -INFINITY && l[off + i] == 0.0);
                else CHECK(isfinite(l[off + i]));
            }
            ++n2;
        }
        CHECK(star_oracle_partial(qr, nr, k, v, dtype, L, 5, 4, -1, hq, hkv, d, scale, a, m, l, 1) == -1);
        CHECK(star_oracle_partial(qr, nr, k, v, dtype, L, 0, L + 1, -1, hq, hkv, d, scale, a, m, l, 1) == -1);
        double *om = malloc(sizeof(double) * (size_t)(hq * nr * d)), *lm = malloc(sizeof(double) * (size_t)(hq * nr));
        star_oracle_merge(a, m, l, P, (int64_t)hq * nr, d, om, lm);
        CHECK(all_finite(om, (int64_t)hq * nr * d));
        ++n3;
        free(om);
        free(lm);
        free(a);
        free(m);
        free(l);
        free(qr);
        free(k);
        free(v);
    }
    printf("ok: %d phase-1 calls, %d partials, %d merges\n", n1, n2, n3);
    return 0;
}
