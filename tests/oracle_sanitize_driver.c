/*
 * oracle_sanitize_driver.c -- calls every function of the fp64 oracle on
 * exactly sized heap buffers, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py).  Shapes cover
 * row and channel ranges, W larger than a sequence, one-token sequences,
 * decoding, the prefill hand-off and the rotary embedding, plus argument
 * errors that must return before touching memory.  Exits 0 when every call
 * returns the expected code; the sanitizers abort on any invalid access.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_headwise_fwd(int64_t, int64_t, int64_t, int32_t, int32_t, const double *, const double *,
                        const int32_t *, int32_t, int32_t, int64_t, int64_t, double *);
int oracle_headwise_bwd(int64_t, int64_t, int64_t, int32_t, int32_t, const double *, const double *,
                        const double *, const int32_t *, int32_t, int32_t, int64_t, int64_t, double *, double *);
int oracle_lowrank_fwd(int64_t, int64_t, int64_t, int32_t, int32_t, const double *, const double *,
                       const double *, const int32_t *, int32_t, int32_t, int64_t, int64_t, double *);
int oracle_lowrank_bwd(int64_t, int64_t, int64_t, int32_t, int32_t, const double *, const double *,
                       const double *, const double *, const int32_t *, int32_t, int32_t, int64_t, int64_t,
                       double *, double *, int64_t, int64_t, double *);
int oracle_static_fwd(int64_t, int64_t, int64_t, int32_t, const double *, const double *, const int32_t *,
                      int32_t, int32_t, int64_t, int64_t, double *);
int oracle_static_bwd(int64_t, int64_t, int64_t, int32_t, const double *, const double *, const double *,
                      const int32_t *, int32_t, int32_t, int64_t, int64_t, double *, double *);
int oracle_headwise_decode(int64_t, int64_t, int32_t, int32_t, const double *, const double *, double *,
                           int32_t, double *);
int oracle_lowrank_decode(int64_t, int64_t, int32_t, int32_t, const double *, const double *,
                          const double *, double *, int32_t, double *);
int oracle_state_from_prefill(int64_t, int64_t, int64_t, int32_t, const double *, const int32_t *, int32_t,
                              double *);
int oracle_rope_table(int64_t, int32_t, double, double *);
int oracle_rope(int64_t, int64_t, int64_t, int64_t, int32_t, double, const int32_t *, int32_t, int32_t, int64_t,
                int64_t, const double *, double *);
int oracle_rope_at(int64_t, int64_t, int64_t, int32_t, double, const int32_t *, const double *, double *);

static int failures = 0;

static void expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: returned %d, expected %d\n", what, got, want);
        ++failures;
    }
}

/* a buffer of exactly n doubles with a deterministic fill (NULL-safe for n = 0) */
static double *buf(int64_t n, unsigned seed)
{
    double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof *p);
    for (int64_t i = 0; i < n; ++i) p[i] = (double)((seed * 2654435761u + (unsigned)i * 40503u) % 2001) / 1000.0 - 1.0;
    return p;
}

static void run_shape(int64_t B, int64_t T, int64_t D, int32_t W, int32_t H, int32_t R, const int32_t *cu,
                      int32_t ns)
{
    const int64_t N = B * T, G = D / H;
    double *x = buf(N * D, 1), *w = buf(N * G * W, 2), *g = buf(N * D, 3), *z = buf(N * R, 4);
    double *U = buf((int64_t)R * D * W, 5), *c = buf(D * W, 6);
    const int64_t lo = N > 2 ? 1 : 0, hi = N > 2 ? N - 1 : N;  /* a row range inside the batch */
    const int64_t rows = hi - lo;
    double *y = buf(rows * D, 0), *dx = buf(rows * D, 0), *dw = buf(rows * G * W, 0), *dz = buf(rows * R, 0);
    const int64_t dlo = D > 1 ? 1 : 0, dhi = D;
    double *dU = buf((int64_t)R * (dhi - dlo) * W, 0), *dc = buf(D * W, 0);
    for (int32_t res = 0; res < 2; ++res) {
        expect(oracle_headwise_fwd(B, T, D, W, H, x, w, cu, ns, res, lo, hi, y), 0, "headwise_fwd");
        expect(oracle_headwise_bwd(B, T, D, W, H, x, w, g, cu, ns, res, lo, hi, dx, dw), 0, "headwise_bwd");
        expect(oracle_lowrank_fwd(B, T, D, W, R, x, z, U, cu, ns, res, lo, hi, y), 0, "lowrank_fwd");
        expect(oracle_lowrank_bwd(B, T, D, W, R, x, z, U, g, cu, ns, res, lo, hi, dx, dz, dlo, dhi, dU), 0,
               "lowrank_bwd");
        expect(oracle_static_fwd(B, T, D, W, x, c, cu, ns, res, lo, hi, y), 0, "static_fwd");
        expect(oracle_static_bwd(B, T, D, W, x, c, g, cu, ns, res, lo, hi, dx, dc), 0, "static_bwd");
    }
    /* the rotary embedding of the row range: one head of 2 channels when D allows */
    if (D % 2 == 0) {
        expect(oracle_rope(B, T, D, D, 2, 10000.0, cu, ns, 0, lo, hi, g + lo * D, y), 0, "rope");
        expect(oracle_rope(B, T, D, D, 2, 10000.0, cu, ns, 1, lo, hi, g + lo * D, y), 0, "rope inverse");
    }
    /* the prefill state: one slot row of W-1 per sequence */
    const int64_t S = cu ? ns : B;
    double *st = buf(S * (W - 1) * D, 0);
    expect(oracle_state_from_prefill(B, T, D, W, x, cu, ns, st), 0, "state_from_prefill");
    free(x); free(w); free(g); free(z); free(U); free(c); free(y); free(dx); free(dw); free(dz); free(dU);
    free(dc); free(st);
}

static void run_decode(int64_t B, int64_t D, int32_t W, int32_t H, int32_t R)
{
    double *x = buf(B * D, 7), *w = buf(B * (D / H) * W, 8), *z = buf(B * R, 9), *U = buf((int64_t)R * D * W, 10);
    double *st = buf(B * (W - 1) * D, 11), *y = buf(B * D, 0);
    int32_t *pos = (int32_t *)malloc((size_t)(B > 0 ? B : 1) * sizeof *pos);
    for (int64_t b = 0; b < B; ++b) pos[b] = (int32_t)(3 * b);
    expect(oracle_headwise_decode(B, D, W, H, x, w, st, 1, y), 0, "headwise_decode");
    expect(oracle_lowrank_decode(B, D, W, R, x, z, U, st, 0, y), 0, "lowrank_decode");
    /* half the channels rotated, in heads of 4 (2 where half is not a multiple of 4) */
    if (D % 4 == 0) expect(oracle_rope_at(B, D, D / 2, (D / 2) % 4 ? 2 : 4, 500.0, pos, x, y), 0, "rope_at");
    free(x); free(w); free(z); free(U); free(st); free(y); free(pos);
}

int main(void)
{
    /* rows, each one sequence; W above T */
    run_shape(2, 3, 4, 5, 2, 3, NULL, 0);
    run_shape(1, 9, 6, 1, 6, 1, NULL, 0);
    /* packed sequences of 1, 2 and 7 tokens crossing the row boundary */
    const int32_t cu[4] = {0, 1, 3, 10};
    run_shape(2, 5, 8, 4, 4, 2, cu, 3);
    run_decode(3, 8, 4, 2, 3);
    run_decode(1, 4, 1, 1, 1);
    double *tab = buf(7 * 3 * 2, 0);
    expect(oracle_rope_table(7, 6, 10000.0, tab), 0, "rope_table");
    free(tab);
    /* argument errors return before any access */
    double *x = buf(16, 1), *y = buf(16, 0);
    const int32_t bad_cu[3] = {0, 3, 2};
    expect(oracle_headwise_fwd(1, 4, 4, 2, 3, x, x, NULL, 0, 0, 0, 4, y), -2, "D % H != 0");
    expect(oracle_headwise_fwd(1, 4, 4, 2, 2, x, x, bad_cu, 2, 0, 0, 4, y), -2, "decreasing offsets");
    expect(oracle_headwise_fwd(1, 4, 4, 2, 2, x, x, NULL, 0, 0, 2, 5, y), -2, "rows past the batch");
    expect(oracle_rope(1, 4, 4, 3, 2, 10000.0, NULL, 0, 0, 0, 4, x, y), -2, "rot not a multiple of head_dim");
    const int32_t neg[1] = {-1};
    expect(oracle_rope_at(1, 4, 4, 2, 10000.0, neg, x, y), -2, "negative position");
    free(x); free(y);
    if (failures) return 1;
    printf("oracle calls ok\n");
    return 0;
}
