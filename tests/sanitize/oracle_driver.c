/* Drives every entry point of the C oracle on small inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: each array is allocated at
 * exactly the size the call documents, so any read or write past it, any use
 * of freed memory and any undefined arithmetic stops the run.  Also checks the
 * argument errors.  Exit status 0 when every call returned as documented and
 * every output is finite. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int kda_oracle_forward(const double *q, const double *k, const double *v, const double *alpha,
                       const double *beta, const double *s0, double *o, double *sT, long n_units,
                       long T, int dk, int dv, double scale, int n_threads);
int kda_oracle_step(const double *q, const double *k, const double *v, const double *alpha,
                    const double *beta, double *state, double *o, long n_units, int dk, int dv,
                    double scale, int n_threads);
int kda_oracle_backward(const double *q, const double *k, const double *v, const double *alpha,
                        const double *beta, const double *s0, const double *dout,
                        const double *dsT, double *gq, double *gk, double *gv, double *ga,
                        double *gb, double *gs0, long n_units, long T, int dk, int dv,
                        double scale, int n_threads);
int gdn2_oracle_forward(const double *q, const double *k, const double *v, const double *alpha,
                        const double *erase, const double *write, const double *s0, double *o,
                        double *sT, long n_units, long T, int dk, int dv, double scale,
                        int n_threads);

static unsigned long long rng = 88172645463325252ULL;
static double uni(void) { /* xorshift64, in (0, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return ((rng >> 11) + 0.5) / 9007199254740992.0;
}
static double *arr(long n, double lo, double hi) {
    double *p = malloc(sizeof(double) * (n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
    return p;
}
static int finite_all(const double *p, long n) {
    for (long i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

static void run(long U, long T, int dk, int dv, int threads) {
    const long nk = U * T * dk, nv = U * T * dv, nt = U * T, ns = U * (long)dk * dv;
    double *q = arr(nk, -1, 1), *k = arr(nk, -1, 1), *v = arr(nv, -1, 1);
    double *a = arr(nk, 0.05, 1), *b = arr(nt, 0, 1), *e = arr(nk, 0, 1), *w = arr(nk, 0, 1);
    double *s0 = arr(ns, -0.5, 0.5), *dout = arr(nv, -1, 1), *dsT = arr(ns, -1, 1);
    double *o = arr(nv, 0, 0), *sT = arr(ns, 0, 0);
    double *gq = arr(nk, 0, 0), *gk = arr(nk, 0, 0), *gv = arr(nv, 0, 0), *ga = arr(nk, 0, 0);
    double *gb = arr(nt, 0, 0), *gs0 = arr(ns, 0, 0);

    CHECK(kda_oracle_forward(q, k, v, a, b, s0, o, sT, U, T, dk, dv, 0.3, threads) == 0);
    CHECK(finite_all(o, nv) && finite_all(sT, ns));
    CHECK(kda_oracle_forward(q, k, v, a, b, NULL, NULL, sT, U, T, dk, dv, 0.3, threads) == 0);
    CHECK(kda_oracle_backward(q, k, v, a, b, s0, dout, dsT, gq, gk, gv, ga, gb, gs0, U, T, dk,
                              dv, 0.3, threads) == 0);
    CHECK(finite_all(gq, nk) && finite_all(gk, nk) && finite_all(gv, nv) && finite_all(ga, nk) &&
          finite_all(gb, nt) && finite_all(gs0, ns));
    CHECK(kda_oracle_backward(q, k, v, a, b, NULL, dout, NULL, gq, gk, gv, ga, gb, gs0, U, T, dk,
                              dv, 0.3, threads) == 0);
    CHECK(gdn2_oracle_forward(q, k, v, a, e, w, s0, o, sT, U, T, dk, dv, 0.3, threads) == 0);
    CHECK(gdn2_oracle_forward(q, k, v, a, e, w, NULL, o, NULL, U, T, dk, dv, 0.3, threads) == 0);
    CHECK(finite_all(o, nv));
    /* alpha is required whenever there are tokens (the binding passes ones) */
    CHECK(gdn2_oracle_forward(q, k, v, NULL, e, w, NULL, o, NULL, U, T, dk, dv, 0.3, threads) ==
          (T > 0 ? -1 : 0));
    if (T >= 1) {  /* one decode step in place on the first token of every unit */
        double *st = arr(ns, -0.5, 0.5), *o1 = arr(U * dv, 0, 0);
        double *q1 = arr(U * dk, -1, 1), *k1 = arr(U * dk, -1, 1), *v1 = arr(U * dv, -1, 1);
        double *a1 = arr(U * dk, 0.05, 1), *b1 = arr(U, 0, 1);
        CHECK(kda_oracle_step(q1, k1, v1, a1, b1, st, o1, U, dk, dv, 0.3, threads) == 0);
        CHECK(finite_all(st, ns) && finite_all(o1, U * dv));
        free(st); free(o1); free(q1); free(k1); free(v1); free(a1); free(b1);
    }
    double *all[] = {q, k, v, a, b, e, w, s0, dout, dsT, o, sT, gq, gk, gv, ga, gb, gs0};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
}

int main(void) {
    run(3, 37, 8, 6, 2);
    run(2, 1, 16, 16, 1);
    run(4, 0, 8, 8, 3);    /* units without tokens */
    run(1, 70, 5, 9, 0);   /* odd sizes, one thread per CPU */
    /* argument errors */
    double x = 0;
    CHECK(kda_oracle_forward(&x, &x, &x, &x, &x, NULL, &x, &x, -1, 1, 1, 1, 1.0, 1) == -1);
    CHECK(kda_oracle_forward(NULL, &x, &x, &x, &x, NULL, &x, &x, 1, 1, 1, 1, 1.0, 1) == -1);
    CHECK(kda_oracle_step(&x, &x, &x, &x, &x, NULL, &x, 1, 1, 1, 1.0, 1) == -1);
    CHECK(kda_oracle_forward(&x, &x, &x, &x, &x, NULL, &x, &x, 0, 1, 1, 1, 1.0, 1) == 0);
    if (fails) return 1;
    printf("oracle sanitizer run: ok\n");
    return 0;
}
