/* oracle_sanitize_check.c -- the fp64 oracle (oracle/rehyat_oracle.c) built
 * with AddressSanitizer and UndefinedBehaviorSanitizer and run over tiny
 * geometries: every feature map, both partitions, row subsets, partial
 * outputs, invalid arguments and the non-finite report.  Besides the
 * sanitizers' own checks it tests one invariant of the hybrid attention
 * (each output is a convex combination of values, so v = c everywhere gives
 * y = c) and that the partials recombine to y.  Prints "oracle sanitize check:
 * N cases, 0 failures" and exits 0 on success. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int rehyat_oracle_fwd(const double* q, const double* k, const double* v, double* y, int B, int H, int F, int HW,
                      int d, int Tc, int To, int phi_kind, double scale, int causal, const long long* rows,
                      long long nrows, double* part_m, double* part_nt, double* part_oS, double* part_oL,
                      double* part_nL, int nthreads, const double* fq, const double* fk, int Dg);

static unsigned long long g_state = 88172645463325252ull;
static double uniform(void) { /* xorshift64, mapped to [-1, 1) */
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (double)(g_state >> 11) / 4503599627370496.0 - 1.0;
}

static int cases = 0, failures = 0;
static void check(int ok, const char* what, int a, int b, int c) {
    ++cases;
    if (!ok) {
        ++failures;
        printf("FAIL %s (%d %d %d)\n", what, a, b, c);
    }
}

int main(void) {
    const int B = 1, H = 2, d = 8;
    for (int F = 1; F <= 5; ++F)
        for (int Tc = 1; Tc <= 3; ++Tc)
            for (int To = 0; To <= 3; ++To)
                for (int phi = 0; phi <= 3; ++phi)
                    for (int causal = 0; causal <= 1; ++causal) {
                        const int HW = 3, N = F * HW, Dg = phi == 3 ? 5 : 0;
                        const size_t n = (size_t)B * H * N * d;
                        double *q = malloc(n * sizeof *q), *k = malloc(n * sizeof *k), *v = malloc(n * sizeof *v);
                        double *y = malloc(n * sizeof *y), *yc = malloc(n * sizeof *yc);
                        double *fq = NULL, *fk = NULL;
                        for (size_t i = 0; i < n; ++i) {
                            q[i] = uniform();
                            k[i] = uniform();
                            v[i] = 0.25;
                        }
                        if (phi == 3) {
                            fq = malloc((size_t)B * H * N * Dg * sizeof *fq);
                            fk = malloc((size_t)B * H * N * Dg * sizeof *fk);
                            for (long i = 0; i < (long)B * H * N * Dg; ++i) {
                                fq[i] = 1.0 + uniform();
                                fk[i] = 1.0 + uniform();
                            }
                        }
                        int st = rehyat_oracle_fwd(q, k, v, y, B, H, F, HW, d, Tc, To, phi, 1.0, causal, NULL, 0,
                                                   NULL, NULL, NULL, NULL, NULL, 2, fq, fk, Dg);
                        check(st == 0, "status", F, Tc, To);
                        double err = 0.0;
                        for (size_t i = 0; i < n; ++i) err = fmax(err, fabs(y[i] - 0.25));
                        check(err < 1e-12, "constant values", F, Tc, To);
                        /* random values: a row subset with every partial, recombined */
                        for (size_t i = 0; i < n; ++i) v[i] = uniform();
                        st = rehyat_oracle_fwd(q, k, v, y, B, H, F, HW, d, Tc, To, phi, 0.5, causal, NULL, 0,
                                               NULL, NULL, NULL, NULL, NULL, 2, fq, fk, Dg);
                        check(st == 0, "status random", F, Tc, To);
                        long long rows[2] = {N - 1, 0};
                        double m[4], nt[4], nl[4], os[4 * 8], ol[4 * 8];
                        st = rehyat_oracle_fwd(q, k, v, yc, B, H, F, HW, d, Tc, To, phi, 0.5, causal, rows, 2, m, nt,
                                               os, ol, nl, 1, fq, fk, Dg);
                        check(st == 0, "status rows", F, Tc, To);
                        for (int bh = 0; bh < B * H; ++bh)
                            for (int r = 0; r < 2; ++r) {
                                const double ns = nt[bh * 2 + r] * exp(m[bh * 2 + r]), nL = nl[bh * 2 + r];
                                for (int c = 0; c < d; ++c) {
                                    const double rec = (ns * os[(bh * 2 + r) * d + c] + nL * ol[(bh * 2 + r) * d + c]) /
                                                       (ns + nL);
                                    const double full = y[((size_t)bh * N + rows[r]) * d + c];
                                    check(fabs(yc[(bh * 2 + r) * d + c] - full) < 1e-13 && fabs(rec - full) < 1e-12,
                                          "rows and partials", F, Tc, To);
                                }
                            }
                        free(q); free(k); free(v); free(y); free(yc); free(fq); free(fk);
                    }
    /* invalid arguments and a sum that overflows fp64 */
    double x[16] = {0}, out[16];
    long long bad_row = 5;
    check(rehyat_oracle_fwd(NULL, x, x, out, 1, 1, 1, 2, 8, 1, 0, 1, 1.0, 1, NULL, 0, NULL, NULL, NULL, NULL, NULL, 1,
                            NULL, NULL, 0) == 1, "null q", 0, 0, 0);
    check(rehyat_oracle_fwd(x, x, x, out, 1, 1, 1, 2, 8, 0, 0, 1, 1.0, 1, NULL, 0, NULL, NULL, NULL, NULL, NULL, 1,
                            NULL, NULL, 0) == 1, "Tc = 0", 0, 0, 0);
    check(rehyat_oracle_fwd(x, x, x, out, 1, 1, 1, 2, 8, 1, 0, 1, 1.0, 1, &bad_row, 1, NULL, NULL, NULL, NULL, NULL,
                            1, NULL, NULL, 0) == 1, "row out of range", 0, 0, 0);
    check(rehyat_oracle_fwd(x, x, x, out, 1, 1, 1, 2, 8, 1, 0, 3, 1.0, 1, NULL, 0, NULL, NULL, NULL, NULL, NULL, 1,
                            NULL, NULL, 0) == 1, "given phi without rows", 0, 0, 0);
    for (int i = 0; i < 16; ++i) x[i] = 30.0; /* q.k = 7200: exp overflows */
    check(rehyat_oracle_fwd(x, x, x, out, 1, 1, 1, 2, 8, 1, 0, 1, 1.0, 1, NULL, 0, NULL, NULL, NULL, NULL, NULL, 1,
                            NULL, NULL, 0) == 2, "overflow reported", 0, 0, 0);
    printf("oracle sanitize check: %d cases, %d failures\n", cases, failures);
    return failures == 0 ? 0 : 1;
}
