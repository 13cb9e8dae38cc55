/*
 * oracle_sanitize.c -- a driver that exercises every code path of the fp64
 * oracle (oracle/falcon_oracle.c) in one process, built by
 * tests/test_oracle_sanitize.py with AddressSanitizer and
 * UndefinedBehaviorSanitizer (any invalid access or undefined operation
 * aborts the run).  Test infrastructure only.
 *
 * It runs the recurrent form for all six variants (windows 1, 3 and 8 for the
 * window rules), both alignments, the three feature maps, with and without
 * S0 and halos, at lengths 0, 1 and 37, on more threads than sequences and
 * fewer; the decode steps likewise; and checks two facts that need no second
 * implementation: interpolation (alpha = eta = 1, eps = 0: reading with the
 * step's own key returns the step's target, Falcon-1) and the invalid-
 * argument codes.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_recurrent_ex(int variant, int B, int H, int T, int dk, int dv, int W, int lag,
                        int phi, double eps, const double* q, const double* k, const double* v,
                        const double* alpha, const double* eta, const double* S0,
                        const double* k_prev, const double* v_prev, double* o, double* S_out,
                        int nthreads);
int oracle_decode_step_ex(int variant, int N, int H, int dk, int dv, int lag, int phi,
                          double eps, double* S, double* k_cache, const double* q,
                          const double* k, const double* v, const double* alpha,
                          const double* eta, double* o);
int oracle_decode_step_window_ex(int variant, int N, int H, int dk, int dv, int W, int lag,
                                 int phi, double eps, double* S, double* k_cache,
                                 double* v_cache, const double* q, const double* k,
                                 const double* v, const double* alpha, const double* eta,
                                 double* o);

static unsigned long long rng_state = 88172645463325252ULL;
static double urand(void) { /* xorshift64, uniform in [-1, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) / 4503599627370496.0 - 1.0;
}
static double* fill(size_t n, double lo, double hi) {
    double* p = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (urand() + 1.0);
    return p;
}

static int failures = 0;
#define CHECK(c, ...)                          \
    do {                                       \
        if (!(c)) {                            \
            fprintf(stderr, __VA_ARGS__);      \
            fprintf(stderr, "\n");             \
            ++failures;                        \
        }                                      \
    } while (0)

static void recurrent_paths(void) {
    const int variants[6] = {1, 2, 3, 11, 12, 13};
    const int lengths[3] = {0, 1, 37};
    for (int vi = 0; vi < 6; ++vi) {
        const int var = variants[vi];
        const int win = var == 3 || var == 13;
        for (int wi = 0; wi < (win ? 3 : 1); ++wi) {
            const int W = win ? (wi == 0 ? 1 : (wi == 1 ? 3 : 8)) : 1;
            for (int li = 0; li < 3; ++li)
                for (int lag = 0; lag <= 1; ++lag)
                    for (int phi = 0; phi <= 2; ++phi)
                        for (int opt = 0; opt <= 1; ++opt) {
                            const int B = 2, H = 3, T = lengths[li], dk = 5, dv = 4;
                            const size_t n = (size_t)B * H;
                            double* q = fill(n * T * dk, -1, 1);
                            double* k = fill(n * T * dk, -1, 1);
                            double* v = fill(n * T * dv, -1, 1);
                            double* al = fill(n * T, 0.5, 1.0);
                            double* et = fill(n * T, 0.0, 1.0);
                            double* S0 = opt ? fill(n * dv * dk, -1, 1) : NULL;
                            double* kp = opt ? fill(n * W * dk, -1, 1) : NULL;
                            double* vp = (opt && W > 1) ? fill(n * (W - 1) * dv, -1, 1) : NULL;
                            double* o = fill(n * T * dv, 0, 0);
                            double* S = fill(n * dv * dk, 0, 0);
                            const int th = (li + lag + phi) % 2 ? 1 : 16;
                            int rc = oracle_recurrent_ex(var, B, H, T, dk, dv, W, lag, phi, 1e-6,
                                                         q, k, v, al, et, S0, kp, vp, o, S, th);
                            CHECK(rc > 0, "recurrent var %d W %d T %d lag %d phi %d: rc %d", var,
                                  W, T, lag, phi, rc);
                            for (size_t i = 0; i < n * T * dv; ++i)
                                CHECK(isfinite(o[i]), "non-finite output var %d", var);
                            free(q), free(k), free(v), free(al), free(et), free(S0), free(kp),
                                free(vp), free(o), free(S);
                        }
        }
    }
}

static void interpolation(void) {
    /* alpha = eta = 1, eps = 0: S_t x_t = y_t after step t (Falcon-1); with
     * q_t = x_t = k_{t-1} the read returns v_t */
    const int T = 12, d = 6;
    double* k = fill((size_t)T * d, -1, 1);
    double* v = fill((size_t)T * d, -1, 1);
    double* q = fill((size_t)T * d, 0, 0);
    double* kp = fill((size_t)d, -1, 1);
    double* al = fill(T, 1, 1);
    double* et = fill(T, 1, 1);
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < d; ++c) q[t * d + c] = t == 0 ? kp[c] : k[(t - 1) * d + c];
    double* o = fill((size_t)T * d, 0, 0);
    int rc = oracle_recurrent_ex(1, 1, 1, T, d, d, 1, 1, 0, 0.0, q, k, v, al, et, NULL, kp, NULL,
                                 o, NULL, 1);
    CHECK(rc > 0, "interpolation: rc %d", rc);
    for (int i = 0; i < T * d; ++i)
        CHECK(fabs(o[i] - v[i]) <= 1e-10, "interpolation: o %g v %g at %d", o[i], v[i], i);
    free(k), free(v), free(q), free(kp), free(al), free(et), free(o);
}

static void decode_paths(void) {
    const int variants[4] = {1, 2, 11, 12};
    for (int vi = 0; vi < 4; ++vi)
        for (int lag = 0; lag <= 1; ++lag)
            for (int phi = 0; phi <= 2; ++phi) {
                const int N = 2, H = 3, dk = 5, dv = 4;
                const size_t n = (size_t)N * H;
                double* S = fill(n * dv * dk, -1, 1);
                double* kc = fill(n * dk, -1, 1);
                double* q = fill(n * dk, -1, 1);
                double* k = fill(n * dk, -1, 1);
                double* v = fill(n * dv, -1, 1);
                double* al = fill(n, 0.5, 1);
                double* et = fill(n, 0, 1);
                double* o = fill(n * dv, 0, 0);
                int rc = oracle_decode_step_ex(variants[vi], N, H, dk, dv, lag, phi, 1e-6, S, kc,
                                               q, k, v, al, et, o);
                CHECK(rc >= 0, "decode var %d: rc %d", variants[vi], rc);
                free(S), free(kc), free(q), free(k), free(v), free(al), free(et), free(o);
            }
    for (int var = 3; var <= 13; var += 10)
        for (int W = 1; W <= 8; W += 3)
            for (int lag = 0; lag <= 1; ++lag)
                for (int phi = 0; phi <= 2; ++phi) {
                    const int N = 2, H = 2, dk = 5, dv = 4;
                    const size_t n = (size_t)N * H;
                    double* S = fill(n * dv * dk, -1, 1);
                    double* kc = fill(n * W * dk, -1, 1);
                    double* vc = fill(n * (W > 1 ? W - 1 : 1) * dv, -1, 1);
                    double* q = fill(n * dk, -1, 1);
                    double* k = fill(n * dk, -1, 1);
                    double* v = fill(n * dv, -1, 1);
                    double* al = fill(n, 0.5, 1);
                    double* et = fill(n, 0, 1);
                    double* o = fill(n * dv, 0, 0);
                    int rc = oracle_decode_step_window_ex(var, N, H, dk, dv, W, lag, phi, 1e-6, S,
                                                          kc, vc, q, k, v, al, et, o);
                    CHECK(rc >= 0, "decode window var %d W %d: rc %d", var, W, rc);
                    free(S), free(kc), free(vc), free(q), free(k), free(v), free(al), free(et),
                        free(o);
                }
}

static void invalid_arguments(void) {
    double x[64] = {0};
    CHECK(oracle_recurrent_ex(7, 1, 1, 1, 2, 2, 1, 1, 0, 0, x, x, x, x, x, NULL, NULL, NULL, x,
                              NULL, 1) == -3, "unknown variant accepted");
    CHECK(oracle_recurrent_ex(1, 1, 1, 1, 2, 2, 2, 1, 0, 0, x, x, x, x, x, NULL, NULL, NULL, x,
                              NULL, 1) == -2, "window 2 accepted for Falcon-1");
    CHECK(oracle_recurrent_ex(1, 1, 1, 1, 2, 2, 1, 1, 0, 0, NULL, x, x, x, x, NULL, NULL, NULL, x,
                              NULL, 1) == -1, "NULL queries accepted");
}

int main(void) {
    recurrent_paths();
    interpolation();
    decode_paths();
    invalid_arguments();
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle paths ok\n");
    return 0;
}
