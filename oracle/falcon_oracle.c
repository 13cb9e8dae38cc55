/*
 * falcon_oracle.c -- fp64 CPU oracle for the Falcon fast-weight recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it: only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg do.  It shares no source
 * with the GPU library.
 *
 * What it computes is the plain step-by-step (recurrent) form, one time step
 * after another, independently per (batch, head), in double precision on the
 * exact input values handed in (bf16 or fp32 bits already widened to double
 * by the caller).
 *
 * Sources ("Fast Weight Attention for Continual Learning", the authors'
 * abstract as reproduced on its listing pages, and the KLA abstract shown on
 * the same listing):
 *   - the state is a fixed-size fast-weight matrix updated once per token as
 *     one step of an online learner, and it is read after the write
 *     (authors' abstract: read-after-write autoregressive semantics);
 *   - step t learns from the key one step back paired with the current
 *     value, x_t = phi(k_{t-1}), y_t = v_t ("Fast Weight Attention for
 *     Continual Learning", authors' abstract; phi = identity here);
 *     the same-step pair x_t = k_t, y_t = v_t (the alignment of the KLA/GDN
 *     recurrences the pages contrast it with) is an option: `lag` = 1 is the
 *     prefix alignment, lag = 0 the same-step one;
 *   - phi is left open by the pages; identity is the default, and a feature
 *     map applied to every key and every query (halo keys included) is an
 *     option: `phi` = 1 is L2 normalization x / ||x|| (0 for x = 0), 2 is
 *     SiLU x / (1 + exp(-x)), elementwise;
 *   - the updates are normalized first-order steps on a squared-error
 *     regression loss (Falcon-1/2/3) or a negative inner-product loss
 *     (Falcon-1A/2A/3A) (authors' abstract, the variant list);
 *   - the step is normalized by the key norm, eta_t / (||x_t||^2 + eps)
 *     (KLA abstract, its Kaczmarz step-size formula), and the state is first
 *     decayed by the positive gate alpha_t, then corrected with a residual
 *     taken at the decayed state (KLA abstract: KLA keeps GDN's gated decay
 *     followed by a delta-rule residual write).
 *
 * Readings where the pages leave a step open (each is listed with its reason
 * in the design notes):
 *   Falcon-2  ("per-column extension", a separate normalization per column):
 *             u_j = eta * x_j / (|x_j| * ||x||_1 + eps), i.e. a diagonal
 *             per-column normalizer whose gain x.u is eta at eps = 0.
 *   Falcon-3  ("sliding-window mini-batch"): one first-order step on the W
 *             most recent prefix-aligned pairs, every residual taken at the
 *             decayed state, step eta / (sum_w ||x_{t-w}||^2 + eps).
 *   A family: the same write vector as the regression counterpart, with the
 *             target itself written instead of the residual.
 *   Start:    keys before the sequence come from k_prev (or are 0), values
 *             before it from v_prev (or are 0); a zero pair writes nothing.
 */
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F1 = 1, OR_F2 = 2, OR_F3 = 3, OR_F1A = 11, OR_F2A = 12, OR_F3A = 13 };

typedef struct {
    int variant, B, H, T, dk, dv, W, lag, phi;
    double eps;
    const double *q, *k, *v, *alpha, *eta, *S0, *k_prev, *v_prev;
    double *o, *S_out;
    int nthreads, tid;
} seq_job;

static int is_known_variant(int var) {
    return var == OR_F1 || var == OR_F2 || var == OR_F3 || var == OR_F1A || var == OR_F2A ||
           var == OR_F3A;
}

/* Key k_tau of one (b,h) sequence for tau in [-W, T-1]; tau < 0 reads the
 * carried halo k_prev[W + tau] (oldest first) or 0 when there is none.  The
 * key of step t's pair w is k_{t-w-lag}. */
static const double* key_at(const seq_job* j, const double* kseq, const double* kprev, int tau,
                            const double* zeros) {
    if (tau >= 0) return kseq + (size_t)tau * j->dk;
    if (kprev && tau >= -j->W) return kprev + (size_t)(j->W + tau) * j->dk;
    return zeros;
}

/* Value v_tau for tau in [-(W-1), T-1]; tau < 0 reads v_prev[W-1+tau]. */
static const double* val_at(const seq_job* j, const double* vseq, const double* vprev, int tau,
                            const double* zeros) {
    if (tau >= 0) return vseq + (size_t)tau * j->dv;
    if (vprev && tau >= -(j->W - 1)) return vprev + (size_t)(j->W - 1 + tau) * j->dv;
    return zeros;
}

/* The feature map phi applied to one vector of n entries, into out. */
static void apply_phi(int phi, const double* x, double* out, int n) {
    if (phi == 1) {
        double nrm = 0.0;
        for (int c = 0; c < n; ++c) nrm += x[c] * x[c];
        const double s = nrm > 0.0 ? 1.0 / sqrt(nrm) : 0.0;
        for (int c = 0; c < n; ++c) out[c] = x[c] * s;
    } else if (phi == 2) {
        for (int c = 0; c < n; ++c) out[c] = x[c] / (1.0 + exp(-x[c]));
    } else {
        for (int c = 0; c < n; ++c) out[c] = x[c];
    }
}

/* A copy of `rows` vectors of length n with phi applied to each (NULL in,
 * NULL out). */
static double* phi_copy(int phi, const double* x, int rows, int n) {
    if (!x) return NULL;
    double* out = malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) * n);
    for (int r = 0; r < rows; ++r) apply_phi(phi, x + (size_t)r * n, out + (size_t)r * n, n);
    return out;
}

/* One (b,h) sequence, t = 0..T-1, in the order the recurrence defines. */
static void run_sequence(const seq_job* j, int bh) {
    const int T = j->T, dk = j->dk, dv = j->dv, W = j->W, var = j->variant;
    /* the feature map on the keys (halo included) and queries, up front */
    double* qphi = phi_copy(j->phi, j->q + (size_t)bh * T * dk, T, dk);
    double* kphi = phi_copy(j->phi, j->k + (size_t)bh * T * dk, T, dk);
    double* kpphi = phi_copy(j->phi, j->k_prev ? j->k_prev + (size_t)bh * W * dk : NULL, W, dk);
    const double* q = qphi;
    const double* k = kphi;
    const double* v = j->v + (size_t)bh * T * dv;
    const double* al = j->alpha + (size_t)bh * T;
    const double* et = j->eta + (size_t)bh * T;
    const double* kprev = kpphi;
    const double* vprev = (j->v_prev && W > 1) ? j->v_prev + (size_t)bh * (W - 1) * dv : NULL;
    double* o = j->o + (size_t)bh * T * dv;

    double* S = calloc((size_t)dv * dk, sizeof(double));      /* S[i][c], i: value row, c: key col */
    double* u = calloc((size_t)dk, sizeof(double));           /* write vector */
    double* pred = calloc((size_t)W * dv, sizeof(double));    /* S' x for each window pair */
    double* zeros = calloc((size_t)(dk > dv ? dk : dv), sizeof(double));
    if (j->S0) memcpy(S, j->S0 + (size_t)bh * dv * dk, sizeof(double) * dv * dk);

    for (int t = 0; t < T; ++t) {
        const double a = al[t], e = et[t];
        /* decay first: S' = alpha_t S */
        for (size_t n = 0; n < (size_t)dv * dk; ++n) S[n] *= a;

        if (var == OR_F1 || var == OR_F1A || var == OR_F2 || var == OR_F2A) {
            const double* x = key_at(j, k, kprev, t - j->lag, zeros); /* x_t = k_{t-lag} */
            const double* y = v + (size_t)t * dv;                /* y_t = v_t */
            if (var == OR_F1 || var == OR_F1A) {
                double nrm = 0.0;
                for (int c = 0; c < dk; ++c) nrm += x[c] * x[c];
                for (int c = 0; c < dk; ++c) u[c] = e * x[c] / (nrm + j->eps);
            } else {
                double l1 = 0.0;
                for (int c = 0; c < dk; ++c) l1 += fabs(x[c]);
                for (int c = 0; c < dk; ++c) u[c] = e * x[c] / (fabs(x[c]) * l1 + j->eps);
            }
            if (var == OR_F1 || var == OR_F2) {
                /* residual at the decayed state, then S = S' + (y - S'x) u^T */
                for (int i = 0; i < dv; ++i) {
                    double s = 0.0;
                    for (int c = 0; c < dk; ++c) s += S[(size_t)i * dk + c] * x[c];
                    pred[i] = y[i] - s;
                }
                for (int i = 0; i < dv; ++i)
                    for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] += pred[i] * u[c];
            } else {
                /* inner-product objective: S = S' + y u^T */
                for (int i = 0; i < dv; ++i)
                    for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] += y[i] * u[c];
            }
        } else { /* Falcon-3 / 3A: the W most recent pairs (k_{t-w-lag}, v_{t-w}), w = 0..W-1 */
            double nrm = 0.0;
            for (int w = 0; w < W; ++w) {
                const double* x = key_at(j, k, kprev, t - w - j->lag, zeros);
                for (int c = 0; c < dk; ++c) nrm += x[c] * x[c];
            }
            const double bstep = e / (nrm + j->eps);
            if (var == OR_F3) {
                /* every residual is taken at the same decayed state S' */
                for (int w = 0; w < W; ++w) {
                    const double* x = key_at(j, k, kprev, t - w - j->lag, zeros);
                    const double* y = val_at(j, v, vprev, t - w, zeros);
                    for (int i = 0; i < dv; ++i) {
                        double s = 0.0;
                        for (int c = 0; c < dk; ++c) s += S[(size_t)i * dk + c] * x[c];
                        pred[(size_t)w * dv + i] = y[i] - s;
                    }
                }
                for (int w = 0; w < W; ++w) {
                    const double* x = key_at(j, k, kprev, t - w - j->lag, zeros);
                    for (int i = 0; i < dv; ++i) {
                        const double r = bstep * pred[(size_t)w * dv + i];
                        for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] += r * x[c];
                    }
                }
            } else {
                for (int w = 0; w < W; ++w) {
                    const double* x = key_at(j, k, kprev, t - w - j->lag, zeros);
                    const double* y = val_at(j, v, vprev, t - w, zeros);
                    for (int i = 0; i < dv; ++i) {
                        const double r = bstep * y[i];
                        for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] += r * x[c];
                    }
                }
            }
        }
        /* read after the write: o_t = S_t q_t */
        const double* qt = q + (size_t)t * dk;
        for (int i = 0; i < dv; ++i) {
            double s = 0.0;
            for (int c = 0; c < dk; ++c) s += S[(size_t)i * dk + c] * qt[c];
            o[(size_t)t * dv + i] = s;
        }
    }
    if (j->S_out) memcpy(j->S_out + (size_t)bh * dv * dk, S, sizeof(double) * dv * dk);
    free(qphi);
    free(kphi);
    free(kpphi);
    free(S);
    free(u);
    free(pred);
    free(zeros);
}

static void* seq_worker(void* arg) {
    const seq_job* j = (const seq_job*)arg;
    const int n = j->B * j->H;
    for (int bh = j->tid; bh < n; bh += j->nthreads) run_sequence(j, bh);
    return NULL;
}

/* Number of CPUs this process may run on. */
int oracle_num_cpus(void) {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int c = CPU_COUNT(&set);
        if (c > 0) return c;
    }
    return 1;
}

/* Recurrent form over [B,H,T,*] inputs.  Shapes: q,k [B,H,T,dk]; v [B,H,T,dv];
 * alpha, eta [B,H,T]; S0 [B,H,dv,dk] or NULL; k_prev [B,H,W,dk] or NULL;
 * v_prev [B,H,W-1,dv] or NULL.  Outputs o [B,H,T,dv], S_out [B,H,dv,dk] (or
 * NULL).  W must be 1 unless the variant is Falcon-3/3A; lag is 1 (prefix
 * alignment) or 0 (same-step).  Returns the number of threads used, or a
 * negative value for an invalid argument. */
int oracle_recurrent_ex(int variant, int B, int H, int T, int dk, int dv, int W, int lag,
                        int phi, double eps, const double* q, const double* k, const double* v,
                        const double* alpha, const double* eta, const double* S0,
                        const double* k_prev, const double* v_prev, double* o, double* S_out,
                        int nthreads) {
    if (!is_known_variant(variant)) return -3;
    if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1 || W < 1) return -2;
    if (lag != 0 && lag != 1) return -2;
    if (phi < 0 || phi > 2) return -2;
    if (W != 1 && variant != OR_F3 && variant != OR_F3A) return -2;
    if (!q || !k || !v || !alpha || !eta || !o) return -1;
    int n = B * H;
    if (nthreads <= 0) nthreads = oracle_num_cpus();
    if (nthreads > n) nthreads = n;
    seq_job* jobs = calloc((size_t)nthreads, sizeof(seq_job));
    pthread_t* th = calloc((size_t)nthreads, sizeof(pthread_t));
    for (int i = 0; i < nthreads; ++i) {
        seq_job jb = {variant, B, H, T, dk, dv, W, lag, phi, eps, q, k, v, alpha, eta, S0,
                      k_prev, v_prev, o, S_out, nthreads, i};
        jobs[i] = jb;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, seq_worker, &jobs[i]);
    seq_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(jobs);
    free(th);
    return nthreads;
}

/* The identity feature map. */
int oracle_recurrent_lag(int variant, int B, int H, int T, int dk, int dv, int W, int lag,
                         double eps, const double* q, const double* k, const double* v,
                         const double* alpha, const double* eta, const double* S0,
                         const double* k_prev, const double* v_prev, double* o, double* S_out,
                         int nthreads) {
    return oracle_recurrent_ex(variant, B, H, T, dk, dv, W, lag, 0, eps, q, k, v, alpha, eta, S0,
                               k_prev, v_prev, o, S_out, nthreads);
}

/* The prefix-aligned form (lag 1), identity feature map. */
int oracle_recurrent(int variant, int B, int H, int T, int dk, int dv, int W, double eps,
                     const double* q, const double* k, const double* v, const double* alpha,
                     const double* eta, const double* S0, const double* k_prev,
                     const double* v_prev, double* o, double* S_out, int nthreads) {
    return oracle_recurrent_lag(variant, B, H, T, dk, dv, W, 1, eps, q, k, v, alpha, eta, S0,
                                k_prev, v_prev, o, S_out, nthreads);
}

/* One decode step for N*H independent heads (Falcon-1/1A/2/2A, window 1):
 * x = k_cache (the previous key; lag 0: the new key k), then decay, write and
 * read exactly as one iteration of the recurrence; afterwards k_cache holds
 * the new key.  S [N,H,dv,dk] and k_cache [N,H,dk] are updated in place;
 * q, k [N,H,dk]; v [N,H,dv]; alpha, eta [N,H]; o [N,H,dv]. */
int oracle_decode_step_ex(int variant, int N, int H, int dk, int dv, int lag, int phi,
                          double eps, double* S, double* k_cache, const double* q,
                          const double* k, const double* v, const double* alpha,
                          const double* eta, double* o) {
    if (variant != OR_F1 && variant != OR_F2 && variant != OR_F1A && variant != OR_F2A) return -3;
    if (N < 1 || H < 1 || dk < 1 || dv < 1 || (lag != 0 && lag != 1)) return -2;
    if (phi < 0 || phi > 2) return -2;
    double* u = calloc((size_t)dk, sizeof(double));
    double* r = calloc((size_t)dv, sizeof(double));
    double* xb = calloc((size_t)dk, sizeof(double));
    double* qb = calloc((size_t)dk, sizeof(double));
    for (size_t n = 0; n < (size_t)N * H; ++n) {
        double* Sh = S + n * dv * dk;
        double* kc = k_cache + n * dk;
        const double *kh = k + n * dk, *vh = v + n * dv;
        apply_phi(phi, lag ? kc : kh, xb, dk);  /* the caches keep the raw keys */
        apply_phi(phi, q + n * dk, qb, dk);
        const double* x = xb;
        const double* qh = qb;
        const double a = alpha[n], e = eta[n];
        for (size_t m = 0; m < (size_t)dv * dk; ++m) Sh[m] *= a;
        if (variant == OR_F1 || variant == OR_F1A) {
            double nrm = 0.0;
            for (int c = 0; c < dk; ++c) nrm += x[c] * x[c];
            for (int c = 0; c < dk; ++c) u[c] = e * x[c] / (nrm + eps);
        } else {
            double l1 = 0.0;
            for (int c = 0; c < dk; ++c) l1 += fabs(x[c]);
            for (int c = 0; c < dk; ++c) u[c] = e * x[c] / (fabs(x[c]) * l1 + eps);
        }
        for (int i = 0; i < dv; ++i) {
            if (variant == OR_F1 || variant == OR_F2) {
                double s = 0.0;
                for (int c = 0; c < dk; ++c) s += Sh[(size_t)i * dk + c] * x[c];
                r[i] = vh[i] - s;
            } else {
                r[i] = vh[i];
            }
        }
        for (int i = 0; i < dv; ++i)
            for (int c = 0; c < dk; ++c) Sh[(size_t)i * dk + c] += r[i] * u[c];
        for (int i = 0; i < dv; ++i) {
            double s = 0.0;
            for (int c = 0; c < dk; ++c) s += Sh[(size_t)i * dk + c] * qh[c];
            o[n * dv + i] = s;
        }
        memcpy(kc, kh, sizeof(double) * dk);
    }
    free(u);
    free(r);
    free(xb);
    free(qb);
    return 0;
}

int oracle_decode_step_lag(int variant, int N, int H, int dk, int dv, int lag, double eps,
                           double* S, double* k_cache, const double* q, const double* k,
                           const double* v, const double* alpha, const double* eta, double* o) {
    return oracle_decode_step_ex(variant, N, H, dk, dv, lag, 0, eps, S, k_cache, q, k, v, alpha,
                                 eta, o);
}

int oracle_decode_step(int variant, int N, int H, int dk, int dv, double eps, double* S,
                       double* k_cache, const double* q, const double* k, const double* v,
                       const double* alpha, const double* eta, double* o) {
    return oracle_decode_step_lag(variant, N, H, dk, dv, 1, eps, S, k_cache, q, k, v, alpha, eta,
                                  o);
}

/*
 * One step of Falcon-3 / Falcon-3A for N x H heads, carrying the window in
 * caches (newest first):
 *   k_cache [N,H,W,dk]:  k_cache[w] = k_{t-1-w}, so x_{t-w} = k_cache[w];
 *   v_cache [N,H,W-1,dv]: v_cache[w-1] = v_{t-w} for w >= 1 (y_t = v, the new
 *                         value).
 * The step is the same one the recurrent form takes at step t: S' = alpha S,
 * b = eta / (sum_w ||x_{t-w}||^2 + eps), then S = S' + b sum_w R_w x_{t-w}^T
 * with every residual R_w = y_{t-w} - S' x_{t-w} taken at S' (Falcon-3A:
 * R_w = y_{t-w}), and o = S q.  Both caches then move one slot: the new key
 * and value enter at slot 0 and the oldest leave.  With lag 0 (same-step
 * pairs) pair w's key is k_{t-w}: the new key for w = 0, k_cache[w-1] after.
 */
int oracle_decode_step_window_ex(int variant, int N, int H, int dk, int dv, int W, int lag,
                                 int phi, double eps, double* S, double* k_cache,
                                 double* v_cache, const double* q, const double* k,
                                 const double* v, const double* alpha, const double* eta,
                                 double* o) {
    if (variant != OR_F3 && variant != OR_F3A) return -3;
    if (N < 1 || H < 1 || dk < 1 || dv < 1 || W < 1 || (lag != 0 && lag != 1)) return -2;
    if (phi < 0 || phi > 2) return -2;
    double* R = calloc((size_t)W * dv, sizeof(double));
    const double** y = calloc((size_t)W, sizeof(double*));
    const double** xs = calloc((size_t)W, sizeof(double*));
    double* xb = calloc((size_t)W * dk, sizeof(double));
    double* qb = calloc((size_t)dk, sizeof(double));
    for (size_t n = 0; n < (size_t)N * H; ++n) {
        double* Sh = S + n * dv * dk;
        double* kc = k_cache + n * W * dk;
        double* vc = v_cache + n * (W - 1) * dv;
        const double *kh = k + n * dk, *vh = v + n * dv;
        apply_phi(phi, q + n * dk, qb, dk);
        const double* qh = qb;
        const double a = alpha[n], e = eta[n];
        for (int w = 0; w < W; ++w) {
            y[w] = (w == 0) ? vh : vc + (size_t)(w - 1) * dv;
            /* the caches keep the raw keys; phi is applied to each pair's key */
            apply_phi(phi, (w + lag == 0) ? kh : kc + (size_t)(w + lag - 1) * dk,
                      xb + (size_t)w * dk, dk);
            xs[w] = xb + (size_t)w * dk;
        }
        for (size_t m = 0; m < (size_t)dv * dk; ++m) Sh[m] *= a;
        double nrm = 0.0;
        for (int w = 0; w < W; ++w)
            for (int c = 0; c < dk; ++c) nrm += xs[w][c] * xs[w][c];
        const double b = e / (nrm + eps);
        for (int w = 0; w < W; ++w) {
            const double* x = xs[w];
            for (int i = 0; i < dv; ++i) {
                double s = 0.0;
                if (variant == OR_F3)
                    for (int c = 0; c < dk; ++c) s += Sh[(size_t)i * dk + c] * x[c];
                R[(size_t)w * dv + i] = y[w][i] - s;
            }
        }
        for (int w = 0; w < W; ++w) {
            const double* x = xs[w];
            for (int i = 0; i < dv; ++i)
                for (int c = 0; c < dk; ++c) Sh[(size_t)i * dk + c] += b * R[(size_t)w * dv + i] * x[c];
        }
        for (int i = 0; i < dv; ++i) {
            double s = 0.0;
            for (int c = 0; c < dk; ++c) s += Sh[(size_t)i * dk + c] * qh[c];
            o[n * dv + i] = s;
        }
        for (int w = W - 1; w >= 1; --w) memcpy(kc + (size_t)w * dk, kc + (size_t)(w - 1) * dk, sizeof(double) * dk);
        memcpy(kc, kh, sizeof(double) * dk);
        for (int w = W - 2; w >= 1; --w) memcpy(vc + (size_t)w * dv, vc + (size_t)(w - 1) * dv, sizeof(double) * dv);
        if (W > 1) memcpy(vc, vh, sizeof(double) * dv);
    }
    free(R);
    free(y);
    free(xs);
    free(xb);
    free(qb);
    return 0;
}

int oracle_decode_step_window_lag(int variant, int N, int H, int dk, int dv, int W, int lag,
                                  double eps, double* S, double* k_cache, double* v_cache,
                                  const double* q, const double* k, const double* v,
                                  const double* alpha, const double* eta, double* o) {
    return oracle_decode_step_window_ex(variant, N, H, dk, dv, W, lag, 0, eps, S, k_cache,
                                        v_cache, q, k, v, alpha, eta, o);
}

int oracle_decode_step_window(int variant, int N, int H, int dk, int dv, int W, double eps,
                              double* S, double* k_cache, double* v_cache, const double* q,
                              const double* k, const double* v, const double* alpha,
                              const double* eta, double* o) {
    return oracle_decode_step_window_lag(variant, N, H, dk, dv, W, 1, eps, S, k_cache, v_cache, q,
                                         k, v, alpha, eta, o);
}
