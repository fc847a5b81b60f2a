/*
 * kdn_oracle.c -- plain fp64 CPU oracle of the Kalman Delta Network (KDN)
 * layer forward pass and of its one-token decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists so that tests, the smoke check
 * and the benchmark's CPU-baseline leg can check the GPU library against an
 * obviously correct reference.  No product code path may link, load or call
 * it, and it shares no code, header, table or helper with the GPU library.
 *
 * What it computes (sources: "Kalman Delta Networks: Uncertainty-aware
 * Associative Memory", English abstract; ai-feeds.com summary, section
 * "方法 / 关键模块" steps 1-3):
 *
 *   Each head carries a memory S (d_v x d_k).  The memory is the latent state
 *   of a linear-Gaussian state-space model and every token is a noisy linear
 *   observation of it:  v_t = S k_t + N(0, r_t I).  The transition scales the
 *   mean by a_t and adds process noise of variance nu_t.  The rows of S share
 *   one covariance, kept either diagonal (precision lambda, one value per key
 *   dimension: "Diagonal KDN", online mean-field projection of each one-step
 *   posterior) or isotropic (one precision scalar per head: "Isotropic KDN").
 *
 *   Per token, in this order (plain reading of predict -> update):
 *     predict:    lambda^-   = lambda / (a^2 + nu * lambda)         (elementwise)
 *                 P^-        = 1 / lambda^-
 *     gain:       diagonal:  w = (P^- . k) / (sum_i k_i^2 P^-_i + r)
 *                 isotropic: w = P^- k / (P^- |k|^2 + r)
 *     projection: diagonal:  lambda = lambda^- + k.k / r
 *                 isotropic: lambda = lambda^- + |k|^2 / (d_k r)
 *     mean:       S <- a S;  u = v - S k;  S <- S + u w^T;  o = S q
 *
 *   The gain is the exact Kalman gain of the projected predictive prior; the
 *   projection keeps the diagonal of the posterior precision (diagonal) or
 *   its mean over the key dimensions (isotropic), which are the reverse-KL
 *   optima over diagonal / isotropic Gaussians.  The read-out uses the
 *   memory after the write.  lambda0 and S0 are the posterior at t = 0, so
 *   token 1 starts with a prediction step.
 *
 * Layouts (all contiguous, head-major):
 *   q, k  [B,H,T,d_k]    v [B,H,T,d_v]    a, nu, r [B,H,T]
 *   lambda0 [B,H,d_k] (diagonal) or [B,H] (isotropic), NULL -> all ones
 *   S0 [B,H,d_v,d_k] row-major, NULL -> zeros
 *   o [B,H,T,d_v]   S_T like S0   lambda_T like lambda0
 *   dbg_lambda_minus: NULL or [B,H,T,d_k] (diagonal) / [B,H,T] (isotropic)
 *   dbg_w: NULL or [B,H,T,d_k]
 * Inputs are single precision (bf16 inputs arrive already widened to float,
 * exactly); every operation is done in double.
 *
 * Return value: 0 on success, negative on a rejected argument:
 *   -1 bad sizes or variant, -2 NULL pointer, -3 a precondition on the input
 *   values failed (need 0 < a <= 1, nu >= 0, r > 0, lambda0 > 0).
 */
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define KDN_ORACLE_DIAGONAL 0
#define KDN_ORACLE_ISOTROPIC 1

typedef struct {
    int H, T, dk, dv, variant;
    const float *q, *k, *v, *a, *nu, *r, *lambda0, *S0;
    double *o, *S_T, *lambda_T, *dbg_lm, *dbg_w;
    int n_heads, n_threads, tid;
} job_t;

/* One token of the filter for one head.  S is d_v x d_k row-major, lam is
 * d_k values (diagonal) or one value (isotropic).  lm and w are d_k scratch
 * values; on return lm holds lambda^- and w the gain key. */
static void kdn_token(int dk, int dv, int variant, const float *qt, const float *kt,
                      const float *vt, double a, double nu, double r, double *S,
                      double *lam, double *lm, double *w, double *ot)
{
    int i, j;
    if (variant == KDN_ORACLE_DIAGONAL) {
        double den = r;
        for (i = 0; i < dk; ++i) {
            lm[i] = lam[i] / (a * a + nu * lam[i]);
            den += (double)kt[i] * (double)kt[i] / lm[i];
        }
        for (i = 0; i < dk; ++i) {
            w[i] = ((double)kt[i] / lm[i]) / den;
            lam[i] = lm[i] + (double)kt[i] * (double)kt[i] / r;
        }
    } else {
        double kk = 0.0, lmin, pmin;
        for (i = 0; i < dk; ++i) kk += (double)kt[i] * (double)kt[i];
        lmin = lam[0] / (a * a + nu * lam[0]);
        pmin = 1.0 / lmin;
        for (i = 0; i < dk; ++i) {
            lm[i] = lmin;
            w[i] = pmin * (double)kt[i] / (pmin * kk + r);
        }
        lam[0] = lmin + kk / ((double)dk * r);
    }
    for (j = 0; j < dv; ++j) {
        double *row = S + (size_t)j * dk;
        double sk = 0.0, sq = 0.0, u;
        for (i = 0; i < dk; ++i) {
            row[i] *= a;
            sk += row[i] * (double)kt[i];
        }
        u = (double)vt[j] - sk;
        for (i = 0; i < dk; ++i) {
            row[i] += u * w[i];
            sq += row[i] * (double)qt[i];
        }
        ot[j] = sq;
    }
}

static void *run_heads(void *arg)
{
    const job_t *J = (const job_t *)arg;
    const int dk = J->dk, dv = J->dv, T = J->T;
    const int nl = (J->variant == KDN_ORACLE_DIAGONAL) ? dk : 1;
    double *lm = (double *)malloc(sizeof(double) * (size_t)dk);
    double *w = (double *)malloc(sizeof(double) * (size_t)dk);
    int bh, t, i;
    for (bh = J->tid; bh < J->n_heads; bh += J->n_threads) {
        double *S = J->S_T + (size_t)bh * dv * dk;
        double *lam = J->lambda_T + (size_t)bh * nl;
        for (i = 0; i < dv * dk; ++i)
            S[i] = J->S0 ? (double)J->S0[(size_t)bh * dv * dk + i] : 0.0;
        for (i = 0; i < nl; ++i)
            lam[i] = J->lambda0 ? (double)J->lambda0[(size_t)bh * nl + i] : 1.0;
        for (t = 0; t < T; ++t) {
            size_t tok = (size_t)bh * T + t;
            kdn_token(dk, dv, J->variant, J->q + tok * dk, J->k + tok * dk, J->v + tok * dv,
                      (double)J->a[tok], (double)J->nu[tok], (double)J->r[tok], S, lam, lm, w,
                      J->o + tok * dv);
            if (J->dbg_lm)
                for (i = 0; i < nl; ++i) J->dbg_lm[tok * nl + i] = lm[i];
            if (J->dbg_w)
                for (i = 0; i < dk; ++i) J->dbg_w[tok * dk + i] = w[i];
        }
    }
    free(lm);
    free(w);
    return NULL;
}

static int check_values(size_t n_tok, size_t n_lam, const float *a, const float *nu,
                        const float *r, const float *lambda0)
{
    size_t i;
    for (i = 0; i < n_tok; ++i)
        if (!(a[i] > 0.0f && a[i] <= 1.0f && nu[i] >= 0.0f && r[i] > 0.0f)) return -3;
    if (lambda0)
        for (i = 0; i < n_lam; ++i)
            if (!(lambda0[i] > 0.0f)) return -3;
    return 0;
}

static int run_threads(job_t *base, int n_threads)
{
    pthread_t *th;
    job_t *jobs;
    int i;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > base->n_heads) n_threads = base->n_heads > 0 ? base->n_heads : 1;
    th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    jobs = (job_t *)malloc(sizeof(job_t) * (size_t)n_threads);
    for (i = 0; i < n_threads; ++i) {
        jobs[i] = *base;
        jobs[i].tid = i;
        jobs[i].n_threads = n_threads;
    }
    for (i = 1; i < n_threads; ++i) pthread_create(&th[i], NULL, run_heads, &jobs[i]);
    run_heads(&jobs[0]);
    for (i = 1; i < n_threads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
    return 0;
}

int kdn_oracle_forward(int B, int H, int T, int dk, int dv, int variant, const float *q,
                       const float *k, const float *v, const float *a, const float *nu,
                       const float *r, const float *lambda0, const float *S0, double *o,
                       double *S_T, double *lambda_T, double *dbg_lambda_minus, double *dbg_w,
                       int n_threads)
{
    job_t J;
    int rc;
    size_t nl;
    if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1) return -1;
    if (variant != KDN_ORACLE_DIAGONAL && variant != KDN_ORACLE_ISOTROPIC) return -1;
    if (!S_T || !lambda_T) return -2;
    if (T > 0 && (!q || !k || !v || !a || !nu || !r || !o)) return -2;
    nl = (variant == KDN_ORACLE_DIAGONAL) ? (size_t)dk : 1;
    rc = check_values((size_t)B * H * T, (size_t)B * H * nl, a, nu, r, lambda0);
    if (rc) return rc;
    J.H = H; J.T = T; J.dk = dk; J.dv = dv; J.variant = variant;
    J.q = q; J.k = k; J.v = v; J.a = a; J.nu = nu; J.r = r;
    J.lambda0 = lambda0; J.S0 = S0;
    J.o = o; J.S_T = S_T; J.lambda_T = lambda_T;
    J.dbg_lm = dbg_lambda_minus; J.dbg_w = dbg_w;
    J.n_heads = B * H; J.n_threads = n_threads; J.tid = 0;
    return run_threads(&J, n_threads);
}

/* One decode step in place: the t-loop body above applied once to cached
 * (S, lambda) of N sequences x H heads.  q, k [N,H,d_k]; v [N,H,d_v];
 * a, nu, r [N,H]; S [N,H,d_v,d_k] and lambda [N,H,d_k] or [N,H] are read
 * and overwritten; o [N,H,d_v]. */
typedef struct {
    int dk, dv, variant, n_states, n_threads, tid;
    const float *q, *k, *v, *a, *nu, *r;
    double *S, *lam, *o;
} djob_t;

static void *run_decode(void *arg)
{
    const djob_t *J = (const djob_t *)arg;
    const int dk = J->dk, dv = J->dv;
    const int nl = (J->variant == KDN_ORACLE_DIAGONAL) ? dk : 1;
    double *lm = (double *)malloc(sizeof(double) * (size_t)dk);
    double *w = (double *)malloc(sizeof(double) * (size_t)dk);
    int s;
    for (s = J->tid; s < J->n_states; s += J->n_threads)
        kdn_token(dk, dv, J->variant, J->q + (size_t)s * dk, J->k + (size_t)s * dk,
                  J->v + (size_t)s * dv, (double)J->a[s], (double)J->nu[s], (double)J->r[s],
                  J->S + (size_t)s * dv * dk, J->lam + (size_t)s * nl, lm, w,
                  J->o + (size_t)s * dv);
    free(lm);
    free(w);
    return NULL;
}

int kdn_oracle_decode_step(int N, int H, int dk, int dv, int variant, const float *q,
                           const float *k, const float *v, const float *a, const float *nu,
                           const float *r, double *S, double *lambda, double *o, int n_threads)
{
    djob_t base, *jobs;
    pthread_t *th;
    int i, n_states = N * H;
    size_t s;
    if (N < 0 || H < 0 || dk < 1 || dv < 1) return -1;
    if (variant != KDN_ORACLE_DIAGONAL && variant != KDN_ORACLE_ISOTROPIC) return -1;
    if (n_states == 0) return 0;
    if (!q || !k || !v || !a || !nu || !r || !S || !lambda || !o) return -2;
    if (check_values((size_t)n_states, 0, a, nu, r, NULL)) return -3;
    for (s = 0; s < (size_t)n_states * ((variant == KDN_ORACLE_DIAGONAL) ? dk : 1); ++s)
        if (!(lambda[s] > 0.0)) return -3;
    base.dk = dk; base.dv = dv; base.variant = variant; base.n_states = n_states;
    base.q = q; base.k = k; base.v = v; base.a = a; base.nu = nu; base.r = r;
    base.S = S; base.lam = lambda; base.o = o;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > n_states) n_threads = n_states;
    th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    jobs = (djob_t *)malloc(sizeof(djob_t) * (size_t)n_threads);
    for (i = 0; i < n_threads; ++i) {
        jobs[i] = base;
        jobs[i].tid = i;
        jobs[i].n_threads = n_threads;
    }
    for (i = 1; i < n_threads; ++i) pthread_create(&th[i], NULL, run_decode, &jobs[i]);
    run_decode(&jobs[0]);
    for (i = 1; i < n_threads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
    return 0;
}

/* ------------------------------------------------------------------------
 * Reverse-mode derivative of kdn_oracle_forward (a vector-Jacobian product).
 *
 * Given the cotangents dO [B,H,T,d_v], dS_T [B,H,d_v,d_k] (NULL: zero) and
 * dlambda_T (NULL: zero), it returns the gradient of
 *     L = <dO, o> + <dS_T, S_T> + <dlambda_T, lambda_T>
 * with respect to every input: dq, dk [B,H,T,d_k], dv [B,H,T,d_v],
 * da, dnu, dr [B,H,T], dlambda0 (like lambda0) and dS0 (like S0).  Training
 * the layer needs exactly these ("Kalman Delta Networks", English abstract:
 * the variants are pretrained inside language models of 750M and 1.3B
 * parameters).
 *
 * It differentiates the per-token steps of kdn_token above, in the reverse of
 * their order, by the chain rule written out; nothing is re-associated.  The
 * rows of S evolve independently given the gains, so the mean part runs row
 * by row; the precision recursion (which does not see S) runs per head.
 *
 * Mean, for one row s of S (u = v_j - a s_{t-1}.k, s_t = a s_{t-1} + u w,
 * o_j = s_t.q), with sigma the adjoint of s_t:
 *     sigma += do_j q;  dq += do_j s_t;  du = sigma.w;  dw += u sigma;
 *     dv_j = du;  dk -= du a s_{t-1};  da += sigma.s_{t-1} - du (s_{t-1}.k);
 *     sigma <- a sigma - a du k.
 * Precision, per token in reverse with Lambda the adjoint of lambda_t:
 *     lambda_t = lambda^- + (k.k)/r   (isotropic: + |k|^2/(d_k r))
 *     w = P^- k / D,  D = r + sum_i k_i^2 P^-_i   (isotropic: D = P^- |k|^2 + r)
 *     lambda^- = lambda_{t-1} / (a^2 + nu lambda_{t-1}),  P^- = 1/lambda^-.
 * Inputs are single precision as in the forward; every operation is double.
 * Return value as kdn_oracle_forward.
 * ------------------------------------------------------------------------ */
typedef struct {
    int T, dk, dv, variant;
    const float *q, *k, *v, *a, *nu, *r, *lambda0, *S0, *dO, *dS_T, *dlam_T;
    double *dq, *dk_, *dv_, *da, *dnu, *dr, *dlam0, *dS0;
    int n_heads, n_threads, tid;
} bjob_t;

static void *run_heads_backward(void *arg)
{
    const bjob_t *J = (const bjob_t *)arg;
    const int T = J->T, dk = J->dk, dv = J->dv;
    const int diag = J->variant == KDN_ORACLE_DIAGONAL;
    const int nl = diag ? dk : 1;
    double *lamprev = (double *)malloc(sizeof(double) * ((size_t)T * nl + 1));
    double *lmh = (double *)malloc(sizeof(double) * ((size_t)T * nl + 1));
    double *wh = (double *)malloc(sizeof(double) * ((size_t)T * dk + 1));
    double *Dh = (double *)malloc(sizeof(double) * ((size_t)T + 1));
    double *hist = (double *)malloc(sizeof(double) * ((size_t)(T + 1) * dk));
    double *dw = (double *)malloc(sizeof(double) * ((size_t)T * dk + 1));
    double *lam = (double *)malloc(sizeof(double) * (size_t)nl);
    double *Lam = (double *)malloc(sizeof(double) * (size_t)nl);
    double *sig = (double *)malloc(sizeof(double) * (size_t)dk);
    int bh, t, i, j;
    for (bh = J->tid; bh < J->n_heads; bh += J->n_threads) {
        const size_t tok0 = (size_t)bh * T;
        double *dq = J->dq + tok0 * dk, *dkk = J->dk_ + tok0 * dk, *dvv = J->dv_ + tok0 * dv;
        double *da = J->da + tok0, *dnu = J->dnu + tok0, *dr = J->dr + tok0;
        /* precision recursion forward: lambda_{t-1}, lambda^-_t, w_t, D_t */
        for (i = 0; i < nl; ++i)
            lam[i] = J->lambda0 ? (double)J->lambda0[(size_t)bh * nl + i] : 1.0;
        for (t = 0; t < T; ++t) {
            const float *kt = J->k + (tok0 + t) * dk;
            const double a = J->a[tok0 + t], nu = J->nu[tok0 + t], r = J->r[tok0 + t];
            double D;
            for (i = 0; i < nl; ++i) {
                lamprev[(size_t)t * nl + i] = lam[i];
                lmh[(size_t)t * nl + i] = lam[i] / (a * a + nu * lam[i]);
            }
            if (diag) {
                D = r;
                for (i = 0; i < dk; ++i) D += (double)kt[i] * (double)kt[i] / lmh[(size_t)t * dk + i];
                for (i = 0; i < dk; ++i) {
                    wh[(size_t)t * dk + i] = ((double)kt[i] / lmh[(size_t)t * dk + i]) / D;
                    lam[i] = lmh[(size_t)t * dk + i] + (double)kt[i] * (double)kt[i] / r;
                }
            } else {
                double kk = 0.0, p = 1.0 / lmh[t];
                for (i = 0; i < dk; ++i) kk += (double)kt[i] * (double)kt[i];
                D = p * kk + r;
                for (i = 0; i < dk; ++i) wh[(size_t)t * dk + i] = p * (double)kt[i] / D;
                lam[0] = lmh[t] + kk / ((double)dk * r);
            }
            Dh[t] = D;
        }
        for (i = 0; i < T * dk; ++i) { dq[i] = 0.0; dkk[i] = 0.0; dw[i] = 0.0; }
        for (t = 0; t < T; ++t) { da[t] = 0.0; dnu[t] = 0.0; dr[t] = 0.0; }
        /* mean: one row of S at a time, forward (keeping every s_t) then reverse */
        for (j = 0; j < dv; ++j) {
            for (i = 0; i < dk; ++i)
                hist[i] = J->S0 ? (double)J->S0[((size_t)bh * dv + j) * dk + i] : 0.0;
            for (t = 0; t < T; ++t) {
                const float *kt = J->k + (tok0 + t) * dk;
                const double a = J->a[tok0 + t];
                const double *sp = hist + (size_t)t * dk;
                double *sn = hist + (size_t)(t + 1) * dk;
                double sk = 0.0, u;
                for (i = 0; i < dk; ++i) sk += a * sp[i] * (double)kt[i];
                u = (double)J->v[(tok0 + t) * dv + j] - sk;
                for (i = 0; i < dk; ++i) sn[i] = a * sp[i] + u * wh[(size_t)t * dk + i];
            }
            for (i = 0; i < dk; ++i)
                sig[i] = J->dS_T ? (double)J->dS_T[((size_t)bh * dv + j) * dk + i] : 0.0;
            for (t = T - 1; t >= 0; --t) {
                const float *kt = J->k + (tok0 + t) * dk, *qt = J->q + (tok0 + t) * dk;
                const double a = J->a[tok0 + t];
                const double doj = J->dO[(tok0 + t) * dv + j];
                const double *sp = hist + (size_t)t * dk, *sn = hist + (size_t)(t + 1) * dk;
                const double *wt = wh + (size_t)t * dk;
                double sk = 0.0, du = 0.0, ss = 0.0, u;
                for (i = 0; i < dk; ++i) {
                    sig[i] += doj * (double)qt[i];
                    dq[(size_t)t * dk + i] += doj * sn[i];
                    sk += sp[i] * (double)kt[i];
                }
                u = (double)J->v[(tok0 + t) * dv + j] - a * sk;
                for (i = 0; i < dk; ++i) {
                    du += sig[i] * wt[i];
                    dw[(size_t)t * dk + i] += u * sig[i];
                    ss += sig[i] * sp[i];
                }
                dvv[(size_t)t * dv + j] = du;
                da[t] += ss - du * sk;
                for (i = 0; i < dk; ++i) {
                    dkk[(size_t)t * dk + i] -= du * a * sp[i];
                    sig[i] = a * sig[i] - a * du * (double)kt[i];
                }
            }
            if (J->dS0)
                for (i = 0; i < dk; ++i) J->dS0[((size_t)bh * dv + j) * dk + i] = sig[i];
        }
        /* precision recursion in reverse */
        for (i = 0; i < nl; ++i) Lam[i] = J->dlam_T ? (double)J->dlam_T[(size_t)bh * nl + i] : 0.0;
        for (t = T - 1; t >= 0; --t) {
            const float *kt = J->k + (tok0 + t) * dk;
            const double a = J->a[tok0 + t], nu = J->nu[tok0 + t], r = J->r[tok0 + t];
            const double D = Dh[t];
            const double *wt = wh + (size_t)t * dk, *dwt = dw + (size_t)t * dk;
            double s = 0.0;
            for (i = 0; i < dk; ++i) s += dwt[i] * wt[i];
            dr[t] += -s / D;
            if (diag) {
                for (i = 0; i < dk; ++i) {
                    const double ki = kt[i], lm = lmh[(size_t)t * dk + i], p = 1.0 / lm;
                    const double lp = lamprev[(size_t)t * dk + i], e = a * a + nu * lp;
                    double dlm = Lam[i], dp;
                    /* lambda_t = lambda^- + k^2 / r */
                    dkk[(size_t)t * dk + i] += Lam[i] * 2.0 * ki / r;
                    dr[t] += -Lam[i] * ki * ki / (r * r);
                    /* w = P^- k / D */
                    dp = (ki / D) * (dwt[i] - ki * s);
                    dkk[(size_t)t * dk + i] += (p / D) * (dwt[i] - 2.0 * ki * s);
                    dlm += -dp * p * p;
                    /* lambda^- = lambda_{t-1} / (a^2 + nu lambda_{t-1}) */
                    Lam[i] = dlm * a * a / (e * e);
                    da[t] += dlm * (-2.0 * a * lp) / (e * e);
                    dnu[t] += dlm * (-lp * lp) / (e * e);
                }
            } else {
                double kk = 0.0, z = 0.0, dkap, dp, dlm;
                const double lm = lmh[t], p = 1.0 / lm, lp = lamprev[t], e = a * a + nu * lp;
                for (i = 0; i < dk; ++i) {
                    kk += (double)kt[i] * (double)kt[i];
                    z += dwt[i] * (double)kt[i];
                }
                /* lambda_t = lambda^- + |k|^2 / (d_k r) */
                dlm = Lam[0];
                dkap = Lam[0] / ((double)dk * r);
                dr[t] += -Lam[0] * kk / ((double)dk * r * r);
                /* w = P^- k / (P^- |k|^2 + r) */
                dp = z / D - s * kk / D;
                dkap += -p * s / D;
                for (i = 0; i < dk; ++i)
                    dkk[(size_t)t * dk + i] += dwt[i] * p / D + dkap * 2.0 * (double)kt[i];
                dlm += -dp * p * p;
                Lam[0] = dlm * a * a / (e * e);
                da[t] += dlm * (-2.0 * a * lp) / (e * e);
                dnu[t] += dlm * (-lp * lp) / (e * e);
            }
        }
        if (J->dlam0)
            for (i = 0; i < nl; ++i) J->dlam0[(size_t)bh * nl + i] = Lam[i];
    }
    free(lamprev); free(lmh); free(wh); free(Dh); free(hist); free(dw);
    free(lam); free(Lam); free(sig);
    return NULL;
}

int kdn_oracle_backward(int B, int H, int T, int dk, int dv, int variant, const float *q,
                        const float *k, const float *v, const float *a, const float *nu,
                        const float *r, const float *lambda0, const float *S0, const float *dO,
                        const float *dS_T, const float *dlambda_T, double *dq, double *dk_,
                        double *dv_, double *da, double *dnu, double *dr, double *dlambda0,
                        double *dS0, int n_threads)
{
    bjob_t base, *jobs;
    pthread_t *th;
    int i, rc, n_heads = B * H;
    size_t nl;
    if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1) return -1;
    if (variant != KDN_ORACLE_DIAGONAL && variant != KDN_ORACLE_ISOTROPIC) return -1;
    if (T > 0 && (!q || !k || !v || !a || !nu || !r || !dO || !dq || !dk_ || !dv_ || !da ||
                  !dnu || !dr))
        return -2;
    nl = (variant == KDN_ORACLE_DIAGONAL) ? (size_t)dk : 1;
    rc = check_values((size_t)B * H * T, (size_t)B * H * nl, a, nu, r, lambda0);
    if (rc) return rc;
    if (n_heads == 0) return 0;
    base.T = T; base.dk = dk; base.dv = dv; base.variant = variant;
    base.q = q; base.k = k; base.v = v; base.a = a; base.nu = nu; base.r = r;
    base.lambda0 = lambda0; base.S0 = S0; base.dO = dO; base.dS_T = dS_T;
    base.dlam_T = dlambda_T;
    base.dq = dq; base.dk_ = dk_; base.dv_ = dv_; base.da = da; base.dnu = dnu; base.dr = dr;
    base.dlam0 = dlambda0; base.dS0 = dS0;
    base.n_heads = n_heads;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > n_heads) n_threads = n_heads;
    th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    jobs = (bjob_t *)malloc(sizeof(bjob_t) * (size_t)n_threads);
    for (i = 0; i < n_threads; ++i) {
        jobs[i] = base;
        jobs[i].tid = i;
        jobs[i].n_threads = n_threads;
    }
    for (i = 1; i < n_threads; ++i) pthread_create(&th[i], NULL, run_heads_backward, &jobs[i]);
    run_heads_backward(&jobs[0]);
    for (i = 1; i < n_threads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
    return 0;
}

/* ------------------------------------------------------------------------
 * Exact KDN: the dense Riccati recursion that the two approximations replace
 * ("Kalman Delta Networks", English abstract: exact tracking of the key-space
 * posterior needs a full covariance whose Riccati update depends on the
 * state).  One d_k x d_k covariance P per head,
 * shared by the rows of S; per token, in the order of kdn_token:
 *     predict:  P^- = a^2 P + nu I
 *     gain:     w = P^- k / (k^T P^- k + r)
 *     update:   P = P^- - (P^- k)(P^- k)^T / (k^T P^- k + r)
 *     mean:     S <- a S;  u = v - S k;  S <- S + u w^T;  o = S q
 * P0 [B,H,d_k,d_k] (NULL: identity) is the posterior covariance at t = 0.
 * Outputs o, S_T as kdn_oracle_forward, P_T [B,H,d_k,d_k], and optionally the
 * gains dbg_w [B,H,T,d_k].  Return value as kdn_oracle_forward (-3 also for a
 * P0 with a non-positive diagonal).
 * ------------------------------------------------------------------------ */
typedef struct {
    int T, dk, dv;
    const float *q, *k, *v, *a, *nu, *r, *P0, *S0;
    double *o, *S_T, *P_T, *dbg_w;
    int n_heads, n_threads, tid;
} djob2_t;

static void *run_heads_dense(void *arg)
{
    const djob2_t *J = (const djob2_t *)arg;
    const int T = J->T, dk = J->dk, dv = J->dv;
    double *pk = (double *)malloc(sizeof(double) * (size_t)dk);
    double *w = (double *)malloc(sizeof(double) * (size_t)dk);
    int bh, t, i, j;
    for (bh = J->tid; bh < J->n_heads; bh += J->n_threads) {
        double *P = J->P_T + (size_t)bh * dk * dk;
        double *S = J->S_T + (size_t)bh * dv * dk;
        for (i = 0; i < dk * dk; ++i)
            P[i] = J->P0 ? (double)J->P0[(size_t)bh * dk * dk + i] : (i % (dk + 1) == 0 ? 1.0 : 0.0);
        for (i = 0; i < dv * dk; ++i) S[i] = J->S0 ? (double)J->S0[(size_t)bh * dv * dk + i] : 0.0;
        for (t = 0; t < T; ++t) {
            const size_t tok = (size_t)bh * T + t;
            const float *kt = J->k + tok * dk, *qt = J->q + tok * dk, *vt = J->v + tok * dv;
            const double a = J->a[tok], nu = J->nu[tok], r = J->r[tok];
            double den = r;
            for (i = 0; i < dk * dk; ++i) P[i] *= a * a;
            for (i = 0; i < dk; ++i) P[(size_t)i * dk + i] += nu;
            for (i = 0; i < dk; ++i) {
                double s = 0.0;
                for (j = 0; j < dk; ++j) s += P[(size_t)i * dk + j] * (double)kt[j];
                pk[i] = s;
            }
            for (i = 0; i < dk; ++i) den += (double)kt[i] * pk[i];
            for (i = 0; i < dk; ++i) w[i] = pk[i] / den;
            for (i = 0; i < dk; ++i)
                for (j = 0; j < dk; ++j) P[(size_t)i * dk + j] -= pk[i] * pk[j] / den;
            if (J->dbg_w)
                for (i = 0; i < dk; ++i) J->dbg_w[tok * dk + i] = w[i];
            for (j = 0; j < dv; ++j) {
                double *row = S + (size_t)j * dk;
                double sk = 0.0, sq = 0.0, u;
                for (i = 0; i < dk; ++i) {
                    row[i] *= a;
                    sk += row[i] * (double)kt[i];
                }
                u = (double)vt[j] - sk;
                for (i = 0; i < dk; ++i) {
                    row[i] += u * w[i];
                    sq += row[i] * (double)qt[i];
                }
                J->o[tok * dv + j] = sq;
            }
        }
    }
    free(pk);
    free(w);
    return NULL;
}

int kdn_oracle_forward_dense(int B, int H, int T, int dk, int dv, const float *q, const float *k,
                             const float *v, const float *a, const float *nu, const float *r,
                             const float *P0, const float *S0, double *o, double *S_T,
                             double *P_T, double *dbg_w, int n_threads)
{
    djob2_t base, *jobs;
    pthread_t *th;
    int i, n_heads = B * H;
    size_t h;
    if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1) return -1;
    if (!S_T || !P_T) return -2;
    if (T > 0 && (!q || !k || !v || !a || !nu || !r || !o)) return -2;
    if (check_values((size_t)B * H * T, 0, a, nu, r, NULL)) return -3;
    if (P0)
        for (h = 0; h < (size_t)n_heads; ++h)
            for (i = 0; i < dk; ++i)
                if (!(P0[h * dk * dk + (size_t)i * dk + i] > 0.0f)) return -3;
    if (n_heads == 0) return 0;
    base.T = T; base.dk = dk; base.dv = dv;
    base.q = q; base.k = k; base.v = v; base.a = a; base.nu = nu; base.r = r;
    base.P0 = P0; base.S0 = S0; base.o = o; base.S_T = S_T; base.P_T = P_T; base.dbg_w = dbg_w;
    base.n_heads = n_heads;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > n_heads) n_threads = n_heads;
    th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    jobs = (djob2_t *)malloc(sizeof(djob2_t) * (size_t)n_threads);
    for (i = 0; i < n_threads; ++i) {
        jobs[i] = base;
        jobs[i].tid = i;
        jobs[i].n_threads = n_threads;
    }
    for (i = 1; i < n_threads; ++i) pthread_create(&th[i], NULL, run_heads_dense, &jobs[i]);
    run_heads_dense(&jobs[0]);
    for (i = 1; i < n_threads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
    return 0;
}
