/*
 * rt_oracle.c -- plain, slow, fp64 CPU oracle of the routed sparse attention
 * layer of the Routing Transformer (Roy, Saffar, Vaswani, Grangier,
 * "Efficient Content-Based Sparse Attention with Routing Transformers",
 * TACL 9, 2021).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library; it reads float64 copies of the exact (already rounded) input
 * values and computes everything in float64 with straightforward loops.
 *
 * Page citations below are to the paperlayer.ai "Source-linked AI summary" of
 * the paper (written "summary §N") and to the arXiv abstract as shown on the
 * mlsanity.com index page ("abstract").  The pages describe the method in
 * words only; the steps here are the plainest reading of them:
 *
 *   O1 normalise   q^ = x / max(||x||_2, 1e-12)            summary §1, §4
 *   O2 score       s[c][t] = <q^_t, mu_c>                   summary §2, §4
 *   O3 select      per centroid, the w tokens with the largest score
 *                  (ties: lower position first), listed by position
 *                                                           summary §4 (balanced)
 *   O4 attend      per cluster, causal softmax attention among its members,
 *                  masked by original position (self included) summary §3, §4
 *   O5 scatter     out[t] = sum over the clusters holding t, centroid order
 *   O6 EMA         mu <- lam*mu + (1-lam)/2 * (sum of member q^ + member k^),
 *                  members summed over the whole batch       summary §2, §4
 *                  (online mini-batch spherical k-means; the update rule is
 *                  not printed on the pages -- this exponential-moving-average
 *                  form is the reading taken)
 *   O7 local       sliding-window softmax attention over the W most recent
 *                  positions (self included)                 abstract; summary §6
 *   O8 backward    gradients of O4+O5 w.r.t. q^, k^, v (routing and the
 *                  normalisation are held fixed)
 *   O9 local bwd   gradients of O7 w.r.t. q, k, v
 * Variants (readings the pages leave open, built beside the main path):
 *   O10 blocked    blocked (chunked) local attention: blocks of `block`
 *                  positions, position i sees the positions of its own block
 *                  and of the `lookback` blocks before it, not later than i
 *   O11 argmax     each token's nearest centroid (largest score, ties to the
 *                  lower index), and the EMA of O6 over those assignments
 *                  (every token counts once, for its own centroid)
 *   O12 partition  one cluster per token, all clusters of n/k tokens: tokens
 *                  ordered by (argmax centroid, descending score against it,
 *                  position) and cut into k consecutive groups   summary §4
 *                  (a token's assigned cluster; a sort)
 *
 * Every function is sequential over its unit; the *_all drivers only hand
 * independent (batch, head) units to worker threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- O1 ---- */
/* Unit-normalise each of the n rows of x [n][d].  Summary §4: queries and
 * keys are unit-normalised so that nearest-centroid routing relates to
 * maximum inner product search.  inv_norm[t] = 1 / max(||x_t||, 1e-12). */
void orc_normalize(const double *x, long n, int d, double *xhat, double *inv_norm)
{
    for (long t = 0; t < n; ++t) {
        double ss = 0.0;
        for (int i = 0; i < d; ++i)
            ss += x[t * d + i] * x[t * d + i];
        double r = sqrt(ss);
        if (r < 1e-12)
            r = 1e-12;
        if (inv_norm)
            inv_norm[t] = 1.0 / r;
        for (int i = 0; i < d; ++i)
            xhat[t * d + i] = x[t * d + i] / r;
    }
}

/* ---------------------------------------------------------------- O2 ---- */
/* Score every token against every centroid: s[c][t] = <xhat_t, mu_c>.
 * For unit xhat, ||xhat - mu||^2 = 1 - 2<xhat,mu> + ||mu||^2, so the largest
 * score is the nearest centroid (summary §2, §4). */
void orc_scores(const double *xhat, const double *mu, long n, int d, int k, double *s)
{
    for (int c = 0; c < k; ++c)
        for (long t = 0; t < n; ++t) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += xhat[t * d + i] * mu[c * d + i];
            s[(long)c * n + t] = acc;
        }
}

/* ---------------------------------------------------------------- O3 ---- */
typedef struct {
    double s;
    long t;
} scored_t;

/* larger score first; equal scores: lower position first */
static int by_score_then_pos(const void *a, const void *b)
{
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->t < y->t) ? -1 : (x->t > y->t);
}

static int by_int(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Balanced clusters (summary §4: each query meets about n/k keys): centroid c
 * takes the w tokens with the largest scores.  idx[c][*] lists them by
 * ascending position.  margin[c] is the gap between the w-th and the
 * (w+1)-th largest score (+inf when w == n): where it is tiny, rounding may
 * legitimately choose another member. */
void orc_select(const double *s, long n, int k, long w, int32_t *idx, double *margin)
{
    scored_t *buf = (scored_t *)malloc(sizeof(scored_t) * (size_t)n);
    for (int c = 0; c < k; ++c) {
        for (long t = 0; t < n; ++t) {
            buf[t].s = s[(long)c * n + t];
            buf[t].t = t;
        }
        qsort(buf, (size_t)n, sizeof(scored_t), by_score_then_pos);
        for (long r = 0; r < w; ++r)
            idx[(long)c * w + r] = (int32_t)buf[r].t;
        qsort(idx + (long)c * w, (size_t)w, sizeof(int32_t), by_int);
        if (margin)
            margin[c] = (w < n) ? buf[w - 1].s - buf[w].s : INFINITY;
    }
    free(buf);
}

/* ---------------------------------------------------------------- O4 ---- */
/* Attention inside each cluster (summary §3: softmax-normalised weights over
 * the allowed keys, output = weighted sum of values; §4: only query-key pairs
 * routed to the same cluster are considered).  Member s is visible to member
 * r when its original position is not later (causal) or always (causal==0).
 * o[c][r][*] is the output row of member r of cluster c; lse[c][r] is the
 * log of the softmax denominator (max + log sum exp), -inf for an empty row,
 * whose output is 0. */
void orc_attend(const double *qhat, const double *khat, const double *v, const int32_t *idx,
                long n, int d, int k, long w, double scale, int causal, double *o, double *lse)
{
    (void)n;
    double *logit = (double *)malloc(sizeof(double) * (size_t)w);
    char *ok = (char *)malloc((size_t)w);
    for (int c = 0; c < k; ++c) {
        const int32_t *p = idx + (long)c * w;
        for (long r = 0; r < w; ++r) {
            double *orow = o + ((long)c * w + r) * d;
            double m = -INFINITY;
            for (long s = 0; s < w; ++s) {
                ok[s] = (!causal) || (p[s] <= p[r]);
                if (!ok[s])
                    continue;
                double dot = 0.0;
                for (int i = 0; i < d; ++i)
                    dot += qhat[(long)p[r] * d + i] * khat[(long)p[s] * d + i];
                logit[s] = scale * dot;
                if (logit[s] > m)
                    m = logit[s];
            }
            for (int i = 0; i < d; ++i)
                orow[i] = 0.0;
            if (m == -INFINITY) {
                if (lse)
                    lse[(long)c * w + r] = -INFINITY;
                continue;
            }
            double z = 0.0;
            for (long s = 0; s < w; ++s)
                if (ok[s])
                    z += exp(logit[s] - m);
            for (long s = 0; s < w; ++s) {
                if (!ok[s])
                    continue;
                double pr = exp(logit[s] - m) / z;
                for (int i = 0; i < d; ++i)
                    orow[i] += pr * v[(long)p[s] * d + i];
            }
            if (lse)
                lse[(long)c * w + r] = m + log(z);
        }
    }
    free(logit);
    free(ok);
}

/* ---------------------------------------------------------------- O5 ---- */
/* Scatter-add back to token order: a token gets the sum of its rows over all
 * clusters that hold it (taken in ascending centroid order); a token in no
 * cluster gets 0. */
void orc_scatter(const double *o, const int32_t *idx, long n, int d, int k, long w, double *out)
{
    memset(out, 0, sizeof(double) * (size_t)n * (size_t)d);
    for (int c = 0; c < k; ++c)
        for (long r = 0; r < w; ++r) {
            long t = idx[(long)c * w + r];
            for (int i = 0; i < d; ++i)
                out[t * d + i] += o[((long)c * w + r) * d + i];
        }
}

/* ---------------------------------------------------------------- O6 ---- */
/* acc[c][*] += sum over the members of cluster c of xhat (ascending member
 * order).  Called once per batch row, in ascending batch order, since the
 * centroids are shared across sequences (summary §4). */
void orc_cluster_sums(const double *xhat, const int32_t *idx, long n, int d, int k, long w,
                      double *acc)
{
    (void)n;
    for (int c = 0; c < k; ++c)
        for (long r = 0; r < w; ++r) {
            long t = idx[(long)c * w + r];
            for (int i = 0; i < d; ++i)
                acc[(long)c * d + i] += xhat[t * d + i];
        }
}

/* mu <- lam*mu + (1-lam)/2 * (sum_q + sum_k), in place, no renormalisation. */
void orc_ema(double *mu, const double *sum_q, const double *sum_k, int k, int d, double lam)
{
    for (long j = 0; j < (long)k * d; ++j)
        mu[j] = lam * mu[j] + (1.0 - lam) * 0.5 * (sum_q[j] + sum_k[j]);
}

/* ---------------------------------------------------------------- O7 ---- */
/* Local (sliding-window) attention: position i attends to the `window`
 * positions ending at i (causal), or to positions within window-1 on either
 * side (causal == 0).  Plain softmax(scale * q_i . k_j) v_j over that set. */
void orc_local(const double *q, const double *kk, const double *v, long n, int d, long window,
               double scale, int causal, double *out)
{
    double *logit = (double *)malloc(sizeof(double) * (size_t)(2 * window + 1));
    for (long i = 0; i < n; ++i) {
        long lo = i - window + 1;
        if (lo < 0)
            lo = 0;
        long hi = causal ? i : i + window - 1;
        if (hi > n - 1)
            hi = n - 1;
        double m = -INFINITY;
        for (long j = lo; j <= hi; ++j) {
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += q[i * d + e] * kk[j * d + e];
            logit[j - lo] = scale * dot;
            if (logit[j - lo] > m)
                m = logit[j - lo];
        }
        double z = 0.0;
        for (long j = lo; j <= hi; ++j)
            z += exp(logit[j - lo] - m);
        for (int e = 0; e < d; ++e)
            out[i * d + e] = 0.0;
        for (long j = lo; j <= hi; ++j) {
            double pr = exp(logit[j - lo] - m) / z;
            for (int e = 0; e < d; ++e)
                out[i * d + e] += pr * v[j * d + e];
        }
    }
    free(logit);
}

/* ---------------------------------------------------------------- O8 ---- */
/* Backward of O4+O5 for a fixed membership.  The scatter-add hands every
 * membership the token's full output gradient; inside a cluster the softmax
 * backward is dl = P .* (dP - rowsum(P .* dP)).  Gradients accumulate into
 * dqhat, dkhat, dv (token order, caller-zeroed) in ascending centroid order. */
void orc_attend_bwd(const double *qhat, const double *khat, const double *v, const int32_t *idx,
                    const double *dout, long n, int d, int k, long w, double scale, int causal,
                    double *dqhat, double *dkhat, double *dv)
{
    (void)n;
    double *P = (double *)malloc(sizeof(double) * (size_t)w * (size_t)w);
    double *dP = (double *)malloc(sizeof(double) * (size_t)w * (size_t)w);
    for (int c = 0; c < k; ++c) {
        const int32_t *p = idx + (long)c * w;
        /* recompute the softmax rows */
        for (long r = 0; r < w; ++r) {
            double m = -INFINITY;
            for (long s = 0; s < w; ++s) {
                P[r * w + s] = -INFINITY;
                if (causal && p[s] > p[r])
                    continue;
                double dot = 0.0;
                for (int i = 0; i < d; ++i)
                    dot += qhat[(long)p[r] * d + i] * khat[(long)p[s] * d + i];
                P[r * w + s] = scale * dot;
                if (P[r * w + s] > m)
                    m = P[r * w + s];
            }
            double z = 0.0;
            for (long s = 0; s < w; ++s)
                if (P[r * w + s] != -INFINITY)
                    z += exp(P[r * w + s] - m);
            for (long s = 0; s < w; ++s)
                P[r * w + s] = (P[r * w + s] == -INFINITY) ? 0.0 : exp(P[r * w + s] - m) / z;
        }
        /* dV and dP */
        for (long r = 0; r < w; ++r) {
            const double *g = dout + (long)p[r] * d;
            for (long s = 0; s < w; ++s) {
                double pr = P[r * w + s];
                double acc = 0.0;
                for (int i = 0; i < d; ++i) {
                    dv[(long)p[s] * d + i] += pr * g[i];
                    acc += g[i] * v[(long)p[s] * d + i];
                }
                dP[r * w + s] = acc;
            }
        }
        /* softmax backward and the two logit gradients */
        for (long r = 0; r < w; ++r) {
            double D = 0.0;
            for (long s = 0; s < w; ++s)
                D += P[r * w + s] * dP[r * w + s];
            for (long s = 0; s < w; ++s) {
                double dl = P[r * w + s] * (dP[r * w + s] - D);
                if (dl == 0.0)
                    continue;
                for (int i = 0; i < d; ++i) {
                    dqhat[(long)p[r] * d + i] += scale * dl * khat[(long)p[s] * d + i];
                    dkhat[(long)p[s] * d + i] += scale * dl * qhat[(long)p[r] * d + i];
                }
            }
        }
    }
    free(P);
    free(dP);
}

/* ---------------------------------------------------------------- O9 ---- */
/* Backward of O7 for the output gradients dout: with P the softmax row of
 * query i over its window, dV[j] += P[i][j] dO[i], dP[i][j] = <dO[i], v[j]>,
 * dl[i][j] = P[i][j] (dP[i][j] - sum_j' P[i][j'] dP[i][j']), and the logit
 * gradient goes back through the scaled product: dQ[i] += scale dl k[j],
 * dK[j] += scale dl q[i].  Outputs are zeroed here. */
void orc_local_bwd(const double *q, const double *kk, const double *v, const double *dout, long n,
                   int d, long window, double scale, int causal, double *dq, double *dk, double *dv)
{
    memset(dq, 0, sizeof(double) * (size_t)n * (size_t)d);
    memset(dk, 0, sizeof(double) * (size_t)n * (size_t)d);
    memset(dv, 0, sizeof(double) * (size_t)n * (size_t)d);
    double *P = (double *)malloc(sizeof(double) * (size_t)(2 * window + 1));
    double *dP = (double *)malloc(sizeof(double) * (size_t)(2 * window + 1));
    for (long i = 0; i < n; ++i) {
        long lo = i - window + 1;
        if (lo < 0)
            lo = 0;
        long hi = causal ? i : i + window - 1;
        if (hi > n - 1)
            hi = n - 1;
        double m = -INFINITY;
        for (long j = lo; j <= hi; ++j) {
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += q[i * d + e] * kk[j * d + e];
            P[j - lo] = scale * dot;
            if (P[j - lo] > m)
                m = P[j - lo];
        }
        double z = 0.0;
        for (long j = lo; j <= hi; ++j)
            z += exp(P[j - lo] - m);
        double D = 0.0;
        for (long j = lo; j <= hi; ++j) {
            P[j - lo] = exp(P[j - lo] - m) / z;
            double dot = 0.0;
            for (int e = 0; e < d; ++e) {
                dot += dout[i * d + e] * v[j * d + e];
                dv[j * d + e] += P[j - lo] * dout[i * d + e];
            }
            dP[j - lo] = dot;
            D += P[j - lo] * dot;
        }
        for (long j = lo; j <= hi; ++j) {
            double dl = P[j - lo] * (dP[j - lo] - D);
            for (int e = 0; e < d; ++e) {
                dq[i * d + e] += scale * dl * kk[j * d + e];
                dk[j * d + e] += scale * dl * q[i * d + e];
            }
        }
    }
    free(P);
    free(dP);
}

/* --------------------------------------------------------------- O10 ---- */
/* Blocked local attention: position i, in block b = i / block, attends to the
 * positions of blocks b - lookback .. b that are not later than i. */
void orc_local_blocked(const double *q, const double *kk, const double *v, long n, int d,
                       long block, long lookback, double scale, double *out)
{
    double *logit = (double *)malloc(sizeof(double) * (size_t)((lookback + 1) * block));
    for (long i = 0; i < n; ++i) {
        long lo = (i / block - lookback) * block;
        if (lo < 0)
            lo = 0;
        double m = -INFINITY;
        for (long j = lo; j <= i; ++j) {
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += q[i * d + e] * kk[j * d + e];
            logit[j - lo] = scale * dot;
            if (logit[j - lo] > m)
                m = logit[j - lo];
        }
        double z = 0.0;
        for (long j = lo; j <= i; ++j)
            z += exp(logit[j - lo] - m);
        for (int e = 0; e < d; ++e)
            out[i * d + e] = 0.0;
        for (long j = lo; j <= i; ++j) {
            double pr = exp(logit[j - lo] - m) / z;
            for (int e = 0; e < d; ++e)
                out[i * d + e] += pr * v[j * d + e];
        }
    }
    free(logit);
}

/* --------------------------------------------------------------- O11 ---- */
/* Nearest centroid of each token from the scores s[c][t]: the largest score,
 * ties to the lower centroid index.  margin[t] (nullable) is the gap to the
 * second largest score (+inf when k == 1). */
void orc_argmax(const double *s, long n, int k, int32_t *label, double *margin)
{
    for (long t = 0; t < n; ++t) {
        int best = 0;
        double b1 = s[t], b2 = -INFINITY;
        for (int c = 1; c < k; ++c) {
            double x = s[(long)c * n + t];
            if (x > b1) {
                b2 = b1;
                b1 = x;
                best = c;
            } else if (x > b2) {
                b2 = x;
            }
        }
        label[t] = best;
        if (margin)
            margin[t] = b1 - b2;
    }
}

/* acc[label[t]][*] += xhat[t][*] in ascending t. */
void orc_label_sums(const double *xhat, const int32_t *label, long n, int d, double *acc)
{
    for (long t = 0; t < n; ++t)
        for (int i = 0; i < d; ++i)
            acc[(long)label[t] * d + i] += xhat[t * d + i];
}

/* --------------------------------------------------------------- O12 ---- */
typedef struct {
    int c;
    double s;
    long t;
} labelled_t;

/* lower centroid first; then larger score; then lower position */
static int by_label_score_pos(const void *a, const void *b)
{
    const labelled_t *x = (const labelled_t *)a, *y = (const labelled_t *)b;
    if (x->c != y->c) return (x->c < y->c) ? -1 : 1;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->t < y->t) ? -1 : (x->t > y->t);
}

/* Partition-style balanced clusters of w = n / k tokens (n a multiple of k):
 * idx[c][*] are the tokens at ranks c*w .. c*w + w - 1 of the order above,
 * listed by ascending position. */
void orc_partition(const double *s, long n, int k, int32_t *idx)
{
    long w = n / k;
    labelled_t *buf = (labelled_t *)malloc(sizeof(labelled_t) * (size_t)n);
    int32_t *label = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    orc_argmax(s, n, k, label, NULL);
    for (long t = 0; t < n; ++t) {
        buf[t].c = label[t];
        buf[t].s = s[(long)label[t] * n + t];
        buf[t].t = t;
    }
    qsort(buf, (size_t)n, sizeof(labelled_t), by_label_score_pos);
    for (int c = 0; c < k; ++c) {
        for (long r = 0; r < w; ++r)
            idx[(long)c * w + r] = (int32_t)buf[(long)c * w + r].t;
        qsort(idx + (long)c * w, (size_t)w, sizeof(int32_t), by_int);
    }
    free(buf);
    free(label);
}

/* ------------------------------------------------ whole-tensor drivers ---- */
/* Tensors are contiguous row-major [B][H][n][d] (qk, v, out), [H][k][d] (mu),
 * [B][H][n] (inv_norm), [B][H][k][w] (idx, lse), [B][H][k] (margin),
 * [B][H][k][n] (scores).  Units (b, h) are independent and go to threads. */

typedef struct {
    void (*fn)(void *arg, long unit);
    void *arg;
    long units;
    int nthreads;
    int tid;
} job_t;

static void *job_main(void *p)
{
    job_t *j = (job_t *)p;
    for (long u = j->tid; u < j->units; u += j->nthreads)
        j->fn(j->arg, u);
    return NULL;
}

static void parallel_units(void (*fn)(void *, long), void *arg, long units, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > units)
        nthreads = (int)units;
    if (nthreads <= 1) {
        for (long u = 0; u < units; ++u)
            fn(arg, u);
        return;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) {
        jobs[i].fn = fn;
        jobs[i].arg = arg;
        jobs[i].units = units;
        jobs[i].nthreads = nthreads;
        jobs[i].tid = i;
        pthread_create(&th[i], NULL, job_main, &jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i)
        pthread_join(th[i], NULL);
    free(th);
    free(jobs);
}

typedef struct {
    const double *qk, *mu;
    int H, d, k;
    long n, w;
    double *inv_norm, *margin, *scores;
    int32_t *idx;
} route_args;

static void route_unit(void *p, long u)
{
    route_args *a = (route_args *)p;
    long n = a->n;
    int d = a->d, k = a->k, h = (int)(u % a->H);
    double *xhat = (double *)malloc(sizeof(double) * (size_t)n * (size_t)d);
    double *s = (double *)malloc(sizeof(double) * (size_t)k * (size_t)n);
    orc_normalize(a->qk + u * n * d, n, d, xhat, a->inv_norm + u * n);
    orc_scores(xhat, a->mu + (long)h * k * d, n, d, k, s);
    orc_select(s, n, k, a->w, a->idx + u * k * a->w, a->margin ? a->margin + u * k : NULL);
    if (a->scores)
        memcpy(a->scores + u * k * n, s, sizeof(double) * (size_t)k * (size_t)n);
    free(xhat);
    free(s);
}

/* O1-O3 for every (b, h). */
void orc_route_all(const double *qk, const double *mu, int B, int H, long n, int d, int k, long w,
                   double *inv_norm, int32_t *idx, double *margin, double *scores, int nthreads)
{
    route_args a = {qk, mu, H, d, k, n, w, inv_norm, margin, scores, idx};
    parallel_units(route_unit, &a, (long)B * H, nthreads);
}

typedef struct {
    const double *q, *kk, *v;
    const int32_t *idx;
    int d, k, causal, normalize;
    long n, w;
    double scale;
    double *out, *lse, *o_clusters;
} attn_args;

static void attn_unit(void *p, long u)
{
    attn_args *a = (attn_args *)p;
    long n = a->n, w = a->w;
    int d = a->d, k = a->k;
    const double *q = a->q + u * n * d, *kk = a->kk + u * n * d;
    double *qhat = (double *)malloc(sizeof(double) * (size_t)n * (size_t)d);
    double *khat = (double *)malloc(sizeof(double) * (size_t)n * (size_t)d);
    double *o = a->o_clusters ? a->o_clusters + u * k * w * d
                              : (double *)malloc(sizeof(double) * (size_t)k * (size_t)w * (size_t)d);
    if (a->normalize) {
        orc_normalize(q, n, d, qhat, NULL);
        orc_normalize(kk, n, d, khat, NULL);
    } else {
        memcpy(qhat, q, sizeof(double) * (size_t)n * (size_t)d);
        memcpy(khat, kk, sizeof(double) * (size_t)n * (size_t)d);
    }
    orc_attend(qhat, khat, a->v + u * n * d, a->idx + u * k * w, n, d, k, w, a->scale, a->causal, o,
               a->lse ? a->lse + u * k * w : NULL);
    orc_scatter(o, a->idx + u * k * w, n, d, k, w, a->out + u * n * d);
    if (!a->o_clusters)
        free(o);
    free(qhat);
    free(khat);
}

/* O1 (when normalize != 0), O4, O5 for every (b, h) with the given membership.
 * o_clusters (nullable, [B][H][k][w][d]) receives the per-cluster rows. */
void orc_routed_attn_all(const double *q, const double *kk, const double *v, const int32_t *idx,
                         int B, int H, long n, int d, int k, long w, double scale, int causal,
                         int normalize, double *out, double *lse, double *o_clusters, int nthreads)
{
    attn_args a = {q, kk, v, idx, d, k, causal, normalize, n, w, scale, out, lse, o_clusters};
    parallel_units(attn_unit, &a, (long)B * H, nthreads);
}

/* O1 + O6: one EMA step of every head's centroids, with the members of all
 * batch rows (b ascending) contributing.  mu [H][k][d] is updated in place. */
void orc_centroid_update_all(double *mu, const double *q, const double *kk, const int32_t *idx,
                             int B, int H, long n, int d, int k, long w, double lam)
{
    double *xhat = (double *)malloc(sizeof(double) * (size_t)n * (size_t)d);
    double *sq = (double *)malloc(sizeof(double) * (size_t)k * (size_t)d);
    double *sk = (double *)malloc(sizeof(double) * (size_t)k * (size_t)d);
    for (int h = 0; h < H; ++h) {
        memset(sq, 0, sizeof(double) * (size_t)k * (size_t)d);
        memset(sk, 0, sizeof(double) * (size_t)k * (size_t)d);
        for (int b = 0; b < B; ++b) {
            long u = (long)b * H + h;
            orc_normalize(q + u * n * d, n, d, xhat, NULL);
            orc_cluster_sums(xhat, idx + u * k * w, n, d, k, w, sq);
            orc_normalize(kk + u * n * d, n, d, xhat, NULL);
            orc_cluster_sums(xhat, idx + u * k * w, n, d, k, w, sk);
        }
        orc_ema(mu + (long)h * k * d, sq, sk, k, d, lam);
    }
    free(xhat);
    free(sq);
    free(sk);
}

typedef struct {
    const double *q, *kk, *v;
    long n, window;
    int d, causal;
    double scale;
    double *out;
} local_args;

static void local_unit(void *p, long u)
{
    local_args *a = (local_args *)p;
    long off = u * a->n * a->d;
    orc_local(a->q + off, a->kk + off, a->v + off, a->n, a->d, a->window, a->scale, a->causal,
              a->out + off);
}

/* O7 for every (b, h). */
void orc_local_attn_all(const double *q, const double *kk, const double *v, int B, int H, long n,
                        int d, long window, double scale, int causal, double *out, int nthreads)
{
    local_args a = {q, kk, v, n, window, d, causal, scale, out};
    parallel_units(local_unit, &a, (long)B * H, nthreads);
}

typedef struct {
    const double *q, *kk, *v, *dout;
    const int32_t *idx;
    long n, w;
    int d, k, causal;
    double scale;
    double *dq, *dk, *dv;
} bwd_args;

static void bwd_unit(void *p, long u)
{
    bwd_args *a = (bwd_args *)p;
    long n = a->n, w = a->w;
    int d = a->d, k = a->k;
    long off = u * n * d;
    double *qhat = (double *)malloc(sizeof(double) * (size_t)n * (size_t)d);
    double *khat = (double *)malloc(sizeof(double) * (size_t)n * (size_t)d);
    orc_normalize(a->q + off, n, d, qhat, NULL);
    orc_normalize(a->kk + off, n, d, khat, NULL);
    memset(a->dq + off, 0, sizeof(double) * (size_t)n * (size_t)d);
    memset(a->dk + off, 0, sizeof(double) * (size_t)n * (size_t)d);
    memset(a->dv + off, 0, sizeof(double) * (size_t)n * (size_t)d);
    orc_attend_bwd(qhat, khat, a->v + off, a->idx + u * k * w, a->dout + off, n, d, k, w,
                   a->scale, a->causal, a->dq + off, a->dk + off, a->dv + off);
    free(qhat);
    free(khat);
}

/* O1 + O8 for every (b, h): gradients w.r.t. the normalised q^, k^ and v. */
void orc_routed_attn_bwd_all(const double *q, const double *kk, const double *v, const int32_t *idx,
                             const double *dout, int B, int H, long n, int d, int k, long w,
                             double scale, int causal, double *dq, double *dk, double *dv,
                             int nthreads)
{
    bwd_args a = {q, kk, v, dout, idx, n, w, d, k, causal, scale, dq, dk, dv};
    parallel_units(bwd_unit, &a, (long)B * H, nthreads);
}

typedef struct {
    const double *q, *kk, *v, *dout;
    long n, window;
    int d, causal;
    double scale;
    double *dq, *dk, *dv;
} local_bwd_args;

static void local_bwd_unit(void *p, long u)
{
    local_bwd_args *a = (local_bwd_args *)p;
    long off = u * a->n * a->d;
    orc_local_bwd(a->q + off, a->kk + off, a->v + off, a->dout + off, a->n, a->d, a->window,
                  a->scale, a->causal, a->dq + off, a->dk + off, a->dv + off);
}

/* O9 for every (b, h). */
void orc_local_attn_bwd_all(const double *q, const double *kk, const double *v, const double *dout,
                            int B, int H, long n, int d, long window, double scale, int causal,
                            double *dq, double *dk, double *dv, int nthreads)
{
    local_bwd_args a = {q, kk, v, dout, n, window, d, causal, scale, dq, dk, dv};
    parallel_units(local_bwd_unit, &a, (long)B * H, nthreads);
}

typedef struct {
    const double *q, *kk, *v;
    long n, block, lookback;
    int d;
    double scale;
    double *out;
} blocked_args;

static void blocked_unit(void *p, long u)
{
    blocked_args *a = (blocked_args *)p;
    long off = u * a->n * a->d;
    orc_local_blocked(a->q + off, a->kk + off, a->v + off, a->n, a->d, a->block, a->lookback,
                      a->scale, a->out + off);
}

/* O10 for every (b, h). */
void orc_local_blocked_all(const double *q, const double *kk, const double *v, int B, int H,
                           long n, int d, long block, long lookback, double scale, double *out,
                           int nthreads)
{
    blocked_args a = {q, kk, v, n, block, lookback, d, scale, out};
    parallel_units(blocked_unit, &a, (long)B * H, nthreads);
}

/* O1 + O2 + O11 for every (b, h): labels [B][H][n] and margins [B][H][n]. */
void orc_argmax_all(const double *x, const double *mu, int B, int H, long n, int d, int k,
                    int32_t *label, double *margin)
{
    double *xhat = (double *)malloc(sizeof(double) * (size_t)n * (size_t)d);
    double *s = (double *)malloc(sizeof(double) * (size_t)k * (size_t)n);
    for (long u = 0; u < (long)B * H; ++u) {
        int h = (int)(u % H);
        orc_normalize(x + u * n * d, n, d, xhat, NULL);
        orc_scores(xhat, mu + (long)h * k * d, n, d, k, s);
        orc_argmax(s, n, k, label + u * n, margin ? margin + u * n : NULL);
    }
    free(xhat);
    free(s);
}

/* O1 + O11: one EMA step of every head's centroids with each query and each
 * key counted for its own nearest centroid (batch rows in ascending order).
 * mu [H][k][d] is updated in place. */
void orc_centroid_update_argmax_all(double *mu, const double *q, const double *kk, int B, int H,
                                    long n, int d, int k, double lam)
{
    double *xhat = (double *)malloc(sizeof(double) * (size_t)n * (size_t)d);
    double *s = (double *)malloc(sizeof(double) * (size_t)k * (size_t)n);
    int32_t *label = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    double *sq = (double *)malloc(sizeof(double) * (size_t)k * (size_t)d);
    double *sk = (double *)malloc(sizeof(double) * (size_t)k * (size_t)d);
    for (int h = 0; h < H; ++h) {
        const double *muh = mu + (long)h * k * d;
        memset(sq, 0, sizeof(double) * (size_t)k * (size_t)d);
        memset(sk, 0, sizeof(double) * (size_t)k * (size_t)d);
        for (int b = 0; b < B; ++b) {
            long u = (long)b * H + h;
            orc_normalize(q + u * n * d, n, d, xhat, NULL);
            orc_scores(xhat, muh, n, d, k, s);
            orc_argmax(s, n, k, label, NULL);
            orc_label_sums(xhat, label, n, d, sq);
            orc_normalize(kk + u * n * d, n, d, xhat, NULL);
            orc_scores(xhat, muh, n, d, k, s);
            orc_argmax(s, n, k, label, NULL);
            orc_label_sums(xhat, label, n, d, sk);
        }
        orc_ema(mu + (long)h * k * d, sq, sk, k, d, lam);
    }
    free(xhat);
    free(s);
    free(label);
    free(sq);
    free(sk);
}

/* O1 + O2 + O12 for every (b, h): idx [B][H][k][n/k]. */
void orc_route_partition_all(const double *x, const double *mu, int B, int H, long n, int d,
                             int k, int32_t *idx)
{
    double *xhat = (double *)malloc(sizeof(double) * (size_t)n * (size_t)d);
    double *s = (double *)malloc(sizeof(double) * (size_t)k * (size_t)n);
    for (long u = 0; u < (long)B * H; ++u) {
        int h = (int)(u % H);
        orc_normalize(x + u * n * d, n, d, xhat, NULL);
        orc_scores(xhat, mu + (long)h * k * d, n, d, k, s);
        orc_partition(s, n, k, idx + u * n);
    }
    free(xhat);
    free(s);
}
