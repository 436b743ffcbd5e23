/*
 * csa_attn_oracle.c -- plain CPU oracle for sparse attention over the keys
 * the lightning indexer selected.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code with the HIP
 * library.
 *
 * What it computes (StreamIndex: Memory-Bounded Compressed Sparse Attention
 * via Streaming Top-k, Abstract: after the indexer picks each query's keys,
 * an attention kernel reads only those keys).  The pages give no formula for
 * that attention; the reading used here is ordinary softmax attention
 * restricted to the selected compressed entries, with one key row and one
 * value row per compressed entry shared by all query heads:
 *
 *     for query row r (batch b) and head h, let E(r) be the entries e of the
 *     row's index list with 0 <= idx[r, e] < T (others are padding);
 *     z_e   = scale * (q[r, h, :] . k[idx[r, e], :])
 *     M     = max_e z_e,   p_e = exp(z_e - M),   L = sum_e p_e
 *     o[r, h, :] = sum_e p_e * v[idx[r, e], :] / L
 *     lse[r, h]  = M + log(L)
 *
 * Every list entry counts once (the indexer never repeats a key).  A row
 * with no valid entry has o = 0 and lse = -infinity.
 *
 * The oracle also returns a[r, h, x] = sum_e (p_e / L) * |v[idx[r, e], x]|,
 * the weighted magnitude that bounds how far a result computed with rounded
 * weights may stray from o.
 *
 * Arithmetic: bf16 inputs are decoded exactly to double; every sum is a
 * plain loop in double, in list order.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

double csa_oracle_decode_bf16(uint16_t bits);

typedef struct {
    const uint16_t *q;    /* [n, H, D] bf16 bits, the requested rows */
    const uint16_t *k;    /* [T, D] bf16 bits */
    const uint16_t *v;    /* [T, D] bf16 bits */
    const int32_t *idx;   /* [n, L] */
    int64_t n, T;
    int H, D, L;
    double scale;
    double *o, *lse, *a;  /* [n, H, D], [n, H], [n, H, D] (a may be NULL) */
    double *kd, *vd;      /* decoded k and v, [T, D] */
} attn_problem;

static void attend_row(const attn_problem *p, int64_t r, double *z, double *qd)
{
    const int32_t *list = p->idx + r * p->L;
    for (int h = 0; h < p->H; h++) {
        for (int x = 0; x < p->D; x++)
            qd[x] = csa_oracle_decode_bf16(p->q[(r * p->H + h) * p->D + x]);
        double *o = p->o + (r * p->H + h) * p->D;
        double *a = p->a ? p->a + (r * p->H + h) * p->D : NULL;
        for (int x = 0; x < p->D; x++) {
            o[x] = 0.0;
            if (a) a[x] = 0.0;
        }
        /* scores of the valid entries, and their maximum */
        double M = -INFINITY;
        int any = 0;
        for (int e = 0; e < p->L; e++) {
            const int64_t s = list[e];
            if (s < 0 || s >= p->T) continue;
            double dot = 0.0;
            for (int x = 0; x < p->D; x++) dot += qd[x] * p->kd[s * p->D + x];
            z[e] = p->scale * dot;
            if (!any || z[e] > M) M = z[e];
            any = 1;
        }
        if (!any) {
            p->lse[r * p->H + h] = -INFINITY;
            continue;
        }
        double L = 0.0;
        for (int e = 0; e < p->L; e++) {
            const int64_t s = list[e];
            if (s < 0 || s >= p->T) continue;
            const double pe = exp(z[e] - M);
            L += pe;
            for (int x = 0; x < p->D; x++) {
                o[x] += pe * p->vd[s * p->D + x];
                if (a) a[x] += pe * fabs(p->vd[s * p->D + x]);
            }
        }
        for (int x = 0; x < p->D; x++) {
            o[x] /= L;
            if (a) a[x] /= L;
        }
        p->lse[r * p->H + h] = M + log(L);
    }
}

typedef struct {
    const attn_problem *p;
    int64_t first, stride;
    int status;
} attn_job;

static void *attn_run(void *arg)
{
    attn_job *jb = (attn_job *)arg;
    const attn_problem *p = jb->p;
    double *z = (double *)malloc((size_t)(p->L > 0 ? p->L : 1) * sizeof(double));
    double *qd = (double *)malloc((size_t)p->D * sizeof(double));
    if (!z || !qd) {
        free(z);
        free(qd);
        jb->status = -1;
        return NULL;
    }
    for (int64_t r = jb->first; r < p->n; r += jb->stride)
        attend_row(p, r, z, qd);
    free(z);
    free(qd);
    jb->status = 0;
    return NULL;
}

/*
 * Sparse attention for `n` query rows.  q holds only those rows; idx holds
 * their L-entry index lists; k and v hold the batch entry's T compressed
 * rows.  Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int csa_oracle_sparse_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const int32_t *idx, int64_t n, int64_t T, int H, int D,
                                int L, double scale, int nthreads, double *out_o,
                                double *out_lse, double *out_a)
{
    if (!q || !idx || !out_o || !out_lse || (T > 0 && (!k || !v))) return -1;
    if (n < 0 || T < 0 || H < 1 || D < 1 || L < 0) return -1;
    double *kd = (double *)malloc((size_t)(T > 0 ? T : 1) * D * sizeof(double));
    double *vd = (double *)malloc((size_t)(T > 0 ? T : 1) * D * sizeof(double));
    if (!kd || !vd) {
        free(kd);
        free(vd);
        return -1;
    }
    for (int64_t i = 0; i < T * D; i++) {
        kd[i] = csa_oracle_decode_bf16(k[i]);
        vd[i] = csa_oracle_decode_bf16(v[i]);
    }
    attn_problem p = {q, k, v, idx, n, T, H, D, L, scale, out_o, out_lse, out_a, kd, vd};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n) nthreads = n > 0 ? (int)n : 1;
    attn_job *jobs = (attn_job *)calloc((size_t)nthreads, sizeof(attn_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        free(kd);
        free(vd);
        return -1;
    }
    int status = 0;
    for (int i = 0; i < nthreads; i++) {
        jobs[i].p = &p;
        jobs[i].first = i;
        jobs[i].stride = nthreads;
        if (pthread_create(&th[i], NULL, attn_run, &jobs[i]) != 0) {
            attn_run(&jobs[i]);
            th[i] = 0;
        }
    }
    for (int i = 0; i < nthreads; i++) {
        if (th[i]) pthread_join(th[i], NULL);
        if (jobs[i].status != 0) status = -1;
    }
    free(jobs);
    free(th);
    free(kd);
    free(vd);
    return status;
}
