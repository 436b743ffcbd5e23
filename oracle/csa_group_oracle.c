/*
 * csa_group_oracle.c -- plain CPU oracle for the grouped (approximate)
 * indexer: the query-group shared scan of the PIVOT news item
 * (themodelwire, "PIVOT reduces sparse attention indexing bottleneck":
 * nearby queries share one scan of their common prefix, then each refines
 * the shared result).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * The item gives no formula; the reading implemented here, step by step:
 *   groups     q rows 0..S-1 in groups of g consecutive rows; row i is
 *              position t = row_offset + i; group r holds rows r*g ..
 *              min(S, r*g+g) - 1, its first member t0 = row_offset + r*g.
 *   pooling    per head j and dimension x the pooled query is the mean of
 *              the members' values, formed in binary32: a binary32 sum in
 *              member order divided by the member count in binary32, then
 *              rounded to bfloat16 (nearest, ties to the even significand);
 *              the pooled weight of head j is the binary32 mean of the
 *              members' weights, formed the same way (not rounded further).
 *   shared     the pooled query's indexer score of every key s visible to
 *   scan       the first member (s < n_vis(t0)), in double from the
 *              decoded values, and the C best of them by (score desc,
 *              key asc).
 *   re-rank    for each member t: its own exact score (the plain
 *              definition) of every shared candidate and of every key
 *              n_vis(t0) <= s < n_vis(t); the top-k of those by (score
 *              desc, key asc), padded with (-1, -inf).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t bits)
{
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* Round a finite binary32 value to bfloat16, nearest, ties to even: the two
 * bfloat16 neighbours are the value truncated to its top 16 bits and the
 * next one away from zero; pick the closer, on a tie the one whose last
 * significand bit is 0. */
static double round_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lo = u & 0xFFFF0000u;
    uint32_t hi = lo + 0x10000u;
    float flo, fhi;
    memcpy(&flo, &lo, sizeof flo);
    memcpy(&fhi, &hi, sizeof fhi);
    double dlo = fabs((double)f - (double)flo), dhi = fabs((double)fhi - (double)f);
    if (dlo < dhi) return (double)flo;
    if (dhi < dlo) return (double)fhi;
    return ((lo >> 16) & 1u) ? (double)fhi : (double)flo;
}

static int64_t n_vis(int64_t t, int64_t T, int m)
{
    int64_t n = (t + 1) / m;
    if (n < 0) n = 0;
    return n < T ? n : T;
}

typedef struct {
    double score;
    int32_t idx;
} gentry;

static int cmp_gentry(const void *pa, const void *pb)
{
    const gentry *a = (const gentry *)pa, *b = (const gentry *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

typedef struct {
    const uint16_t *q;   /* [S, H, D] bf16 bits, one batch entry */
    const float *w;      /* [S, H] */
    const double *kd;    /* [T, D] decoded keys */
    int64_t S, T, row_offset;
    int H, D, m, topk, g, C;
    const int64_t *rows; /* requested rows */
    int64_t nrows;
    int32_t *out_idx;    /* [nrows, topk] */
    double *out_score;   /* [nrows, topk] */
} gproblem;

/* sum over heads of w * max(0, q . k) in double */
static double indexer_score(const double *qd, const double *wd, const double *kd, int H, int D)
{
    double total = 0.0;
    for (int j = 0; j < H; j++) {
        double dot = 0.0;
        for (int x = 0; x < D; x++) dot += qd[j * D + x] * kd[x];
        total += wd[j] * (dot > 0.0 ? dot : 0.0);
    }
    return total;
}

/*
 * The pooled query of the group holding row i: pq [H, D] (bfloat16 values
 * as doubles) and pw [H].  Returns the group's first row.
 */
int64_t csa_oracle_group_pool(const uint16_t *q, const float *w, int64_t S, int H, int D, int g,
                              int64_t i, double *pq, double *pw)
{
    const int64_t i0 = (i / g) * g;
    const int64_t n_mem = (S - i0) < g ? (S - i0) : g;
    for (int j = 0; j < H; j++) {
        for (int x = 0; x < D; x++) {
            float acc = 0.0f;
            for (int64_t u = 0; u < n_mem; u++)
                acc = acc + (float)bf16_value(q[((i0 + u) * H + j) * D + x]);
            pq[j * D + x] = round_bf16(acc / (float)n_mem);
        }
        float accw = 0.0f;
        for (int64_t u = 0; u < n_mem; u++) accw = accw + w[(i0 + u) * H + j];
        pw[j] = (double)(accw / (float)n_mem);
    }
    return i0;
}

static void solve_group_row(const gproblem *p, int64_t ri, double *pq, double *pw, double *qd,
                            double *wd, gentry *buf)
{
    const int64_t i = p->rows[ri];
    const int H = p->H, D = p->D;
    const int64_t i0 = csa_oracle_group_pool(p->q, p->w, p->S, H, D, p->g, i, pq, pw);
    /* shared scan over the first member's visible keys */
    const int64_t n0 = n_vis(p->row_offset + i0, p->T, p->m);
    for (int64_t s = 0; s < n0; s++) {
        buf[s].score = indexer_score(pq, pw, p->kd + s * D, H, D);
        buf[s].idx = (int32_t)s;
    }
    qsort(buf, (size_t)n0, sizeof(gentry), cmp_gentry);
    const int64_t nc = n0 < p->C ? n0 : p->C;
    /* re-rank with the member's own query: candidates, then its extra keys */
    for (int j = 0; j < H; j++) {
        for (int x = 0; x < D; x++) qd[j * D + x] = bf16_value(p->q[(i * H + j) * D + x]);
        wd[j] = (double)p->w[i * H + j];
    }
    const int64_t nt = n_vis(p->row_offset + i, p->T, p->m);
    int64_t n = 0;
    for (int64_t c = 0; c < nc; c++) {
        const int32_t s = buf[c].idx;
        buf[n].idx = s;
        buf[n].score = indexer_score(qd, wd, p->kd + (int64_t)s * D, H, D);
        n++;
    }
    for (int64_t s = n0; s < nt; s++) {
        buf[n].idx = (int32_t)s;
        buf[n].score = indexer_score(qd, wd, p->kd + s * D, H, D);
        n++;
    }
    qsort(buf, (size_t)n, sizeof(gentry), cmp_gentry);
    for (int e = 0; e < p->topk; e++) {
        const int64_t o = ri * p->topk + e;
        if (e < n) {
            p->out_idx[o] = buf[e].idx;
            p->out_score[o] = buf[e].score;
        } else {
            p->out_idx[o] = -1;
            p->out_score[o] = -INFINITY;
        }
    }
}

typedef struct {
    const gproblem *p;
    int64_t first, stride;
    int status;
} gjob;

static void *run_gjob(void *arg)
{
    gjob *jb = (gjob *)arg;
    const gproblem *p = jb->p;
    const size_t hd = (size_t)p->H * p->D;
    double *pq = (double *)malloc(hd * sizeof(double));
    double *qd = (double *)malloc(hd * sizeof(double));
    double *pw = (double *)malloc((size_t)p->H * sizeof(double));
    double *wd = (double *)malloc((size_t)p->H * sizeof(double));
    gentry *buf = (gentry *)malloc((size_t)(p->T + p->C + 1) * sizeof(gentry));
    jb->status = (pq && qd && pw && wd && buf) ? 0 : -1;
    if (jb->status == 0)
        for (int64_t ri = jb->first; ri < p->nrows; ri += jb->stride)
            solve_group_row(p, ri, pq, pw, qd, wd, buf);
    free(pq);
    free(qd);
    free(pw);
    free(wd);
    free(buf);
    return NULL;
}

/*
 * Grouped top-k of the requested rows of one batch entry.  q [S, H, D] bf16
 * bits, w [S, H], k [T, D] bf16 bits hold the whole entry (pooling reads
 * every member of a row's group).  Returns 0, or -1 on bad arguments or
 * allocation failure.
 */
int csa_oracle_grouped(const uint16_t *q, const float *w, const uint16_t *k, int64_t S,
                       int64_t T, int H, int D, int m, int topk, int g, int C,
                       int64_t row_offset, const int64_t *rows, int64_t nrows, int nthreads,
                       int32_t *out_idx, double *out_score)
{
    if (!q || !w || !k || !rows || !out_idx || !out_score) return -1;
    if (S < 0 || T < 0 || H < 1 || D < 1 || m < 1 || topk < 1 || g < 1 || C < 1 ||
        row_offset < 0)
        return -1;
    for (int64_t ri = 0; ri < nrows; ri++)
        if (rows[ri] < 0 || rows[ri] >= S) return -1;
    double *kd = (double *)malloc((size_t)(T > 0 ? T : 1) * D * sizeof(double));
    if (!kd) return -1;
    for (int64_t e = 0; e < T * D; e++) kd[e] = bf16_value(k[e]);
    gproblem p = {q, w, kd, S, T, row_offset, H, D, m, topk, g, C, rows, nrows,
                  out_idx, out_score};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    gjob *jobs = (gjob *)calloc((size_t)nthreads, sizeof(gjob));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    int status = 0;
    if (!jobs || !th) {
        status = -1;
    } else {
        for (int t = 0; t < nthreads; t++) {
            jobs[t].p = &p;
            jobs[t].first = t;
            jobs[t].stride = nthreads;
            if (pthread_create(&th[t], NULL, run_gjob, &jobs[t]) != 0) {
                run_gjob(&jobs[t]);
                th[t] = 0;
            }
        }
        for (int t = 0; t < nthreads; t++) {
            if (th[t]) pthread_join(th[t], NULL);
            if (jobs[t].status != 0) status = -1;
        }
    }
    free(jobs);
    free(th);
    free(kd);
    return status;
}
