/*
 * MSA forward oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU implementation of what the MiniMax Sparse Attention
 * (MSA) forward path computes, used to check the GPU library.  Only the
 * tests, the package's smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code with the GPU library.
 *
 * Source: "MiniMax Sparse Attention" explainer
 * (minimax-sparse-attention-danialwang.pages.dev), sections 01-05.
 *
 * Conventions
 *   - Positions are 0-based; query i sees keys j <= i (section 02: the
 *     indexer picks a subset of {1..i} in the page's 1-based numbering).
 *   - Blocks are fixed, aligned at position 0, B_k tokens each; the local
 *     block of query i is lb(i) = floor(i / B_k).
 *   - Head h belongs to GQA group r = floor(h / G), G = H_q / H_kv
 *     (section 01: G adjacent query heads share one KV head).
 *   - bf16 inputs arrive as their uint16 bit patterns and are widened
 *     exactly to double; every sum is accumulated in fp64, one term at a
 *     time, in ascending index order.
 *
 * Layouts (row-major, token-major):
 *   q_idx rows [nrows, H_kv, d_idx], k_idx [Nk, H_kv, d_idx]
 *   Q rows [nrows, H_q, d_h], K and V [Nk, H_kv, d_h]
 *   sel [nrows, H_kv, k] int32, ascending block ids, -1 padded
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------ */
/* Index Branch                                                       */
/* ------------------------------------------------------------------ */

/*
 * Block scores of one (query row, group): for every block b = 0..lb(i),
 *   P[b] = max over tokens j of block b with j <= i of  q_idx[i,r,:] . k_idx[j,r,:]
 * The token score is a plain dot product (Figure 1: the index query and
 * key produce a score); block max pooling turns token scores into block
 * scores (Figure 1 caption, "Block Max Pooling").
 */
void oracle_block_scores(const uint16_t *q_row /* [H_kv, d_idx] */,
                         const uint16_t *k_idx, int64_t i, int r, int H_kv,
                         int d_idx, int B_k, double *P /* [lb(i)+1] */)
{
    int64_t lb = i / B_k;
    for (int64_t b = 0; b <= lb; ++b) {
        double best = -INFINITY;
        for (int64_t j = b * B_k; j < (b + 1) * B_k && j <= i; ++j) {
            double s = 0.0;
            for (int d = 0; d < d_idx; ++d)
                s += widen_bf16(q_row[(int64_t)r * d_idx + d]) *
                     widen_bf16(k_idx[(j * H_kv + r) * d_idx + d]);
            if (s > best)
                best = s;
        }
        P[b] = best;
    }
}

/*
 * Block selection for one (query row, group), given its block scores.
 * The local block lb(i) is always kept and counts toward k (Figure 1
 * caption; section 03, forced local block).  The other k-1 blocks are the
 * highest-scoring earlier blocks, chosen on the raw scores with no
 * softmax: softmax preserves order, so the Top-k is the same (section 05,
 * part 1).  Ties go to the lower block index.  If fewer than k blocks are
 * visible, all of them are taken.  Output: ascending ids, -1 padded.
 */
static void select_from_scores(const double *P, int64_t lb, int k,
                               int32_t *out /* [k] */, char *taken)
{
    int n = 0;
    memset(taken, 0, (size_t)(lb + 1));
    taken[lb] = 1;
    for (int t = 0; t < k - 1; ++t) {
        int64_t best = -1;
        for (int64_t b = 0; b < lb; ++b) {
            if (taken[b])
                continue;
            if (best < 0 || P[b] > P[best])
                best = b;
        }
        if (best < 0)
            break;
        taken[best] = 1;
    }
    for (int64_t b = 0; b <= lb; ++b)
        if (taken[b])
            out[n++] = (int32_t)b;
    for (; n < k; ++n)
        out[n] = -1;
}

/* ------------------------------------------------------------------ */
/* Main Branch                                                        */
/* ------------------------------------------------------------------ */

/*
 * Exact softmax attention of one (query row, head) over the tokens of its
 * group's selected blocks, j <= i inside each block (section 02: Main
 * Branch = scaled dot-product softmax attention over the selected set;
 * section 03: the visible token set induced by the selected blocks).
 * One softmax over the union of all selected tokens.
 *   s_j = scale * Q[i,h,:] . K[j,r,:]
 *   O   = sum_j exp(s_j) V[j,r,:] / sum_j exp(s_j)
 *   lse = ln sum_j exp(s_j)          (the max is subtracted for range only)
 */
static void attend_one(const uint16_t *q_vec /* [d_h] */, const uint16_t *K,
                       const uint16_t *V, int64_t i, int r, int H_kv, int d_h,
                       int B_k, const int32_t *sel_row, int k, double scale,
                       double *s_buf, double *O /* [d_h] */, double *lse)
{
    int64_t n = 0;
    for (int t = 0; t < k; ++t) {
        int32_t b = sel_row[t];
        if (b < 0)
            continue;
        for (int64_t j = (int64_t)b * B_k; j < ((int64_t)b + 1) * B_k && j <= i; ++j) {
            double s = 0.0;
            for (int d = 0; d < d_h; ++d)
                s += widen_bf16(q_vec[d]) * widen_bf16(K[(j * H_kv + r) * d_h + d]);
            s_buf[n++] = s * scale;
        }
    }
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t)
        if (s_buf[t] > m)
            m = s_buf[t];
    double l = 0.0;
    for (int d = 0; d < d_h; ++d)
        O[d] = 0.0;
    n = 0;
    for (int t = 0; t < k; ++t) {
        int32_t b = sel_row[t];
        if (b < 0)
            continue;
        for (int64_t j = (int64_t)b * B_k; j < ((int64_t)b + 1) * B_k && j <= i; ++j) {
            double p = exp(s_buf[n++] - m);
            l += p;
            for (int d = 0; d < d_h; ++d)
                O[d] += p * widen_bf16(V[(j * H_kv + r) * d_h + d]);
        }
    }
    for (int d = 0; d < d_h; ++d)
        O[d] /= l;
    *lse = m + log(l);
}

/*
 * Index-alignment KL of one (query row, group) over the token set T of
 * its selection (section 03, "KL Loss": on the visible token set induced by
 * the selected blocks, the student is the softmax of the index scores and
 * the teacher is the mean over the group's G query heads of their Main
 * Branch attention distributions; the indexer minimises KL(teacher ||
 * student), averaged over positions and groups).
 *   teacher t_j = (1/G) sum_h softmax_T(scale * Q[i,h,:] . K[j,r,:])_j
 *   student u_j = softmax_T(q_idx[i,r,:] . k_idx[j,r,:])_j
 *   KL = sum_{j in T, t_j > 0} t_j (ln t_j - ln u_j)
 * Every softmax is taken over the whole of T at once, in fp64.
 */
static double kl_one(const uint16_t *q_row /* [d_idx] */, const uint16_t *k_idx,
                     const uint16_t *Q_heads /* [G, d_h] */, const uint16_t *K,
                     int64_t i, int r, int G, int H_kv, int d_h, int d_idx, int B_k,
                     const int32_t *sel_row, int k, double scale, double *buf /* 3*k*B_k */)
{
    double *tok = buf;                    /* token ids of T, as doubles */
    double *t = buf + (int64_t)k * B_k;   /* teacher */
    double *s = t + (int64_t)k * B_k;     /* scores, reused */
    int64_t n = 0;
    for (int u = 0; u < k; ++u) {
        int32_t b = sel_row[u];
        if (b < 0)
            continue;
        for (int64_t j = (int64_t)b * B_k; j < ((int64_t)b + 1) * B_k && j <= i; ++j)
            tok[n++] = (double)j;
    }
    for (int64_t a = 0; a < n; ++a)
        t[a] = 0.0;
    for (int g = 0; g < G; ++g) {
        const uint16_t *qv = Q_heads + (int64_t)g * d_h;
        double m = -INFINITY;
        for (int64_t a = 0; a < n; ++a) {
            int64_t j = (int64_t)tok[a];
            double dot = 0.0;
            for (int d = 0; d < d_h; ++d)
                dot += widen_bf16(qv[d]) * widen_bf16(K[(j * H_kv + r) * d_h + d]);
            s[a] = dot * scale;
            if (s[a] > m)
                m = s[a];
        }
        double z = 0.0;
        for (int64_t a = 0; a < n; ++a)
            z += exp(s[a] - m);
        for (int64_t a = 0; a < n; ++a)
            t[a] += exp(s[a] - m) / z / (double)G;
    }
    double m = -INFINITY;
    for (int64_t a = 0; a < n; ++a) {
        int64_t j = (int64_t)tok[a];
        double dot = 0.0;
        for (int d = 0; d < d_idx; ++d)
            dot += widen_bf16(q_row[d]) * widen_bf16(k_idx[(j * H_kv + r) * d_idx + d]);
        s[a] = dot;
        if (dot > m)
            m = dot;
    }
    double z = 0.0;
    for (int64_t a = 0; a < n; ++a)
        z += exp(s[a] - m);
    double lse = m + log(z);
    double kl = 0.0;
    for (int64_t a = 0; a < n; ++a)
        if (t[a] > 0.0)
            kl += t[a] * (log(t[a]) - (s[a] - lse));
    return kl;
}

/* ------------------------------------------------------------------ */
/* Threaded drivers over query rows                                   */
/* ------------------------------------------------------------------ */

typedef struct {
    /* shared */
    const uint16_t *q_rows, *k_idx, *Q_rows, *K, *V;
    const int64_t *rows;
    int64_t nrows;
    int H_q, H_kv, d_h, d_idx, B_k, k;
    double scale;
    int32_t *sel;      /* select: output; attend: input */
    double *O, *lse;
    double *kl;        /* index KL: output [nrows, H_kv] */
    int mode;          /* 0 select, 1 attend, 2 index KL */
    /* per thread */
    int tid, nthreads;
} job_t;

/* Work units are (row, group) pairs for selection and (row, head) pairs
 * for attention, dealt to the threads round-robin. */
static void *run_rows(void *arg)
{
    job_t *jb = (job_t *)arg;
    int64_t maxrow = 0;
    for (int64_t n = 0; n < jb->nrows; ++n)
        if (jb->rows[n] > maxrow)
            maxrow = jb->rows[n];
    if (jb->mode == 0) {
        int64_t nb = maxrow / jb->B_k + 1;
        double *P = (double *)malloc(sizeof(double) * (size_t)nb);
        char *taken = (char *)malloc((size_t)nb);
        for (int64_t u = jb->tid; u < jb->nrows * jb->H_kv; u += jb->nthreads) {
            int64_t n = u / jb->H_kv;
            int r = (int)(u % jb->H_kv);
            int64_t i = jb->rows[n];
            oracle_block_scores(jb->q_rows + n * jb->H_kv * jb->d_idx, jb->k_idx, i,
                                r, jb->H_kv, jb->d_idx, jb->B_k, P);
            select_from_scores(P, i / jb->B_k, jb->k,
                               jb->sel + (n * jb->H_kv + r) * jb->k, taken);
        }
        free(P);
        free(taken);
    } else if (jb->mode == 2) {
        int G = jb->H_q / jb->H_kv;
        double *buf = (double *)malloc(sizeof(double) * 3 * (size_t)jb->k * jb->B_k);
        for (int64_t u = jb->tid; u < jb->nrows * jb->H_kv; u += jb->nthreads) {
            int64_t n = u / jb->H_kv;
            int r = (int)(u % jb->H_kv);
            int64_t i = jb->rows[n];
            jb->kl[n * jb->H_kv + r] =
                kl_one(jb->q_rows + (n * jb->H_kv + r) * jb->d_idx, jb->k_idx,
                       jb->Q_rows + (n * jb->H_q + (int64_t)r * G) * jb->d_h, jb->K, i, r, G,
                       jb->H_kv, jb->d_h, jb->d_idx, jb->B_k,
                       jb->sel + (n * jb->H_kv + r) * jb->k, jb->k, jb->scale, buf);
        }
        free(buf);
    } else {
        int G = jb->H_q / jb->H_kv;
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)jb->k * jb->B_k);
        for (int64_t u = jb->tid; u < jb->nrows * jb->H_q; u += jb->nthreads) {
            int64_t n = u / jb->H_q;
            int h = (int)(u % jb->H_q);
            int64_t i = jb->rows[n];
            int r = h / G;
            attend_one(jb->Q_rows + (n * jb->H_q + h) * jb->d_h, jb->K, jb->V, i, r,
                       jb->H_kv, jb->d_h, jb->B_k, jb->sel + (n * jb->H_kv + r) * jb->k,
                       jb->k, jb->scale, s_buf, jb->O + (n * jb->H_q + h) * jb->d_h,
                       jb->lse + n * jb->H_q + h);
        }
        free(s_buf);
    }
    return NULL;
}

static void run_threads(job_t *base, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *base;
        jobs[t].tid = t;
        jobs[t].nthreads = nthreads;
        pthread_create(&th[t], NULL, run_rows, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

/*
 * Index Branch for a list of query rows: block scores, then selection.
 *   q_rows: the index queries of those rows, [nrows, H_kv, d_idx]
 *   k_idx:  index keys of the whole prefix, [Nk, H_kv, d_idx], Nk > max row
 *   sel:    out [nrows, H_kv, k]
 */
void oracle_select(const uint16_t *q_rows, const uint16_t *k_idx,
                   const int64_t *rows, int64_t nrows, int H_kv, int d_idx,
                   int B_k, int k, int32_t *sel, int nthreads)
{
    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.q_rows = q_rows;
    jb.k_idx = k_idx;
    jb.rows = rows;
    jb.nrows = nrows;
    jb.H_kv = H_kv;
    jb.d_idx = d_idx;
    jb.B_k = B_k;
    jb.k = k;
    jb.sel = sel;
    jb.mode = 0;
    run_threads(&jb, nthreads);
}

/*
 * Main Branch for a list of query rows, given their selection.
 *   Q_rows: [nrows, H_q, d_h]; K, V: [Nk, H_kv, d_h]
 *   O: out [nrows, H_q, d_h] fp64; lse: out [nrows, H_q] fp64 (natural log)
 */
void oracle_attend(const uint16_t *Q_rows, const uint16_t *K, const uint16_t *V,
                   const int32_t *sel, const int64_t *rows, int64_t nrows,
                   int H_q, int H_kv, int d_h, int B_k, int k, double scale,
                   double *O, double *lse, int nthreads)
{
    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.Q_rows = Q_rows;
    jb.K = K;
    jb.V = V;
    jb.sel = (int32_t *)sel;
    jb.rows = rows;
    jb.nrows = nrows;
    jb.H_q = H_q;
    jb.H_kv = H_kv;
    jb.d_h = d_h;
    jb.B_k = B_k;
    jb.k = k;
    jb.scale = scale;
    jb.O = O;
    jb.lse = lse;
    jb.mode = 1;
    run_threads(&jb, nthreads);
}

/*
 * Index-alignment KL (see kl_one) for a list of query rows, given their
 * selection.
 *   q_rows: [nrows, H_kv, d_idx]; k_idx: [Nk, H_kv, d_idx]
 *   Q_rows: [nrows, H_q, d_h]; K: [Nk, H_kv, d_h]
 *   kl: out [nrows, H_kv] fp64
 */
void oracle_index_kl(const uint16_t *q_rows, const uint16_t *k_idx, const uint16_t *Q_rows,
                     const uint16_t *K, const int32_t *sel, const int64_t *rows, int64_t nrows,
                     int H_q, int H_kv, int d_h, int d_idx, int B_k, int k, double scale,
                     double *kl, int nthreads)
{
    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.q_rows = q_rows;
    jb.k_idx = k_idx;
    jb.Q_rows = Q_rows;
    jb.K = K;
    jb.sel = (int32_t *)sel;
    jb.rows = rows;
    jb.nrows = nrows;
    jb.H_q = H_q;
    jb.H_kv = H_kv;
    jb.d_h = d_h;
    jb.d_idx = d_idx;
    jb.B_k = B_k;
    jb.k = k;
    jb.scale = scale;
    jb.kl = kl;
    jb.mode = 2;
    run_threads(&jb, nthreads);
}

/*
 * Main Branch backward over the selected token sets: the gradients of a
 * scalar loss with output gradient dO, for the forward above (section 02:
 * Main Branch = exact softmax attention over the selected blocks; the
 * selection itself is not differentiable -- section 03 -- so no gradient
 * reaches the Index Branch from this loss).  Per query row i and head h
 * (group r), over T = the tokens j <= i of the row's selected blocks:
 *   s_j = scale * Q[i,h].K[j,r],  p = softmax_T(s),  O = sum_j p_j V[j,r]
 *   dp_j = dO[i,h].V[j,r],  ds_j = p_j (dp_j - dO[i,h].O)
 *   dQ[i,h]  = scale * sum_j ds_j K[j,r]
 *   dK[j,r] += scale * ds_j Q[i,h]        dV[j,r] += p_j dO[i,h]
 * Every softmax is taken over the whole of T at once, in fp64; dK and dV
 * sum over every (row, head) whose T contains j.
 *   Q, dO: [N, H_q, d_h] (all rows 0..N-1); K, V: [N, H_kv, d_h]
 *   sel: [N, H_kv, k]; dQ out [N, H_q, d_h]; dK, dV out [N, H_kv, d_h]
 */
typedef struct {
    const uint16_t *Q, *K, *V, *dO;
    const int32_t *sel;
    int64_t N;              /* rows of Q, dO, sel, dQ */
    const int64_t *pos;     /* their positions (NULL: row i is position i) */
    int H_q, H_kv, d_h, B_k, k;
    double scale;
    double *dQ, *dK, *dV;   /* dK, dV: this thread's private accumulators (NULL: dQ only) */
    int tid, nthreads;
} bwd_job_t;

static void *run_bwd(void *arg)
{
    bwd_job_t *jb = (bwd_job_t *)arg;
    const int G = jb->H_q / jb->H_kv, d_h = jb->d_h, B_k = jb->B_k;
    const int64_t cap = (int64_t)jb->k * B_k;
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
    double *p = (double *)malloc(sizeof(double) * (size_t)cap);
    double *O = (double *)malloc(sizeof(double) * (size_t)d_h);
    for (int64_t u = jb->tid; u < jb->N * jb->H_q; u += jb->nthreads) {
        const int64_t ii = u / jb->H_q;                 /* row of the inputs */
        const int64_t i = jb->pos ? jb->pos[ii] : ii;   /* its position */
        const int h = (int)(u % jb->H_q), r = h / G;
        const uint16_t *q = jb->Q + (ii * jb->H_q + h) * d_h;
        const uint16_t *go = jb->dO + (ii * jb->H_q + h) * d_h;
        const int32_t *srow = jb->sel + (ii * jb->H_kv + r) * jb->k;
        int64_t n = 0;
        for (int t = 0; t < jb->k; ++t) {
            if (srow[t] < 0)
                continue;
            for (int64_t j = (int64_t)srow[t] * B_k; j < ((int64_t)srow[t] + 1) * B_k && j <= i; ++j)
                tok[n++] = j;
        }
        double m = -INFINITY;
        for (int64_t a = 0; a < n; ++a) {
            double dot = 0.0;
            for (int d = 0; d < d_h; ++d)
                dot += widen_bf16(q[d]) * widen_bf16(jb->K[(tok[a] * jb->H_kv + r) * d_h + d]);
            p[a] = dot * jb->scale;
            if (p[a] > m)
                m = p[a];
        }
        double z = 0.0;
        for (int64_t a = 0; a < n; ++a) {
            p[a] = exp(p[a] - m);
            z += p[a];
        }
        for (int d = 0; d < d_h; ++d)
            O[d] = 0.0;
        for (int64_t a = 0; a < n; ++a) {
            p[a] /= z;
            for (int d = 0; d < d_h; ++d)
                O[d] += p[a] * widen_bf16(jb->V[(tok[a] * jb->H_kv + r) * d_h + d]);
        }
        double Dv = 0.0;
        for (int d = 0; d < d_h; ++d)
            Dv += widen_bf16(go[d]) * O[d];
        double *dq = jb->dQ + (ii * jb->H_q + h) * d_h;
        for (int d = 0; d < d_h; ++d)
            dq[d] = 0.0;
        for (int64_t a = 0; a < n; ++a) {
            const int64_t base = (tok[a] * jb->H_kv + r) * d_h;
            double dp = 0.0;
            for (int d = 0; d < d_h; ++d)
                dp += widen_bf16(go[d]) * widen_bf16(jb->V[base + d]);
            const double ds = p[a] * (dp - Dv);
            for (int d = 0; d < d_h; ++d)
                dq[d] += jb->scale * ds * widen_bf16(jb->K[base + d]);
            if (jb->dK) {
                for (int d = 0; d < d_h; ++d) {
                    jb->dK[base + d] += jb->scale * ds * widen_bf16(q[d]);
                    jb->dV[base + d] += p[a] * widen_bf16(go[d]);
                }
            }
        }
    }
    free(tok);
    free(p);
    free(O);
    return NULL;
}

void oracle_attend_backward(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                            const uint16_t *dO, const int32_t *sel, int64_t N, int H_q,
                            int H_kv, int d_h, int B_k, int k, double scale, double *dQ,
                            double *dK, double *dV, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    const size_t kv = (size_t)N * H_kv * d_h;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    bwd_job_t *jobs = (bwd_job_t *)malloc(sizeof(bwd_job_t) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) {
        bwd_job_t *jb = &jobs[t];
        jb->Q = Q; jb->K = K; jb->V = V; jb->dO = dO; jb->sel = sel;
        jb->N = N; jb->pos = NULL;
        jb->H_q = H_q; jb->H_kv = H_kv; jb->d_h = d_h; jb->B_k = B_k; jb->k = k;
        jb->scale = scale; jb->dQ = dQ;
        jb->dK = (double *)calloc(kv, sizeof(double));
        jb->dV = (double *)calloc(kv, sizeof(double));
        jb->tid = t;
        jb->nthreads = nthreads;
        pthread_create(&th[t], NULL, run_bwd, jb);
    }
    for (size_t e = 0; e < kv; ++e)
        dK[e] = dV[e] = 0.0;
    for (int t = 0; t < nthreads; ++t) {
        pthread_join(th[t], NULL);
        for (size_t e = 0; e < kv; ++e) {
            dK[e] += jobs[t].dK[e];
            dV[e] += jobs[t].dV[e];
        }
        free(jobs[t].dK);
        free(jobs[t].dV);
    }
    free(th);
    free(jobs);
}

/*
 * dQ alone for chosen query rows: the same per-row computation as
 * oracle_attend_backward, for rows at positions pos[0..n_rows) (their Q,
 * dO and selection rows given compactly), without the dK/dV sums.
 *   Q_rows, dO_rows: [n_rows, H_q, d_h]; sel_rows: [n_rows, H_kv, k]
 *   K, V: [>= max(pos)+1, H_kv, d_h]; dQ_rows out [n_rows, H_q, d_h]
 */
void oracle_attend_backward_dq_rows(const uint16_t *Q_rows, const uint16_t *K,
                                    const uint16_t *V, const uint16_t *dO_rows,
                                    const int32_t *sel_rows, const int64_t *pos, int64_t n_rows,
                                    int H_q, int H_kv, int d_h, int B_k, int k, double scale,
                                    double *dQ_rows, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    bwd_job_t *jobs = (bwd_job_t *)malloc(sizeof(bwd_job_t) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) {
        bwd_job_t *jb = &jobs[t];
        jb->Q = Q_rows; jb->K = K; jb->V = V; jb->dO = dO_rows; jb->sel = sel_rows;
        jb->N = n_rows; jb->pos = pos;
        jb->H_q = H_q; jb->H_kv = H_kv; jb->d_h = d_h; jb->B_k = B_k; jb->k = k;
        jb->scale = scale; jb->dQ = dQ_rows; jb->dK = NULL; jb->dV = NULL;
        jb->tid = t;
        jb->nthreads = nthreads;
        pthread_create(&th[t], NULL, run_bwd, jb);
    }
    for (int t = 0; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

/*
 * Inverted index: the selection table turned around, from "which blocks
 * does each query read" to "which queries hit each block" (section 05,
 * part 2: KV-outer execution gathers, per KV block, the queries that
 * selected it).  Buckets are (group r, block b) in r-major order; inside a
 * bucket the queries are in ascending position; slot is the rank of the
 * block inside that query's selection row.  A plain counting sort.
 *   sel: [Nq, H_kv, k] for query positions q_start .. q_start+Nq-1
 *   row_ptr: out [H_kv*nblk + 1]; col, slot: out [nnz]
 * Returns nnz.
 */
int64_t oracle_invert(const int32_t *sel, int64_t q_start, int64_t Nq, int H_kv,
                      int k, int64_t nblk, int64_t *row_ptr, int64_t *col,
                      int32_t *slot)
{
    int64_t nb = (int64_t)H_kv * nblk;
    int64_t *fill = (int64_t *)calloc((size_t)nb, sizeof(int64_t));
    for (int64_t x = 0; x <= nb; ++x)
        row_ptr[x] = 0;
    for (int64_t iq = 0; iq < Nq; ++iq)
        for (int r = 0; r < H_kv; ++r)
            for (int s = 0; s < k; ++s) {
                int32_t b = sel[(iq * H_kv + r) * k + s];
                if (b >= 0)
                    row_ptr[(int64_t)r * nblk + b + 1] += 1;
            }
    for (int64_t x = 0; x < nb; ++x)
        row_ptr[x + 1] += row_ptr[x];
    for (int64_t iq = 0; iq < Nq; ++iq)
        for (int r = 0; r < H_kv; ++r)
            for (int s = 0; s < k; ++s) {
                int32_t b = sel[(iq * H_kv + r) * k + s];
                if (b < 0)
                    continue;
                int64_t bucket = (int64_t)r * nblk + b;
                int64_t pos = row_ptr[bucket] + fill[bucket]++;
                col[pos] = q_start + iq;
                slot[pos] = s;
            }
    free(fill);
    return row_ptr[nb];
}

/*
 * Decode for one sequence: the new query is the last cache row
 * (position N-1), so it sees the whole cache and its local block is the
 * last block.  Selection and attention are exactly those of that prefill
 * row.
 *   q [H_q, d_h], q_idx [H_kv, d_idx]; K, V [N, H_kv, d_h]; k_idx [N, H_kv, d_idx]
 *   sel out [H_kv, k]; O out [H_q, d_h]; lse out [H_q]
 */
void oracle_decode_one(const uint16_t *q, const uint16_t *q_idx, const uint16_t *K,
                       const uint16_t *V, const uint16_t *k_idx, int64_t N, int H_q,
                       int H_kv, int d_h, int d_idx, int B_k, int k, double scale,
                       int32_t *sel, double *O, double *lse, int nthreads)
{
    int64_t row = N - 1;
    oracle_select(q_idx, k_idx, &row, 1, H_kv, d_idx, B_k, k, sel, nthreads);
    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.Q_rows = q;
    jb.K = K;
    jb.V = V;
    jb.sel = sel;
    jb.rows = &row;
    jb.nrows = 1;
    jb.H_q = H_q;
    jb.H_kv = H_kv;
    jb.d_h = d_h;
    jb.B_k = B_k;
    jb.k = k;
    jb.scale = scale;
    jb.O = O;
    jb.lse = lse;
    jb.mode = 1;
    run_threads(&jb, nthreads);
}
