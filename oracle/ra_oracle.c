/*
 * ra_oracle.c -- plain fp64 CPU oracle for the ring-attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * source with the HIP library and includes no HIP header.
 *
 * Pages cited (short names used below):
 *   [P1] "Ring Attention如何让大模型突破百万token上下文：从环形通信到计算重叠的技术突围"
 *        (answer.freetools.me blog post)
 *   [P2] "Ring Attention with Blockwise Transformers for Near Infinite Context"
 *        (reading notes on arXiv 2310.01889, papers.chlience.com)
 *   [P3] aiqz.cc Ring Attention explainer (sections 分块注意力, 环状拓扑, 工程实现)
 *
 * What it computes is the plain definition, not the blocked algorithm:
 *   - scaled dot-product attention softmax(Q K^T / sqrt(d)) V
 *     ([P2] section 5.1, "基础 attention 语义"; [P3] 分块注意力 formula for S_b),
 *     with d the head dimension;
 *   - an explicit per-element causal mask: key token t_k is visible to query
 *     token t_q iff t_k <= t_q ([P3] 工程实现: a token sees tokens whose index
 *     does not exceed its own);
 *   - token index of local row r on host h: contiguous h*c + r, striped r*N + h
 *     ([P1] 因果掩码的负载均衡挑战, the striped device/token lists);
 *   - the log-sum-exp of each row in natural-log units ([P1] Online Softmax,
 *     LogSumExp form);
 *   - the backward is the closed-form gradient of the same function (the pages
 *     say only that the backward accumulates dQ, dK, dV along the ring,
 *     [P2] section 5.2): with P = exp(S - LSE) on visible pairs,
 *     D = rowsum(dO * O), dV = P^T dO, dS = P * (dO V^T - D),
 *     dQ = scale * dS K, dK = scale * dS^T Q.
 * Grouped heads: query head g reads key/value head g / (Hq / Hkv).
 *
 * Arrays are float32 in host-major layout [hosts][B][H][c][d]; every value
 * is widened to double before use and every sum is accumulated in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_LAYOUT_CONTIGUOUS 0
#define OR_LAYOUT_STRIPED 1
#define OR_LAYOUT_ZIGZAG 2

/* Global token index of local row r on host h.
 * Contiguous: host h holds tokens [h c, (h+1) c).  Striped: token r N + h.
 * Zigzag (named beside Striped as the causal load-balancing variant in P1,
 * "工程实践指南", item "因果掩码"; the pages give no definition, the reading
 * used here): the sequence is cut into 2N chunks of c/2 tokens and host h
 * holds chunk h (its rows 0..c/2-1) and chunk 2N-1-h (rows c/2..c-1). */
static inline long long token_index(int layout, int n_hosts, long long block_len, int host,
                                    long long r)
{
    if (layout == OR_LAYOUT_STRIPED)
        return r * (long long)n_hosts + host;
    if (layout == OR_LAYOUT_ZIGZAG) {
        const long long half = block_len / 2;
        if (r < half)
            return (long long)host * half + r;
        return (long long)(2 * n_hosts - 1 - host) * half + (r - half);
    }
    return (long long)host * block_len + r;
}

/* 1 if key token tk is visible to query token tq. */
static inline int visible(int causal, long long tq, long long tk)
{
    if (!causal)
        return 1;
    return tk <= tq ? 1 : 0;
}

long long oracle_token_index(int layout, int n_hosts, long long block_len, int host,
                             long long r)
{
    return token_index(layout, n_hosts, block_len, host, r);
}

int oracle_visible(int causal, long long tq, long long tk)
{
    return visible(causal, tq, tk);
}

/* Explicit mask of query block qhost against key block khost: out[r*c + r']. */
void oracle_block_mask(int layout, int causal, int n_hosts, int block_len, int qhost,
                       int khost, unsigned char *out)
{
    for (long long r = 0; r < block_len; ++r) {
        long long tq = token_index(layout, n_hosts, block_len, qhost, r);
        for (long long rk = 0; rk < block_len; ++rk) {
            long long tk = token_index(layout, n_hosts, block_len, khost, rk);
            out[r * block_len + rk] = (unsigned char)visible(causal, tq, tk);
        }
    }
}

typedef struct {
    int n_hosts, batch, hq, hkv, c, d, layout, causal;
    double scale;
    const float *K, *V;
} or_dims;

static size_t idx_row(const or_dims *g, int heads, int host, int b, int h, long long r)
{
    return ((((size_t)host * g->batch + b) * heads + h) * (size_t)g->c + (size_t)r) *
           (size_t)g->d;
}

/* Dot product of two double vectors.  The definition fixes no summation
 * order; the reduction clause lets the compiler split the sum over vector
 * lanes.  One out-of-line copy, so every caller sums in the same order. */
__attribute__((noinline)) static double dot_d(const double *a, const double *b, int d)
{
    double s = 0.0;
#pragma omp simd reduction(+ : s)
    for (int e = 0; e < d; ++e)
        s += a[e] * b[e];
    return s;
}

#define K_ROW(g, j, b, kvh, rk) ((g)->K + idx_row((g), (g)->hkv, (j), (b), (kvh), (rk)))
#define V_ROW(g, j, b, kvh, rk) ((g)->V + idx_row((g), (g)->hkv, (j), (b), (kvh), (rk)))

static double dot_f32(const float *a, const double *qd, int d)
{
    double s = 0.0;
#pragma omp simd reduction(+ : s)
    for (int e = 0; e < d; ++e)
        s += (double)a[e] * qd[e];
    return s;
}

/* One query row, the definition written out ([P2] 5.1; [P3] 分块注意力):
 * the scaled scores of the visible keys and their max, then the exp-sum and
 * the weighted sum of values, then O = sum / l and LSE = max + ln l.  A row
 * that sees no key gets O = 0 and LSE = -inf.  sc: N*c doubles of scratch
 * (the row's scores, kept for the backward). */
static void fwd_row(const or_dims *g, const double *q, long long r, int qhost, int b,
                    int kvh, double *sc, double *O, double *mx_out, double *l_out,
                    double *lse_out)
{
    const int d = g->d;
    const long long c = g->c;
    const long long tq = token_index(g->layout, g->n_hosts, c, qhost, r);
    double kd[512];
    double mx = -INFINITY, l = 0.0;
    for (int j = 0; j < g->n_hosts; ++j)
        for (long long rk = 0; rk < c; ++rk) {
            if (!visible(g->causal, tq, token_index(g->layout, g->n_hosts, c, j, rk)))
                continue;
            const float *k = K_ROW(g, j, b, kvh, rk);
            for (int e = 0; e < d; ++e)
                kd[e] = (double)k[e];
            double s = g->scale * dot_d(kd, q, d);
            sc[j * c + rk] = s;
            if (s > mx)
                mx = s;
        }
    for (int e = 0; e < d; ++e)
        O[e] = 0.0;
    for (int j = 0; j < g->n_hosts; ++j)
        for (long long rk = 0; rk < c; ++rk) {
            if (!visible(g->causal, tq, token_index(g->layout, g->n_hosts, c, j, rk)))
                continue;
            const float *v = V_ROW(g, j, b, kvh, rk);
            double p = exp(sc[j * c + rk] - mx);
            l += p;
            for (int e = 0; e < d; ++e)
                O[e] += p * (double)v[e];
        }
    *mx_out = mx;
    if (mx == -INFINITY) {
        *l_out = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    for (int e = 0; e < d; ++e)
        O[e] /= l;
    *l_out = l;
    *lse_out = mx + log(l);
}

/* dQ of one query row after fwd_row: D = dO . O, and over the visible keys
 * P = exp(s - LSE), dS = P (dO . v - D), dQ = scale * sum dS k. */
static void bwd_q_row(const or_dims *g, const double *dov, const double *O, long long r,
                      int qhost, int b, int kvh, const double *sc, double lse, double *D_out,
                      double *dq)
{
    const int d = g->d;
    const long long c = g->c;
    const long long tq = token_index(g->layout, g->n_hosts, c, qhost, r);
    double vd[512];
    double D = 0.0;
    for (int e = 0; e < d; ++e)
        D += dov[e] * O[e];
    *D_out = D;
    for (int e = 0; e < d; ++e)
        dq[e] = 0.0;
    if (lse == -INFINITY)
        return;
    for (int j = 0; j < g->n_hosts; ++j)
        for (long long rk = 0; rk < c; ++rk) {
            if (!visible(g->causal, tq, token_index(g->layout, g->n_hosts, c, j, rk)))
                continue;
            const float *k = K_ROW(g, j, b, kvh, rk);
            const float *v = V_ROW(g, j, b, kvh, rk);
            for (int e = 0; e < d; ++e)
                vd[e] = (double)v[e];
            double p = exp(sc[j * c + rk] - lse);
            double ds = p * (dot_d(vd, dov, d) - D);
            for (int e = 0; e < d; ++e)
                dq[e] += g->scale * ds * (double)k[e];
        }
}

/* The row-set functions below compute exactly what fwd_row and bwd_q_row
 * compute, for up to OR_SET rows at once; oracle_attn_rows_plain and
 * oracle_attn_bwd_q_rows_plain run the per-row forms, and a CPU test checks
 * that both give bitwise equal results. */

/* Up to OR_SET query rows of one (host, batch, head) are evaluated in one
 * sweep over the keys, so each key/value row is read once per set instead of
 * once per query row.  Every row's arithmetic is exactly fwd_row's. */
#define OR_SET 16

static void fwd_rowset(const or_dims *g, int nset, const double *const *q, const long long *r,
                       int qhost, int b, int kvh, double *const *sc, double *const *O,
                       double *mx, double *l, double *lse)
{
    const int d = g->d;
    const long long c = g->c;
    long long tq[OR_SET];
    double kd[512];
    for (int i = 0; i < nset; ++i) {
        tq[i] = token_index(g->layout, g->n_hosts, c, qhost, r[i]);
        mx[i] = -INFINITY;
        l[i] = 0.0;
        for (int e = 0; e < d; ++e)
            O[i][e] = 0.0;
    }
    /* scores of the visible keys, and each row's max */
    for (int j = 0; j < g->n_hosts; ++j)
        for (long long rk = 0; rk < c; ++rk) {
            long long tk = token_index(g->layout, g->n_hosts, c, j, rk);
            const float *k = K_ROW(g, j, b, kvh, rk);
            int any = 0;
            for (int i = 0; i < nset; ++i)
                any |= visible(g->causal, tq[i], tk);
            if (!any)
                continue;
            for (int e = 0; e < d; ++e)
                kd[e] = (double)k[e];
            for (int i = 0; i < nset; ++i) {
                if (!visible(g->causal, tq[i], tk))
                    continue;
                double s = g->scale * dot_d(kd, q[i], d);
                sc[i][j * c + rk] = s;
                if (s > mx[i])
                    mx[i] = s;
            }
        }
    /* exp-sum and weighted sum of values */
    for (int j = 0; j < g->n_hosts; ++j)
        for (long long rk = 0; rk < c; ++rk) {
            long long tk = token_index(g->layout, g->n_hosts, c, j, rk);
            const float *v = V_ROW(g, j, b, kvh, rk);
            int any = 0;
            for (int i = 0; i < nset; ++i)
                any |= visible(g->causal, tq[i], tk);
            if (!any)
                continue;
            for (int e = 0; e < d; ++e)
                kd[e] = (double)v[e];
            for (int i = 0; i < nset; ++i) {
                if (!visible(g->causal, tq[i], tk))
                    continue;
                double p = exp(sc[i][j * c + rk] - mx[i]);
                l[i] += p;
                double *oi = O[i];
#pragma omp simd
                for (int e = 0; e < d; ++e)
                    oi[e] += p * kd[e];
            }
        }
    for (int i = 0; i < nset; ++i) {
        if (mx[i] == -INFINITY) {
            lse[i] = -INFINITY;
            l[i] = 0.0;
            continue;
        }
        for (int e = 0; e < d; ++e)
            O[i][e] /= l[i];
        lse[i] = mx[i] + log(l[i]);
    }
}

/*
 * Forward attention for a list of query rows.
 *   Q: [n_q_hosts][B][Hq][c][d], host index h stored at h - q_host_base
 *   (rows outside [q_host_base, q_host_base + n_q_hosts) are rejected)
 *   K, V: [N][B][Hkv][c][d]
 *   rows: n_rows x 4 int64 (host, batch, q_head, local row)
 * Outputs (n_rows each; O is n_rows x d): O, LSE, max score, denominator.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_attn_rows(const float *Q, const float *K, const float *V, int n_hosts,
                     int batch, int hq, int hkv, int c, int d, int layout, int causal,
                     double scale, int q_host_base, int n_q_hosts, long long n_rows,
                     const long long *rows, double *O, double *lse, double *mx,
                     double *l)
{
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || d > 512 || c <= 0 || n_hosts <= 0)
        return -1;
    or_dims g = {n_hosts, batch, hq, hkv, c, d, layout, causal, scale, K, V};
    const int group = hq / hkv;
    for (long long i = 0; i < n_rows; ++i) {
        const long long *rd = rows + 4 * i;
        int host = (int)rd[0], b = (int)rd[1], h = (int)rd[2];
        long long r = rd[3];
        if (host < 0 || host >= n_hosts || host < q_host_base ||
            host >= q_host_base + n_q_hosts || b < 0 || b >= batch || h < 0 || h >= hq ||
            r < 0 || r >= c)
            return -1;
    }
    /* sets: runs of up to OR_SET consecutive rows with the same (host, batch, head) */
    long long *set_start = (long long *)malloc(sizeof(long long) * (size_t)(n_rows + 1));
    long long n_sets = 0;
    for (long long i = 0; i < n_rows;) {
        long long j = i + 1;
        while (j < n_rows && j - i < OR_SET && rows[4 * j] == rows[4 * i] &&
               rows[4 * j + 1] == rows[4 * i + 1] && rows[4 * j + 2] == rows[4 * i + 2])
            ++j;
        set_start[n_sets++] = i;
        i = j;
    }
    set_start[n_sets] = n_rows;
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (size_t)OR_SET *
                                       ((size_t)d + (size_t)n_hosts * c));
#pragma omp for schedule(dynamic, 1)
        for (long long s = 0; s < n_sets; ++s) {
            const long long i0 = set_start[s];
            const int nset = (int)(set_start[s + 1] - i0);
            const long long *rd = rows + 4 * i0;
            const int host = (int)rd[0], b = (int)rd[1], h = (int)rd[2];
            double *qp[OR_SET], *scp[OR_SET], *op[OR_SET];
            long long rr[OR_SET];
            for (int i = 0; i < nset; ++i) {
                qp[i] = buf + (size_t)i * d;
                scp[i] = buf + (size_t)OR_SET * d + (size_t)i * n_hosts * c;
                op[i] = O + (size_t)(i0 + i) * d;
                rr[i] = rows[4 * (i0 + i) + 3];
                const float *qs = Q + idx_row(&g, hq, host - q_host_base, b, h, rr[i]);
                for (int e = 0; e < d; ++e)
                    qp[i][e] = (double)qs[e];
            }
            fwd_rowset(&g, nset, (const double *const *)qp, rr, host, b, h / group,
                       (double *const *)scp, (double *const *)op, mx + i0, l + i0, lse + i0);
        }
        free(buf);
    }
    free(set_start);
    return 0;
}

/* Backward of a row set: after fwd_rowset, D = dO . O per row, then one more
 * sweep over the keys accumulates dQ = scale * sum_k P (dO.v_k - D) k. */
static void bwd_q_rowset(const or_dims *g, int nset, const double *const *dov,
                         const long long *r, int qhost, int b, int kvh,
                         double *const *sc, double *const *O, const double *lse,
                         const double *D, double *const *dq)
{
    const int d = g->d;
    const long long c = g->c;
    long long tq[OR_SET];
    double kd[512], vd[512];
    for (int i = 0; i < nset; ++i) {
        tq[i] = token_index(g->layout, g->n_hosts, c, qhost, r[i]);
        for (int e = 0; e < d; ++e)
            dq[i][e] = 0.0;
    }
    (void)O;
    for (int j = 0; j < g->n_hosts; ++j)
        for (long long rk = 0; rk < c; ++rk) {
            long long tk = token_index(g->layout, g->n_hosts, c, j, rk);
            int any = 0;
            for (int i = 0; i < nset; ++i)
                any |= visible(g->causal, tq[i], tk) && lse[i] != -INFINITY;
            if (!any)
                continue;
            const float *k = K_ROW(g, j, b, kvh, rk);
            const float *v = V_ROW(g, j, b, kvh, rk);
            for (int e = 0; e < d; ++e) {
                kd[e] = (double)k[e];
                vd[e] = (double)v[e];
            }
            for (int i = 0; i < nset; ++i) {
                if (!visible(g->causal, tq[i], tk) || lse[i] == -INFINITY)
                    continue;
                double p = exp(sc[i][j * c + rk] - lse[i]);
                double dp = dot_d(vd, dov[i], d);
                double ds = p * (dp - D[i]);
                double *dqi = dq[i];
#pragma omp simd
                for (int e = 0; e < d; ++e)
                    dqi[e] += g->scale * ds * kd[e];
            }
        }
}

/*
 * Backward for a list of query rows: dQ (n_rows x d), plus the row's LSE and
 * D = rowsum(dO * O) with O the oracle's own fp64 output.
 *   dO: same layout and host base as Q.
 */
int oracle_attn_bwd_q_rows(const float *Q, const float *K, const float *V,
                           const float *dO, int n_hosts, int batch, int hq, int hkv,
                           int c, int d, int layout, int causal, double scale,
                           int q_host_base, int n_q_hosts, long long n_rows,
                           const long long *rows, double *dQ, double *lse_out,
                           double *D_out)
{
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || d > 512 || c <= 0 || n_hosts <= 0)
        return -1;
    or_dims g = {n_hosts, batch, hq, hkv, c, d, layout, causal, scale, K, V};
    const int group = hq / hkv;
    for (long long i = 0; i < n_rows; ++i) {
        const long long *rd = rows + 4 * i;
        int host = (int)rd[0], b = (int)rd[1], h = (int)rd[2];
        long long r = rd[3];
        if (host < 0 || host >= n_hosts || host < q_host_base ||
            host >= q_host_base + n_q_hosts || b < 0 || b >= batch || h < 0 || h >= hq ||
            r < 0 || r >= c)
            return -1;
    }
    long long *set_start = (long long *)malloc(sizeof(long long) * (size_t)(n_rows + 1));
    long long n_sets = 0;
    for (long long i = 0; i < n_rows;) {
        long long j = i + 1;
        while (j < n_rows && j - i < OR_SET && rows[4 * j] == rows[4 * i] &&
               rows[4 * j + 1] == rows[4 * i + 1] && rows[4 * j + 2] == rows[4 * i + 2])
            ++j;
        set_start[n_sets++] = i;
        i = j;
    }
    set_start[n_sets] = n_rows;
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (size_t)OR_SET *
                                       (3 * (size_t)d + (size_t)n_hosts * c + 2));
#pragma omp for schedule(dynamic, 1)
        for (long long s = 0; s < n_sets; ++s) {
            const long long i0 = set_start[s];
            const int nset = (int)(set_start[s + 1] - i0);
            const long long *rd = rows + 4 * i0;
            const int host = (int)rd[0], b = (int)rd[1], h = (int)rd[2];
            double *qp[OR_SET], *op[OR_SET], *dop[OR_SET], *scp[OR_SET], *dqp[OR_SET];
            double mx[OR_SET], lv[OR_SET], Dv[OR_SET];
            long long rr[OR_SET];
            double *area = buf + (size_t)OR_SET * 3 * d;
            for (int i = 0; i < nset; ++i) {
                qp[i] = buf + (size_t)i * 3 * d;
                op[i] = qp[i] + d;
                dop[i] = qp[i] + 2 * d;
                scp[i] = area + (size_t)i * n_hosts * c;
                dqp[i] = dQ + (size_t)(i0 + i) * d;
                rr[i] = rows[4 * (i0 + i) + 3];
                size_t qo = idx_row(&g, hq, host - q_host_base, b, h, rr[i]);
                for (int e = 0; e < d; ++e) {
                    qp[i][e] = (double)Q[qo + e];
                    dop[i][e] = (double)dO[qo + e];
                }
            }
            fwd_rowset(&g, nset, (const double *const *)qp, rr, host, b, h / group,
                       (double *const *)scp, (double *const *)op, mx, lv, lse_out + i0);
            for (int i = 0; i < nset; ++i) {
                double acc = 0.0;
                for (int e = 0; e < d; ++e)
                    acc += dop[i][e] * op[i][e];
                Dv[i] = acc;
                D_out[i0 + i] = acc;
            }
            bwd_q_rowset(&g, nset, (const double *const *)dop, rr, host, b, h / group,
                         (double *const *)scp, (double *const *)op, lse_out + i0, Dv,
                         (double *const *)dqp);
        }
        free(buf);
    }
    free(set_start);
    return 0;
}

/*
 * oracle_attn_rows and oracle_attn_bwd_q_rows, one row at a time through
 * fwd_row and bwd_q_row (same arguments; dQ and D are NULL for the forward).
 * They exist to check the row-set forms, which must agree with them bit for
 * bit; they read every key row once per query row, so they suit small inputs.
 */
static int rows_plain(const float *Q, const float *K, const float *V, const float *dO,
                      int n_hosts, int batch, int hq, int hkv, int c, int d, int layout,
                      int causal, double scale, int q_host_base, int n_q_hosts,
                      long long n_rows, const long long *rows, double *O, double *lse,
                      double *mx, double *l, double *dQ, double *D)
{
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || d > 512 || c <= 0 || n_hosts <= 0)
        return -1;
    or_dims g = {n_hosts, batch, hq, hkv, c, d, layout, causal, scale, K, V};
    const int group = hq / hkv;
    for (long long i = 0; i < n_rows; ++i) {
        const long long *rd = rows + 4 * i;
        int host = (int)rd[0], b = (int)rd[1], h = (int)rd[2];
        long long r = rd[3];
        if (host < 0 || host >= n_hosts || host < q_host_base ||
            host >= q_host_base + n_q_hosts || b < 0 || b >= batch || h < 0 || h >= hq ||
            r < 0 || r >= c)
            return -1;
    }
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (3 * (size_t)d + (size_t)n_hosts * c));
        double *qd = buf, *od = buf + d, *dod = buf + 2 * (size_t)d, *sc = buf + 3 * (size_t)d;
#pragma omp for schedule(dynamic, 1)
        for (long long i = 0; i < n_rows; ++i) {
            const long long *rd = rows + 4 * i;
            const int host = (int)rd[0], b = (int)rd[1], h = (int)rd[2];
            const long long r = rd[3];
            const size_t qo = idx_row(&g, hq, host - q_host_base, b, h, r);
            for (int e = 0; e < d; ++e)
                qd[e] = (double)Q[qo + e];
            double m, den, ls;
            fwd_row(&g, qd, r, host, b, h / group, sc, O ? O + (size_t)i * d : od, &m, &den,
                    &ls);
            if (mx)
                mx[i] = m;
            if (l)
                l[i] = den;
            lse[i] = ls;
            if (dQ) {
                for (int e = 0; e < d; ++e)
                    dod[e] = (double)dO[qo + e];
                bwd_q_row(&g, dod, od, r, host, b, h / group, sc, ls, D + i,
                          dQ + (size_t)i * d);
            }
        }
        free(buf);
    }
    return 0;
}

int oracle_attn_rows_plain(const float *Q, const float *K, const float *V, int n_hosts,
                           int batch, int hq, int hkv, int c, int d, int layout, int causal,
                           double scale, int q_host_base, int n_q_hosts, long long n_rows,
                           const long long *rows, double *O, double *lse, double *mx,
                           double *l)
{
    return rows_plain(Q, K, V, NULL, n_hosts, batch, hq, hkv, c, d, layout, causal, scale,
                      q_host_base, n_q_hosts, n_rows, rows, O, lse, mx, l, NULL, NULL);
}

int oracle_attn_bwd_q_rows_plain(const float *Q, const float *K, const float *V,
                                 const float *dO, int n_hosts, int batch, int hq, int hkv,
                                 int c, int d, int layout, int causal, double scale,
                                 int q_host_base, int n_q_hosts, long long n_rows,
                                 const long long *rows, double *dQ, double *lse_out,
                                 double *D_out)
{
    return rows_plain(Q, K, V, dO, n_hosts, batch, hq, hkv, c, d, layout, causal, scale,
                      q_host_base, n_q_hosts, n_rows, rows, NULL, lse_out, NULL, NULL, dQ,
                      D_out);
}

/*
 * Backward for a list of key rows: dK and dV (n_rows x d each).
 *   rows: n_rows x 4 int64 (host, batch, kv_head, local row)
 *   lse_all, D_all: [N][B][Hq][c] doubles for every query row of every host
 *   (from the oracle's own forward); Q and dO hold all N hosts.
 */
int oracle_attn_bwd_kv_rows(const float *Q, const float *K, const float *V,
                            const float *dO, const double *lse_all, const double *D_all,
                            int n_hosts, int batch, int hq, int hkv, int c, int d,
                            int layout, int causal, double scale, long long n_rows,
                            const long long *rows, double *dK, double *dV)
{
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || c <= 0 || n_hosts <= 0)
        return -1;
    or_dims g = {n_hosts, batch, hq, hkv, c, d, layout, causal, scale, K, V};
    const int group = hq / hkv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long long i = 0; i < n_rows; ++i) {
        const long long *rd = rows + 4 * i;
        int host = (int)rd[0], b = (int)rd[1], kvh = (int)rd[2];
        long long rk = rd[3];
        if (host < 0 || host >= n_hosts || b < 0 || b >= batch || kvh < 0 || kvh >= hkv ||
            rk < 0 || rk >= c) {
            bad = 1;
            continue;
        }
        double *kv = (double *)malloc(sizeof(double) * (size_t)d * 2);
        double *vv = kv + d;
        size_t ko = idx_row(&g, hkv, host, b, kvh, rk);
        for (int e = 0; e < d; ++e) {
            kv[e] = (double)K[ko + e];
            vv[e] = (double)V[ko + e];
        }
        double *dk = dK + (size_t)i * d, *dv = dV + (size_t)i * d;
        for (int e = 0; e < d; ++e) {
            dk[e] = 0.0;
            dv[e] = 0.0;
        }
        const long long tk = token_index(layout, n_hosts, c, host, rk);
        for (int h = kvh * group; h < (kvh + 1) * group; ++h)
            for (int j = 0; j < n_hosts; ++j)
                for (long long r = 0; r < c; ++r) {
                    long long tq = token_index(layout, n_hosts, c, j, r);
                    if (!visible(causal, tq, tk))
                        continue;
                    size_t qo = idx_row(&g, hq, j, b, h, r);
                    size_t so = (((size_t)j * batch + b) * hq + h) * (size_t)c + (size_t)r;
                    double lse = lse_all[so];
                    if (lse == -INFINITY)
                        continue;
                    double p = exp(scale * dot_f32(Q + qo, kv, d) - lse);
                    double dp = dot_f32(dO + qo, vv, d);
                    double ds = p * (dp - D_all[so]);
#pragma omp simd
                    for (int e = 0; e < d; ++e) {
                        dv[e] += p * (double)dO[qo + e];
                        dk[e] += scale * ds * (double)Q[qo + e];
                    }
                }
        free(kv);
    }
    return bad ? -1 : 0;
}

/* Number of threads OpenMP will use (for reporting the CPU baseline). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
