/*
 * oracle.c -- plain fp64 CPU oracle for segmented exact softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes, and where the pages state it:
 *  - exact softmax attention of a block of queries against one segment of
 *    keys/values ("Ultra-Long Sequence Distributed Transformer", Abstract:
 *    each GPU computes a partial self-attention for its segment; "Boosting
 *    Spec Eagle: USP For Long-Context Training", The Solution: each device
 *    holds a slice of the sequence and talks only to its ring neighbours);
 *  - the log-sum-exp merge of two partial (O, LSE) results, which is what
 *    makes a segment-by-segment result exact (no page prints it; it is the
 *    only combination under which the segmented result equals attention over
 *    the union of the segments);
 *  - LongNet dilated attention ("LongNet: Scaling Transformers to
 *    1,000,000,000 Tokens", Abstract and Results: it takes the place of
 *    dense attention with the same interface, a mixture of segment lengths w and dilation ratios
 *    r).  The page's formula slots are empty; the reading used here is: for
 *    branch (w, r) the sequence is cut into segments of length w (the last
 *    one may be shorter), a position p is selected iff its offset inside its
 *    segment is a multiple of r, and selected queries attend to the selected
 *    keys of the same segment; the branch partials are folded with the
 *    log-sum-exp merge;
 *  - the backward of the attention (dQ, dK, dV) given dO, using the global
 *    (all-segment) softmax statistics ("LongNet ...", Distributed Trainer:
 *    the backward turns the all-gather into a reduce-scatter, so a per-device
 *    backward over local queries and gathered keys exists).
 *
 * Conventions (readings where the pages are silent):
 *  - scale sigma = 1/sqrt(d) unless a positive scale is given;
 *  - key j of a segment is visible to query i iff j <= i + delta, where
 *    delta = q_start - k_start; delta = ORACLE_NONCAUSAL means all visible;
 *  - a row with no visible key has O = 0 and LSE = -inf;
 *  - LSE uses the natural logarithm;
 *  - grouped KV heads: query head h of Hq reads KV head floor(h*Hkv/Hq).
 *
 * Inputs are float32 arrays (bf16 and fp32 values are exact in float32);
 * every sum, product, exp and log is taken in double.  Layout is contiguous
 * [B][H][N][d].  Rows are independent, so most entry points take an optional
 * list of flat row indices ((b*Hq + h)*Nq + i) and compute only those.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_NONCAUSAL INT64_MAX

static int64_t kv_head_of(int64_t h, int64_t hq, int64_t hkv)
{
    return (h * hkv) / hq;
}

static int visible(int64_t i, int64_t j, int64_t delta)
{
    if (delta == ORACLE_NONCAUSAL)
        return 1;
    /* j <= i + delta, written without overflow for large |delta| */
    return (j - i) <= delta;
}

static double pick_scale(double scale, int64_t d)
{
    return scale > 0.0 ? scale : 1.0 / sqrt((double)d);
}

/*
 * Attention of one query row against an explicit list of key rows.
 * keys[t] are row indices into kb/vb (each of length d).  s is scratch of
 * length nkeys.  Writes o[d] and *lse.  An empty list gives O = 0, LSE = -inf.
 */
static void row_attention(const float *qrow, const float *kb, const float *vb,
                          const int64_t *keys, int64_t nkeys, int64_t d,
                          double sigma, double *s, double *o, double *lse)
{
    for (int64_t c = 0; c < d; ++c)
        o[c] = 0.0;
    if (nkeys == 0) {
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t t = 0; t < nkeys; ++t) {
        const float *krow = kb + keys[t] * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += (double)qrow[c] * (double)krow[c];
        s[t] = sigma * dot;
        if (s[t] > m)
            m = s[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < nkeys; ++t) {
        double p = exp(s[t] - m);
        l += p;
        const float *vrow = vb + keys[t] * d;
        for (int64_t c = 0; c < d; ++c)
            o[c] += p * (double)vrow[c];
    }
    for (int64_t c = 0; c < d; ++c)
        o[c] /= l;
    *lse = m + log(l);
}

/*
 * Merge of two partials over disjoint key sets:
 *   L = log(exp(La) + exp(Lb)),  O = exp(La - L) Oa + exp(Lb - L) Ob,
 * evaluated with the max shift.  (0, -inf) is the identity element; two
 * empty partials merge to (0, -inf).
 */
static void merge_row(const double *oa, double la, const double *ob, double lb,
                      int64_t d, double *o, double *l)
{
    if (la == -INFINITY && lb == -INFINITY) {
        for (int64_t c = 0; c < d; ++c)
            o[c] = 0.0;
        *l = -INFINITY;
        return;
    }
    double mx = la > lb ? la : lb;
    double wa = exp(la - mx), wb = exp(lb - mx);
    double tot = wa + wb;
    for (int64_t c = 0; c < d; ++c)
        o[c] = (wa * oa[c] + wb * ob[c]) / tot;
    *l = mx + log(tot);
}

/* ------------------------------------------------------------------------- */
/* Segment forward                                                           */
/* ------------------------------------------------------------------------- */

/*
 * oracle_attn_fwd: (O, LSE) of queries q[B][Hq][Nq][d] against k, v
 * [B][Hkv][Nk][d] with the visibility rule j <= i + delta.
 * rows: flat row ids to compute (NULL = all B*Hq*Nq rows, in order);
 * o_out[nrows][d], lse_out[nrows].
 */
void oracle_attn_fwd(const float *q, const float *k, const float *v,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                     int64_t Nk, int64_t d, int64_t delta, double scale,
                     const int64_t *rows, int64_t nrows,
                     double *o_out, double *lse_out)
{
    const double sigma = pick_scale(scale, d);
    if (rows == NULL)
        nrows = B * Hq * Nq;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (Nk > 0 ? Nk : 1));
        double *s = (double *)malloc(sizeof(double) * (Nk > 0 ? Nk : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t flat = rows ? rows[r] : r;
            const int64_t i = flat % Nq;
            const int64_t bh = flat / Nq;
            const int64_t b = bh / Hq, h = bh % Hq;
            const int64_t g = kv_head_of(h, Hq, Hkv);
            const float *kb = k + (b * Hkv + g) * Nk * d;
            const float *vb = v + (b * Hkv + g) * Nk * d;
            int64_t n = 0;
            for (int64_t j = 0; j < Nk; ++j)
                if (visible(i, j, delta))
                    keys[n++] = j;
            row_attention(q + flat * d, kb, vb, keys, n, d, sigma, s,
                          o_out + r * d, lse_out + r);
        }
        free(keys);
        free(s);
    }
}

/* ------------------------------------------------------------------------- */
/* Log-sum-exp merge                                                         */
/* ------------------------------------------------------------------------- */

void oracle_lse_merge(const double *oa, const double *la, const double *ob,
                      const double *lb, int64_t nrows, int64_t d,
                      double *o_out, double *lse_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r)
        merge_row(oa + r * d, la[r], ob + r * d, lb[r], d, o_out + r * d,
                  lse_out + r);
}

/* ------------------------------------------------------------------------- */
/* Dilated attention                                                         */
/* ------------------------------------------------------------------------- */

/* Key list of query p in a branch (segment length w, dilation r, offset s
 * inside the segment; causal keeps keys at original positions <= p).
 * Returns the count, or -1 if the branch does not select p. */
static int64_t dilated_keys(int64_t p, int64_t N, int64_t w, int64_t r,
                            int64_t s, int32_t causal, int64_t *keys)
{
    const int64_t seg0 = (p / w) * w;
    if (p - seg0 < s || (p - seg0 - s) % r != 0)
        return -1;
    int64_t n = 0;
    for (int64_t t = seg0 + s; t < seg0 + w && t < N; t += r)
        if (!causal || t <= p)
            keys[n++] = t;
    return n;
}

/*
 * oracle_dilated_fwd: for each branch b (segment length w[b], dilation
 * r[b]) a position p is selected iff (p mod w[b]) - s is a non-negative
 * multiple of r[b], where the offset s is 0, or h mod r[b] for query head h
 * when head_shift != 0 (LongNet's multi-head variant: heads spread over the
 * r[b] residue classes).  A selected query p attends to the keys of its
 * segment floor(p / w[b]) at the same offsets (and, when causal != 0, only
 * to keys at original positions <= p).  Each branch gives a partial
 * (O_b, LSE_b) -- (0, -inf) for an unselected p -- and the partials are
 * folded with the log-sum-exp merge in branch order.
 * q, k, v share the length N.  rows as in oracle_attn_fwd.
 */
void oracle_dilated_fwd(const float *q, const float *k, const float *v,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                        int64_t d, const int64_t *w, const int64_t *r,
                        int32_t nb, int32_t causal, int32_t head_shift,
                        double scale, const int64_t *rows, int64_t nrows,
                        double *o_out, double *lse_out)
{
    const double sigma = pick_scale(scale, d);
    if (rows == NULL)
        nrows = B * Hq * N;
    int64_t wmax = 1;
    for (int32_t b = 0; b < nb; ++b)
        if (w[b] > wmax)
            wmax = w[b];
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * wmax);
        double *s = (double *)malloc(sizeof(double) * wmax);
        double *ob = (double *)malloc(sizeof(double) * d);
        double *acc = (double *)malloc(sizeof(double) * d);
        double *tmp = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 4)
        for (int64_t rr = 0; rr < nrows; ++rr) {
            const int64_t flat = rows ? rows[rr] : rr;
            const int64_t p = flat % N;
            const int64_t bh = flat / N;
            const int64_t bt = bh / Hq, h = bh % Hq;
            const int64_t g = kv_head_of(h, Hq, Hkv);
            const float *kb = k + (bt * Hkv + g) * N * d;
            const float *vb = v + (bt * Hkv + g) * N * d;
            double lacc = -INFINITY, lb, lnew;
            for (int64_t c = 0; c < d; ++c)
                acc[c] = 0.0;
            for (int32_t b = 0; b < nb; ++b) {
                const int64_t off = head_shift ? h % r[b] : 0;
                const int64_t n = dilated_keys(p, N, w[b], r[b], off, causal, keys);
                if (n < 0)
                    continue; /* (0, -inf): the merge identity */
                row_attention(q + flat * d, kb, vb, keys, n, d, sigma, s, ob,
                              &lb);
                merge_row(acc, lacc, ob, lb, d, tmp, &lnew);
                memcpy(acc, tmp, sizeof(double) * d);
                lacc = lnew;
            }
            memcpy(o_out + rr * d, acc, sizeof(double) * d);
            lse_out[rr] = lacc;
        }
        free(keys);
        free(s);
        free(ob);
        free(acc);
        free(tmp);
    }
}

/* ------------------------------------------------------------------------- */
/* Backward                                                                  */
/* ------------------------------------------------------------------------- */

/*
 * Softmax statistics of one query row over all its visible keys:
 * returns LSE and fills o[d]; D = sum_c dO_c O_c is then formed by the
 * caller.  This is the same definition as the forward, evaluated in full.
 */
static void row_stats(const float *qrow, const float *kb, const float *vb,
                      int64_t i, int64_t Nk, int64_t d, int64_t delta,
                      double sigma, int64_t *keys, double *s, double *o,
                      double *lse)
{
    int64_t n = 0;
    for (int64_t j = 0; j < Nk; ++j)
        if (visible(i, j, delta))
            keys[n++] = j;
    row_attention(qrow, kb, vb, keys, n, d, sigma, s, o, lse);
}

/*
 * oracle_attn_bwd_rows: dQ for a list of query rows (rows as in
 * oracle_attn_fwd; NULL = all).  For each row i:
 *   P_ij = exp(s_ij - LSE_i), D_i = sum_c dO_ic O_ic,
 *   dQ_i = sigma * sum_j P_ij (dO_i . v_j - D_i) k_j.
 * Also returns the row's O and LSE (o_out, lse_out may be NULL).
 */
void oracle_attn_bwd_dq_rows(const float *q, const float *k, const float *v,
                             const float *dout, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                             int64_t delta, double scale, const int64_t *rows,
                             int64_t nrows, double *dq_out, double *o_out,
                             double *lse_out)
{
    const double sigma = pick_scale(scale, d);
    if (rows == NULL)
        nrows = B * Hq * Nq;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (Nk > 0 ? Nk : 1));
        double *s = (double *)malloc(sizeof(double) * (Nk > 0 ? Nk : 1));
        double *o = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t flat = rows ? rows[r] : r;
            const int64_t i = flat % Nq;
            const int64_t bh = flat / Nq;
            const int64_t b = bh / Hq, h = bh % Hq;
            const int64_t g = kv_head_of(h, Hq, Hkv);
            const float *kb = k + (b * Hkv + g) * Nk * d;
            const float *vb = v + (b * Hkv + g) * Nk * d;
            const float *qrow = q + flat * d;
            const float *dorow = dout + flat * d;
            double lse;
            row_stats(qrow, kb, vb, i, Nk, d, delta, sigma, keys, s, o, &lse);
            double D = 0.0;
            for (int64_t c = 0; c < d; ++c)
                D += (double)dorow[c] * o[c];
            double *dq = dq_out + r * d;
            for (int64_t c = 0; c < d; ++c)
                dq[c] = 0.0;
            for (int64_t j = 0; j < Nk; ++j) {
                if (!visible(i, j, delta))
                    continue;
                const float *krow = kb + j * d, *vrow = vb + j * d;
                double dot = 0.0, dp = 0.0;
                for (int64_t c = 0; c < d; ++c) {
                    dot += (double)qrow[c] * (double)krow[c];
                    dp += (double)dorow[c] * (double)vrow[c];
                }
                const double p = exp(sigma * dot - lse);
                const double ds = p * (dp - D);
                for (int64_t c = 0; c < d; ++c)
                    dq[c] += sigma * ds * (double)krow[c];
            }
            if (o_out)
                memcpy(o_out + r * d, o, sizeof(double) * d);
            if (lse_out)
                lse_out[r] = lse;
        }
        free(keys);
        free(s);
        free(o);
    }
}

/*
 * oracle_attn_bwd: full dQ [B][Hq][Nq][d], dK and dV [B][Hkv][Nk][d].
 *   dV_j = sum_i P_ij dO_i,
 *   dK_j = sigma * sum_i P_ij (dO_i . v_j - D_i) q_i,
 * summed over the query heads that share the KV head.  First every row's
 * LSE_i and D_i is formed, then dQ per query row, then dK, dV per key row.
 */
void oracle_attn_bwd(const float *q, const float *k, const float *v,
                     const float *dout, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nk, int64_t d, int64_t delta,
                     double scale, double *dq_out, double *dk_out,
                     double *dv_out)
{
    const double sigma = pick_scale(scale, d);
    const int64_t nq_rows = B * Hq * Nq;
    double *lse = (double *)malloc(sizeof(double) * (nq_rows > 0 ? nq_rows : 1));
    double *D = (double *)malloc(sizeof(double) * (nq_rows > 0 ? nq_rows : 1));
    double *otmp = (double *)malloc(sizeof(double) * (nq_rows > 0 ? nq_rows : 1) * d);

    oracle_attn_bwd_dq_rows(q, k, v, dout, B, Hq, Hkv, Nq, Nk, d, delta, scale,
                            NULL, nq_rows, dq_out, otmp, lse);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nq_rows; ++r) {
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c)
            acc += (double)dout[r * d + c] * otmp[r * d + c];
        D[r] = acc;
    }

    const int64_t nk_rows = B * Hkv * Nk;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t kr = 0; kr < nk_rows; ++kr) {
        const int64_t j = kr % Nk;
        const int64_t bg = kr / Nk;
        const int64_t b = bg / Hkv, g = bg % Hkv;
        const float *krow = k + kr * d, *vrow = v + kr * d;
        double *dk = dk_out + kr * d, *dv = dv_out + kr * d;
        for (int64_t c = 0; c < d; ++c)
            dk[c] = dv[c] = 0.0;
        for (int64_t h = 0; h < Hq; ++h) {
            if (kv_head_of(h, Hq, Hkv) != g)
                continue;
            for (int64_t i = 0; i < Nq; ++i) {
                if (!visible(i, j, delta))
                    continue;
                const int64_t qr = (b * Hq + h) * Nq + i;
                const float *qrow = q + qr * d, *dorow = dout + qr * d;
                double dot = 0.0, dp = 0.0;
                for (int64_t c = 0; c < d; ++c) {
                    dot += (double)qrow[c] * (double)krow[c];
                    dp += (double)dorow[c] * (double)vrow[c];
                }
                const double p = exp(sigma * dot - lse[qr]);
                const double ds = p * (dp - D[qr]);
                for (int64_t c = 0; c < d; ++c) {
                    dv[c] += p * (double)dorow[c];
                    dk[c] += sigma * ds * (double)qrow[c];
                }
            }
        }
    }
    free(lse);
    free(D);
    free(otmp);
}

int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* ------------------------------------------------------------------------- */
/* Dilated attention backward                                                */
/* ------------------------------------------------------------------------- */

/*
 * oracle_dilated_bwd: gradients of L = sum(dO * O) for the dilated attention
 * of oracle_dilated_fwd.  Folding branch partials with the log-sum-exp merge
 * is one softmax over the list of (branch, key) occurrences of query p, so
 * with the global O_p, LSE_p and D_p = dO_p . O_p, every occurrence (b, j)
 * contributes P = exp(s_pj - LSE_p), dS = P (dO_p . v_j - D_p):
 *   dV_j += P dO_p,  dQ_p += sigma dS k_j,  dK_j += sigma dS q_p.
 * Full outputs: dq [B][Hq][N][d], dk and dv [B][Hkv][N][d].
 */
void oracle_dilated_bwd(const float *q, const float *k, const float *v,
                        const float *dout, int64_t B, int64_t Hq, int64_t Hkv,
                        int64_t N, int64_t d, const int64_t *w, const int64_t *r,
                        int32_t nb, int32_t causal, int32_t head_shift,
                        double scale, double *dq_out, double *dk_out,
                        double *dv_out)
{
    const double sigma = pick_scale(scale, d);
    const int64_t nq_rows = B * Hq * N;
    double *o = (double *)malloc(sizeof(double) * (nq_rows > 0 ? nq_rows : 1) * d);
    double *lse = (double *)malloc(sizeof(double) * (nq_rows > 0 ? nq_rows : 1));
    double *D = (double *)malloc(sizeof(double) * (nq_rows > 0 ? nq_rows : 1));
    int64_t wmax = 1;
    for (int32_t b = 0; b < nb; ++b)
        if (w[b] > wmax)
            wmax = w[b];

    /* global O, LSE (the forward definition) and D per query row */
    oracle_dilated_fwd(q, k, v, B, Hq, Hkv, N, d, w, r, nb, causal, head_shift,
                       scale, NULL, nq_rows, o, lse);
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < nq_rows; ++row) {
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c)
            acc += (double)dout[row * d + c] * o[row * d + c];
        D[row] = acc;
    }

    /* dQ per query row */
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * wmax);
#pragma omp for schedule(dynamic, 4)
        for (int64_t row = 0; row < nq_rows; ++row) {
            const int64_t p = row % N, bh = row / N;
            const int64_t bt = bh / Hq, h = bh % Hq;
            const int64_t g = kv_head_of(h, Hq, Hkv);
            const float *qrow = q + row * d, *dorow = dout + row * d;
            double *dq = dq_out + row * d;
            for (int64_t c = 0; c < d; ++c)
                dq[c] = 0.0;
            for (int32_t b = 0; b < nb; ++b) {
                const int64_t off = head_shift ? h % r[b] : 0;
                const int64_t n = dilated_keys(p, N, w[b], r[b], off, causal, keys);
                for (int64_t t = 0; t < n; ++t) {
                    const float *krow = k + ((bt * Hkv + g) * N + keys[t]) * d;
                    const float *vrow = v + ((bt * Hkv + g) * N + keys[t]) * d;
                    double dot = 0.0, dp = 0.0;
                    for (int64_t c = 0; c < d; ++c) {
                        dot += (double)qrow[c] * (double)krow[c];
                        dp += (double)dorow[c] * (double)vrow[c];
                    }
                    const double P = exp(sigma * dot - lse[row]);
                    const double ds = P * (dp - D[row]);
                    for (int64_t c = 0; c < d; ++c)
                        dq[c] += sigma * ds * (double)krow[c];
                }
            }
        }
        free(keys);
    }

    /* dK, dV per key row: every (branch, query) that lists the key */
    const int64_t nk_rows = B * Hkv * N;
#pragma omp parallel
    {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * wmax);
#pragma omp for schedule(dynamic, 4)
        for (int64_t kr = 0; kr < nk_rows; ++kr) {
            const int64_t j = kr % N, bg = kr / N;
            const int64_t bt = bg / Hkv, g = bg % Hkv;
            const float *krow = k + kr * d, *vrow = v + kr * d;
            double *dk = dk_out + kr * d, *dv = dv_out + kr * d;
            for (int64_t c = 0; c < d; ++c)
                dk[c] = dv[c] = 0.0;
            for (int64_t h = 0; h < Hq; ++h) {
                if (kv_head_of(h, Hq, Hkv) != g)
                    continue;
                for (int32_t b = 0; b < nb; ++b) {
                    const int64_t seg0 = (j / w[b]) * w[b];
                    const int64_t off = head_shift ? h % r[b] : 0;
                    for (int64_t p = seg0; p < seg0 + w[b] && p < N; ++p) {
                        const int64_t n = dilated_keys(p, N, w[b], r[b], off, causal, keys);
                        int listed = 0;
                        for (int64_t t = 0; t < n; ++t)
                            if (keys[t] == j)
                                listed = 1;
                        if (!listed)
                            continue;
                        const int64_t row = (bt * Hq + h) * N + p;
                        const float *qrow = q + row * d, *dorow = dout + row * d;
                        double dot = 0.0, dp = 0.0;
                        for (int64_t c = 0; c < d; ++c) {
                            dot += (double)qrow[c] * (double)krow[c];
                            dp += (double)dorow[c] * (double)vrow[c];
                        }
                        const double P = exp(sigma * dot - lse[row]);
                        const double ds = P * (dp - D[row]);
                        for (int64_t c = 0; c < d; ++c) {
                            dv[c] += P * (double)dorow[c];
                            dk[c] += sigma * ds * (double)qrow[c];
                        }
                    }
                }
            }
        }
        free(keys);
    }
    free(o);
    free(lse);
    free(D);
}
