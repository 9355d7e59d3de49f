/*
 * fmha_oracle.c -- plain, slow, fp64 CPU attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker for the HIP library,
 * not part of it: only the tests, the smoke check and the bench's CPU
 * baseline leg load it.  It shares no code, header, table or helper with
 * the GPU path and includes nothing from it.
 *
 * What it computes (written from the pages' problem statement, not from
 * any kernel):
 *
 *   For batch b, query head h, query row i (0 <= i < T):
 *     kv      = h / (n_h / n_kv_h)                 (contiguous GQA groups;
 *                                                    MQA = one KV head, or a
 *                                                    K/V head stride of 0)
 *     pos_i   = s_k - T + i                        (queries are the last T
 *                                                    positions of the sequence)
 *     key j is visible iff  lo <= j < hi  and  j < s_k
 *                      and (causal == 0 or j <= pos_i)
 *                      and (window == 0 or j > pos_i - window)
 *     s_j     = scale * sum_d q[d] * k_j[d]        (the dot product is taken
 *                                                    unscaled and the scale is
 *                                                    applied afterwards: page 2,
 *                                                    "Key lessons")
 *     m       = max_j s_j,  p_j = exp(s_j - m),  l = sum_j p_j
 *     O[d]    = sum_j p_j * v_j[d] / l             (page 2, "What's working":
 *                                                    QK -> softmax -> PV)
 *     lse     = m + ln(l)                          (natural log)
 *   A row with no visible key gets O = 0 and lse = -inf.
 *
 *   Split partitions (page 2, "Next steps" item 4): partition p covers keys
 *   [p*split_len, min((p+1)*split_len, s_k)); each partition is the same
 *   definition restricted to its range.  The merge is the D5 formula
 *   O = sum_p exp(lse_p) O_p / sum_p exp(lse_p), evaluated with the common
 *   factor exp(max_p lse_p) taken out so that it does not overflow; the
 *   merged lse is ln(sum_p exp(lse_p)).
 *
 * Inputs are bf16 bit patterns (uint16_t); each is widened exactly to
 * double.  scale arrives as a float (the value the GPU receives) and is
 * widened exactly.  All arithmetic is double; libm's exp and log.
 *
 * Strides are in elements, three per tensor: batch, token, head.  The head
 * dimension is contiguous.  Outputs are dense:
 *   o   [batch][T][n_h][hd]            lse  [batch][n_h][T]
 *   o_part [batch][n_h][T][n_split][hd]   lse_part [batch][n_h][T][n_split]
 *
 * Work is split over (batch, head) units across threads; each unit is
 * computed by exactly one thread in a fixed order, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v;
    int batch, n_h, n_kv_h, T, s_k, hd;
    int64_t qs[3], ks[3], vs[3];
    double scale;
    int window, causal;
    /* key range restriction: [lo, hi) per partition, n_split partitions of
     * split_len keys each (n_split == 1, split_len >= s_k: plain attention) */
    int split_len, n_split;
    /* outputs: exactly one of (o, lse) / (o_part, lse_part) / w is used */
    double *o, *lse, *o_part, *lse_part, *w;
    int next_unit;
    pthread_mutex_t lock;
} job_t;

static int key_visible(const job_t *J, int i, int j, int lo, int hi) {
    int pos = J->s_k - J->T + i;
    if (j < lo || j >= hi || j >= J->s_k) return 0;
    if (J->causal && j > pos) return 0;
    if (J->window > 0 && j <= pos - J->window) return 0;
    return 1;
}

/* One query row over keys [lo, hi): writes O (hd doubles), lse, and,
 * if wrow != NULL, the full weight row p_j / l (exact 0 for masked keys). */
static void one_row(const job_t *J, int b, int h, int i, int lo, int hi,
                    double *s_buf, double *orow, double *lse_out, double *wrow) {
    const int hd = J->hd;
    const int kv = h / (J->n_h / J->n_kv_h);
    const uint16_t *qp = J->q + b * J->qs[0] + (int64_t)i * J->qs[1] + h * J->qs[2];
    double m = -INFINITY;
    int any = 0;
    for (int j = 0; j < J->s_k; ++j) {
        if (!key_visible(J, i, j, lo, hi)) continue;
        const uint16_t *kp = J->k + b * J->ks[0] + (int64_t)j * J->ks[1] + kv * J->ks[2];
        double dot = 0.0;
        for (int d = 0; d < hd; ++d) dot += bf16_to_double(qp[d]) * bf16_to_double(kp[d]);
        s_buf[j] = J->scale * dot;
        if (!any || s_buf[j] > m) m = s_buf[j];
        any = 1;
    }
    for (int d = 0; d < hd; ++d) orow[d] = 0.0;
    if (wrow)
        for (int j = 0; j < J->s_k; ++j) wrow[j] = 0.0;
    if (!any) {
        *lse_out = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int j = 0; j < J->s_k; ++j) {
        if (!key_visible(J, i, j, lo, hi)) continue;
        double p = exp(s_buf[j] - m);
        s_buf[j] = p;
        l += p;
        const uint16_t *vp = J->v + b * J->vs[0] + (int64_t)j * J->vs[1] + kv * J->vs[2];
        for (int d = 0; d < hd; ++d) orow[d] += p * bf16_to_double(vp[d]);
    }
    for (int d = 0; d < hd; ++d) orow[d] /= l;
    if (wrow)
        for (int j = 0; j < J->s_k; ++j)
            if (key_visible(J, i, j, lo, hi)) wrow[j] = s_buf[j] / l;
    *lse_out = m + log(l);
}

static void run_unit(const job_t *J, int unit, double *s_buf) {
    const int b = unit / J->n_h, h = unit % J->n_h;
    const int T = J->T, hd = J->hd, ns = J->n_split;
    for (int i = 0; i < T; ++i) {
        if (J->o_part) {
            for (int p = 0; p < ns; ++p) {
                int lo = p * J->split_len;
                int hi = lo + J->split_len < J->s_k ? lo + J->split_len : J->s_k;
                int64_t r = (((int64_t)b * J->n_h + h) * T + i) * ns + p;
                one_row(J, b, h, i, lo, hi, s_buf, J->o_part + r * hd, J->lse_part + r, NULL);
            }
        } else {
            double lse;
            double *orow = J->o + (((int64_t)b * T + i) * J->n_h + h) * hd;
            double *wrow = J->w ? J->w + (((int64_t)b * J->n_h + h) * T + i) * J->s_k : NULL;
            one_row(J, b, h, i, 0, J->s_k, s_buf, orow, &lse, wrow);
            if (J->lse) J->lse[((int64_t)b * J->n_h + h) * T + i] = lse;
        }
    }
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    double *s_buf = (double *)malloc(sizeof(double) * (size_t)J->s_k);
    if (!s_buf) return (void *)1;
    const int units = J->batch * J->n_h;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int u = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (u >= units) break;
        run_unit(J, u, s_buf);
    }
    free(s_buf);
    return NULL;
}

static int check_dims(int batch, int n_h, int n_kv_h, int T, int s_k, int hd) {
    if (batch <= 0 || n_h <= 0 || n_kv_h <= 0 || T <= 0 || s_k <= 0 || hd <= 0) return 1;
    if (n_h % n_kv_h != 0) return 1;
    return 0;
}

static int run_job(job_t *J, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    J->next_unit = 0;
    pthread_mutex_init(&J->lock, NULL);
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, J) != 0) break;
        ++started;
    }
    if (worker(J) != NULL) rc = 3;
    for (int t = 1; t <= started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret != NULL) rc = 3;
    }
    pthread_mutex_destroy(&J->lock);
    return rc;
}

static void fill_job(job_t *J, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                     const int64_t *q_st, const int64_t *k_st, const int64_t *v_st,
                     float scale, int window, int causal) {
    memset(J, 0, sizeof *J);
    J->q = q; J->k = k; J->v = v;
    J->batch = batch; J->n_h = n_h; J->n_kv_h = n_kv_h;
    J->T = T; J->s_k = s_k; J->hd = hd;
    for (int x = 0; x < 3; ++x) { J->qs[x] = q_st[x]; J->ks[x] = k_st[x]; J->vs[x] = v_st[x]; }
    J->scale = (double)scale;
    J->window = window; J->causal = causal;
    J->split_len = s_k; J->n_split = 1;
}

/* Full attention.  Returns 0 on success, 1 on bad arguments, 3 on thread
 * or allocation failure.  lse may be NULL. */
int oracle_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     double *o, double *lse,
                     int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                     const int64_t *q_st, const int64_t *k_st, const int64_t *v_st,
                     float scale, int window, int causal, int nthreads) {
    if (!q || !k || !v || !o || check_dims(batch, n_h, n_kv_h, T, s_k, hd) || window < 0) return 1;
    job_t J;
    fill_job(&J, q, k, v, batch, n_h, n_kv_h, T, s_k, hd, q_st, k_st, v_st, scale, window, causal);
    J.o = o; J.lse = lse;
    return run_job(&J, nthreads);
}

/* Per-partition attention: o_part [batch][n_h][T][n_split][hd], lse_part
 * [batch][n_h][T][n_split], n_split = ceil(s_k / split_len).  A partition
 * with no visible key gets O_p = 0 and lse_p = -inf. */
int oracle_split(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                 double *o_part, double *lse_part,
                 int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                 const int64_t *q_st, const int64_t *k_st, const int64_t *v_st,
                 float scale, int window, int causal, int split_len, int nthreads) {
    if (!q || !k || !v || !o_part || !lse_part || check_dims(batch, n_h, n_kv_h, T, s_k, hd) ||
        window < 0 || split_len <= 0)
        return 1;
    job_t J;
    fill_job(&J, q, k, v, batch, n_h, n_kv_h, T, s_k, hd, q_st, k_st, v_st, scale, window, causal);
    J.split_len = split_len;
    J.n_split = (s_k + split_len - 1) / split_len;
    J.o_part = o_part; J.lse_part = lse_part;
    return run_job(&J, nthreads);
}

/* The D5 merge of n_split partials per row (rows = batch*n_h*T, dense).
 * o [rows][hd], lse [rows] (lse may be NULL).  Partials with lse = -inf
 * carry zero weight; if all are -inf the row is O = 0, lse = -inf. */
int oracle_merge(const double *o_part, const double *lse_part, double *o, double *lse,
                 int rows, int hd, int n_split) {
    if (!o_part || !lse_part || !o || rows <= 0 || hd <= 0 || n_split <= 0) return 1;
    for (int r = 0; r < rows; ++r) {
        const double *lp = lse_part + (int64_t)r * n_split;
        const double *op = o_part + (int64_t)r * n_split * hd;
        double *orow = o + (int64_t)r * hd;
        double mx = -INFINITY;
        for (int p = 0; p < n_split; ++p)
            if (lp[p] > mx) mx = lp[p];
        for (int d = 0; d < hd; ++d) orow[d] = 0.0;
        if (mx == -INFINITY) {
            if (lse) lse[r] = -INFINITY;
            continue;
        }
        double den = 0.0;
        for (int p = 0; p < n_split; ++p) {
            if (lp[p] == -INFINITY) continue;
            double wgt = exp(lp[p] - mx);
            den += wgt;
            for (int d = 0; d < hd; ++d) orow[d] += wgt * op[(int64_t)p * hd + d];
        }
        for (int d = 0; d < hd; ++d) orow[d] /= den;
        if (lse) lse[r] = mx + log(den);
    }
    return 0;
}

/* Debug entry for tiny shapes: the full softmax weight row p_j / l per
 * (b, h, i), w [batch][n_h][T][s_k], exactly 0.0 at masked keys. */
int oracle_weights(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   double *w, int batch, int n_h, int n_kv_h, int T, int s_k, int hd,
                   const int64_t *q_st, const int64_t *k_st, const int64_t *v_st,
                   float scale, int window, int causal) {
    if (!q || !k || !v || !w || check_dims(batch, n_h, n_kv_h, T, s_k, hd) || window < 0) return 1;
    double *o = (double *)malloc(sizeof(double) * (size_t)batch * T * n_h * hd);
    if (!o) return 3;
    job_t J;
    fill_job(&J, q, k, v, batch, n_h, n_kv_h, T, s_k, hd, q_st, k_st, v_st, scale, window, causal);
    J.o = o; J.w = w;
    int rc = run_job(&J, 1);
    free(o);
    return rc;
}
