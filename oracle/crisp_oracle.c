/*
 * CRISP sparse-prefill oracle: a plain, slow CPU implementation written from
 * the paper "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
 * Structural-Mass-Motivated Routing" (arXiv 2609.01925).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP library never
 * links, includes or calls it, and it shares no source with that library.
 *
 * Arithmetic: bf16 inputs are widened exactly; every score, softmax, sum and
 * attention output is computed in IEEE double.  Where a floating-point value
 * decides an integer result (the routing bit, a selected block, the PE
 * cut-off), the decision is taken on the value rounded to float, with the
 * threshold formula evaluated in float in the order the paper writes it --
 * the precision the GPU kernels decide in.
 *
 * Layouts: Q is [hq][n][d], K and V are [hkv][n][d], row-major bf16 bit
 * patterns (uint16).  Query head h reads KV head h / (hq / hkv).
 *
 * Pins: every function here is checked by tests against brute force in numpy,
 * closed forms and invariants (see the test-suite); none is "parity unpinned".
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the OpenMP loops below run on. */
int orc_threads(void) { return omp_get_max_threads(); }

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Widen one [n][d] slab of bf16 to float (exact). */
static float *widen(const uint16_t *src, int64_t count)
{
    float *dst = (float *)malloc((size_t)count * sizeof(float));
    if (!dst) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) dst[i] = bf16_to_f32(src[i]);
    return dst;
}

static double dot(const float *a, const float *b, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += (double)a[c] * (double)b[c];
    return s;
}

/*
 * Proxy attention of one query head (Alg. 2): the representative
 * query block Q^ is the last R = min(b, n) query rows (b = B); A^ =
 * Softmax(Q^ K^T / sqrt(d)).  Causal reading: row i sits at position
 * q_i = n - R + i and sees keys k <= q_i; entries with k > q_i are exactly 0.
 * Output ahat is [R][n], doubles.
 */
static void proxy_rows(const float *qh, const float *kg, int n, int d, int R, double *ahat)
{
    const double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < R; ++i) {
        const int64_t qi = (int64_t)n - R + i;
        const float *qrow = qh + qi * d;
        double *row = ahat + (int64_t)i * n;
        double m = -INFINITY;
        for (int64_t k = 0; k <= qi; ++k) {
            double s = scale * dot(qrow, kg + k * d, d);
            row[k] = s;
            if (s > m) m = s;
        }
        double l = 0.0;
        for (int64_t k = 0; k <= qi; ++k) {
            row[k] = exp(row[k] - m);
            l += row[k];
        }
        for (int64_t k = 0; k <= qi; ++k) row[k] /= l;
        for (int64_t k = qi + 1; k < n; ++k) row[k] = 0.0;
    }
}

/*
 * Directional block scores (Alg. 3) and C_struct (Eq. 2).
 * Blocks partition the n tokens into N_b = ceil(n / B) blocks (Section 4.3);
 * the last one holds n - (N_b - 1) B tokens.
 *   a_v = colmean(A^): a_v[k] = (1/R) sum_i A^[i,k]
 *   a_s = diagmean(A^): entry (i,k) lies on the diagonal of offset
 *         o = q_i - k >= 0; diagonals are grouped into offset blocks
 *         floor(o / B), and slash block j is offset block N_b - 1 - j, so
 *         slash block N_b - 1 is the recency band (offsets 0 .. B-1) and
 *         slash block 0 the farthest diagonals (the sink region).
 *   p_d = blockpool(a_d): sum over the positions of each block.
 *   C_struct = (1/R) sum_i sum_{k in anchor} A^[i,k], anchor = the first
 *              and the last block (the w_sink = w_local = B windows of
 *              Section 4.3), one block when N_b = 1.
 */
static void block_scores(const double *ahat, int n, int B, int R, double *pv, double *ps,
                         double *cstruct)
{
    const int nb = (n + B - 1) / B;
#pragma omp parallel for schedule(static)
    for (int j = 0; j < nb; ++j) {
        double sv = 0.0, ss = 0.0;
        for (int i = 0; i < R; ++i) {
            const int64_t qi = (int64_t)n - R + i;
            const double *row = ahat + (int64_t)i * n;
            /* key block j: keys jB .. min(jB + B, n) - 1 (zero past q_i) */
            for (int64_t k = (int64_t)j * B; k < (int64_t)(j + 1) * B && k < n; ++k) sv += row[k];
            /* slash block j: offsets (Nb-1-j)B .. (Nb-j)B - 1, keys q_i - o >= 0 */
            for (int64_t o = (int64_t)(nb - 1 - j) * B; o < (int64_t)(nb - j) * B && o <= qi; ++o)
                ss += row[qi - o];
        }
        pv[j] = sv / R;
        ps[j] = ss / R;
    }
    double cs = 0.0;
    const int64_t last0 = (int64_t)(nb - 1) * B;
    for (int i = 0; i < R; ++i) {
        const double *row = ahat + (int64_t)i * n;
        for (int64_t k = 0; k < n; ++k)
            if (k < B || k >= last0) cs += row[k];
    }
    *cstruct = cs / R;
}

/* Single-head proxy map, exported for the brute-force pins; ahat is [R][n]. */
int orc_proxy_map(const uint16_t *q, const uint16_t *k, int n, int hq, int hkv, int d, int B,
                  int h, double *ahat)
{
    if (n < 1 || B < 1 || hq % hkv || h < 0 || h >= hq) return 1;
    const int g = h / (hq / hkv), R = n < B ? n : B;
    float *qh = widen(q + (int64_t)h * n * d, (int64_t)n * d);
    float *kg = widen(k + (int64_t)g * n * d, (int64_t)n * d);
    if (!qh || !kg) { free(qh); free(kg); return 2; }
    proxy_rows(qh, kg, n, d, R, ahat);
    free(qh);
    free(kg);
    return 0;
}

/* ahat is [R][n] with R = min(B, n); the anchor windows must equal B. */
int orc_block_scores(const double *ahat, int n, int B, int w_sink, int w_local,
                     double *pv, double *ps, double *cstruct)
{
    if (n < 1 || B < 1 || w_sink != B || w_local != B) return 1;
    block_scores(ahat, n, B, n < B ? n : B, pv, ps, cstruct);
    return 0;
}

/*
 * PatSearch (Alg. 2) for every query head: proxy map, block scores,
 * C_struct (Eq. 2) and the routing rule "VS iff C_struct >= tau_proxy"
 * (Alg. 2), the comparison taken in float.
 * pattern: 1 = VS, 0 = PE.  p_v and p_s are [hq][N_b].
 */
int orc_route(const uint16_t *q, const uint16_t *k, int n, int hq, int hkv, int d, int B,
              float tau, int w_sink, int w_local,
              double *pv, double *ps, double *cstruct, uint8_t *pattern)
{
    if (n < 1 || B < 1 || hq % hkv || w_sink != B || w_local != B) return 1;
    const int nb = (n + B - 1) / B, G = hq / hkv, R = n < B ? n : B;
    double *ahat = (double *)malloc((size_t)R * n * sizeof(double));
    float *qlast = (float *)malloc((size_t)n * d * sizeof(float));
    if (!ahat || !qlast) { free(ahat); free(qlast); return 2; }
    for (int g = 0; g < hkv; ++g) {
        float *kg = widen(k + (int64_t)g * n * d, (int64_t)n * d);
        if (!kg) { free(ahat); free(qlast); return 2; }
        for (int h = g * G; h < (g + 1) * G; ++h) {
            /* only the last R query rows are read; widen those */
            const uint16_t *qh = q + (int64_t)h * n * d;
            for (int64_t e = (int64_t)(n - R) * d; e < (int64_t)n * d; ++e)
                qlast[e] = bf16_to_f32(qh[e]);
            proxy_rows(qlast, kg, n, d, R, ahat);
            block_scores(ahat, n, B, R, pv + (int64_t)h * nb, ps + (int64_t)h * nb, cstruct + h);
            pattern[h] = ((float)cstruct[h] >= tau) ? 1 : 0;
        }
        free(kg);
    }
    free(ahat);
    free(qlast);
    return 0;
}

/*
 * FlexPrefill's pattern search (Alg. 5), the routing CRISP replaces:
 *   abar = Softmax(pool(Q^) pool(K)^T / sqrt(d)) over the N_b key blocks,
 *          pool(Q^) the mean of the R = min(B, n) representative rows and
 *          pool(K) the per-block key means (over the tokens each block holds);
 *   ahat = sumpool(Softmax(Q^ K^T / sqrt(d))) = p_v (per-query mean, pooled);
 *   D_JS = sqrt(KL(ahat||m) / 2 + KL(abar||m) / 2), m = (ahat + abar) / 2,
 *          natural logarithms, 0 log 0 = 0.
 * pv holds the head's p_v (from orc_route); returns D_JS in *djs.  The
 * routing bit "VS iff D_JS >= tau" is taken in float by the caller.
 */
int orc_jsd(const uint16_t *q, const uint16_t *k, int n, int hq, int hkv, int d, int B, int h,
            const double *pv, double *djs)
{
    if (n < 1 || B < 1 || hq % hkv || h < 0 || h >= hq) return 1;
    const int nb = (n + B - 1) / B, g = h / (hq / hkv), R = n < B ? n : B;
    const double scale = 1.0 / sqrt((double)d);
    double *qbar = (double *)calloc((size_t)d, sizeof(double));
    double *abar = (double *)malloc((size_t)nb * sizeof(double));
    if (!qbar || !abar) { free(qbar); free(abar); return 2; }
    const uint16_t *qh = q + (int64_t)h * n * d, *kg = k + (int64_t)g * n * d;
    for (int i = 0; i < R; ++i)
        for (int c = 0; c < d; ++c) qbar[c] += (double)bf16_to_f32(qh[((int64_t)n - R + i) * d + c]);
    for (int c = 0; c < d; ++c) qbar[c] /= R;
    double m = -INFINITY;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < nb; ++b) {
        const int len = (b == nb - 1) ? n - b * B : B;
        double s = 0.0;
        for (int c = 0; c < d; ++c) {
            double kb = 0.0;
            for (int t = 0; t < len; ++t) kb += (double)bf16_to_f32(kg[((int64_t)b * B + t) * d + c]);
            s += qbar[c] * (kb / len);
        }
        abar[b] = scale * s;
    }
    for (int b = 0; b < nb; ++b) if (abar[b] > m) m = abar[b];
    double l = 0.0;
    for (int b = 0; b < nb; ++b) { abar[b] = exp(abar[b] - m); l += abar[b]; }
    double kl_hat = 0.0, kl_bar = 0.0;
    for (int b = 0; b < nb; ++b) {
        abar[b] /= l;
        const double mb = 0.5 * (pv[b] + abar[b]);
        if (pv[b] > 0.0) kl_hat += pv[b] * log(pv[b] / mb);
        if (abar[b] > 0.0) kl_bar += abar[b] * log(abar[b] / mb);
    }
    double js = 0.5 * kl_hat + 0.5 * kl_bar;
    *djs = sqrt(js > 0.0 ? js : 0.0);
    free(qbar);
    free(abar);
    return 0;
}

/* ---- ordering helpers: (value desc, index asc) on float-rounded values ---- */
typedef struct { float v; int64_t i; } vi_t;

static int cmp_desc(const void *a, const void *b)
{
    const vi_t *x = (const vi_t *)a, *y = (const vi_t *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->i < y->i) ? -1 : (x->i > y->i);
}

static int cmp_int(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/*
 * Budget and top-k shared by both noise floors (Alg. 3; Eq. 4):
 *   k = #{j : p[j] > theta}, counted over all Nb blocks
 *   k = clip(k, k_min, Nb);  S = top-k(p), ties to the lower block index.
 * pf holds p rounded to float.  Writes S ascending to sel, returns |S|.
 */
static int floor_topk(const float *pf, int nb, float theta, int kmin, int32_t *sel,
                      float *kth_out, int *clipped_out)
{
    vi_t *ord = (vi_t *)malloc((size_t)nb * sizeof(vi_t));
    int count = 0;
    for (int j = 0; j < nb; ++j) count += (pf[j] > theta);
    int kk = count < kmin ? kmin : count;
    if (kk > nb) kk = nb;
    for (int j = 0; j < nb; ++j) { ord[j].v = pf[j]; ord[j].i = j; }
    qsort(ord, nb, sizeof(vi_t), cmp_desc);
    for (int t = 0; t < kk; ++t) sel[t] = (int32_t)ord[t].i;
    qsort(sel, kk, sizeof(int32_t), cmp_int);
    *kth_out = ord[kk - 1].v;
    *clipped_out = (count < kk);
    free(ord);
    return kk;
}

/*
 * Sink-aware selection in one direction (Alg. 3; Eq. 3 and 4):
 *   r = max(1 - p[0] - p[Nb-1], 0);  mu = r / (Nb - 2);  theta = alpha * mu
 *   then floor_topk.  All in float, in that order.  theta_out receives
 *   theta and kth_out the k-th largest value (the decisive value when the
 *   clip binds).  Nb <= 2 (mu undefined): every block is selected.
 */
int orc_vs_select(const double *p, int nb, float alpha, int kmin, int32_t *sel,
                  float *theta_out, float *kth_out, int *clipped_out)
{
    if (nb <= 2) {
        for (int j = 0; j < nb; ++j) sel[j] = j;
        *theta_out = 0.0f;
        *kth_out = 0.0f;
        *clipped_out = 0;
        return nb;
    }
    float *pf = (float *)malloc((size_t)nb * sizeof(float));
    for (int j = 0; j < nb; ++j) pf[j] = (float)p[j];
    float r = 1.0f - pf[0];
    r = r - pf[nb - 1];
    if (r < 0.0f) r = 0.0f;
    float mu = r / (float)(nb - 2);
    float theta = alpha * mu;
    *theta_out = theta;
    int kk = floor_topk(pf, nb, theta, kmin, sel, kth_out, clipped_out);
    free(pf);
    return kk;
}

static int cmp_float(const void *a, const void *b)
{
    float x = *(const float *)a, y = *(const float *)b;
    return (x > y) - (x < y);
}

/*
 * The median noise floor of Appendix H ("Median instead of mean as the noise
 * floor"): the floor is the median of the non-retained blocks 1 .. Nb-2
 * instead of their mean r / (Nb - 2); for an even count the mean of the two
 * middle values.  theta = alpha * median, then floor_topk.  In float.
 */
int orc_vs_select_median(const double *p, int nb, float alpha, int kmin, int32_t *sel,
                         float *theta_out, float *kth_out, int *clipped_out)
{
    if (nb <= 2) return orc_vs_select(p, nb, alpha, kmin, sel, theta_out, kth_out, clipped_out);
    const int m = nb - 2;
    float *pf = (float *)malloc((size_t)nb * sizeof(float));
    float *mid = (float *)malloc((size_t)m * sizeof(float));
    for (int j = 0; j < nb; ++j) pf[j] = (float)p[j];
    for (int j = 0; j < m; ++j) mid[j] = pf[j + 1];
    qsort(mid, m, sizeof(float), cmp_float);
    const float med = (m & 1) ? mid[m / 2] : (mid[m / 2 - 1] + mid[m / 2]) * 0.5f;
    const float theta = alpha * med;
    *theta_out = theta;
    int kk = floor_topk(pf, nb, theta, kmin, sel, kth_out, clipped_out);
    free(pf);
    free(mid);
    return kk;
}

/*
 * Cumulative-gamma selection in one direction, the FlexPrefill rule the
 * paper compares against (Alg. 6): p already sums to one, order
 * it (desc, ties to the lower index), keep the shortest prefix whose
 * running sum reaches gamma.  kmin > 0 additionally clips the size to at
 * least kmin (FlexPrefill as configured in Section 5, "Setup").
 */
int orc_gamma_select(const double *p, int nb, float gamma, int kmin, int32_t *sel)
{
    vi_t *ord = (vi_t *)malloc((size_t)nb * sizeof(vi_t));
    for (int j = 0; j < nb; ++j) { ord[j].v = (float)p[j]; ord[j].i = j; }
    qsort(ord, nb, sizeof(vi_t), cmp_desc);
    double cum = 0.0;
    int kk = nb;
    for (int t = 0; t < nb; ++t) {
        cum += (double)ord[t].v;
        if (cum >= (double)gamma) { kk = t + 1; break; }
    }
    if (kk < kmin) kk = kmin < nb ? kmin : nb;
    for (int t = 0; t < kk; ++t) sel[t] = (int32_t)ord[t].i;
    qsort(sel, kk, sizeof(int32_t), cmp_int);
    free(ord);
    return kk;
}

/*
 * Pooled map of one query head for the PE path (Alg. 4):
 *   Qbar[qb] = mean of Q over the tokens of query block qb (all queries; the
 *              last block may hold fewer than B),
 *   Kbar[kb] = mean of K over key block kb,
 *   Abar = row softmax of Qbar Kbar^T / sqrt(d) over the causal key blocks
 *          kb <= qb (entries kb > qb are 0),
 *   Abar = Abar / sum(Abar).
 * abar is [Nb][Nb], doubles.
 */
int orc_pe_map(const uint16_t *q, const uint16_t *k, int n, int hq, int hkv, int d, int B,
               int h, double *abar)
{
    if (n < 1 || B < 1 || hq % hkv || h < 0 || h >= hq) return 1;
    const int nb = (n + B - 1) / B, g = h / (hq / hkv);
    const double scale = 1.0 / sqrt((double)d);
    double *qbar = (double *)calloc((size_t)nb * d, sizeof(double));
    double *kbar = (double *)calloc((size_t)nb * d, sizeof(double));
    if (!qbar || !kbar) { free(qbar); free(kbar); return 2; }
    const uint16_t *qh = q + (int64_t)h * n * d, *kg = k + (int64_t)g * n * d;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < nb; ++b) {
        const int len = (b == nb - 1) ? n - b * B : B;   /* tokens in block b */
        for (int t = 0; t < len; ++t) {
            int64_t pos = (int64_t)b * B + t;
            for (int c = 0; c < d; ++c) {
                qbar[(int64_t)b * d + c] += (double)bf16_to_f32(qh[pos * d + c]);
                kbar[(int64_t)b * d + c] += (double)bf16_to_f32(kg[pos * d + c]);
            }
        }
        for (int c = 0; c < d; ++c) {
            qbar[(int64_t)b * d + c] /= len;
            kbar[(int64_t)b * d + c] /= len;
        }
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (int qb = 0; qb < nb; ++qb) {
        double *row = abar + (int64_t)qb * nb;
        double m = -INFINITY;
        for (int kb = 0; kb <= qb; ++kb) {
            double s = 0.0;
            for (int c = 0; c < d; ++c) s += qbar[(int64_t)qb * d + c] * kbar[(int64_t)kb * d + c];
            row[kb] = scale * s;
            if (row[kb] > m) m = row[kb];
        }
        double l = 0.0;
        for (int kb = 0; kb <= qb; ++kb) { row[kb] = exp(row[kb] - m); l += row[kb]; }
        for (int kb = 0; kb <= qb; ++kb) row[kb] /= l;
        for (int kb = qb + 1; kb < nb; ++kb) row[kb] = 0.0;
    }
    double total = 0.0;
    for (int64_t e = 0; e < (int64_t)nb * nb; ++e) total += abar[e];
    for (int64_t e = 0; e < (int64_t)nb * nb; ++e) abar[e] /= total;
    free(qbar);
    free(kbar);
    return 0;
}

/*
 * gamma-cumsum over the flattened pooled map (Alg. 4):
 * order the causal entries by (value desc, flat index qb*Nb+kb asc) on the
 * float-rounded values, K* = min{k : running sum >= gamma}, S = first K*.
 * selmask[qb*Nb+kb] = 1 for the selected entries.  Returns K*; vstar gets
 * the K*-th value and cum_before the running sum of the first K*-1 entries.
 */
int64_t orc_pe_select(const double *abar, int nb, float gamma, uint8_t *selmask,
                      float *vstar, double *cum_before)
{
    const int64_t ncausal = (int64_t)nb * (nb + 1) / 2;
    vi_t *ord = (vi_t *)malloc((size_t)ncausal * sizeof(vi_t));
    int64_t t = 0;
    for (int qb = 0; qb < nb; ++qb)
        for (int kb = 0; kb <= qb; ++kb) {
            ord[t].v = (float)abar[(int64_t)qb * nb + kb];
            ord[t].i = (int64_t)qb * nb + kb;
            ++t;
        }
    qsort(ord, ncausal, sizeof(vi_t), cmp_desc);
    double cum = 0.0, before = 0.0;
    int64_t kstar = ncausal;
    for (t = 0; t < ncausal; ++t) {
        before = cum;
        cum += (double)ord[t].v;
        if (cum >= (double)gamma) { kstar = t + 1; break; }
    }
    memset(selmask, 0, (size_t)nb * nb);
    for (t = 0; t < kstar; ++t) selmask[ord[t].i] = 1;
    *vstar = ord[kstar - 1].v;
    *cum_before = before;
    free(ord);
    return kstar;
}

/*
 * Block index lists of one head: the mask M_S of Eq. 1 at block level.
 * VS (Alg. 3): S_v holds key-block columns; S_s holds slash blocks,
 *   slash block j being the diagonal band of offset block Nb-1-j, which for
 *   query block qb lands on key block qb-(Nb-1-j); {0, Nb-1} are the sink
 *   column and the recency diagonal (key block qb).
 *   R(qb) = sorted unique {0, qb} u {v in S_v : v <= qb}
 *           u {qb-(Nb-1-j) : j in S_s, qb-(Nb-1-j) >= 0}.
 * PE (Alg. 4 plus the first and last blocks, as VS):
 *   R(qb) = {kb : selmask[qb][kb]} u {0, qb}.
 * row_ptr gets Nb+1 offsets starting at base; returns the entry count.
 */
int64_t orc_expand(int nb, int vs, const int32_t *sv, int nv, const int32_t *ss, int ns,
                   const uint8_t *pe_mask, int64_t base, int32_t *row_ptr, int32_t *col_idx)
{
    uint8_t *mark = (uint8_t *)malloc((size_t)nb);
    int64_t pos = base;
    for (int qb = 0; qb < nb; ++qb) {
        memset(mark, 0, (size_t)nb);
        mark[0] = 1;
        mark[qb] = 1;
        if (vs) {
            for (int t = 0; t < nv; ++t)
                if (sv[t] <= qb) mark[sv[t]] = 1;
            for (int t = 0; t < ns; ++t) {
                int kb = qb - (nb - 1 - ss[t]);
                if (kb >= 0) mark[kb] = 1;
            }
        } else {
            for (int kb = 0; kb <= qb; ++kb)
                if (pe_mask[(int64_t)qb * nb + kb]) mark[kb] = 1;
        }
        row_ptr[qb] = (int32_t)pos;
        for (int kb = 0; kb <= qb; ++kb)
            if (mark[kb]) col_idx[pos++] = kb;
    }
    row_ptr[nb] = (int32_t)pos;
    free(mark);
    return pos - base;
}

/*
 * Masked attention, Eq. 1: O = Softmax(Q K^T / sqrt(d) + M_S) V, where for a
 * query at position t in block qb the allowed keys are the tokens of the
 * listed key blocks that are not in its future (k <= t).
 * row_ptr is [hq][Nb+1] (absolute offsets into col_idx); rows lists the
 * (h*Nb + qb) query blocks to compute; out is [nrows][B][d] doubles (rows of
 * positions >= n in a partial last block are left 0).  Keys k >= n do not
 * exist: k <= t < n excludes them.
 */
int orc_attend(const uint16_t *q, const uint16_t *k, const uint16_t *v, int n, int hq, int hkv,
               int d, int B, const int32_t *row_ptr, const int32_t *col_idx,
               const int32_t *rows, int nrows, double *out)
{
    if (n < 1 || B < 1 || hq % hkv) return 1;
    const int nb = (n + B - 1) / B, G = hq / hkv;
    const double scale = 1.0 / sqrt((double)d);
    for (int g = 0; g < hkv; ++g) {
        int any = 0;
        for (int r = 0; r < nrows; ++r) any |= (rows[r] / nb) / G == g;
        if (!any) continue;
        float *kg = widen(k + (int64_t)g * n * d, (int64_t)n * d);
        float *vg = widen(v + (int64_t)g * n * d, (int64_t)n * d);
        if (!kg || !vg) { free(kg); free(vg); return 2; }
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
        for (int r = 0; r < nrows; ++r) {
            for (int t = 0; t < B; ++t) {
                const int h = rows[r] / nb, qb = rows[r] % nb;
                if (h / G != g) continue;
                const int64_t qpos = (int64_t)qb * B + t;
                double *o = out + ((int64_t)r * B + t) * d;
                if (qpos >= n) {                 /* past the end: rows are 0 */
                    for (int c = 0; c < d; ++c) o[c] = 0.0;
                    continue;
                }
                float qrow[1024];
                const uint16_t *qsrc = q + ((int64_t)h * n + qpos) * d;
                for (int c = 0; c < d; ++c) qrow[c] = bf16_to_f32(qsrc[c]);
                const int32_t *list = col_idx + row_ptr[h * (nb + 1) + qb];
                const int len = row_ptr[h * (nb + 1) + qb + 1] - row_ptr[h * (nb + 1) + qb];
                double m = -INFINITY;
                for (int e = 0; e < len; ++e)
                    for (int c = 0; c < B; ++c) {
                        int64_t key = (int64_t)list[e] * B + c;
                        if (key > qpos) continue;
                        double s = scale * dot(qrow, kg + key * d, d);
                        if (s > m) m = s;
                    }
                double l = 0.0;
                for (int c = 0; c < d; ++c) o[c] = 0.0;
                for (int e = 0; e < len; ++e)
                    for (int c = 0; c < B; ++c) {
                        int64_t key = (int64_t)list[e] * B + c;
                        if (key > qpos) continue;
                        double w = exp(scale * dot(qrow, kg + key * d, d) - m);
                        l += w;
                        const float *vr = vg + key * d;
                        for (int x = 0; x < d; ++x) o[x] += w * (double)vr[x];
                    }
                for (int x = 0; x < d; ++x) o[x] /= l;
            }
        }
        free(kg);
        free(vg);
    }
    return 0;
}

/*
 * Eq. 1 for individual queries: qsel lists (h, position) pairs; out is
 * [nsel][d] doubles.  Same arithmetic as orc_attend, one query at a time,
 * for sampled checks of long sequences.
 */
int orc_attend_queries(const uint16_t *q, const uint16_t *k, const uint16_t *v, int n, int hq,
                       int hkv, int d, int B, const int32_t *row_ptr, const int32_t *col_idx,
                       const int32_t *qsel, int nsel, double *out)
{
    if (n < 1 || B < 1 || hq % hkv || d > 1024) return 1;
    const int nb = (n + B - 1) / B, G = hq / hkv;
    const double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nsel; ++r) {
        const int h = qsel[2 * r], g = h / G;
        const int64_t qpos = qsel[2 * r + 1];
        const int qb = (int)(qpos / B);
        const uint16_t *kg = k + (int64_t)g * n * d, *vg = v + (int64_t)g * n * d;
        float qrow[1024];
        const uint16_t *qsrc = q + ((int64_t)h * n + qpos) * d;
        for (int c = 0; c < d; ++c) qrow[c] = bf16_to_f32(qsrc[c]);
        const int32_t *list = col_idx + row_ptr[h * (nb + 1) + qb];
        const int len = row_ptr[h * (nb + 1) + qb + 1] - row_ptr[h * (nb + 1) + qb];
        double m = -INFINITY;
        for (int e = 0; e < len; ++e)
            for (int c = 0; c < B; ++c) {
                const int64_t key = (int64_t)list[e] * B + c;
                if (key > qpos) continue;
                double s = 0.0;
                for (int x = 0; x < d; ++x) s += (double)qrow[x] * (double)bf16_to_f32(kg[key * d + x]);
                s *= scale;
                if (s > m) m = s;
            }
        double l = 0.0;
        double *o = out + (int64_t)r * d;
        for (int x = 0; x < d; ++x) o[x] = 0.0;
        for (int e = 0; e < len; ++e)
            for (int c = 0; c < B; ++c) {
                const int64_t key = (int64_t)list[e] * B + c;
                if (key > qpos) continue;
                double s = 0.0;
                for (int x = 0; x < d; ++x) s += (double)qrow[x] * (double)bf16_to_f32(kg[key * d + x]);
                const double w = exp(scale * s - m);
                l += w;
                for (int x = 0; x < d; ++x) o[x] += w * (double)bf16_to_f32(vg[key * d + x]);
            }
        for (int x = 0; x < d; ++x) o[x] /= l;
    }
    return 0;
}
