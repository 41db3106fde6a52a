/*
 * pkm_oracle.c -- plain, slow fp64 CPU oracle of the product-key memory layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the
 * package entry module and the CPU-baseline leg of the benchmark may load
 * this library.  The GPU library never calls it, and the two share no source,
 * header, table or helper: this file includes only the C standard library and
 * OpenMP.
 *
 * What it computes follows the pages' statement of the method:
 *
 *  - "Large Memory Layers with Product Keys" (gptget.net summary), section
 *    "Methodology" and the methodology list of its "Deep Analysis": the query q
 *    is split into halves q1, q2; two sub-key sets C and C' of n vectors of
 *    dimension d_k/2 each; the implied key set is their Cartesian product; the
 *    k keys of largest inner product are selected; the output is the weighted
 *    sum of their value rows; several heads are combined; every parameter is
 *    trained by backprop and only the selected slots get a value update.
 *  - "Product Keys Give Transformers Million-Slot Memory Layers", section
 *    "Implied keys vs stored sub-keys": key (i, j) is left sub-key i
 *    concatenated with right sub-key j, so its score against q is
 *    <q1, C_i> + <q2, C'_j>.
 *
 * The oracle does not use the product-key shortcut.  For every (token, head)
 * it scores ALL n*n implied keys (flat search, the baseline of section
 * "Search cost: flat vs product keys" of the second page), fully sorts them,
 * and keeps the first k.  That the shortcut reaches the same set (section
 * "Why top-k of each half is enough") is checked by the tests, not assumed.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *  - slot index of key (i, j) is f = i*n + j; q1 is the first d_k/2 entries;
 *  - order is (score descending, slot ascending) -- ties go to the lowest slot;
 *  - the weights are a softmax over the k selected scores of one head (the
 *    pages only say "weighted sum"); heads are summed into one output row and
 *    share one value table; every head has its own pair of codebooks;
 *  - the selection is a constant for the gradient: only the k selected scores
 *    carry gradient, each to its own left and right sub-key score.
 *
 * Array layouts (row-major, element offsets):
 *   q       [T][H][d_k]          left half = first d_k/2
 *   keys    [H][2][n][d_k/2]     [h][0] = C (left), [h][1] = C' (right)
 *   values  [n*n][d_v]           row f = i*n + j
 *   dy, y   [T][d_v]
 *   idx, scores, weights, dw, ds   [T][H][k]
 *   dq      [T][H][d_k];  dkeys [H][2][n][d_k/2];  dvalues [n*n][d_v]
 *
 * Input arrays carry a storage-type code: 0 = float32, 1 = bfloat16 (raw
 * 16-bit patterns), 2 = float64.  Every value is widened exactly to double
 * before any arithmetic; all arithmetic is in double.
 *
 * Return value: 0 on success, a negative code on bad arguments or non-finite
 * inputs (see ORC_E* below).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_OK = 0, ORC_EARG = -1, ORC_ENONFINITE = -2, ORC_ENOMEM = -3 };
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

/* Widen element i of an array stored with type code dt to double (exact). */
static double elem(const void *base, int dt, int64_t i)
{
    if (dt == ORC_F32)
        return (double)((const float *)base)[i];
    if (dt == ORC_BF16) {
        /* a bfloat16 is the upper 16 bits of a float32 */
        uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double *)base)[i];
}

static int dtype_ok(int dt) { return dt == ORC_F32 || dt == ORC_BF16 || dt == ORC_F64; }

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int pkm_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int check_finite(const void *a, int dt, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        if (!isfinite(elem(a, dt, i)))
            return 0;
    return 1;
}

/* Inner product of the left (s = 0) or right (s = 1) half of q[t][h] with
 * sub-key `i` of codebook s of head h. */
static double half_score(int64_t t, int h, int s, int i, int H, int n, int d_k,
                         const void *q, int q_dt, const void *keys, int k_dt)
{
    const int half = d_k / 2;
    const int64_t q_off = (t * H + h) * (int64_t)d_k + (int64_t)s * half;
    const int64_t k_off = (((int64_t)h * 2 + s) * n + i) * (int64_t)half;
    double acc = 0.0;
    for (int c = 0; c < half; ++c)
        acc += elem(q, q_dt, q_off + c) * elem(keys, k_dt, k_off + c);
    return acc;
}

/* Score of every implied key f = i*n + j for one (token, head):
 * out[f] = <q1, C_i> + <q2, C'_j>  (section "Implied keys vs stored sub-keys"). */
int pkm_oracle_flat_scores(int64_t t, int h, int64_t T, int H, int n, int d_k,
                           const void *q, int q_dt, const void *keys, int k_dt,
                           double *out)
{
    if (t < 0 || t >= T || h < 0 || h >= H || n < 1 || d_k < 2 || (d_k & 1) ||
        !dtype_ok(q_dt) || !dtype_ok(k_dt) || !q || !keys || !out)
        return ORC_EARG;
    double *left = malloc(sizeof(double) * (size_t)n);
    double *right = malloc(sizeof(double) * (size_t)n);
    if (!left || !right) {
        free(left);
        free(right);
        return ORC_ENOMEM;
    }
    for (int i = 0; i < n; ++i) {
        left[i] = half_score(t, h, 0, i, H, n, d_k, q, q_dt, keys, k_dt);
        right[i] = half_score(t, h, 1, i, H, n, d_k, q, q_dt, keys, k_dt);
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j)
            out[(int64_t)i * n + j] = left[i] + right[j];
    free(left);
    free(right);
    return ORC_OK;
}

typedef struct {
    double score;
    int32_t slot;
} scored_slot;

/* Total order used everywhere: higher score first; on equal scores the lower
 * slot index first. */
static int by_score_desc_slot_asc(const void *a, const void *b)
{
    const scored_slot *x = a, *y = b;
    if (x->score > y->score)
        return -1;
    if (x->score < y->score)
        return 1;
    return (x->slot > y->slot) - (x->slot < y->slot);
}

/* Softmax over the k scores of one head, shifted by their maximum. */
static void softmax(const double *s, int k, double *w)
{
    double m = s[0];
    for (int r = 1; r < k; ++r)
        if (s[r] > m)
            m = s[r];
    double z = 0.0;
    for (int r = 0; r < k; ++r) {
        w[r] = exp(s[r] - m);
        z += w[r];
    }
    for (int r = 0; r < k; ++r)
        w[r] /= z;
}

/* y[t] = sum over heads h and picks r of w[t][h][r] * values[idx[t][h][r]]. */
static void weighted_sum(int64_t t, int H, int k, int d_v, const int32_t *idx,
                         const double *w, const void *values, int v_dt, double *y)
{
    double *yt = y + t * (int64_t)d_v;
    for (int x = 0; x < d_v; ++x)
        yt[x] = 0.0;
    for (int h = 0; h < H; ++h)
        for (int r = 0; r < k; ++r) {
            const int64_t e = (t * H + h) * (int64_t)k + r;
            const int64_t row = (int64_t)idx[e] * d_v;
            for (int x = 0; x < d_v; ++x)
                yt[x] += w[e] * elem(values, v_dt, row + x);
        }
}

static int common_args_ok(int64_t T, int H, int n, int k, int d_k, int d_v)
{
    return T >= 0 && H >= 1 && n >= 1 && d_k >= 2 && !(d_k & 1) && d_v >= 1 &&
           k >= 1 && (int64_t)k <= (int64_t)n * n && (int64_t)n * n <= INT32_MAX;
}

/*
 * Forward pass by flat search.
 * Outputs idx, scores, weights [T][H][k] in (score desc, slot asc) order,
 * y [T][d_v], and for the parity rule the k-th and (k+1)-th largest flat
 * scores kth[T][H], kth1[T][H] (kth1 = -inf when k = n*n).  kth/kth1 may be
 * NULL.
 */
int pkm_oracle_forward(int64_t T, int H, int n, int k, int d_k, int d_v,
                       const void *q, int q_dt, const void *keys, int k_dt,
                       const void *values, int v_dt,
                       int32_t *idx, double *scores, double *weights, double *y,
                       double *kth, double *kth1, int nthreads)
{
    if (!common_args_ok(T, H, n, k, d_k, d_v) || !dtype_ok(q_dt) || !dtype_ok(k_dt) ||
        !dtype_ok(v_dt) || !q || !keys || !values || !idx || !scores || !weights || !y)
        return ORC_EARG;
    if (!check_finite(q, q_dt, T * H * (int64_t)d_k) ||
        !check_finite(keys, k_dt, (int64_t)H * 2 * n * (d_k / 2)))
        return ORC_ENONFINITE;
    set_threads(nthreads);
    const int64_t nn = (int64_t)n * n;
    int status = ORC_OK;

#pragma omp parallel
    {
        scored_slot *all = malloc(sizeof(scored_slot) * (size_t)nn);
        double *flat = malloc(sizeof(double) * (size_t)nn);
        if (!all || !flat) {
#pragma omp atomic write
            status = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            if (!all || !flat)
                continue;
            for (int h = 0; h < H; ++h) {
                pkm_oracle_flat_scores(t, h, T, H, n, d_k, q, q_dt, keys, k_dt, flat);
                for (int64_t f = 0; f < nn; ++f) {
                    all[f].score = flat[f];
                    all[f].slot = (int32_t)f;
                }
                qsort(all, (size_t)nn, sizeof(scored_slot), by_score_desc_slot_asc);
                const int64_t base = (t * H + h) * (int64_t)k;
                for (int r = 0; r < k; ++r) {
                    idx[base + r] = all[r].slot;
                    scores[base + r] = all[r].score;
                }
                softmax(scores + base, k, weights + base);
                if (kth)
                    kth[t * H + h] = all[k - 1].score;
                if (kth1)
                    kth1[t * H + h] = (k < nn) ? all[k].score : -INFINITY;
            }
            weighted_sum(t, H, k, d_v, idx, weights, values, v_dt, y);
        }
        free(all);
        free(flat);
    }
    return status;
}

/*
 * Forward pass on a GIVEN selection: scores of the listed slots recomputed
 * from their definition, softmax, weighted sum.  Used to judge a GPU result
 * whose selection legitimately differs from the oracle's at a near-tie.
 */
int pkm_oracle_forward_given_idx(int64_t T, int H, int n, int k, int d_k, int d_v,
                                 const void *q, int q_dt, const void *keys, int k_dt,
                                 const void *values, int v_dt, const int32_t *idx,
                                 double *scores, double *weights, double *y, int nthreads)
{
    if (!common_args_ok(T, H, n, k, d_k, d_v) || !dtype_ok(q_dt) || !dtype_ok(k_dt) ||
        !dtype_ok(v_dt) || !q || !keys || !values || !idx || !scores || !weights || !y)
        return ORC_EARG;
    const int64_t nn = (int64_t)n * n;
    for (int64_t e = 0; e < T * H * (int64_t)k; ++e)
        if (idx[e] < 0 || idx[e] >= nn)
            return ORC_EARG;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            const int64_t base = (t * H + h) * (int64_t)k;
            for (int r = 0; r < k; ++r) {
                const int f = idx[base + r];
                scores[base + r] = half_score(t, h, 0, f / n, H, n, d_k, q, q_dt, keys, k_dt) +
                                   half_score(t, h, 1, f % n, H, n, d_k, q, q_dt, keys, k_dt);
            }
            softmax(scores + base, k, weights + base);
        }
        weighted_sum(t, H, k, d_v, idx, weights, values, v_dt, y);
    }
    return ORC_OK;
}

/*
 * Backward pass for the loss L = sum_t <dy[t], y[t]>, given the selection
 * idx and weights of the forward pass.
 *   dw[t][h][r] = <dy[t], values[idx]>
 *   ds[t][h][r] = w_r * (dw_r - sum_r' w_r' dw_r')          (softmax backward)
 *   dvalues     = dense n*n x d_v array, zero except the selected rows, which
 *                 receive w * dy[t] for every pick (overwritten, not added)
 *   dS[t][h][s] = dense length-n vector: ds of every pick added at its left
 *                 index i (s = 0) and at its right index j (s = 1)
 *   dq[t][h][s] = sum_i dS[t][h][s][i] * C_s[i]            (all n sub-keys)
 *   dkeys[h][s][i] = sum_t dS[t][h][s][i] * q_s[t][h]       (all tokens)
 * Any of dq, dkeys, dvalues, dw, ds may be NULL to skip it (dq and dkeys
 * need ds internally all the same).
 */
int pkm_oracle_backward(int64_t T, int H, int n, int k, int d_k, int d_v,
                        const void *q, int q_dt, const void *keys, int k_dt,
                        const void *values, int v_dt, const int32_t *idx,
                        const double *weights, const void *dy, int dy_dt,
                        double *dq, double *dkeys, double *dvalues, double *dw_out,
                        double *ds_out, int nthreads)
{
    if (!common_args_ok(T, H, n, k, d_k, d_v) || !dtype_ok(q_dt) || !dtype_ok(k_dt) ||
        !dtype_ok(v_dt) || !dtype_ok(dy_dt) || !q || !keys || !values || !idx ||
        !weights || !dy)
        return ORC_EARG;
    const int64_t nn = (int64_t)n * n;
    const int64_t picks = T * H * (int64_t)k;
    for (int64_t e = 0; e < picks; ++e)
        if (idx[e] < 0 || idx[e] >= nn)
            return ORC_EARG;
    if (!check_finite(dy, dy_dt, T * (int64_t)d_v))
        return ORC_ENONFINITE;
    set_threads(nthreads);
    const int half = d_k / 2;

    double *dw = malloc(sizeof(double) * (size_t)(picks > 0 ? picks : 1));
    double *ds = malloc(sizeof(double) * (size_t)(picks > 0 ? picks : 1));
    double *dS = calloc((size_t)(T * H * 2 * (int64_t)n + 1), sizeof(double));
    if (!dw || !ds || !dS) {
        free(dw);
        free(ds);
        free(dS);
        return ORC_ENOMEM;
    }

    /* dw and the softmax backward, one (token, head) at a time */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            const int64_t base = (t * H + h) * (int64_t)k;
            double wdw = 0.0;
            for (int r = 0; r < k; ++r) {
                const int64_t row = (int64_t)idx[base + r] * d_v;
                double acc = 0.0;
                for (int x = 0; x < d_v; ++x)
                    acc += elem(dy, dy_dt, t * d_v + x) * elem(values, v_dt, row + x);
                dw[base + r] = acc;
                wdw += weights[base + r] * acc;
            }
            for (int r = 0; r < k; ++r)
                ds[base + r] = weights[base + r] * (dw[base + r] - wdw);
        }
    }

    /* route every pick's ds to its two sub-keys (dense dS) */
    for (int64_t t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h)
            for (int r = 0; r < k; ++r) {
                const int64_t e = (t * H + h) * (int64_t)k + r;
                const int f = idx[e];
                dS[((t * H + h) * 2 + 0) * (int64_t)n + f / n] += ds[e];
                dS[((t * H + h) * 2 + 1) * (int64_t)n + f % n] += ds[e];
            }

    if (dvalues) {
        memset(dvalues, 0, sizeof(double) * (size_t)(nn * d_v));
        for (int64_t t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h)
                for (int r = 0; r < k; ++r) {
                    const int64_t e = (t * H + h) * (int64_t)k + r;
                    double *row = dvalues + (int64_t)idx[e] * d_v;
                    for (int x = 0; x < d_v; ++x)
                        row[x] += weights[e] * elem(dy, dy_dt, t * d_v + x);
                }
    }

    if (dq) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h)
                for (int s = 0; s < 2; ++s) {
                    const double *g = dS + ((t * H + h) * 2 + s) * (int64_t)n;
                    double *out = dq + (t * H + h) * (int64_t)d_k + (int64_t)s * half;
                    for (int c = 0; c < half; ++c) {
                        double acc = 0.0;
                        for (int i = 0; i < n; ++i)
                            acc += g[i] * elem(keys, k_dt, (((int64_t)h * 2 + s) * n + i) * half + c);
                        out[c] = acc;
                    }
                }
    }

    if (dkeys) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t row = 0; row < (int64_t)H * 2 * n; ++row) {
            const int h = (int)(row / (2 * (int64_t)n));
            const int s = (int)((row / n) % 2);
            const int i = (int)(row % n);
            double *out = dkeys + row * half;
            for (int c = 0; c < half; ++c)
                out[c] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double g = dS[((t * H + h) * 2 + s) * (int64_t)n + i];
                const int64_t q_off = (t * H + h) * (int64_t)d_k + (int64_t)s * half;
                for (int c = 0; c < half; ++c)
                    out[c] += g * elem(q, q_dt, q_off + c);
            }
        }
    }

    if (dw_out)
        memcpy(dw_out, dw, sizeof(double) * (size_t)picks);
    if (ds_out)
        memcpy(ds_out, ds, sizeof(double) * (size_t)picks);
    free(dw);
    free(ds);
    free(dS);
    return ORC_OK;
}
