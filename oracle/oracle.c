/*
 * oracle.c -- plain CPU reference for the routed MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): loaded by the tests, the package
 * smoke check and the benchmark's CPU-baseline leg, never by the product path.
 * Shares no code with the HIP library.
 *
 * The method reaches plain definitions (a linear map, a sigmoid, a top-k by
 * value, a normalisation, an elementwise activation, a weighted sum), so each
 * function below is that definition written out in double precision, in the
 * order the pages give the steps ([glm5next] "MoE FFN" and "What Executes vs.
 * TODO"):
 *   1. logits z = W_router x + b                    (bias inside the sigmoid)
 *   2. top-8 of sigmoid(z) over the 288 experts      (= top-8 of z, ties -> lower id)
 *   3. weights normalised to sum to one
 *   4. per selected expert: gate and up projections, clamped SwiGLU
 *      (gate clamped to at most 10 then SiLU, up clamped to [-10, 10];
 *      [glm5next] "Architecture"), down projection
 *   5. one always-on shared expert (same clamped SwiGLU), added with weight 1
 *      to the weighted sum of the routed expert outputs.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_E_ARG (-1)
#define ORC_E_MEM (-2)

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ */
/* scalar helpers                                                      */
/* ------------------------------------------------------------------ */

/* Logistic sigmoid, evaluated so that neither branch overflows. */
double oracle_sigmoid(double z)
{
    if (z >= 0.0)
        return 1.0 / (1.0 + exp(-z));
    double e = exp(z);
    return e / (1.0 + e);
}

/* SiLU(a) = a * sigmoid(a). */
double oracle_silu(double a)
{
    return a * oracle_sigmoid(a);
}

/* Clamped SwiGLU of one (gate, up) pair ([glm5next] "Architecture"):
 * the gate is limited from above at 10 (no lower limit) before the SiLU,
 * the up value is limited to the closed interval [-10, 10]. */
double oracle_swiglu(double g, double u)
{
    double gc = g > 10.0 ? 10.0 : g;
    double uc = u;
    if (uc > 10.0) uc = 10.0;
    if (uc < -10.0) uc = -10.0;
    return oracle_silu(gc) * uc;
}

/* bf16 bit pattern -> double (exact: bf16 is the top half of an fp32). */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16 bit pattern -> double (exact), decoded field by field. */
double oracle_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)mant, -24);               /* subnormal: mant * 2^-24 */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(mant + 1024), expo - 25); /* (1024+mant) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* Round a double to the nearest bf16 (ties to even), directly from the double
 * (no intermediate fp32 rounding).  bf16 keeps 8 significant bits and fp32's
 * exponent range; the smallest subnormal is 2^-133. */
uint16_t oracle_bf16_from_double(double v)
{
    if (isnan(v)) return 0x7fc0;
    double a = fabs(v);
    double q;
    if (a == 0.0) {
        q = 0.0;
    } else {
        int e;
        frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
        int quantum_exp = e - 8;      /* 8 significant bits */
        if (quantum_exp < -133) quantum_exp = -133;
        q = ldexp(nearbyint(ldexp(a, -quantum_exp)), quantum_exp);   /* RNE */
    }
    uint16_t bits;
    if (q >= ldexp(1.0, 128)) {
        bits = 0x7f80;                /* overflow to infinity */
    } else {
        float f = (float)q;           /* exact: q has at most 8 significant bits */
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        bits = (uint16_t)(u >> 16);
    }
    if (signbit(v)) bits |= 0x8000;
    return bits;
}

double oracle_mat_elem(const orc_mat *a, int64_t m, int64_t rows, int64_t K,
                       int64_t row, int64_t k)
{
    int64_t r = m * rows + row;
    switch (a->kind) {
    case ORC_F32:
        return (double)((const float *)a->data)[r * K + k];
    case ORC_BF16:
        return oracle_bf16_to_double(((const uint16_t *)a->data)[r * K + k]);
    case ORC_INT4: {
        uint8_t byte = ((const uint8_t *)a->data)[r * (K / 2) + k / 2];
        int nib = (k & 1) ? (byte >> 4) : (byte & 0x0f);
        double s = oracle_fp16_to_double(a->scales[r * (K / a->group) + k / a->group]);
        return (double)(nib - 8) * s;
    }
    default:
        return NAN;
    }
}

static int mat_ok(const orc_mat *a, int64_t K)
{
    if (!a || !a->data) return 0;
    if (a->kind == ORC_INT4)
        return a->scales && a->group > 0 && K % a->group == 0 && K % 2 == 0;
    return a->kind == ORC_F32 || a->kind == ORC_BF16;
}

/* Widen row `row` of a [rows][K] operand into a double vector. */
static void widen_row(const orc_mat *a, int64_t m, int64_t rows, int64_t K,
                      int64_t row, double *out)
{
    for (int64_t k = 0; k < K; ++k)
        out[k] = oracle_mat_elem(a, m, rows, K, row, k);
}

/* dot(W[m][row][:], v) with the index ascending. */
static double dot_row(const orc_mat *a, int64_t m, int64_t rows, int64_t K,
                      int64_t row, const double *v)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += oracle_mat_elem(a, m, rows, K, row, k) * v[k];
    return acc;
}

/* ------------------------------------------------------------------ */
/* 1. router logits                                                    */
/* ------------------------------------------------------------------ */

int oracle_router_logits(int64_t T, int64_t D, int64_t E, const orc_mat *x,
                         const orc_mat *wr, const float *bias, double *z)
{
    if (T < 0 || D <= 0 || E <= 0 || !mat_ok(x, D) || !mat_ok(wr, D) || !bias || !z)
        return ORC_E_ARG;
    int64_t t;
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < T; ++t) {
        double *xr = (double *)malloc((size_t)D * sizeof(double));
        if (!xr) continue;
        widen_row(x, 0, T, D, t, xr);
        for (int64_t e = 0; e < E; ++e)
            z[t * E + e] = dot_row(wr, 0, E, D, e, xr) + (double)bias[e];
        free(xr);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* 2-4. selection, sigmoid, normalisation, canonical order             */
/* ------------------------------------------------------------------ */

/* a ranks before b: larger logit first, then lower expert index. */
static int ranks_before(double za, int64_t a, double zb, int64_t b)
{
    if (za > zb) return 1;
    if (za < zb) return 0;
    return a < b;
}

int oracle_select_topk(int64_t T, int64_t E, int K, const double *z,
                       int32_t *ids, double *w)
{
    if (T < 0 || E <= 0 || K <= 0 || K > E || !z || !ids || !w)
        return ORC_E_ARG;
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        const double *zt = z + t * E;
        char *taken = (char *)calloc((size_t)E, 1);
        int64_t *pick = (int64_t *)malloc((size_t)K * sizeof(int64_t));
        if (!taken || !pick) { free(taken); free(pick); continue; }
        /* K passes; each pass takes the best expert not yet taken. */
        for (int j = 0; j < K; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(zt[e], e, zt[best], best)) best = e;
            }
            taken[best] = 1;
            pick[j] = best;
        }
        /* canonical order: ascending expert id (insertion sort of K ids) */
        for (int a = 1; a < K; ++a) {
            int64_t v = pick[a];
            int b = a - 1;
            while (b >= 0 && pick[b] > v) { pick[b + 1] = pick[b]; --b; }
            pick[b + 1] = v;
        }
        double psum = 0.0;
        for (int j = 0; j < K; ++j) psum += oracle_sigmoid(zt[pick[j]]);
        for (int j = 0; j < K; ++j) {
            ids[t * K + j] = (int32_t)pick[j];
            w[t * K + j] = oracle_sigmoid(zt[pick[j]]) / psum;
        }
        free(taken);
        free(pick);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* routing bookkeeping (stable counting sort)                          */
/* ------------------------------------------------------------------ */

int oracle_permutation(int64_t T, int64_t E, int K, const int32_t *ids,
                       int32_t *count, int32_t *offset, int32_t *perm, int32_t *inv)
{
    if (T < 0 || E <= 0 || K <= 0 || !ids || !count || !offset || !perm || !inv)
        return ORC_E_ARG;
    for (int64_t e = 0; e < E; ++e) count[e] = 0;
    for (int64_t i = 0; i < T * K; ++i) {
        if (ids[i] < 0 || ids[i] >= E) return ORC_E_ARG;
        count[ids[i]]++;
    }
    offset[0] = 0;
    for (int64_t e = 0; e < E; ++e) offset[e + 1] = offset[e] + count[e];
    /* walk experts in order, and within an expert tokens in order */
    int64_t row = 0;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t t = 0; t < T; ++t)
            for (int j = 0; j < K; ++j)
                if (ids[t * K + j] == e) {
                    perm[row] = (int32_t)(t * K + j);
                    inv[t * K + j] = (int32_t)row;
                    ++row;
                }
    return 0;
}

/* ------------------------------------------------------------------ */
/* 5. expert FFN                                                       */
/* ------------------------------------------------------------------ */

int oracle_expert_hidden(int64_t D, int64_t F, const double *xrow,
                         const orc_mat *gate, const orc_mat *up, int64_t n_mat,
                         int64_t e, double *h)
{
    if (!xrow || !h || !mat_ok(gate, D) || !mat_ok(up, D) || e < 0 || e >= n_mat)
        return ORC_E_ARG;
    for (int64_t f = 0; f < F; ++f) {
        double g = dot_row(gate, e, F, D, f, xrow);
        double u = dot_row(up, e, F, D, f, xrow);
        h[f] = oracle_swiglu(g, u);
    }
    return 0;
}

int oracle_expert_down(int64_t D, int64_t F, const double *h, const orc_mat *down,
                       int64_t n_mat, int64_t e, double *o)
{
    if (!h || !o || !mat_ok(down, F) || e < 0 || e >= n_mat)
        return ORC_E_ARG;
    for (int64_t d = 0; d < D; ++d)
        o[d] = dot_row(down, e, D, F, d, h);
    return 0;
}

int oracle_moe_ffn(int64_t T, int64_t D, int64_t E, int K, int64_t F,
                   const orc_mat *x, const int32_t *ids, const double *w,
                   const orc_mat *gate, const orc_mat *up, const orc_mat *down,
                   const orc_mat *s_gate, const orc_mat *s_up, const orc_mat *s_down,
                   const double *residual, const int64_t *tokens, int64_t n_tokens,
                   double *y)
{
    if (T < 0 || D <= 0 || E <= 0 || K <= 0 || F <= 0 || !ids || !w || !y)
        return ORC_E_ARG;
    if (!mat_ok(x, D) || !mat_ok(gate, D) || !mat_ok(up, D) || !mat_ok(down, F) ||
        !mat_ok(s_gate, D) || !mat_ok(s_up, D) || !mat_ok(s_down, F))
        return ORC_E_ARG;
    if (!tokens) n_tokens = T;
    int bad = 0;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (i = 0; i < n_tokens; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        if (t < 0 || t >= T) { bad = 1; continue; }
        double *xr = (double *)malloc((size_t)D * sizeof(double));
        double *h = (double *)malloc((size_t)F * sizeof(double));
        double *o = (double *)malloc((size_t)D * sizeof(double));
        double *acc = y + i * D;
        if (!xr || !h || !o) { bad = 1; free(xr); free(h); free(o); continue; }
        widen_row(x, 0, T, D, t, xr);
        /* shared expert, weight one */
        oracle_expert_hidden(D, F, xr, s_gate, s_up, 1, 0, h);
        oracle_expert_down(D, F, h, s_down, 1, 0, o);
        for (int64_t d = 0; d < D; ++d) acc[d] = o[d];
        /* routed experts in the stored (ascending id) order */
        for (int j = 0; j < K; ++j) {
            int64_t e = ids[t * K + j];
            if (e < 0 || e >= E) { bad = 1; break; }
            oracle_expert_hidden(D, F, xr, gate, up, E, e, h);
            oracle_expert_down(D, F, h, down, E, e, o);
            double wj = w[t * K + j];
            for (int64_t d = 0; d < D; ++d) acc[d] += wj * o[d];
        }
        if (residual)
            for (int64_t d = 0; d < D; ++d) acc[d] = residual[t * D + d] + acc[d];
        free(xr);
        free(h);
        free(o);
    }
    return bad ? ORC_E_ARG : 0;
}

/* ------------------------------------------------------------------ */
/* stacked chain, one layer                                             */
/* ------------------------------------------------------------------ */

int oracle_residual_layer(int64_t n, int64_t D, int64_t E, int K, int64_t F,
                          const double *x, const orc_mat *wr, const float *bias,
                          const orc_mat *gate, const orc_mat *up, const orc_mat *down,
                          const orc_mat *s_gate, const orc_mat *s_up, const orc_mat *s_down,
                          uint16_t *xin_bf16, int32_t *ids, double *w, double *z,
                          double *y, double *x_next)
{
    if (n < 0 || !x || !xin_bf16 || !ids || !w || !y || !x_next) return ORC_E_ARG;
    for (int64_t i = 0; i < n * D; ++i) xin_bf16[i] = oracle_bf16_from_double(x[i]);
    orc_mat xin = { ORC_BF16, xin_bf16, NULL, 0 };
    double *zz = z ? z : (double *)malloc((size_t)(n * E > 0 ? n * E : 1) * sizeof(double));
    if (!zz) return ORC_E_MEM;
    int rc = oracle_router_logits(n, D, E, &xin, wr, bias, zz);
    if (rc == 0) rc = oracle_select_topk(n, E, K, zz, ids, w);
    if (rc == 0)
        rc = oracle_moe_ffn(n, D, E, K, F, &xin, ids, w, gate, up, down,
                            s_gate, s_up, s_down, NULL, NULL, n, y);
    if (rc == 0)
        for (int64_t i = 0; i < n * D; ++i) x_next[i] = x[i] + y[i];
    if (!z) free(zz);
    return rc;
}

/* ------------------------------------------------------------------ */
/* dense FFN (layers without experts)                                  */
/* ------------------------------------------------------------------ */

int oracle_dense_ffn(int64_t T, int64_t D, int64_t F, const orc_mat *x,
                     const orc_mat *gate, const orc_mat *up, const orc_mat *down,
                     const double *residual, double *y)
{
    if (T < 0 || D <= 0 || F <= 0 || !y || !mat_ok(x, D) || !mat_ok(gate, D) ||
        !mat_ok(up, D) || !mat_ok(down, F))
        return ORC_E_ARG;
    int bad = 0;
    int64_t t;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (t = 0; t < T; ++t) {
        double *xr = (double *)malloc((size_t)D * sizeof(double));
        double *h = (double *)malloc((size_t)F * sizeof(double));
        if (!xr || !h) { bad = 1; free(xr); free(h); continue; }
        widen_row(x, 0, T, D, t, xr);
        oracle_expert_hidden(D, F, xr, gate, up, 1, 0, h);
        oracle_expert_down(D, F, h, down, 1, 0, y + t * D);
        if (residual)
            for (int64_t d = 0; d < D; ++d) y[t * D + d] = residual[t * D + d] + y[t * D + d];
        free(xr);
        free(h);
    }
    return bad ? ORC_E_ARG : 0;
}

/* ------------------------------------------------------------------ */
/* index selection (top-k over indexer scores, tail always kept)       */
/* ------------------------------------------------------------------ */

typedef struct {
    int tail;      /* 1: one of the always-selected last positions */
    double score;
    int64_t pos;
} orc_cand;

/* a ranks before b: tail positions first, then larger score, then lower position */
static int cand_cmp(const void *pa, const void *pb)
{
    const orc_cand *a = (const orc_cand *)pa, *b = (const orc_cand *)pb;
    if (a->tail != b->tail) return a->tail ? -1 : 1;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->pos < b->pos) ? -1 : (a->pos > b->pos);
}

static int pos_cmp(const void *pa, const void *pb)
{
    const int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

int oracle_index_topk(int64_t rows, int64_t L, int64_t ld, const float *scores,
                      const int32_t *lens, int64_t k, int64_t tail, int32_t *idx)
{
    if (rows < 0 || L < 0 || ld < L || k <= 0 || tail < 0 || (rows > 0 && (!scores || !idx)))
        return ORC_E_ARG;
    int bad = 0;
    int64_t r;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (r = 0; r < rows; ++r) {
        int64_t n = L;
        if (lens) {
            if (lens[r] < 0) { bad = 1; continue; }
            if (lens[r] < n) n = lens[r];
        }
        int32_t *out = idx + r * k;
        if (n <= k) {
            for (int64_t j = 0; j < k; ++j) out[j] = j < n ? (int32_t)j : -1;
            continue;
        }
        orc_cand *c = (orc_cand *)malloc((size_t)n * sizeof(orc_cand));
        if (!c) { bad = 1; continue; }
        const int64_t nt = tail < k ? tail : k;
        for (int64_t i = 0; i < n; ++i) {
            c[i].tail = i >= n - nt;
            c[i].score = (double)scores[r * ld + i];
            c[i].pos = i;
        }
        qsort(c, (size_t)n, sizeof(orc_cand), cand_cmp);
        for (int64_t j = 0; j < k; ++j) out[j] = (int32_t)c[j].pos;
        qsort(out, (size_t)k, sizeof(int32_t), pos_cmp);
        free(c);
    }
    return bad ? ORC_E_ARG : 0;
}
