/*
 * oracle.h -- plain CPU reference ("oracle") for the routed mixture-of-experts
 * FFN layer of GLM-5.3-Flash-style models.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the HIP path.  Only
 * the test suite, the package smoke check and the CPU-baseline leg of the
 * benchmark may load or call it; the product path never does.  It shares no
 * code, header, table or constant with the GPU library (include/coli_moe.h and
 * the package's csrc/), and neither side includes the other.
 *
 * Pages cited (short names used throughout this directory):
 *   [glm5next]  "Add GLM-5.3-Flash (glm5next) support with ROCmFP mix qtypes
 *               (105/106)" -- sections "Architecture", "MoE FFN",
 *               "What Executes vs. TODO".
 *   [glm53-hip] "feat(glm53): add device-resident HIP backend for MI350P" --
 *               sections "Key changes", "Validation results".
 *   [glm5next-prod] "GLM5next Production Readiness: Optional Mix Qtypes +
 *               Cache Allocation" -- section "Architecture".
 *
 * Everything is computed in IEEE double precision with plain loops, in the
 * order the definitions state (ascending reduction index), no BLAS, no
 * blocking.  Inputs are taken in the exact encoding the GPU receives (fp32,
 * bf16 bits, or packed int4 + fp16 scale bits) and widened exactly.
 *
 * Parity pins (tests/test_oracle_pins.py): closed-form SwiGLU and sigmoid
 * points, brute-force top-k, renormalisation invariants, brute-force stable
 * permutation, token-order equivariance, identical-experts and E=K=1
 * reductions to a textbook SwiGLU FFN, dense brute force over all experts,
 * int4 decode points, fp16/bf16 decode and rounding points.  Absolute
 * agreement with the pages' own trained model is "parity unpinned": the pages
 * print no values for this layer.
 */
#ifndef COLI_ORACLE_H
#define COLI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element encodings of a stacked matrix operand. */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_INT4 = 2 };

/*
 * A stack of matrices [n_mat][rows][K] with the reduction index K contiguous.
 *   ORC_F32 : data = float[n_mat*rows*K]
 *   ORC_BF16: data = uint16_t bf16 bit patterns, same shape
 *   ORC_INT4: data = uint8_t[n_mat*rows*K/2]; byte i of a row holds element
 *             2i in its low nibble and 2i+1 in its high nibble; scales =
 *             fp16 bit patterns [n_mat*rows*K/group]; element value =
 *             (nibble - 8) * scale  (offset-binary, [glm53-hip] "Key changes").
 */
typedef struct {
    int kind;
    const void *data;
    const uint16_t *scales;
    int group;
} orc_mat;

/* ---- scalar helpers (exposed so the tests can pin them directly) ---- */
double oracle_sigmoid(double z);
double oracle_silu(double a);
double oracle_swiglu(double g, double u);
double oracle_bf16_to_double(uint16_t b);
double oracle_fp16_to_double(uint16_t h);
uint16_t oracle_bf16_from_double(double v);
/* value of element (row, k) of matrix `m` of a stack with `rows` rows of K */
double oracle_mat_elem(const orc_mat *a, int64_t m, int64_t rows, int64_t K, int64_t row, int64_t k);

/* ---- the layer, step by step ---- */

/* Router logits z[t][e] = sum_d x[t][d] * wr[e][d] + bias[e]  ([glm5next] "MoE FFN"). */
int oracle_router_logits(int64_t T, int64_t D, int64_t E, const orc_mat *x,
                         const orc_mat *wr, const float *bias, double *z);

/* Per token: the K experts with the largest logits (ties: lower index first),
 * p = sigmoid(z) of the chosen ones, w = p / sum(p); ids stored in ascending
 * expert order with w aligned.  Ranking by the logit is ranking by sigmoid(z)
 * because the sigmoid is strictly increasing. */
int oracle_select_topk(int64_t T, int64_t E, int K, const double *z,
                       int32_t *ids, double *w);

/* Stable counting sort of the T*K (token, slot) assignments by expert:
 * count[e]; offset[0..E] exclusive prefix sums; rows ordered by expert
 * ascending then token ascending; perm[row] = t*K + j; inv[t*K + j] = row. */
int oracle_permutation(int64_t T, int64_t E, int K, const int32_t *ids,
                       int32_t *count, int32_t *offset, int32_t *perm, int32_t *inv);

/* One expert's clamped-SwiGLU hidden vector h[F] for input row xrow[D]
 * (gate/up stacks are [n_mat][F][D]). */
int oracle_expert_hidden(int64_t D, int64_t F, const double *xrow,
                         const orc_mat *gate, const orc_mat *up, int64_t n_mat,
                         int64_t e, double *h);

/* One expert's down projection o[D] = Wd[e] h  (down stack [n_mat][D][F]). */
int oracle_expert_down(int64_t D, int64_t F, const double *h, const orc_mat *down,
                       int64_t n_mat, int64_t e, double *o);

/*
 * Routed + shared FFN for a list of tokens (tokens == NULL means all T):
 *   y[i] = residual[tok] + S(x_tok) + sum_{j ascending id} w[tok][j] * E_{ids[tok][j]}(x_tok)
 * ids/w are [T][K]; residual is nullable [T][D]; y is [n_tokens][D].
 */
int oracle_moe_ffn(int64_t T, int64_t D, int64_t E, int K, int64_t F,
                   const orc_mat *x, const int32_t *ids, const double *w,
                   const orc_mat *gate, const orc_mat *up, const orc_mat *down,
                   const orc_mat *s_gate, const orc_mat *s_up, const orc_mat *s_down,
                   const double *residual, const int64_t *tokens, int64_t n_tokens,
                   double *y);

/*
 * One layer of the stacked chain for n rows: the layer input is
 * bf16_rne(x[i]) (returned in xin_bf16), y = FFN(route(xin)), and
 * x_next = x + y.  ids/w/z (nullable) receive the routing of the rows.
 */
int oracle_residual_layer(int64_t n, int64_t D, int64_t E, int K, int64_t F,
                          const double *x, const orc_mat *wr, const float *bias,
                          const orc_mat *gate, const orc_mat *up, const orc_mat *down,
                          const orc_mat *s_gate, const orc_mat *s_up, const orc_mat *s_down,
                          uint16_t *xin_bf16, int32_t *ids, double *w, double *z,
                          double *y, double *x_next);

/*
 * Dense FFN layer ([glm5next] "Architecture" and "MoE FFN": the first three
 * layers run a dense FFN with no experts; the clamped SwiGLU is stated for
 * the model as a whole):
 *   y[t] = residual[t] + W_down swiglu(W_gate x_t, W_up x_t)
 * gate/up [F][D], down [D][F]; residual nullable [T][D]; y [T][D].
 */
int oracle_dense_ffn(int64_t T, int64_t D, int64_t F, const orc_mat *x,
                     const orc_mat *gate, const orc_mat *up, const orc_mat *down,
                     const double *residual, double *y);

/*
 * Index selection of the sparse attention's IndexPool ([glm5next] "MLA/DSA":
 * top-k over the indexer scores with k = 2048, and the last kpool tokens
 * always selected).  Per row r of scores [rows][ld] (fp32), over its first
 * n = min(lens[r], L) positions (n = L when lens is NULL):
 *   - n <= k: every position 0..n-1 is selected;
 *   - otherwise the last min(tail, k) positions n - tail .. n - 1 are
 *     selected, and the remaining slots go to the other positions in order of
 *     score, larger first, ties to the lower position.
 * idx[r][0..k-1] holds the selected positions in ascending order, then -1 in
 * the slots left over when n < k.
 */
int oracle_index_topk(int64_t rows, int64_t L, int64_t ld, const float *scores,
                      const int32_t *lens, int64_t k, int64_t tail, int32_t *idx);

/* Threads the OpenMP loops use (1 when built without OpenMP), and a way to
 * change it (for timing the oracle on one core). */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
