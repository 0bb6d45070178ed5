/*
 * coli_moe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts FFN
 * layer used by GLM-5.3-Flash-style models.
 *
 * The layer, per token x (length D):
 *   z      = W_router x + b                         (E logits, bias inside the sigmoid)
 *   ids    = the K experts with the largest z       (ties: lower expert index)
 *   w      = sigmoid(z_ids) / sum(sigmoid(z_ids))   (routing weights sum to one)
 *   E_e(x) = W_down[e] swiglu(W_gate[e] x, W_up[e] x)
 *   swiglu(g, u) = silu(min(g, 10)) * clamp(u, -10, 10)
 *   y      = residual + S(x) + sum_j w_j E_{ids_j}(x)   (S = the shared expert,
 *                                                        same clamped SwiGLU)
 * Pages: "Add GLM-5.3-Flash (glm5next) support with ROCmFP mix qtypes
 * (105/106)" -- section "Architecture" (288 routed experts, top-8, one shared
 * expert, sigmoid routing, clamped SwiGLU limits) and section "MoE FFN"
 * (router formula, top-8 selection, weight normalisation, gate/up/down expert
 * products, shared expert combined with the routed output);
 * "feat(glm53): add device-resident HIP backend for MI350P" -- section "Key
 * changes" (deterministic top-k routing; grouped int4 weights decoded as
 * offset-binary nibble minus 8) and "Validation results" (bitwise GPU
 * determinism).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises, and keeps no mutable global
 *     state.  Scratch memory is the caller's workspace (`ws`, `ws_bytes`),
 *     sized by coli_moe_workspace_bytes().
 *   - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *     stream).  All work is enqueued on it in order; calls return before the
 *     GPU finishes.
 *   - Shape, pointer, alignment, aliasing and workspace errors are detected on
 *     the host BEFORE anything is enqueued: the call returns the error and no
 *     output is touched.  A launch failure returns COLI_E_LAUNCH; outputs are
 *     then undefined.  The library never prints, aborts or falls back to
 *     another code path.
 *   - Layouts are row-major with the reduction index contiguous:
 *       x [T][D], W_router [E][D], gate/up [E][F][D], down [E][D][F],
 *       shared gate/up [F][D], shared down [D][F], y [T][D].
 *   - Every pointer must be 16-byte aligned.  T = 0 is valid: routing then
 *     writes zero counts and offsets and the FFN enqueues nothing (the
 *     per-assignment routing arrays may be NULL).
 *   - Results are bitwise reproducible run to run for the same inputs and
 *     shape (no floating-point atomics; every reduction has a fixed order).
 */
#ifndef COLI_MOE_H
#define COLI_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    COLI_OK = 0,
    COLI_E_NULL = 1,      /* a required pointer is NULL */
    COLI_E_SHAPE = 2,     /* a size is out of the supported range */
    COLI_E_DTYPE = 3,     /* unknown element type */
    COLI_E_ALIGN = 4,     /* a pointer is not 16-byte aligned */
    COLI_E_WORKSPACE = 5, /* workspace smaller than coli_moe_workspace_bytes() */
    COLI_E_DEVICE = 6,    /* the current device is not a gfx950 GPU */
    COLI_E_LAUNCH = 7,    /* a kernel launch failed */
    COLI_E_ALIAS = 8      /* an output overlaps an input it must not overlap */
} coli_status;

/* Element type of activations and (non-int4) weights.  COLI_F32: everything
 * fp32 with fp32 arithmetic.  COLI_BF16: bf16 storage, fp32 accumulation. */
typedef enum { COLI_F32 = 0, COLI_BF16 = 1 } coli_dtype;

/* Layer shape.  T tokens, model width D, E routed experts, K experts per
 * token, expert (and shared expert) hidden width F.
 * Supported: T >= 0, 1 <= K <= 8, K <= E <= 1024, D and F multiples of 64
 * (int4: also of the group size), D <= 16384, F <= 16384. */
typedef struct {
    int32_t T, D, E, K, F;
    int32_t dtype; /* coli_dtype */
} coli_moe_shape;

/* Routing produced by coli_moe_route and consumed by the FFN entry points.
 *   ids    [T][K] int32  the chosen experts of each token, ascending
 *   w      [T][K] fp32   their routing weights (sum to one per token)
 *   count  [E]    int32  tokens routed to each expert
 *   offset [E+1]  int32  exclusive prefix sums of count (offset[E] = T*K); the
 *                        FFN entry points derive the same sums from count and
 *                        do not read it
 *   perm   [T*K]  int32  row -> t*K + j; rows grouped by expert ascending,
 *                        tokens ascending within an expert (stable sort)
 *   inv    [T*K]  int32  t*K + j -> row (inverse of perm) */
typedef struct {
    int32_t *ids;
    float *w;
    int32_t *count;
    int32_t *offset;
    int32_t *perm;
    int32_t *inv;
} coli_moe_routing;

/* Routed and shared expert weights in the shape's dtype. */
typedef struct {
    const void *gate;   /* [E][F][D] */
    const void *up;     /* [E][F][D] */
    const void *down;   /* [E][D][F] */
    const void *s_gate; /* [F][D] */
    const void *s_up;   /* [F][D] */
    const void *s_down; /* [D][F] */
} coli_moe_weights;

/* Int4 routed experts: element (row, k) = (nibble - 8) * scale, where byte
 * k/2 of the row holds even k in its low nibble and odd k in its high
 * nibble, and scale is the fp16 value of group k/group of that row.  The
 * shared expert stays in the shape's dtype (bf16). */
typedef struct {
    const uint8_t *gate_q;   /* [E][F][D/2] */
    const uint8_t *up_q;     /* [E][F][D/2] */
    const uint8_t *down_q;   /* [E][D][F/2] */
    const uint16_t *gate_s;  /* [E][F][D/group] fp16 bits */
    const uint16_t *up_s;    /* [E][F][D/group] fp16 bits */
    const uint16_t *down_s;  /* [E][D][F/group] fp16 bits */
    int32_t group;           /* elements per scale along the reduction index; 32 */
    const void *s_gate;      /* [F][D] */
    const void *s_up;        /* [F][D] */
    const void *s_down;      /* [D][F] */
} coli_moe_weights_int4;

/* Bytes of workspace an entry point needs for this shape (int4 != 0 for the
 * int4 FFN); at least 256, and 0 for an invalid shape.  The same workspace
 * may serve route and FFN calls of the shape. */
size_t coli_moe_workspace_bytes(const coli_moe_shape *s, int int4);

/* Router, top-K selection, weight normalisation and the stable permutation
 * of the T*K (token, slot) assignments into expert-contiguous rows.
 * x [T][D] and w_router [E][D] in the shape's dtype; bias [E] fp32.
 * Selection ranks the fp32 logits (ranking by the sigmoid is the same order);
 * weights are computed from the sigmoid of the chosen logits in fp32. */
coli_status coli_moe_route(const coli_moe_shape *s, const void *x, const void *w_router,
                           const float *bias, const coli_moe_routing *out, void *ws,
                           size_t ws_bytes, void *stream);

/* Routed + shared expert FFN and the fixed-order combine:
 *   y[t] = residual[t] + S(x_t) + sum_j w[t][j] E_{ids[t][j]}(x_t)
 * with the sum taken in the order of ids (ascending expert id).  residual is
 * nullable [T][D] fp32 and may alias y (in-place residual stream); y [T][D]
 * fp32; y_bf16 nullable [T][D] receives y rounded to bf16 (bf16 shapes only).
 * x must not overlap y or y_bf16. */
coli_status coli_moe_ffn(const coli_moe_shape *s, const void *x, const coli_moe_routing *r,
                         const coli_moe_weights *w, const float *residual, float *y,
                         void *y_bf16, void *ws, size_t ws_bytes, void *stream);

/* As coli_moe_ffn with int4 routed experts (bf16 shapes only).  Arithmetic:
 * fp16 products with fp32 accumulation -- each weight (nibble - 8) * scale
 * rounded once to fp16, the activations and the hidden rows of the routed and
 * shared experts converted to fp16; the combine is as in coli_moe_ffn. */
coli_status coli_moe_ffn_int4(const coli_moe_shape *s, const void *x,
                              const coli_moe_routing *r, const coli_moe_weights_int4 *w,
                              const float *residual, float *y, void *y_bf16, void *ws,
                              size_t ws_bytes, void *stream);

/* Instrumented variants for timing each kernel of a call: the same work and
 * bitwise the same results as the plain entry points, and in addition the
 * caller's HIP events (hipEvent_t handles passed as void*) are recorded on
 * `stream`: events[i] just before stage i is enqueued and events[n_stages]
 * after the last one.  Entries past n_events, and NULL entries, are skipped.
 * Nothing is recorded when the call fails validation or T = 0.
 *   route stages (3): router logits, top-K, permutation
 *   ffn stages (3):   gate+up (+SwiGLU), down (routed and shared), combine;
 *                     a preparation kernel (the tile lists for large batches,
 *                     the x -> fp16 pass for int4) runs before events[0], so
 *                     events[0..1] bracket the gate+up kernel alone */
coli_status coli_moe_route_timed(const coli_moe_shape *s, const void *x, const void *w_router,
                                 const float *bias, const coli_moe_routing *out, void *ws,
                                 size_t ws_bytes, void *stream, void *const *events,
                                 int32_t n_events);
coli_status coli_moe_ffn_timed(const coli_moe_shape *s, const void *x, const coli_moe_routing *r,
                               const coli_moe_weights *w, const float *residual, float *y,
                               void *y_bf16, void *ws, size_t ws_bytes, void *stream,
                               void *const *events, int32_t n_events);
coli_status coli_moe_ffn_int4_timed(const coli_moe_shape *s, const void *x,
                                    const coli_moe_routing *r, const coli_moe_weights_int4 *w,
                                    const float *residual, float *y, void *y_bf16, void *ws,
                                    size_t ws_bytes, void *stream, void *const *events,
                                    int32_t n_events);

/* Static description of a status code. */
const char *coli_moe_status_str(coli_status st);

/* Library version, major*10000 + minor*100 + patch. */
int32_t coli_moe_version(void);

#ifdef __cplusplus
}
#endif
#endif
