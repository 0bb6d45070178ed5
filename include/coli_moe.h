/*
 * coli_moe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts FFN
 * layer used by GLM-5.3-Flash-style models, with the pieces around it that
 * the same pages describe: the dense FFN of the first layers, a double-banked
 * device expert cache, and the sparse attention's index top-k selection.
 *
 * The layer, per token x (length D):
 *   z      = W_router x + b                         (E logits, bias inside the sigmoid)
 *   ids    = the K experts with the largest z       (ties: lower expert index)
 *   w      = sigmoid(z_ids) / sum(sigmoid(z_ids))   (routing weights sum to one)
 *   E_e(x) = W_down[e] swiglu(W_gate[e] x, W_up[e] x)
 *   swiglu(g, u) = silu(min(g, 10)) * clamp(u, -10, 10)
 *   y      = residual + S(x) + sum_j w_j E_{ids_j}(x)   (S = the shared expert,
 *                                                        same clamped SwiGLU)
 * Pages cited below by title:
 *   [glm5next]  "Add GLM-5.3-Flash (glm5next) support with ROCmFP mix qtypes
 *               (105/106)" -- sections "Architecture", "MoE FFN", "MLA/DSA",
 *               "What Executes vs. TODO", "Loader".
 *   [glm53-hip] "feat(glm53): add device-resident HIP backend for MI350P" --
 *               sections "Key changes", "Validation results".
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller (the expert
 *     bank fill also takes pinned HOST pointers, stated there).  The library
 *     never allocates, frees or synchronises.  Its process-wide state is a
 *     per-device cache of the device-architecture check (each entry set once
 *     to a fixed answer) and, for coli_moe_ffn_noalloc only, a per-device
 *     scratch array and its address.  Scratch memory is otherwise the
 *     caller's workspace (`ws`, `ws_bytes`), sized by the matching
 *     *_workspace_bytes() call.
 *   - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *     stream).  All work is enqueued on it in order; calls return before the
 *     GPU finishes.
 *   - Shape, pointer, alignment, aliasing and workspace errors are detected on
 *     the host BEFORE anything is enqueued: the call returns the error and no
 *     output is touched.  A launch failure returns COLI_E_LAUNCH; outputs are
 *     then undefined.  The library never prints, aborts or falls back to
 *     another code path (a missing piece fails outright, as the pages' loader
 *     does: [glm5next] "Loader").
 *   - Layouts are row-major with the reduction index contiguous:
 *       x [T][D], W_router [E][D], gate/up [E][F][D], down [E][D][F],
 *       shared gate/up [F][D], shared down [D][F], y [T][D].
 *   - Every pointer must be 16-byte aligned.  T = 0 is valid: routing then
 *     writes zero counts and offsets and the FFN enqueues nothing (the
 *     per-assignment routing arrays may be NULL).
 *   - Results are bitwise reproducible run to run for the same inputs and
 *     shape (no floating-point atomics; every reduction has a fixed order;
 *     [glm53-hip] "Validation results": bitwise GPU determinism).
 *   - Inputs are finite; NaN inputs give unspecified (but non-faulting)
 *     results.
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
    COLI_E_WORKSPACE = 5, /* workspace smaller than the *_workspace_bytes() answer */
    COLI_E_DEVICE = 6,    /* the current device is not a gfx950 GPU */
    COLI_E_LAUNCH = 7,    /* a kernel launch or copy could not be enqueued */
    COLI_E_ALIAS = 8,     /* an output overlaps an input it must not overlap */
    COLI_E_MEMORY = 9     /* a pointer is not the kind of memory required (device / pinned host) */
} coli_status;

/* Element type of activations and (non-int4) weights.  COLI_F32: everything
 * fp32 with fp32 arithmetic.  COLI_BF16: bf16 storage, fp32 accumulation. */
typedef enum { COLI_F32 = 0, COLI_BF16 = 1 } coli_dtype;

/* Layer shape.  T tokens, model width D, E routed experts, K experts per
 * token, expert (and shared expert) hidden width F.
 * Supported: T >= 0, 1 <= K <= 8 (the pages' layer uses K = 8: [glm5next]
 * "Architecture"), K <= E <= 1024, D and F multiples of 64 (the MFMA tiles'
 * reduction step; the int4 groups need 32), D <= 16384, F <= 16384. */
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

/* Int4 routed experts ([glm53-hip] "Key changes": grouped int4 decoded as
 * offset-binary nibble minus 8): element (row, k) = (nibble - 8) * scale,
 * where byte k/2 of the row holds even k in its low nibble and odd k in its
 * high nibble, and scale is the fp16 value of group k/group of that row.  The
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

/* Bytes of workspace the MoE entry points need for this shape (int4 != 0 for
 * the int4 FFN); at least 256, and 0 for an invalid shape.  The same
 * workspace may serve route and FFN calls of the shape. */
size_t coli_moe_workspace_bytes(const coli_moe_shape *s, int int4);

/* Router, top-K selection, weight normalisation ([glm5next] "MoE FFN":
 * sigmoid of the router projection plus bias, top-8 selection, weight
 * normalisation; [glm53-hip] "Key changes": deterministic top-k routing), and
 * the stable permutation of the T*K (token, slot) assignments into
 * expert-contiguous rows that the grouped expert products read.
 * x [T][D] and w_router [E][D] in the shape's dtype; bias [E] fp32; outputs
 * in `out` (every array written; none may overlap another or an input).
 * Selection ranks the fp32 logits (ranking by the sigmoid is the same order);
 * weights are computed from the sigmoid of the chosen logits in fp32. */
coli_status coli_moe_route(const coli_moe_shape *s, const void *x, const void *w_router,
                           const float *bias, const coli_moe_routing *out, void *ws,
                           size_t ws_bytes, void *stream);

/* Routed + shared expert FFN and the fixed-order combine ([glm5next] "MoE
 * FFN": gate/up/down products of the selected experts with the clamped SwiGLU
 * between them, the shared expert combined with the weighted routed output;
 * "Architecture": the clamp limits):
 *   y[t] = residual[t] + S(x_t) + sum_j w[t][j] E_{ids[t][j]}(x_t)
 * with the sum taken in the order of ids (ascending expert id).  residual is
 * nullable [T][D] fp32 and may be y itself (in-place residual stream; any
 * other overlap is an error); y [T][D] fp32; y_bf16 nullable [T][D] receives
 * y rounded to bf16 (round to nearest even; bf16 shapes only).  x, the
 * routing arrays and the weights must not overlap y, y_bf16 or ws. */
coli_status coli_moe_ffn(const coli_moe_shape *s, const void *x, const coli_moe_routing *r,
                         const coli_moe_weights *w, const float *residual, float *y,
                         void *y_bf16, void *ws, size_t ws_bytes, void *stream);

/* As coli_moe_ffn with int4 routed experts ([glm53-hip] "Key changes"), bf16
 * shapes only.  Arithmetic of the routed experts: fp16 products with fp32
 * accumulation -- each weight (nibble - 8) * scale rounded once to fp16 (for
 * every finite scale), the tokens and the routed hidden rows converted to
 * fp16.  Precondition: |x| < 65504 (fp16's largest finite value); a larger
 * element overflows and makes that token's output non-finite.  The shared
 * expert runs exactly as in coli_moe_ffn (bf16 products, fp32 accumulation);
 * the combine is as in coli_moe_ffn. */
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
 *   route stages (3): router logits, top-K, permutation (for T <= 1024 and
 *                     E <= 512 top-K and the permutation are one kernel,
 *                     timed as the top-K stage; the permutation stage is
 *                     then empty)
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

/* ---- an FFN call that allocates nothing ----------------------------------
 * For callers that cannot allocate device memory or hand over a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): coli_moe_ffn with its workspace taken from a scratch array
 * the library keeps in each GPU's memory (COLI_NOALLOC_SCRATCH_BYTES, held
 * by every GPU the library runs on until the process ends).  A shape whose
 * coli_moe_workspace_bytes(s, 0) exceeds the array returns COLI_E_WORKSPACE
 * before anything is enqueued (the array holds T up to about 540 tokens at
 * D = 2048, F = 768, K = 8).  Every call on one GPU uses the same array:
 * calls that overlap in time on one GPU (other streams, or host threads
 * without an order between their calls) race and give undefined results.
 * Nothing in the array has to start at zero; each call writes every byte it
 * later reads.  Results are bitwise those of coli_moe_ffn. */
#define COLI_NOALLOC_SCRATCH_BYTES (32u << 20)
coli_status coli_moe_ffn_noalloc(const coli_moe_shape *s, const void *x, const coli_moe_routing *r,
                                 const coli_moe_weights *w, const float *residual, float *y,
                                 void *y_bf16, void *stream);

/* ---- dense FFN layers ----------------------------------------------------
 * The model's first layers run a dense FFN instead of the experts
 * ([glm5next] "Architecture": layers 0-2 dense FFN only; "MoE FFN": dense FFN
 * for layers 0-2, no experts), with the model's clamped SwiGLU:
 *   y[t] = residual[t] + W_down swiglu(W_gate x_t, W_up x_t)
 * It runs on the same kernels as the shared expert.  The shape's T, D, F and
 * dtype are used (D, F multiples of 64, D <= 16384, F <= 32768); E and K are
 * ignored.  gate, up [F][D] and down [D][F] in the shape's dtype; residual,
 * y and y_bf16 as in coli_moe_ffn. */
typedef struct {
    const void *gate; /* [F][D] */
    const void *up;   /* [F][D] */
    const void *down; /* [D][F] */
} coli_moe_dense_weights;

size_t coli_moe_dense_workspace_bytes(const coli_moe_shape *s);
coli_status coli_moe_dense_ffn(const coli_moe_shape *s, const void *x,
                               const coli_moe_dense_weights *w, const float *residual, float *y,
                               void *y_bf16, void *ws, size_t ws_bytes, void *stream);

/* ---- double-banked device expert cache -----------------------------------
 * [glm53-hip] "Key changes": a double-banked device expert cache with
 * event-based publication.  A bank is caller-owned device memory laid out
 * exactly like a layer's routed expert tensors, so an FFN call reads a bank
 * as its weights.  While one bank feeds layer l, the next layer's experts are
 * copied from pinned host memory into the other bank on a separate copy
 * stream; an event publishes the copy, and another event tells the copy
 * stream when the compute stream has finished reading a bank:
 *
 *   fill(bank b, layer l+1, copy_stream, wait_event = free[b], ready_event = ready[b])
 *   acquire(compute_stream, ready[b]);  ffn(layer l+1 from bank b);  release(compute_stream, free[b])
 *
 * coli_moe_bank_fill enqueues on copy_stream: a wait for wait_event
 * (nullable: no wait), host-to-device copies of the listed experts' tensors,
 * and a record of ready_event (nullable).  Tensors, in order (int4 = 0 / 1):
 *   bf16/fp32 (3): gate [E][F][D], up [E][F][D], down [E][D][F] in the dtype
 *   int4      (6): gate_q, up_q, down_q, gate_s, up_s, down_s as in
 *                  coli_moe_weights_int4 (with `group`)
 * host[i] must be pinned host memory (hipHostMalloc) and bank[i] device
 * memory, each holding all E experts of tensor i; `experts` is a host array
 * of n_experts distinct ids in [0, E) to copy (NULL: all E); runs of
 * consecutive ids go as one copy.  The shared expert is not part of a bank
 * (it stays resident).  Returns COLI_E_MEMORY for a pointer of the wrong
 * memory kind and COLI_E_SHAPE for a bad expert list; copies run on the
 * DMA engines and use no compute units. */
coli_status coli_moe_bank_fill(const coli_moe_shape *s, int32_t int4, int32_t group,
                               const void *const *host, void *const *bank,
                               const int32_t *experts, int32_t n_experts, void *copy_stream,
                               void *wait_event, void *ready_event);
/* The compute stream waits for ready_event (the bank's copies published). */
coli_status coli_moe_bank_acquire(void *compute_stream, void *ready_event);
/* Records free_event on the compute stream after the work that reads the
 * bank, so that the bank's next fill can wait for it. */
coli_status coli_moe_bank_release(void *compute_stream, void *free_event);

/* ---- sparse attention index selection ------------------------------------
 * [glm5next] "MLA/DSA": IndexPool sparse selection keeps the top-k entries of
 * the indexer scores (k = 2048) and always selects the last kpool (= 4)
 * tokens.  For each row r of scores [rows][ld] (fp32; only the first L
 * columns are read) over its first n = min(lens[r], L) positions (lens
 * nullable: n = L):
 *   - n <= k: every position 0..n-1 is selected;
 *   - otherwise the last min(tail, k) positions are selected and the other
 *     k - min(tail, k) slots go to the remaining positions by score, larger
 *     first, ties to the lower position (+0 and -0 are equal).
 * idx [rows][k] int32 receives the selected positions in ascending order,
 * then -1 for the slots left when n < k.  1 <= k <= 4096, 0 <= tail,
 * 0 <= L <= 1 << 24, ld >= L (a multiple of 4), lens[r] >= 0. */
size_t coli_index_topk_workspace_bytes(int32_t rows, int32_t L, int32_t k);
coli_status coli_index_topk(const float *scores, int32_t rows, int32_t L, int64_t ld,
                            const int32_t *lens, int32_t k, int32_t tail, int32_t *idx,
                            void *ws, size_t ws_bytes, void *stream);

/* Static description of a status code. */
const char *coli_moe_status_str(coli_status st);

/* Library version, major*10000 + minor*100 + patch. */
int32_t coli_moe_version(void);

#ifdef __cplusplus
}
#endif
#endif
