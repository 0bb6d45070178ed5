// kernels.h -- internal launch interface between the C ABI (api.hip) and the
// kernels (route.hip, ffn.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

// Records caller-owned events between stages (instrumented entry points).
struct StageMarks {
    void *const *ev = nullptr;
    int n = 0;
    int next = 0;
    void mark(hipStream_t st)
    {
        if (ev && next < n && ev[next]) (void)hipEventRecord((hipEvent_t)ev[next], st);
        ++next;
    }
};

struct RouteLaunch {
    int T, D, E, K;
    bool bf16;
    const void *x;
    const void *wr;
    const float *bias;
    float *z;              // workspace [router_splits][T][E]: partial logits
    int32_t *tile_count;   // workspace [perm_tiles(T)][E]
    int32_t *done;         // workspace: counter of the fused top-K + permutation (zeroed by the router)
    int32_t *ids;
    float *w;
    int32_t *count, *offset, *perm, *inv;
    StageMarks *marks;     // nullable
};

struct FfnLaunch {
    int T, D, E, K, F;
    bool bf16;
    int bm;                // tile height of the grouped GEMMs (bf16)
    const void *x;
    const int32_t *ids;
    const float *w;
    const int32_t *count, *perm, *inv;
    const void *gate, *up, *down, *s_gate, *s_up, *s_down;
    bool use_int4;         // routed experts in int4 (then gate/up/down above are unused)
    const uint8_t *gate_q, *up_q, *down_q;
    const uint16_t *gate_s, *up_s, *down_s;
    int group;
    const float *residual;
    float *y;
    void *y_bf16;
    void *h;               // workspace [T*K + T][F] (bf16; fp16 in the int4 engine's chunk order for int4)
    uint16_t *x16;         // workspace [T][D] (int4 only): x in fp16, the int4 engine's chunk order
    void *o;               // workspace [T*K][D]
    float *sx;             // workspace [ksplit][T][D] (bf16 path): the shared expert's output (parts)
    int ksplit;            // parts of the down reduction (layers without routed rows; else 1)
    int4 *list_gu;         // workspace [ffn_max_tiles * ffn_col_tiles_gu] (256-row tiles)
    int4 *list_dn;         // workspace [ffn_max_tiles * ffn_col_tiles_dn] (256-row tiles)
    int32_t *n_items;      // workspace [20]: list lengths and per-XCD range starts
    StageMarks *marks;     // nullable
};

hipError_t launch_route(const RouteLaunch &a, hipStream_t st);
hipError_t launch_index_topk(const float *scores, int rows, int L, long ld, const int32_t *lens, int k, int tail,
                             int32_t *idx, hipStream_t st);
hipError_t launch_ffn(const FfnLaunch &a, hipStream_t st);

int perm_tiles(int T);
int router_splits(int T, int D);
int ffn_tile_rows(int T, int E, int K, int int4);
long ffn_max_tiles(int T, int E, int K, int bm);
int ffn_col_tiles_gu(int F);
int ffn_col_tiles_dn(int D);
int ffn_down_splits(int T, int E, int D, int F, int bm);

}  // namespace coli
