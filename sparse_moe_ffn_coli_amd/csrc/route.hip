// route.hip -- router, top-K selection and the deterministic token permutation.
//
// Router: logits z = W_router x + b with the bias inside the sigmoid; the K
// largest are kept and their sigmoid weights normalised to sum to one
// ("Add GLM-5.3-Flash (glm5next) support with ROCmFP mix qtypes (105/106)",
// section "MoE FFN").  Selection is deterministic ("feat(glm53): add
// device-resident HIP backend for MI350P", section "Key changes"): ranking is
// by the fp32 logit (the sigmoid is strictly increasing, so this is the
// ranking by probability without the false ties of a saturated fp32 sigmoid),
// ties go to the lower expert index, and the chosen ids are stored ascending.
//
// Permutation: a stable counting sort of the T*K (token, slot) assignments by
// expert, built from integer work only -- per-64-token-tile expert bitmasks
// (LDS atomic OR, which commutes), a column scan over tiles, and ranks from
// popcounts of the bitmask below each lane -- so it is bitwise reproducible.
#include "device_common.h"
#include "kernels.h"

namespace coli {

// ---------------------------------------------------------------------------
// router logits, bf16 inputs, MFMA.  One workgroup per (16-token block,
// 128-expert block); rows past T and experts past E are zero-padded.
// ---------------------------------------------------------------------------
using RouterCfg = TileCfg<16, 128, 1, 4>;

__global__ __launch_bounds__(256) void router_logits_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, const float *__restrict__ bias,
    int T, int D, int E, float *__restrict__ z)
{
    using C = RouterCfg;
    __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_BYTES / 2];
    const int n_nt = (E + C::BN - 1) / C::BN;
    const int mt = blockIdx.x / n_nt, nt = blockIdx.x % n_nt;
    const int t0 = mt * C::BM, e0 = nt * C::BN;
    const int ch0 = threadIdx.x & 7;

    const uint16_t *ap[C::A_PER_T];
    const uint16_t *bp[C::B_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        int t = min(t0 + a_chunk_row<C>(i), T - 1);      // padding rows reread the last token
        ap[i] = x + (size_t)t * D + ch0 * 8;
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        int e = min(e0 + a_chunk_row<C>(i), E - 1);      // padding rows reread the last expert
        bp[i] = wr + (size_t)e * D + ch0 * 8;
    }
    f32x4 acc[C::FM][C::FN];
    mfma_mainloop<C>(ap, bp, D, lds, acc);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave % C::WAVES_N, wm = wave / C::WAVES_N;
#pragma unroll
    for (int m = 0; m < C::FM; ++m)
#pragma unroll
        for (int n = 0; n < C::FN; ++n) {
            int e = e0 + (wn * C::FN + n) * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int t = t0 + (wm * C::FM + m) * 16 + 4 * (lane >> 4) + i;
                if (t < T && e < E) z[(size_t)t * E + e] = acc[m][n][i] + bias[e];
            }
        }
}

// fp32 router: one thread per (token, expert), plain dot product.
__global__ void router_logits_f32_kernel(const float *__restrict__ x, const float *__restrict__ wr,
                                         const float *__restrict__ bias, int T, int D, int E,
                                         float *__restrict__ z)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * E) return;
    int t = (int)(i / E), e = (int)(i % E);
    const float *xr = x + (size_t)t * D, *wrow = wr + (size_t)e * D;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc = fmaf(xr[d], wrow[d], acc);
    z[i] = acc + bias[e];
}

// ---------------------------------------------------------------------------
// top-K: one wave per token.  Keys are (order-preserving image of the fp32
// logit) << 32 | (0xFFFFFFFF - expert), so the largest key is the largest
// logit with the lowest index on ties; K rounds of a wave-wide max.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o)
{
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint64_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

constexpr int TOPK_MAX_E = 1024;
constexpr int TOPK_SLOTS = TOPK_MAX_E / 64;

__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ z, int T, int E, int K,
                                                   int32_t *__restrict__ ids, float *__restrict__ w)
{
    const int lane = threadIdx.x & 63;
    const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    if (t >= T) return;
    const float *zt = z + (size_t)t * E;

    uint64_t key[TOPK_SLOTS];
#pragma unroll
    for (int s = 0; s < TOPK_SLOTS; ++s) {
        int e = lane + 64 * s;
        key[s] = (e < E) ? ((uint64_t)ordered_bits(zt[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)
                         : 0ull;
    }
    int sel_e[8];
    float sel_z[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j >= K) { sel_e[j] = 0x7fffffff; sel_z[j] = 0.f; continue; }
        uint64_t best = 0;
#pragma unroll
        for (int s = 0; s < TOPK_SLOTS; ++s) best = key[s] > best ? key[s] : best;
        best = wave_max_u64(best);
        int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
        sel_e[j] = e;
        sel_z[j] = from_ordered_bits((uint32_t)(best >> 32));
        if ((e & 63) == lane) {
#pragma unroll
            for (int s = 0; s < TOPK_SLOTS; ++s)
                if (s == (e >> 6)) key[s] = 0ull;
        }
    }
    // canonical order: ascending expert id
#pragma unroll
    for (int a = 1; a < 8; ++a)
#pragma unroll
        for (int b = a; b > 0; --b)
            if (sel_e[b - 1] > sel_e[b]) {
                int te = sel_e[b - 1]; sel_e[b - 1] = sel_e[b]; sel_e[b] = te;
                float tz = sel_z[b - 1]; sel_z[b - 1] = sel_z[b]; sel_z[b] = tz;
            }
    // weights p_j / sum p.  When every chosen logit is negative the ratios are
    // formed relative to the largest one so that tiny sigmoids cannot underflow
    // the sum: sigmoid(a)/sigmoid(m) = e^(a-m) (1+e^m) / (1+e^a).
    float zmax = sel_z[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
        if (j < K) zmax = fmaxf(zmax, sel_z[j]);
    float p[8], psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j >= K) { p[j] = 0.f; continue; }
        if (zmax >= 0.f)
            p[j] = sigmoid_f32(sel_z[j]);
        else
            p[j] = expf(sel_z[j] - zmax) * (1.0f + expf(zmax)) / (1.0f + expf(sel_z[j]));
        psum += p[j];
    }
    if (lane < K) {
        int e = 0;
        float pj = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j == lane) { e = sel_e[j]; pj = p[j]; }
        ids[(size_t)t * K + lane] = e;
        w[(size_t)t * K + lane] = pj / psum;
    }
}

// ---------------------------------------------------------------------------
// permutation
// ---------------------------------------------------------------------------
// Bitmask of the tile's tokens (one bit per lane) that chose each expert.
__device__ __forceinline__ void build_tile_masks(const int32_t *__restrict__ ids, int T, int E, int K,
                                                 uint64_t *masks)
{
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += 64) masks[e] = 0ull;
    __syncthreads();
    const int t = blockIdx.x * 64 + lane;
    if (t < T)
        for (int j = 0; j < K; ++j) atomicOr((unsigned long long *)&masks[ids[(size_t)t * K + j]],
                                             1ull << lane);
    __syncthreads();
}

__global__ __launch_bounds__(64) void perm_hist_kernel(const int32_t *__restrict__ ids, int T, int E,
                                                       int K, int32_t *__restrict__ tile_count)
{
    __shared__ uint64_t masks[TOPK_MAX_E];
    build_tile_masks(ids, T, E, K, masks);
    for (int e = threadIdx.x; e < E; e += 64)
        tile_count[(size_t)blockIdx.x * E + e] = __popcll(masks[e]);
}

// One workgroup: count[e] = sum over tiles; offset = exclusive scan of count;
// tile_base[tile][e] = offset[e] + rows of expert e in earlier tiles.
__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t *__restrict__ tile_count,
                                                         int ntiles, int E, int32_t *__restrict__ tile_base,
                                                         int32_t *__restrict__ count,
                                                         int32_t *__restrict__ offset)
{
    __shared__ int32_t sc[TOPK_MAX_E];
    const int tid = threadIdx.x;
    int c = 0;
    if (tid < E) {
        for (int tl = 0; tl < ntiles; ++tl) c += tile_count[(size_t)tl * E + tid];
        count[tid] = c;
    }
    sc[tid] = (tid < E) ? c : 0;
    __syncthreads();
    // inclusive Hillis-Steele scan over 1024 entries
    for (int off = 1; off < TOPK_MAX_E; off <<= 1) {
        int v = (tid >= off) ? sc[tid - off] : 0;
        __syncthreads();
        sc[tid] += v;
        __syncthreads();
    }
    if (tid < E) {
        int base = sc[tid] - c;           // exclusive prefix
        offset[tid] = base;
        if (tid == E - 1) offset[E] = sc[tid];
        for (int tl = 0; tl < ntiles; ++tl) {
            tile_base[(size_t)tl * E + tid] = base;
            base += tile_count[(size_t)tl * E + tid];
        }
    }
}

__global__ __launch_bounds__(64) void perm_scatter_kernel(const int32_t *__restrict__ ids, int T, int E,
                                                          int K, const int32_t *__restrict__ tile_base,
                                                          int32_t *__restrict__ perm,
                                                          int32_t *__restrict__ inv)
{
    __shared__ uint64_t masks[TOPK_MAX_E];
    build_tile_masks(ids, T, E, K, masks);
    const int lane = threadIdx.x;
    const int t = blockIdx.x * 64 + lane;
    if (t >= T) return;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j = 0; j < K; ++j) {
        int e = ids[(size_t)t * K + j];
        int row = tile_base[(size_t)blockIdx.x * E + e] + __popcll(masks[e] & below);
        perm[row] = t * K + j;
        inv[(size_t)t * K + j] = row;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// T = 0: no tokens, but count and offset are still defined (all zero).
__global__ void route_empty_kernel(int E, int32_t *__restrict__ count, int32_t *__restrict__ offset)
{
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
        if (e < E) count[e] = 0;
        offset[e] = 0;
    }
}

hipError_t launch_route(const RouteLaunch &a, hipStream_t st)
{
    const int T = a.T, D = a.D, E = a.E, K = a.K;
    if (T == 0) {
        route_empty_kernel<<<1, 256, 0, st>>>(E, a.count, a.offset);
        return hipGetLastError();
    }
    StageMarks none;
    StageMarks &mk = a.marks ? *a.marks : none;
    mk.mark(st);
    if (a.bf16) {
        int n_nt = (E + RouterCfg::BN - 1) / RouterCfg::BN;
        int n_mt = (T + RouterCfg::BM - 1) / RouterCfg::BM;
        router_logits_bf16_kernel<<<n_mt * n_nt, 256, 0, st>>>(
            (const uint16_t *)a.x, (const uint16_t *)a.wr, a.bias, T, D, E, a.z);
    } else {
        int64_t n = (int64_t)T * E;
        router_logits_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
            (const float *)a.x, (const float *)a.wr, a.bias, T, D, E, a.z);
    }
    mk.mark(st);
    topk_kernel<<<(T + 3) / 4, 256, 0, st>>>(a.z, T, E, K, a.ids, a.w);
    const int ntiles = (T + 63) / 64;
    mk.mark(st);
    perm_hist_kernel<<<ntiles, 64, 0, st>>>(a.ids, T, E, K, a.tile_count);
    mk.mark(st);
    perm_scan_kernel<<<1, 1024, 0, st>>>(a.tile_count, ntiles, E, a.tile_base, a.count, a.offset);
    mk.mark(st);
    perm_scatter_kernel<<<ntiles, 64, 0, st>>>(a.ids, T, E, K, a.tile_base, a.perm, a.inv);
    mk.mark(st);
    return hipGetLastError();
}

}  // namespace coli
