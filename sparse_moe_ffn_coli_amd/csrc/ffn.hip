// ffn.hip -- routed + shared expert FFN and the fixed-order combine.
//
// Per routed row r (token t, expert e = ids[perm[r]]):
//   h_r = swiglu(W_gate[e] x_t, W_up[e] x_t),  o_r = W_down[e] h_r
// and per token the shared expert S(x_t) = S_down swiglu(S_gate x_t, S_up x_t);
//   y_t = residual_t + S(x_t) + sum_j w_tj o_{inv(t,j)}   (j in ascending expert id)
// ("Add GLM-5.3-Flash (glm5next) support with ROCmFP mix qtypes (105/106)",
// sections "MoE FFN" and "What Executes vs. TODO": gate/up/down matmuls over
// the selected experts, clamped SwiGLU between them, the shared expert
// computed alongside and combined with the weighted routed outputs).
//
// bf16 path: three grouped MFMA GEMMs over a device-built list of
// (expert, first row) tiles -- no host synchronisation is needed to learn the
// per-expert row counts:
//   1. gate+up over the routed rows AND the shared expert (as expert E with
//      all T tokens), clamped SwiGLU in the epilogue, h in bf16;
//   2. down over the routed rows, o in bf16;
//   3. shared down over the T tokens, whose epilogue adds the routed rows of
//      each token with one fixed fmaf chain (no atomics: bitwise repeatable).
// fp32 path: the same three steps with one thread per output value.
#include "device_common.h"
#include "kernels.h"

namespace coli {

// ---------------------------------------------------------------------------
// tile list: for every expert with rows, ceil(count/BM) tiles (expert, m0);
// then the shared expert's tiles (E, m0) over all T tokens.
// n_tiles[0] = routed tiles, n_tiles[1] = routed + shared tiles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void ffn_tiles_kernel(const int32_t *__restrict__ count, int E, int T,
                                                         int BM, int2 *__restrict__ tiles,
                                                         int32_t *__restrict__ n_tiles)
{
    __shared__ int32_t sc[1024];
    const int tid = threadIdx.x;
    const int mt = (tid < E) ? (count[tid] + BM - 1) / BM : 0;
    sc[tid] = mt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int v = (tid >= off) ? sc[tid - off] : 0;
        __syncthreads();
        sc[tid] += v;
        __syncthreads();
    }
    const int start = sc[tid] - mt;
    for (int i = 0; i < mt; ++i) tiles[start + i] = make_int2(tid, i * BM);
    const int routed = sc[1023];
    const int n_sh = (T + BM - 1) / BM;
    for (int i = tid; i < n_sh; i += 1024) tiles[routed + i] = make_int2(E, i * BM);
    if (tid == 0) {
        n_tiles[0] = routed;
        n_tiles[1] = routed + n_sh;
    }
}

// ---------------------------------------------------------------------------
// 1. gate+up grouped GEMM with the clamped SwiGLU epilogue.
// The B tile's BN rows interleave gate and up rows in blocks of 16:
// block b holds rows f0 + (b >> 1)*16 .. +15 of gate (b even) or up (b odd),
// so a wave's fragment pair (2j, 2j+1) holds gate and up of the same columns.
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(256) void gateup_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gate, const uint16_t *__restrict__ up,
    const uint16_t *__restrict__ s_gate, const uint16_t *__restrict__ s_up,
    const int32_t *__restrict__ count, const int32_t *__restrict__ offset,
    const int32_t *__restrict__ perm, const int2 *__restrict__ tiles, const int32_t *__restrict__ n_tiles,
    int T, int D, int E, int K, int F, uint16_t *__restrict__ h)
{
    static_assert(C::FN % 2 == 0, "gate/up fragment pairs");
    __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_BYTES / 2];
    constexpr int FCOLS = C::BN / 2;
    const int n_nt = F / FCOLS;
    const int ti = blockIdx.x / n_nt, nt = blockIdx.x % n_nt;
    if (ti >= n_tiles[1]) return;
    const int2 tile = tiles[ti];
    const int e = tile.x, m0 = tile.y;
    const bool shared = (e == E);
    const int R = T * K;
    const int cnt = shared ? T : count[e];
    const int hbase = shared ? R : offset[e];
    const uint16_t *G = shared ? s_gate : gate + (size_t)e * F * D;
    const uint16_t *U = shared ? s_up : up + (size_t)e * F * D;
    const int f0 = nt * FCOLS;
    const int ch0 = threadIdx.x & 7;

    const uint16_t *ap[C::A_PER_T];
    const uint16_t *bp[C::B_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        // padding rows (past the expert's last row) reread its first row
        int r = m0 + a_chunk_row<C>(i);
        if (a_chunk_row<C>(i) >= C::BM || r >= cnt) r = m0;
        const int t = shared ? r : perm[hbase + r] / K;
        ap[i] = x + (size_t)t * D + ch0 * 8;
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        int rr = a_chunk_row<C>(i);
        int blk = rr >> 4;
        int f = f0 + (blk >> 1) * 16 + (rr & 15);
        bp[i] = ((blk & 1) ? U : G) + (size_t)f * D + ch0 * 8;
    }
    f32x4 acc[C::FM][C::FN];
    mfma_mainloop<C>(ap, bp, D, lds, acc);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave % C::WAVES_N, wm = wave / C::WAVES_N;
#pragma unroll
    for (int m = 0; m < C::FM; ++m)
#pragma unroll
        for (int n = 0; n < C::FN; n += 2) {
            const int f = f0 + ((wn * C::FN + n) >> 1) * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int r = m0 + (wm * C::FM + m) * 16 + 4 * (lane >> 4) + i;
                if (r < cnt)
                    h[(size_t)(hbase + r) * F + f] =
                        f32_to_bf16_bits(swiglu_clamped(acc[m][n][i], acc[m][n + 1][i]));
            }
        }
}

// ---------------------------------------------------------------------------
// 2. down grouped GEMM over the routed rows: o[row] = W_down[e] h[row].
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(256) void down_bf16_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ down,
    const int32_t *__restrict__ count, const int32_t *__restrict__ offset,
    const int2 *__restrict__ tiles, const int32_t *__restrict__ n_tiles, int D, int F,
    uint16_t *__restrict__ o)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_BYTES / 2];
    const int n_nt = (D + C::BN - 1) / C::BN;      // the last n-tile may be ragged
    const int ti = blockIdx.x / n_nt, nt = blockIdx.x % n_nt;
    if (ti >= n_tiles[0]) return;
    const int2 tile = tiles[ti];
    const int e = tile.x, m0 = tile.y;
    const int cnt = count[e];
    const int base = offset[e];
    const int d0 = nt * C::BN;
    const int ch0 = threadIdx.x & 7;

    const uint16_t *ap[C::A_PER_T];
    const uint16_t *bp[C::B_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        int rr = a_chunk_row<C>(i);
        int r = (rr < C::BM && m0 + rr < cnt) ? m0 + rr : m0;
        ap[i] = h + (size_t)(base + r) * F + ch0 * 8;
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        int d = min(d0 + a_chunk_row<C>(i), D - 1);    // rows past D reread the last one
        bp[i] = down + ((size_t)e * D + d) * F + ch0 * 8;
    }
    f32x4 acc[C::FM][C::FN];
    mfma_mainloop<C>(ap, bp, F, lds, acc);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave % C::WAVES_N, wm = wave / C::WAVES_N;
#pragma unroll
    for (int m = 0; m < C::FM; ++m)
#pragma unroll
        for (int n = 0; n < C::FN; ++n) {
            const int d = d0 + (wn * C::FN + n) * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int r = m0 + (wm * C::FM + m) * 16 + 4 * (lane >> 4) + i;
                if (r < cnt && d < D) o[(size_t)(base + r) * D + d] = f32_to_bf16_bits(acc[m][n][i]);
            }
        }
}

// ---------------------------------------------------------------------------
// 3. shared down GEMM over the tokens with the combine in the epilogue:
//    v = S(x_t)[d]; v = fmaf(w_tj, o[inv(t,j)][d], v) for j = 0..K-1;
//    y = residual + v.
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(256) void combine_bf16_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ s_down, const uint16_t *__restrict__ o,
    const float *__restrict__ w, const int32_t *__restrict__ inv, const float *residual, int T, int D,
    int K, int F, float *y, uint16_t *__restrict__ y_bf16)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_BYTES / 2];
    const int n_nt = (D + C::BN - 1) / C::BN;
    const int mt = blockIdx.x / n_nt, nt = blockIdx.x % n_nt;
    const int t0 = mt * C::BM, d0 = nt * C::BN;
    const int R = T * K;
    const int ch0 = threadIdx.x & 7;

    const uint16_t *ap[C::A_PER_T];
    const uint16_t *bp[C::B_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        int rr = a_chunk_row<C>(i);
        int t = (rr < C::BM && t0 + rr < T) ? t0 + rr : t0;
        ap[i] = h + (size_t)(R + t) * F + ch0 * 8;
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        int d = min(d0 + a_chunk_row<C>(i), D - 1);
        bp[i] = s_down + (size_t)d * F + ch0 * 8;
    }
    f32x4 acc[C::FM][C::FN];
    mfma_mainloop<C>(ap, bp, F, lds, acc);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave % C::WAVES_N, wm = wave / C::WAVES_N;
#pragma unroll
    for (int m = 0; m < C::FM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + (wm * C::FM + m) * 16 + 4 * (lane >> 4) + i;
            if (t >= T) continue;
            int rows[8];
            float wt[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < K) {
                    rows[j] = inv[(size_t)t * K + j];
                    wt[j] = w[(size_t)t * K + j];
                }
#pragma unroll
            for (int n = 0; n < C::FN; ++n) {
                const int d = d0 + (wn * C::FN + n) * 16 + (lane & 15);
                if (d >= D) continue;
                float v = acc[m][n][i];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (j < K) v = fmaf(wt[j], bf16_bits_to_f32(o[(size_t)rows[j] * D + d]), v);
                const size_t idx = (size_t)t * D + d;
                if (residual) v = residual[idx] + v;
                y[idx] = v;
                if (y_bf16) y_bf16[idx] = f32_to_bf16_bits(v);
            }
        }
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per output value, plain fp32 dot products.
// ---------------------------------------------------------------------------
__global__ void gateup_f32_kernel(const float *__restrict__ x, const float *__restrict__ gate,
                                  const float *__restrict__ up, const float *__restrict__ s_gate,
                                  const float *__restrict__ s_up, const int32_t *__restrict__ ids,
                                  const int32_t *__restrict__ perm, int T, int D, int K, int F,
                                  float *__restrict__ h)
{
    const int R = T * K;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)(R + T) * F) return;
    const int r = (int)(i / F), f = (int)(i % F);
    const float *G, *U;
    int t;
    if (r < R) {
        const int p = perm[r];
        const int e = ids[p];
        t = p / K;
        G = gate + (size_t)e * F * D;
        U = up + (size_t)e * F * D;
    } else {
        t = r - R;
        G = s_gate;
        U = s_up;
    }
    const float *xr = x + (size_t)t * D;
    float g = 0.f, u = 0.f;
    for (int d = 0; d < D; ++d) {
        g = fmaf(xr[d], G[(size_t)f * D + d], g);
        u = fmaf(xr[d], U[(size_t)f * D + d], u);
    }
    h[i] = swiglu_clamped(g, u);
}

__global__ void down_f32_kernel(const float *__restrict__ h, const float *__restrict__ down,
                                const int32_t *__restrict__ ids, const int32_t *__restrict__ perm, int R,
                                int D, int F, float *__restrict__ o)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)R * D) return;
    const int r = (int)(i / D), d = (int)(i % D);
    const int e = ids[perm[r]];
    const float *hr = h + (size_t)r * F, *wd = down + ((size_t)e * D + d) * F;
    float acc = 0.f;
    for (int f = 0; f < F; ++f) acc = fmaf(hr[f], wd[f], acc);
    o[i] = acc;
}

__global__ void combine_f32_kernel(const float *__restrict__ h, const float *__restrict__ s_down,
                                   const float *__restrict__ o, const float *__restrict__ w,
                                   const int32_t *__restrict__ inv, const float *residual, int T, int D,
                                   int K, int F, float *y)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * D) return;
    const int t = (int)(i / D), d = (int)(i % D);
    const int R = T * K;
    const float *hr = h + (size_t)(R + t) * F, *sd = s_down + (size_t)d * F;
    float v = 0.f;
    for (int f = 0; f < F; ++f) v = fmaf(hr[f], sd[f], v);
    for (int j = 0; j < K; ++j) v = fmaf(w[(size_t)t * K + j], o[(size_t)inv[(size_t)t * K + j] * D + d], v);
    if (residual) v = residual[i] + v;
    y[i] = v;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
using Cfg16 = TileCfg<16, 128, 1, 4>;
using Cfg128 = TileCfg<128, 128, 2, 2>;

int ffn_tile_rows(int T, int E, int K)
{
    // rows per expert on average decides the tile height
    const long R = (long)T * K;
    return (R <= 24L * E) ? 16 : 128;
}

long ffn_max_tiles(int T, int E, int K, int bm)
{
    const long R = (long)T * K;
    return R / bm + (R < E ? R : E) + (T + bm - 1) / bm;
}

template <class C>
static void launch_bf16_gemms(const FfnLaunch &a, StageMarks &mk, hipStream_t st)
{
    const long mt = ffn_max_tiles(a.T, a.E, a.K, C::BM);
    const uint16_t *h = (const uint16_t *)a.h;
    mk.mark(st);
    gateup_bf16_kernel<C><<<(unsigned)(mt * (a.F / (C::BN / 2))), 256, 0, st>>>(
        (const uint16_t *)a.x, (const uint16_t *)a.gate, (const uint16_t *)a.up,
        (const uint16_t *)a.s_gate, (const uint16_t *)a.s_up, a.count, a.offset, a.perm, a.tiles,
        a.n_tiles, a.T, a.D, a.E, a.K, a.F, (uint16_t *)a.h);
    const int n_nt_d = (a.D + C::BN - 1) / C::BN;
    mk.mark(st);
    down_bf16_kernel<C><<<(unsigned)(mt * n_nt_d), 256, 0, st>>>(
        h, (const uint16_t *)a.down, a.count, a.offset, a.tiles, a.n_tiles, a.D, a.F,
        (uint16_t *)a.o);
    const int n_mt = (a.T + C::BM - 1) / C::BM;
    mk.mark(st);
    combine_bf16_kernel<C><<<(unsigned)(n_mt * n_nt_d), 256, 0, st>>>(
        h, (const uint16_t *)a.s_down, (const uint16_t *)a.o, a.w, a.inv, a.residual, a.T, a.D, a.K,
        a.F, a.y, (uint16_t *)a.y_bf16);
    mk.mark(st);
}

hipError_t launch_ffn(const FfnLaunch &a, hipStream_t st)
{
    const int T = a.T, D = a.D, K = a.K, F = a.F;
    const int R = T * K;
    StageMarks none;
    StageMarks &mk = a.marks ? *a.marks : none;
    mk.mark(st);
    if (a.bf16) {
        ffn_tiles_kernel<<<1, 1024, 0, st>>>(a.count, a.E, T, a.bm, a.tiles, a.n_tiles);
        if (a.bm == 16)
            launch_bf16_gemms<Cfg16>(a, mk, st);
        else
            launch_bf16_gemms<Cfg128>(a, mk, st);
    } else {
        const int64_t n1 = (int64_t)(R + T) * F, n2 = (int64_t)R * D, n3 = (int64_t)T * D;
        mk.mark(st);
        gateup_f32_kernel<<<(unsigned)((n1 + 255) / 256), 256, 0, st>>>(
            (const float *)a.x, (const float *)a.gate, (const float *)a.up, (const float *)a.s_gate,
            (const float *)a.s_up, a.ids, a.perm, T, D, K, F, (float *)a.h);
        mk.mark(st);
        if (n2 > 0)
            down_f32_kernel<<<(unsigned)((n2 + 255) / 256), 256, 0, st>>>(
                (const float *)a.h, (const float *)a.down, a.ids, a.perm, R, D, F, (float *)a.o);
        mk.mark(st);
        combine_f32_kernel<<<(unsigned)((n3 + 255) / 256), 256, 0, st>>>(
            (const float *)a.h, (const float *)a.s_down, (const float *)a.o, a.w, a.inv, a.residual, T,
            D, K, F, a.y);
        mk.mark(st);
    }
    return hipGetLastError();
}

}  // namespace coli
