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

#include <algorithm>

namespace coli {

// ---------------------------------------------------------------------------
// router logits, bf16 inputs, MFMA.  One workgroup per (32-token block,
// 32*NF-expert block, reduction split); the four waves split the
// workgroup's part of the reduction dimension into quarters and stream their
// operands straight from global memory into MFMA registers (each wave's data
// is its own, so no LDS staging).  The four partial blocks are added in LDS in
// wave order and stored as split s's partial sums zp[s][t][e]; top-K adds
// the splits in order s = 0, 1, ... and then the bias -- fixed orders, so the
// logits are bitwise reproducible.  Small batches split the reduction over
// several workgroups to occupy the GPU.  Rows past T and experts past E
// reread a valid row; their results are dropped.
// ---------------------------------------------------------------------------
constexpr int RT_M = 32;
constexpr int RT_BATCH = 8;         // reduction steps whose operands are loaded ahead
constexpr int RT_MAX_SPLITS = 8;

template <int NF>                    // 32-expert fragments per workgroup
__global__ __launch_bounds__(256) void router_logits_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, int T, int D, int E, int splits,
    float *__restrict__ zp, int32_t *__restrict__ done)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) *done = 0;     // the fused top-K's counter
    __shared__ float red[4 * NF * 16 * 64];         // [wave][frag][i][lane]
    const int n_nt = (E + 32 * NF - 1) / (32 * NF);
    const int n_mt = (T + RT_M - 1) / RT_M;
    const int sp = blockIdx.x / (n_mt * n_nt), rem = blockIdx.x % (n_mt * n_nt);
    const int mt = rem / n_nt, nt = rem % n_nt;
    const int t0 = mt * RT_M, e0 = nt * 32 * NF;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = D / (4 * splits), kbeg = (sp * 4 + wave) * kq + 8 * (lane >> 5);
    const uint16_t *pa = x + (size_t)min(t0 + (lane & 31), T - 1) * D + kbeg;
    const uint16_t *pb[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) pb[f] = wr + (size_t)min(e0 + 32 * f + (lane & 31), E - 1) * D + kbeg;
    f32x16 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[f][i] = 0.f;
    int k = 0;
    // batches of RT_BATCH steps: all loads of a batch are issued before its MFMAs
    for (; k + 16 * RT_BATCH <= kq; k += 16 * RT_BATCH) {
        bf16x8 a[RT_BATCH], b[RT_BATCH][NF];
#pragma unroll
        for (int u = 0; u < RT_BATCH; ++u) {
            a[u] = *reinterpret_cast<const bf16x8 *>(pa + k + 16 * u);
#pragma unroll
            for (int f = 0; f < NF; ++f) b[u][f] = *reinterpret_cast<const bf16x8 *>(pb[f] + k + 16 * u);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the whole batch of loads ahead of the MFMAs
#pragma unroll
        for (int u = 0; u < RT_BATCH; ++u)
#pragma unroll
            for (int f = 0; f < NF; ++f)
                acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u][f], acc[f], 0, 0, 0);
    }
    for (; k < kq; k += 16) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(pa + k);
#pragma unroll
        for (int f = 0; f < NF; ++f)
            acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, *reinterpret_cast<const bf16x8 *>(pb[f] + k), acc[f], 0, 0, 0);
    }
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[((wave * NF + f) * 16 + i) * 64 + lane] = acc[f][i];
    __syncthreads();
    float *z = zp + (size_t)sp * T * E;
    for (int q = threadIdx.x; q < NF * 16 * 64; q += 256) {
        const int f = q >> 10, i = (q >> 6) & 15, ln = q & 63;
        float v = red[((0 * NF + f) * 16 + i) * 64 + ln];
        v += red[((1 * NF + f) * 16 + i) * 64 + ln];
        v += red[((2 * NF + f) * 16 + i) * 64 + ln];
        v += red[((3 * NF + f) * 16 + i) * 64 + ln];
        const int t = t0 + 8 * (i >> 2) + 4 * (ln >> 5) + (i & 3);
        const int e = e0 + f * 32 + (ln & 31);
        if (t < T && e < E) z[(size_t)t * E + e] = v;
    }
}

// ---------------------------------------------------------------------------
// router logits, bf16 inputs, large batches.  One workgroup of 8 waves per
// (64-token block, reduction split) covers every expert, so each token row is
// fetched once per split and the router matrix is shared by all token blocks
// from L2.  Each 64-wide reduction step needs the block's 64 token rows and
// the E router rows (padded to 32), copied global -> LDS eight 128-byte rows
// per copy instruction into two rings: token-row slots of 8 KB with XS - 1
// steps issued ahead, router-row slots with WS - 1 steps in flight.  Each
// wave waits for its own copies of step kt's router rows (the token rows of
// step kt were issued before them, and copies complete in order), then the
// barrier makes everyone's visible.  Rows are XOR-swizzled in 16-byte chunks
// so the fragment reads are free of bank conflicts.  Wave w computes tokens
// 32 (w / 4) .. +31 of the block against expert fragments w % 4, w % 4 + 4,
// ... over the whole split (two waves per SIMD hide each other's LDS and
// MFMA latencies); split s's partial sums go to zp[s][t][e] (top-K adds the
// splits in order and then the bias).
// ---------------------------------------------------------------------------
constexpr int RL_BK = 64;
constexpr int RL_MAX_E = 512;
constexpr int RL_LDS_BYTES = 160 * 1024;
constexpr int RL_MIN_T = 513;       // smaller batches use the register-streamed kernel above
constexpr int RL_TOK = 64;          // tokens per workgroup
constexpr int RL_XSLOT = RL_TOK * 128;
constexpr int RL_MAX_XS = 6;        // token-row slots

// Ring sizes for E experts: `ws` router-row slots (3, else 2) of
// ceil(E / 32) * 4 KB, then as many token-row slots as fit, at most RL_MAX_XS.
static void router_lds_rings(int E, int *xs, int *ws)
{
    const int wstage = (E + 31) / 32 * 4096;
    *ws = (3 * wstage + RL_MAX_XS * RL_XSLOT <= RL_LDS_BYTES) ? 3 : 2;
    *xs = std::min(RL_MAX_XS, (RL_LDS_BYTES - *ws * wstage) / RL_XSLOT);
}

// s_waitcnt needs an immediate: wave-uniform n in [0, 39] via a jump table
// (a larger n waits for every copy, which is also correct).
__device__ __forceinline__ void wait_vmcnt_rt(int n)
{
    switch (n) {
#define COLI_VM(i) case i: wait_vmcnt_c<i>(); break;
        COLI_VM(0) COLI_VM(1) COLI_VM(2) COLI_VM(3) COLI_VM(4) COLI_VM(5) COLI_VM(6) COLI_VM(7)
        COLI_VM(8) COLI_VM(9) COLI_VM(10) COLI_VM(11) COLI_VM(12) COLI_VM(13) COLI_VM(14) COLI_VM(15)
        COLI_VM(16) COLI_VM(17) COLI_VM(18) COLI_VM(19) COLI_VM(20) COLI_VM(21) COLI_VM(22) COLI_VM(23)
        COLI_VM(24) COLI_VM(25) COLI_VM(26) COLI_VM(27) COLI_VM(28) COLI_VM(29) COLI_VM(30) COLI_VM(31)
        COLI_VM(32) COLI_VM(33) COLI_VM(34) COLI_VM(35) COLI_VM(36) COLI_VM(37) COLI_VM(38) COLI_VM(39)
#undef COLI_VM
        default: wait_vmcnt_c<0>(); break;
    }
}

template <int NFW>                    // expert fragments per wave: nfrag <= 4 * NFW
__global__ __launch_bounds__(512) void router_logits_lds_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, int T, int D, int E, int splits,
    int xs, int ws, float *__restrict__ zp, int32_t *__restrict__ done)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) *done = 0;     // the fused top-K's counter
    constexpr int CPW_MAX = 2 * NFW;              // router-row copies per wave per step
    __shared__ __attribute__((aligned(1024))) char lds[RL_LDS_BYTES];
    const int nfrag = (E + 31) / 32;
    const int wstage = nfrag * 4096;              // router rows of one step
    char *const xl = lds;                         // token-row slots
    char *const wl = lds + xs * RL_XSLOT;         // router-row slots
    const int n_mt = (T + RL_TOK - 1) / RL_TOK;
    const int sp = blockIdx.x / n_mt, mt = blockIdx.x % n_mt;
    const int t0 = mt * RL_TOK;
    const int kq = D / splits, nk = kq / RL_BK;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int th = w >> 2, wc = w & 3;            // token half, expert fragment column

    // a copy fills 8 LDS rows; lane l takes row 8 c + l / 8, whose chunk
    // position l % 8 holds the row's global chunk (l % 8) ^ ((row / 2) % 8).
    // Wave w copies token rows 8 w .. 8 w + 7 and router-row groups q = w + 8 j
    // (rows 8 q .. 8 q + 7) for q < 4 nfrag; rows past T or E reread a valid row.
    const int xr = w * 8 + (lane >> 3);
    const uint16_t *xsrc = x + (size_t)min(t0 + xr, T - 1) * D + (size_t)sp * kq + ((lane & 7) ^ ((xr >> 1) & 7)) * 8;
    const int cw = max(0, (4 * nfrag - w + 7) / 8);   // this wave's router-row copies per step
    const uint16_t *wsrc[CPW_MAX];
#pragma unroll
    for (int j = 0; j < CPW_MAX; ++j) {
        const int r = (w + 8 * j) * 8 + (lane >> 3);
        wsrc[j] = wr + (size_t)min(r, E - 1) * D + (size_t)sp * kq + ((lane & 7) ^ ((r >> 1) & 7)) * 8;
    }
    // the workgroups start their reduction at different steps (rot), so the
    // ones running together read different columns of the shared router rows
    const int rot = mt % nk;
    auto kblock = [&](int s) { return (s + rot < nk) ? s + rot : s + rot - nk; };
    auto issue_x = [&](int s) {
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(xsrc + kblock(s) * RL_BK),
                                         (__attribute__((address_space(3))) void *)(xl + (s % xs) * RL_XSLOT + w * 1024),
                                         16, 0, 0);
    };
    auto issue_w = [&](int s) {
        char *st = wl + (s % ws) * wstage;
        const int kb = kblock(s);
#pragma unroll
        for (int j = 0; j < CPW_MAX; ++j)
            if (j < cw)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(wsrc[j] + kb * RL_BK),
                    (__attribute__((address_space(3))) void *)(st + (w + 8 * j) * 1024), 16, 0, 0);
    };

    // fragment i of wave w: experts (w % 4 + 4i) * 32 ..; past the last
    // fragment the wave recomputes the last one and drops the result
    const int arow = th * 32 + (lane & 31);
    int brow[NFW];
#pragma unroll
    for (int i = 0; i < NFW; ++i) brow[i] = min(wc + 4 * i, nfrag - 1) * 32 + (lane & 31);
    f32x16 acc[NFW];
#pragma unroll
    for (int i = 0; i < NFW; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;

    // issued: this wave's copy instructions so far; f0, f1: its count right
    // after the router rows of the oldest (next) steps in flight were issued
    const int xa = xs - 1;
    int issued = 0, f0 = 0, f1 = 0;
    for (int s = 0; s < min(xa, nk); ++s) {
        issue_x(s);
        ++issued;
    }
    issue_w(0);
    issued += cw;
    f0 = issued;
    if (ws == 3 && nk > 1) {
        issue_w(1);
        issued += cw;
        f1 = issued;
    }
    for (int kt = 0; kt < nk; ++kt) {
        wait_vmcnt_rt(issued - f0);                 // this wave's copies of step kt landed
        f0 = f1;
        asm volatile("s_barrier" ::: "memory");     // everyone's; step kt-1 fully read
        if (kt + xa < nk) {
            issue_x(kt + xa);
            ++issued;
        }
        if (kt + ws - 1 < nk) {
            issue_w(kt + ws - 1);
            issued += cw;
            if (ws == 3) f1 = issued;
            else f0 = issued;
        }
        const char *xst = xl + (kt % xs) * RL_XSLOT;
        const char *wst = wl + (kt % ws) * wstage;
        bf16x8 a[RL_BK / 16], b[RL_BK / 16][NFW];
#pragma unroll
        for (int kk = 0; kk < RL_BK / 16; ++kk) {
            const int c = kk * 2 + (lane >> 5);
            a[kk] = *reinterpret_cast<const bf16x8 *>(xst + swz(arow, c) * 2);
#pragma unroll
            for (int i = 0; i < NFW; ++i) b[kk][i] = *reinterpret_cast<const bf16x8 *>(wst + swz(brow[i], c) * 2);
        }
        __builtin_amdgcn_sched_barrier(0);   // all of the step's fragment reads in flight before its MFMAs
#pragma unroll
        for (int kk = 0; kk < RL_BK / 16; ++kk)
#pragma unroll
            for (int i = 0; i < NFW; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], b[kk][i], acc[i], 0, 0, 0);
    }
    float *z = zp + (size_t)sp * T * E;
#pragma unroll
    for (int i = 0; i < NFW; ++i) {
        const int f = wc + 4 * i;
        if (f >= nfrag) continue;
        const int e = f * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int t = t0 + th * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            if (t < T && e < E) z[(size_t)t * E + e] = acc[i][j];
        }
    }
}

// Reduction splits of the bf16 router: enough workgroups for small batches;
// a split must cover whole 64-element quarters-of-16 (D / (64 splits) integral).
int router_splits(int T, int D)
{
    int want = (T <= 128) ? RT_MAX_SPLITS : (T <= 512) ? 4 : 1;
    if (T >= RL_MIN_T)                          // one 64-token block per workgroup: aim for 256
        while (want < RT_MAX_SPLITS && (T + RL_TOK - 1) / RL_TOK * want < 256) want *= 2;
    int s = want;
    while (s > 1 && (D / 64) % s != 0) --s;
    return s;
}

// fp32 router: one thread per (token, expert), plain dot product (one split).
__global__ void router_logits_f32_kernel(const float *__restrict__ x, const float *__restrict__ wr, int T,
                                         int D, int E, float *__restrict__ z, int32_t *__restrict__ done)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) *done = 0;                        // the fused top-K's counter
    if (i >= (int64_t)T * E) return;
    int t = (int)(i / E), e = (int)(i % E);
    const float *xr = x + (size_t)t * D, *wrow = wr + (size_t)e * D;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc = fmaf(xr[d], wrow[d], acc);
    z[i] = acc;
}

// ---------------------------------------------------------------------------
// top-K: one wave per token.  Lane l holds the logits of experts l, l+64, ...
// (slot s: expert 64 s + l) as order-preserving unsigned images of the fp32
// values.  K rounds each take the largest remaining image (a DPP wave
// maximum) at its lowest expert index (ballots over the slots in order), so
// the K taken are the first K of the order (image desc, index asc): ties go
// to the lower index.  Since the index is 64 s + l, slot-major lane order is
// ascending index order, so each chosen expert's output position is a
// prefix popcount of the chosen masks: the ids come out ascending.
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

constexpr int TOPK_MAX_E = 1024;

// Maximum over the 64 lanes of a wave (all lanes active), returned in every
// lane: pairs, quads, half rows and rows by DPP, then the four row maxima.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}

// The top-K of token t by one wave; sel_e / sel_z: the wave's 8-entry LDS
// scratch.
template <int SLOTS, int NSP>          // NSP >= the number of reduction splits
__device__ __forceinline__ void topk_token(const float *__restrict__ zp, int splits, const float *__restrict__ bias,
                                           int T, int E, int K, int t, int32_t *sel_e, float *sel_z,
                                           int32_t *__restrict__ ids, float *__restrict__ w)
{
    const int lane = threadIdx.x & 63;

    // logit = (split 0 + split 1 + ...) + bias; 0 marks an empty slot, every
    // real logit maps above 0 (NaN aside).  Every partial and bias of the
    // token is loaded before any sum, so the loads cost one memory latency:
    // the loads are unconditional (every slot's index clamped to a real
    // expert -- the slot count is rounded up to a template size, so slots
    // before the last may lie past E as well -- and splits past the last
    // clamped to it), and the empty asm
    // statements take every loaded value before any is used, so the compiler
    // cannot sink a load into a branch.  Slot s of lane l is expert 64 s + l
    // (clamped), so every load of a row is addressed from the row's pointer.
    float part[SLOTS][NSP], bs[SLOTS];
    auto col = [&](int s) { return min(lane + 64 * s, E - 1); };
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) bs[s] = bias[col(s)];
#pragma unroll
    for (int sp = 0; sp < NSP; ++sp) {
        const float *zr = zp + ((size_t)min(sp, splits - 1) * T + t) * E;
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) part[s][sp] = zr[col(s)];
    }
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        asm volatile("" : "+v"(bs[s]));
#pragma unroll
        for (int sp = 0; sp < NSP; ++sp) asm volatile("" : "+v"(part[s][sp]));
    }
    uint32_t key[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        float v = part[s][0];
#pragma unroll
        for (int sp = 1; sp < NSP; ++sp)
            if (sp < splits) v += part[s][sp];
        // real experts map to images >= 1 (only a NaN could map to 0), so a
        // padding slot (image 0) is never among the K taken below
        key[s] = (lane + 64 * s < E) ? max(ordered_bits(v + bs[s]), 1u) : 0u;
    }
    // The K largest images, ties to the lower expert index.  First the K
    // largest lane maxima, one per round (wave maximum of the lanes' heads,
    // one lane holding it retired); tau, the K-th of them, is a lower bound
    // of the K-th largest image, since K distinct lanes hold an image >= tau,
    // so every image of the top K is >= tau.  The candidates (images >= tau;
    // padding slots are 0 < tau) are exactly the top K unless some lane holds
    // two of them or images tie at tau; then the smallest candidates --
    // image ascending, expert index descending -- are dropped one per round
    // until K remain, leaving the first K of the order (image desc, index asc).
    uint32_t head = key[0];
#pragma unroll
    for (int s = 1; s < SLOTS; ++s) head = max(head, key[s]);
    uint32_t tau = 0;
    for (int j = 0; j < K; ++j) {
        const uint32_t m = wave_max_u32(head);
        tau = m;
        const uint64_t b = __ballot(head == m);
        if (lane == __ffsll((unsigned long long)b) - 1) head = 0u;
    }
    uint64_t chosen[SLOTS];
    int ncand = 0;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        chosen[s] = __ballot(key[s] >= tau);
        ncand += __popcll(chosen[s]);
    }
    while (ncand > K) {
        uint32_t mn = 0xffffffffu;                // smallest candidate of this lane
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
            if ((chosen[s] >> lane) & 1ull) mn = min(mn, key[s]);
        mn = wave_reduce_u32(mn, MinU32());
#pragma unroll
        for (int s = SLOTS - 1; s >= 0; --s) {    // highest expert index holding it
            const uint64_t b = chosen[s] & __ballot(key[s] == mn);
            if (b) {
                chosen[s] &= ~(1ull << (63 - __clzll((long long)b)));
                break;
            }
        }
        --ncand;
    }
    // output position of each chosen expert: chosen experts of lower slots,
    // then lower lanes of this slot
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int base = 0;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        if ((chosen[s] >> lane) & 1ull) {
            const int j = base + __popcll(chosen[s] & below);
            sel_e[j] = lane + 64 * s;
            sel_z[j] = from_ordered_bits(key[s]);
        }
        base += __popcll(chosen[s]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // weights p_j / sum p over the chosen experts, lane j holding chosen
    // expert j (ascending id order).  When every chosen logit is negative the
    // ratios are formed relative to the largest one so that tiny sigmoids
    // cannot underflow the sum: sigmoid(a)/sigmoid(m) = e^(a-m) (1+e^m) / (1+e^a).
    // The maximum and the sum over lanes 0..7 are butterflies (every lane
    // ends with the same value, summed in the same order).
    const float zl = (lane < K) ? sel_z[lane] : -INFINITY;
    float zmax = zl;
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, o));
    float pl = 0.f;
    if (lane < K)
        pl = (zmax >= 0.f) ? sigmoid_f32(zl) : expf(zl - zmax) * (1.0f + expf(zmax)) / (1.0f + expf(zl));
    float psum = pl;
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) psum += __shfl_xor(psum, o);
    if (lane < K) {
        ids[(size_t)t * K + lane] = sel_e[lane];
        w[(size_t)t * K + lane] = pl / psum;
    }
}

template <int SLOTS, int NSP>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ zp, int splits,
                                                   const float *__restrict__ bias, int T, int E, int K,
                                                   int32_t *__restrict__ ids, float *__restrict__ w)
{
    __shared__ int32_t sel_e_s[4][8];
    __shared__ float sel_z_s[4][8];
    const int wave = threadIdx.x >> 6;
    const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    if (t >= T) return;                           // whole waves: t is uniform in a wave
    topk_token<SLOTS, NSP>(zp, splits, bias, T, E, K, t, sel_e_s[wave], sel_z_s[wave], ids, w);
}

// ---------------------------------------------------------------------------
// permutation.  Tiles of 256 tokens, one workgroup of 4 waves each; wave w
// builds one bitmask per expert over its 64 tokens (bit l = token 64w + l of
// the tile chose the expert).  A token's rank among the tile's tokens of an
// expert is the popcount of the earlier waves' masks plus the popcount of its
// own wave's mask below its lane.
// ---------------------------------------------------------------------------
constexpr int PERM_TILE = 256;

// The K (<= 8) expert ids of token t in one round of loads: unconditional
// loads (slots past K reread slot K - 1), each value taken by an empty asm
// statement before any use, so the compiler cannot sink a load into the
// per-slot branch of its user (which costs one round trip per slot).
__device__ __forceinline__ void load_token_ids(const int32_t *__restrict__ ids, int t, int K, int (&e)[8])
{
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = ids[(size_t)t * K + min(j, K - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(e[j]));
}

__device__ __forceinline__ void build_tile_masks(const int32_t *__restrict__ ids, int T, int E, int K,
                                                 uint64_t *masks)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < 4 * E; i += PERM_TILE) masks[i] = 0ull;
    __syncthreads();
    const int t = blockIdx.x * PERM_TILE + threadIdx.x;
    if (t < T) {
        int e[8];
        load_token_ids(ids, t, K, e);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < K) atomicOr((unsigned long long *)&masks[wave * E + e[j]], 1ull << lane);
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t *__restrict__ ids, int T, int E,
                                                        int K, int32_t *__restrict__ tile_count)
{
    __shared__ uint64_t masks[4 * TOPK_MAX_E];
    build_tile_masks(ids, T, E, K, masks);
    for (int e = threadIdx.x; e < E; e += PERM_TILE)
        tile_count[(size_t)blockIdx.x * E + e] = __popcll(masks[e]) + __popcll(masks[E + e]) +
                                                 __popcll(masks[2 * E + e]) + __popcll(masks[3 * E + e]);
}

// Every workgroup forms its tile's first row per expert from the counts of
// all tiles: offset[e] (exclusive scan over experts of the totals) plus the
// expert's rows in earlier tiles.  Thread i holds experts 4 i .. 4 i + 3
// (E <= 1024); workgroup 0 also writes count and offset.  Then every
// assignment of the tile is written to its row.  The tile's ids are loaded
// first and every tile's counts right after them (16 tiles per round), so
// the loads cost one memory latency, and the masks are built from the ids
// already in registers (prefill permutation stage 16.4 -> 14.9 us, A/B).
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t *__restrict__ ids, int T, int E,
                                                           int K, const int32_t *__restrict__ tile_count,
                                                           int ntiles, int32_t *__restrict__ count,
                                                           int32_t *__restrict__ offset,
                                                           int32_t *__restrict__ perm,
                                                           int32_t *__restrict__ inv)
{
    __shared__ uint64_t masks[4 * TOPK_MAX_E];
    __shared__ int32_t first_s[TOPK_MAX_E];
    __shared__ int32_t ws[4];
    constexpr int TPR = 16;                       // tiles' counts per round of loads
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t = blockIdx.x * PERM_TILE + tid;
    int ev[8];
    load_token_ids(ids, min(t, T - 1), K, ev);
    for (int i = tid; i < 4 * E; i += PERM_TILE) masks[i] = 0ull;
    int tot[4] = {0, 0, 0, 0}, before[4] = {0, 0, 0, 0};
    // unconditional loads of clamped indices
    for (int tl0 = 0; tl0 < ntiles; tl0 += TPR) {
        int v[TPR][4];
#pragma unroll
        for (int k = 0; k < TPR; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[k][i] = tile_count[(size_t)min(tl0 + k, ntiles - 1) * E + min(4 * tid + i, E - 1)];
#pragma unroll
        for (int k = 0; k < TPR; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tl = tl0 + k;
                tot[i] += (tl < ntiles) ? v[k][i] : 0;
                before[i] += (tl < (int)blockIdx.x) ? v[k][i] : 0;
            }
    }
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (4 * tid + i >= E) tot[i] = 0;
        local += tot[i];
    }
    const int incl = block_scan_incl<4>(local, ws);   // its barriers also order the masks' zeroing
    int run = incl - local;                       // rows of the experts before 4 tid
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * tid + i;
        if (e < E) {
            first_s[e] = run + before[i];
            if (blockIdx.x == 0) {
                count[e] = tot[i];
                offset[e] = run;
            }
        }
        run += tot[i];
    }
    if (blockIdx.x == 0 && tid == 255) offset[E] = incl;
    if (t < T) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < K) atomicOr((unsigned long long *)&masks[wave * E + ev[j]], 1ull << lane);
    }
    __syncthreads();                              // masks and first_s
    if (t >= T) return;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j >= K) break;
        const int e = ev[j];
        int rank = __popcll(masks[wave * E + e] & below);
        for (int w2 = 0; w2 < wave; ++w2) rank += __popcll(masks[w2 * E + e]);
        const int row = first_s[e] + rank;
        perm[row] = t * K + j;
        inv[(size_t)t * K + j] = row;
    }
}

// ---------------------------------------------------------------------------
// permutation of a small batch (T <= PERM_SMALL_T) in one workgroup of 1024
// threads: the same bitmask construction over 16 waves of 64 tokens, the
// counts, the exclusive scan over experts and the scatter, with no global
// round trips between them.  The result is the same stable counting sort.
// ---------------------------------------------------------------------------
constexpr int PERM_SMALL_T = 1024;
constexpr int PERM_SMALL_MAX_E = 512;         // 16 waves x E masks of 8 bytes in LDS

// The small-batch permutation by one workgroup of 1024 threads (T <= 1024,
// E <= 512); ids must be visible to the workgroup.
__device__ __forceinline__ void perm_small_body(const int32_t *__restrict__ ids, int T, int E, int K,
                                                int32_t *__restrict__ count, int32_t *__restrict__ offset,
                                                int32_t *__restrict__ perm, int32_t *__restrict__ inv)
{
    __shared__ uint64_t masks[16 * PERM_SMALL_MAX_E];
    __shared__ int32_t sc[1024];
    __shared__ int32_t ws[16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nw = (T + 63) >> 6;                 // waves that hold tokens
    for (int i = tid; i < nw * E; i += 1024) masks[i] = 0ull;
    __syncthreads();
    int ev[8];
    if (tid < T) {
        load_token_ids(ids, tid, K, ev);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < K) atomicOr((unsigned long long *)&masks[wave * E + ev[j]], 1ull << lane);
    }
    __syncthreads();
    int c = 0;
    if (tid < E)
        for (int w2 = 0; w2 < nw; ++w2) c += __popcll(masks[w2 * E + tid]);
    sc[tid] = block_scan_incl_1024(c, ws);
    __syncthreads();
    if (tid < E) {
        count[tid] = c;
        offset[tid] = sc[tid] - c;
        if (tid == E - 1) offset[E] = sc[tid];
    }
    if (tid < T) {
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j >= K) break;
            const int e = ev[j];
            int rank = __popcll(masks[wave * E + e] & below);
            for (int w2 = 0; w2 < wave; ++w2) rank += __popcll(masks[w2 * E + e]);
            const int row = (e > 0 ? sc[e - 1] : 0) + rank;   // exclusive prefix + rank
            perm[row] = tid * K + j;
            inv[(size_t)tid * K + j] = row;
        }
    }
}

// The same stable counting sort for a batch of at most 64 tokens, by one
// wave with no barriers (lane t holds token t): masks[e] gets bit t when
// token t chose expert e, lane l counts and scans experts l * epl .. + epl
// - 1 (epl = ceil(E / 64)), and a token's rank among an expert's tokens is
// the popcount of the mask below its bit.  Wave-scope fences order the LDS
// phases (the lanes of one wave run in lockstep, but the compiler must not
// move a lane's reads of other lanes' words across them).  ids must be
// visible to the wave.
constexpr int PERM_WAVE_T = 64;

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void perm_wave_body(const int32_t *__restrict__ ids, int T, int E, int K,
                                               int32_t *__restrict__ count, int32_t *__restrict__ offset,
                                               int32_t *__restrict__ perm, int32_t *__restrict__ inv)
{
    __shared__ uint64_t wmask[PERM_SMALL_MAX_E];
    __shared__ int32_t wfirst[PERM_SMALL_MAX_E];
    const int lane = threadIdx.x & 63;
    const int epl = (E + 63) >> 6;                // at most 8 (E <= 512)
    for (int e = lane; e < E; e += 64) wmask[e] = 0ull;
    int ev[8];
    if (lane < T) load_token_ids(ids, lane, K, ev);
    wave_lds_sync();
    if (lane < T) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < K) atomicOr((unsigned long long *)&wmask[ev[j]], 1ull << lane);
    }
    wave_lds_sync();
    int c[8], tot = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = lane * epl + i;
        c[i] = (i < epl && e < E) ? __popcll(wmask[e]) : 0;
        tot += c[i];
    }
    int inc = tot;                                // inclusive scan of the lanes' totals
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(inc, off);
        if (lane >= off) inc += u;
    }
    int run = inc - tot;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = lane * epl + i;
        if (i < epl && e < E) {
            count[e] = c[i];
            offset[e] = run;
            wfirst[e] = run;
            run += c[i];
        }
    }
    if (lane == 63) offset[E] = inc;
    wave_lds_sync();
    if (lane < T) {
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j >= K) break;
            const int e = ev[j];
            const int row = wfirst[e] + __popcll(wmask[e] & below);
            perm[row] = lane * K + j;
            inv[(size_t)lane * K + j] = row;
        }
    }
}

__global__ __launch_bounds__(1024) void perm_small_kernel(const int32_t *__restrict__ ids, int T, int E, int K,
                                                          int32_t *__restrict__ count,
                                                          int32_t *__restrict__ offset,
                                                          int32_t *__restrict__ perm,
                                                          int32_t *__restrict__ inv)
{
    perm_small_body(ids, T, E, K, count, offset, perm, inv);
}

// ---------------------------------------------------------------------------
// top-K and the small-batch permutation in one launch (T <= 1024, E <= 512):
// workgroups of 16 waves, the first TOPK_PER_WG of which take one token each
// (the top-K of a token is bound by instruction issue, so tokens are spread
// over many CUs; the other waves are there for the permutation, which needs
// all 16 in the one workgroup that runs it, or one wave for at most 64
// tokens).  Each workgroup publishes its ids: thread 0 issues an agent-scope
// release fence (the barrier before it makes the other waves' stores part of
// it) and increments a device-scope counter; the workgroup that takes the
// counter to the grid size is the last one, and after thread 0's acquire
// fence (then the barrier) it sees every token's ids and builds the
// permutation.  Release and acquire are one L2 write-back and one L2
// invalidation; a sequentially consistent fence does both, in every
// workgroup (decode step 397.2 -> 395.9 us).  The counter is set to zero by
// the router kernel earlier on the same stream.  The permutation depends
// only on the ids, so it is the same whichever workgroup is last.
// ---------------------------------------------------------------------------
constexpr int TOPK_PER_WG = 4;

template <int SLOTS, int NSP>
__global__ __launch_bounds__(1024) void topk_perm_kernel(const float *__restrict__ zp, int splits,
                                                         const float *__restrict__ bias, int T, int E, int K,
                                                         int32_t *__restrict__ ids, float *__restrict__ w,
                                                         int32_t *__restrict__ done, int32_t *__restrict__ count,
                                                         int32_t *__restrict__ offset, int32_t *__restrict__ perm,
                                                         int32_t *__restrict__ inv)
{
    __shared__ int32_t sel_e_s[TOPK_PER_WG][8];
    __shared__ float sel_z_s[TOPK_PER_WG][8];
    __shared__ int32_t last_s;
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * TOPK_PER_WG + wave;
    if (wave < TOPK_PER_WG && t < T)
        topk_token<SLOTS, NSP>(zp, splits, bias, T, E, K, t, sel_e_s[wave], sel_z_s[wave], ids, w);
    __syncthreads();                              // this workgroup's ids are written
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        last_s = atomicAdd(done, 1) == (int)gridDim.x - 1;
        if (last_s) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (!last_s) return;
    if (T <= PERM_WAVE_T) {
        if (wave == 0) perm_wave_body(ids, T, E, K, count, offset, perm, inv);
    } else {
        perm_small_body(ids, T, E, K, count, offset, perm, inv);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int perm_tiles(int T) { return (T + PERM_TILE - 1) / PERM_TILE; }

// T = 0: no tokens, but count and offset are still defined (all zero).
__global__ void route_empty_kernel(int E, int32_t *__restrict__ count, int32_t *__restrict__ offset)
{
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
        if (e < E) count[e] = 0;
        offset[e] = 0;
    }
}

template <int SLOTS>
static void launch_topk(unsigned g, hipStream_t st, const float *z, int splits, const float *bias, int T, int E,
                        int K, int32_t *ids, float *w)
{
    if (splits <= 1) topk_kernel<SLOTS, 1><<<g, 256, 0, st>>>(z, splits, bias, T, E, K, ids, w);
    else if (splits <= 2) topk_kernel<SLOTS, 2><<<g, 256, 0, st>>>(z, splits, bias, T, E, K, ids, w);
    else if (splits <= 4) topk_kernel<SLOTS, 4><<<g, 256, 0, st>>>(z, splits, bias, T, E, K, ids, w);
    else topk_kernel<SLOTS, RT_MAX_SPLITS><<<g, 256, 0, st>>>(z, splits, bias, T, E, K, ids, w);
}

template <int SLOTS>
static void launch_topk_perm(unsigned g, hipStream_t st, const RouteLaunch &a, int splits)
{
#define COLI_TOPK_PERM(NSP)                                                                               \
    topk_perm_kernel<SLOTS, NSP><<<g, 1024, 0, st>>>(a.z, splits, a.bias, a.T, a.E, a.K, a.ids, a.w, a.done, \
                                                     a.count, a.offset, a.perm, a.inv)
    if (splits <= 1) COLI_TOPK_PERM(1);
    else if (splits <= 2) COLI_TOPK_PERM(2);
    else if (splits <= 4) COLI_TOPK_PERM(4);
    else COLI_TOPK_PERM(RT_MAX_SPLITS);
#undef COLI_TOPK_PERM
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
    int splits = 1;
    if (a.bf16) {
        // small batches: 32-expert blocks and a split reduction for more
        // workgroups; large: 64-expert blocks
        splits = router_splits(T, D);
        const int n_mt = (T + RT_M - 1) / RT_M;
        if (T >= RL_MIN_T && E <= RL_MAX_E) {
            const int nfw = ((E + 31) / 32 + 3) / 4;
            const unsigned g = splits * ((T + RL_TOK - 1) / RL_TOK);
            int xs = 0, ws = 0;
            router_lds_rings(E, &xs, &ws);
            const uint16_t *x = (const uint16_t *)a.x, *wr = (const uint16_t *)a.wr;
            if (nfw == 1) router_logits_lds_kernel<1><<<g, 512, 0, st>>>(x, wr, T, D, E, splits, xs, ws, a.z, a.done);
            else if (nfw == 2) router_logits_lds_kernel<2><<<g, 512, 0, st>>>(x, wr, T, D, E, splits, xs, ws, a.z, a.done);
            else if (nfw == 3) router_logits_lds_kernel<3><<<g, 512, 0, st>>>(x, wr, T, D, E, splits, xs, ws, a.z, a.done);
            else router_logits_lds_kernel<4><<<g, 512, 0, st>>>(x, wr, T, D, E, splits, xs, ws, a.z, a.done);
        } else if (T <= 512)
            router_logits_bf16_kernel<1><<<splits * n_mt * ((E + 31) / 32), 256, 0, st>>>(
                (const uint16_t *)a.x, (const uint16_t *)a.wr, T, D, E, splits, a.z, a.done);
        else
            router_logits_bf16_kernel<2><<<splits * n_mt * ((E + 63) / 64), 256, 0, st>>>(
                (const uint16_t *)a.x, (const uint16_t *)a.wr, T, D, E, splits, a.z, a.done);
    } else {
        int64_t n = (int64_t)T * E;
        router_logits_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
            (const float *)a.x, (const float *)a.wr, T, D, E, a.z, a.done);
    }
    mk.mark(st);
    if (T <= PERM_SMALL_T && E <= PERM_SMALL_MAX_E) {
        // top-K and the permutation in one launch; the permutation stage is empty
        const int g = (T + TOPK_PER_WG - 1) / TOPK_PER_WG, slots = (E + 63) / 64;
        if (slots <= 1) launch_topk_perm<1>(g, st, a, splits);
        else if (slots <= 2) launch_topk_perm<2>(g, st, a, splits);
        else if (slots <= 3) launch_topk_perm<3>(g, st, a, splits);
        else if (slots <= 4) launch_topk_perm<4>(g, st, a, splits);
        else if (slots <= 5) launch_topk_perm<5>(g, st, a, splits);
        else launch_topk_perm<8>(g, st, a, splits);
        mk.mark(st);
        mk.mark(st);
        return hipGetLastError();
    }
    {
        const int g = (T + 3) / 4, slots = (E + 63) / 64;
        if (slots <= 1) launch_topk<1>(g, st, a.z, splits, a.bias, T, E, K, a.ids, a.w);
        else if (slots <= 2) launch_topk<2>(g, st, a.z, splits, a.bias, T, E, K, a.ids, a.w);
        else if (slots <= 3) launch_topk<3>(g, st, a.z, splits, a.bias, T, E, K, a.ids, a.w);
        else if (slots <= 4) launch_topk<4>(g, st, a.z, splits, a.bias, T, E, K, a.ids, a.w);
        else if (slots <= 5) launch_topk<5>(g, st, a.z, splits, a.bias, T, E, K, a.ids, a.w);
        else if (slots <= 8) launch_topk<8>(g, st, a.z, splits, a.bias, T, E, K, a.ids, a.w);
        else launch_topk<16>(g, st, a.z, splits, a.bias, T, E, K, a.ids, a.w);
    }
    mk.mark(st);
    const int ntiles = perm_tiles(T);
    perm_hist_kernel<<<ntiles, PERM_TILE, 0, st>>>(a.ids, T, E, K, a.tile_count);
    perm_scatter_kernel<<<ntiles, PERM_TILE, 0, st>>>(a.ids, T, E, K, a.tile_count, ntiles, a.count, a.offset,
                                                      a.perm, a.inv);
    mk.mark(st);
    return hipGetLastError();
}

}  // namespace coli
