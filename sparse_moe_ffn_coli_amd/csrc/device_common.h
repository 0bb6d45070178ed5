// device_common.h -- device helpers shared by the gfx950 kernels of the routed
// MoE FFN layer: bf16 conversions, the clamped SwiGLU, and the LDS-staged
// MFMA tile engines behind every matrix product of the layer (a register-
// staged engine for row-light tiles and its fp16/int4 variant, and a
// 256 x 256 engine with direct global->LDS copies for row-heavy tiles).
//
// Activation: clamped SwiGLU, gate limited from above at 10 before the SiLU
// and up limited to [-10, 10] ("Add GLM-5.3-Flash (glm5next) support with
// ROCmFP mix qtypes (105/106)", section "Architecture").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 bits, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float sigmoid_f32(float z)
{
    return 1.0f / (1.0f + expf(-z));
}

// silu(min(g, 10)) * clamp(u, -10, 10).  For very negative g, expf(-g)
// overflows to +inf and g / inf = -0, never NaN.
__device__ __forceinline__ float swiglu_clamped(float g, float u)
{
    float gc = fminf(g, 10.0f);
    float uc = fminf(fmaxf(u, -10.0f), 10.0f);
    return gc / (1.0f + expf(-gc)) * uc;
}

// The same with the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32, about
// one ulp each), for results that are rounded to bf16 or fp16 right after:
// a few fp32 ulps are far below that rounding.  Very negative g: the exp2 is
// +inf, its reciprocal 0, the result -0 (never NaN).
__device__ __forceinline__ float swiglu_clamped_fast(float g, float u)
{
    const float gc = fminf(g, 10.0f);
    const float uc = fminf(fmaxf(u, -10.0f), 10.0f);
    const float e = __builtin_amdgcn_exp2f(gc * -1.4426950408889634f);
    return gc * __builtin_amdgcn_rcpf(1.0f + e) * uc;
}

// ---------------------------------------------------------------------------
// Wave-wide reductions on DPP lane permutations (no LDS traffic): within each
// row of 16 lanes, quad swaps, then the half-row and row mirrors; the four
// row results are then combined through readlane.  Every lane returns the
// result.
// ---------------------------------------------------------------------------
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op)
{
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return op(op(r0, r1), op(r2, r3));
}
struct MaxU32 { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };
struct MinU32 { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };

// ---------------------------------------------------------------------------
// Inclusive prefix sum over the NW waves of a workgroup (thread order):
// a shuffle scan inside each wave, then one wave scans the NW wave totals.
// Two barriers; `ws` is NW ints of LDS.  Every thread must call it.
// ---------------------------------------------------------------------------
template <int NW>
__device__ __forceinline__ int block_scan_incl(int v, int32_t *ws)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    if (lane == 63) ws[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int w = (lane < NW) ? ws[lane] : 0;
#pragma unroll
        for (int off = 1; off < NW; off <<= 1) {
            const int u = __shfl_up(w, off);
            if (lane >= off) w += u;
        }
        if (lane < NW) ws[lane] = w;
    }
    __syncthreads();
    return v + (wave > 0 ? ws[wave - 1] : 0);
}
__device__ __forceinline__ int block_scan_incl_1024(int v, int32_t *ws) { return block_scan_incl<16>(v, ws); }

// ---------------------------------------------------------------------------
// bf16 MFMA tile engine
//
// A workgroup of 256 threads (4 waves of 64) computes a BM x BN block of
// C = A * B^T with A [BM][K] and B [BN][K] both K-contiguous (every matrix
// product of the layer has this form: activations times weight rows).  K is
// walked in steps of BK = 64: each step's A and B tiles are copied from
// global memory into LDS (16-byte chunks, one row = 8 chunks), double-buffered
// so the global loads of step k+1 are in flight while step k runs on the
// matrix cores.  The waves form a WAVES_M x WAVES_N grid; each wave owns
// FM x FN fragments of 32x32 and issues v_mfma_f32_32x32x16_bf16 on them
// (on gfx950 this instruction delivers twice the bf16 rate of the 16x16x32
// form, measured 2.36 vs 1.24 PFLOP/s).
//
// Fragment layouts of v_mfma_f32_32x32x16_bf16 (lane l, i = 0..15):
//   A operand: row (l & 31), reduction slots 8*(l >> 5) .. +7
//   B operand: col (l & 31), the same reduction slots
//   result   : row 8*(i >> 2) + 4*(l >> 5) + (i & 3), col (l & 31)
// A and B take the same slots from the same K positions, so the pairing of
// products is exact whatever the hardware's slot order.
//
// LDS layout: chunk c of row r sits at chunk position c ^ ((r >> 1) & 7).
// A fragment read covers 16 lanes = 16 consecutive rows of one logical
// chunk per LDS cycle; with 128-byte rows, even and odd rows fall in
// different bank halves and the XOR spreads each half's 8 rows over 8
// distinct chunk positions, so reads and the row-pair writes are free of
// bank conflicts.
//
// Rows are supplied as per-thread source pointers (gathered activation rows,
// expert weight rows), one per load chunk of the thread.  Every pointer must
// be a readable row: a padding row (past an expert's last token, past the
// weight matrix's last row) points at any valid row instead.  Row m of the
// result depends only on row m of A and column n only on row n of B, so
// padding rows only reach results that the caller discards.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NT = 256;
    static constexpr int BK = 64;
    static constexpr int FM = BM / (WAVES_M * 32);
    static constexpr int FN = BN / (WAVES_N * 32);
    static constexpr int A_CHUNKS = BM * BK / 8;
    static constexpr int B_CHUNKS = BN * BK / 8;
    static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
    static constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
    static constexpr int STAGE = (BM + BN) * BK;      // bf16 elements per stage
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid");
    static_assert(BM % (WAVES_M * 32) == 0 && BN % (WAVES_N * 32) == 0, "tile shape");
};

// Index (in bf16 elements) of chunk `ch` of row `row` inside one tile region.
__device__ __forceinline__ int swz(int row, int ch)
{
    return (row * 8 + (ch ^ ((row >> 1) & 7))) * 8;
}

// Row of this thread's i-th load chunk (the chunk column is tid & 7 for all i).
template <class C>
__device__ __forceinline__ int a_chunk_row(int i) { return (threadIdx.x + i * C::NT) >> 3; }

// Row (within the tile) and column of accumulator element i of fragment
// (m, n) for this lane.
template <class C>
__device__ __forceinline__ int acc_row(int wm, int m, int lane, int i)
{
    return (wm * C::FM + m) * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}
template <class C>
__device__ __forceinline__ int acc_col(int wn, int n, int lane)
{
    return (wn * C::FN + n) * 32 + (lane & 31);
}

template <class C>
__device__ __forceinline__ void mfma_mainloop(const uint16_t *const (&ap)[C::A_PER_T],
                                              const uint16_t *const (&bp)[C::B_PER_T], int K,
                                              uint16_t *lds, f32x16 (&acc)[C::FM][C::FN])
{
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int ch0 = tid & 7;

    // Every thread loads its chunks (threads past the tile's chunk count load
    // a valid duplicate and skip the LDS store), so the staging registers are
    // always fully written and stay in VGPRs.
    u32x4 ra[C::A_PER_T], rb[C::B_PER_T];
#define COLI_GLOAD(kt_)                                                                        \
    do {                                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < C::A_PER_T; ++i_) ra[i_] =                     \
            *reinterpret_cast<const u32x4 *>(ap[i_] + (kt_) * C::BK);                          \
        _Pragma("unroll") for (int i_ = 0; i_ < C::B_PER_T; ++i_) rb[i_] =                     \
            *reinterpret_cast<const u32x4 *>(bp[i_] + (kt_) * C::BK);                          \
    } while (0)
#define COLI_SSTORE(buf_)                                                                      \
    do {                                                                                       \
        uint16_t *sa_ = lds + (buf_) * C::STAGE;                                               \
        uint16_t *sb_ = sa_ + C::BM * C::BK;                                                   \
        _Pragma("unroll") for (int i_ = 0; i_ < C::A_PER_T; ++i_) {                            \
            const int c_ = tid + i_ * C::NT;                                                   \
            if (C::A_CHUNKS % C::NT == 0 || c_ < C::A_CHUNKS)                                  \
                *reinterpret_cast<u32x4 *>(sa_ + swz(c_ >> 3, ch0)) = ra[i_];                  \
        }                                                                                      \
        _Pragma("unroll") for (int i_ = 0; i_ < C::B_PER_T; ++i_) {                            \
            const int c_ = tid + i_ * C::NT;                                                   \
            if (C::B_CHUNKS % C::NT == 0 || c_ < C::B_CHUNKS)                                  \
                *reinterpret_cast<u32x4 *>(sb_ + swz(c_ >> 3, ch0)) = rb[i_];                  \
        }                                                                                      \
    } while (0)

#pragma unroll
    for (int m = 0; m < C::FM; ++m)
#pragma unroll
        for (int n = 0; n < C::FN; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;

    // MFMA operands are double-buffered in registers: the LDS reads of
    // reduction step kk+1 are issued before the MFMAs of step kk, so their
    // latency hides behind matrix-core work even with one wave per SIMD.
    bf16x8 af[2][C::FM], bfr[2][C::FN];
#define COLI_LFRAG(stage_, kk_, slot_)                                                         \
    do {                                                                                       \
        const uint16_t *sa_ = lds + (stage_) * C::STAGE;                                       \
        const uint16_t *sb_ = sa_ + C::BM * C::BK;                                             \
        const int ch_ = (kk_) * 2 + (lane >> 5);                                               \
        _Pragma("unroll") for (int m_ = 0; m_ < C::FM; ++m_) af[slot_][m_] =                   \
            *reinterpret_cast<const bf16x8 *>(sa_ + swz((wm * C::FM + m_) * 32 + (lane & 31), ch_)); \
        _Pragma("unroll") for (int n_ = 0; n_ < C::FN; ++n_) bfr[slot_][n_] =                  \
            *reinterpret_cast<const bf16x8 *>(sb_ + swz((wn * C::FN + n_) * 32 + (lane & 31), ch_)); \
    } while (0)

    const int nk = K / C::BK;
    COLI_GLOAD(0);
    COLI_SSTORE(0);
    __syncthreads();
    COLI_LFRAG(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) COLI_GLOAD(kt + 1);
#pragma unroll
        for (int kk = 0; kk < C::BK / 16; ++kk) {
            const int slot = kk & 1;
            if (kk + 1 < C::BK / 16) COLI_LFRAG(cur, kk + 1, slot ^ 1);
#pragma unroll
            for (int m = 0; m < C::FM; ++m)
#pragma unroll
                for (int n = 0; n < C::FN; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][m], bfr[slot][n],
                                                                        acc[m][n], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            COLI_SSTORE(cur ^ 1);
            __syncthreads();
            COLI_LFRAG(cur ^ 1, 0, 0);
        }
    }
#undef COLI_GLOAD
#undef COLI_SSTORE
#undef COLI_LFRAG
}

// ---------------------------------------------------------------------------
// Large-tile engine: 256 x 256 blocks, eight waves, both operands copied from
// global memory straight into LDS (global_load_lds_dwordx4) through a ring of
// NS stages, NS - 1 of them in flight.
//
// Sized for the row-heavy products (many tokens per expert), whose operands
// come mostly from beyond L2 (weights from HBM, gathered activation rows
// from the memory-side cache): a stage is one reduction step of BK elements
// for 256 A rows and 256 B rows, and keeping NS - 1 stages in flight per CU
// (up to 128 KB) is what covers that latency.  Copy instruction q (0..31 for
// A, 32..63 for B) fills LDS bytes 1024 q .. +1023 of the stage with rows
// RPI q .. RPI q + RPI - 1 of its operand (RPI = 1024 / (2 BK) rows of
// 2 BK bytes); lane l fetches 16 bytes of row RPI q + l / CPR (CPR = BK / 8
// chunks per row), and the source chunk is chosen so that the lane's LDS
// slot holds the swizzled layout read below (chunk c of row r at position
// c ^ ((r >> 1) & 7) for BK = 64, c ^ ((r >> 2) & 3) for BK = 32; either
// makes the 16-lane fragment reads free of bank conflicts).  Wave w issues
// instructions j * 8 + w.
//
// Step kt: wait until this wave's copies of stage kt have landed (vmcnt),
// barrier (everyone's have, and everyone has left step kt-1), issue stage
// kt + NS - 1 into the buffer read in step kt-1, then the MFMAs of stage kt.
//
// Waves form a 4 x 2 grid, each owning 64 rows x 128 columns (2 x 4
// fragments of 32 x 32, v_mfma_f32_32x32x16_bf16); two waves fit per SIMD.
//
// NFW = fragments of this wave that hold real rows (0..2), chosen by the
// caller per wave from the tile's row count: fragments without real rows
// are neither read from LDS nor multiplied.  `valid` = real A rows of the
// tile: A copies whose rows all lie past it are skipped with NS = 2 (every
// step then waits for all of the wave's copies, so the count need not be
// fixed); with a deeper ring they run, rereading a real row.
// ---------------------------------------------------------------------------
template <int BK_, int NS_>
struct BigCfgT {
    static constexpr int NT = 512, BM = 256, BN = 256, BK = BK_, NS = NS_;
    static constexpr int WAVES_M = 4, WAVES_N = 2, FM = 2, FN = 4;
    static constexpr int CPR = BK / 8;                       // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;                     // rows per copy instruction
    static constexpr int OPERAND_BYTES = 256 * BK * 2;
    static constexpr int STAGE_BYTES = 2 * OPERAND_BYTES;
    static constexpr int LDS_BYTES = NS * STAGE_BYTES;
    static constexpr int CPO = 256 / RPI / 8;                // copies per wave per operand per stage
    static constexpr int CPW = 2 * CPO;                      // copies per wave per stage
    static_assert(BK == 32 || BK == 64, "row of 64 or 128 bytes");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(NS >= 2 && (NS - 1) * CPW <= 63, "vmcnt range");
};
using BigCfg = BigCfgT<64, 2>;

// Tile row (within its A or B region) fetched by this lane in copy j of wave w.
template <class C>
__device__ __forceinline__ int big_copy_row(int j, int w)
{
    return ((j % C::CPO) * 8 + w) * C::RPI + (threadIdx.x & 63) / C::CPR;
}
template <class C>
__device__ __forceinline__ int big_swz_pos(int row, int c)
{
    return (C::BK == 64) ? (c ^ ((row >> 1) & 7)) : (c ^ ((row >> 2) & 3));
}
// Source chunk of that lane (its LDS slot is chunk position lane % CPR of the row).
template <class C>
__device__ __forceinline__ int big_copy_chunk(int row)
{
    return big_swz_pos<C>(row, (threadIdx.x & 63) % C::CPR);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_c()
{
    static_assert(N >= 0 && N <= 63, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until at most `pending` stages of this wave's copies are in flight.
template <class C, int P>
__device__ __forceinline__ void big_wait_stages(int pending)
{
    if constexpr (P == 0) {
        wait_vmcnt_c<0>();
    } else {
        if (pending >= P) wait_vmcnt_c<P * C::CPW>();
        else big_wait_stages<C, P - 1>(pending);
    }
}

// One step of a full tile (every A row real, both fragments of every wave
// used) with a two-stage ring, in a fixed instruction order.  The wave reads
// the step's first fragments, then runs its four MFMA groups, reading the
// fragments of group kk + 1 while group kk runs (one LDS read after each of
// the first six MFMAs).  Its eight copies of stage kt + 1 go out one after
// each of MFMAs BASE, BASE + STRIDE, ... of the step: waves 0-3 after MFMAs
// 0..7 (group 0), waves 4-7 (the second wave of each SIMD) after MFMAs 8..15
// (group 1).  A copy instruction moves 1 KB and the CU's address path takes
// about 16 cycles for it, so a wave that issues copies stalls until they are
// accepted; with all eight waves issuing at the start of the step, every
// SIMD's matrix core waited for both of its waves (a timestamped build
// measured the second wave of each SIMD held 44 % of the loop), while
// staggered, one wave of each SIMD multiplies while the other is held.  The
// second wave's copies go out one group later, not two: with two, they were
// still in flight when the next step began (HBM latency is about 1 us) --
// group 1 against group 2 measured 0.62 against 0.63 ms for the prefill step
// and 0.38-0.39 against 0.40 ms for the dense one.  sched_barrier(0) after
// every MFMA keeps this order.
template <class C, bool MORE, int BASE, int STRIDE>
__device__ __forceinline__ void big_full_step(const uint16_t *const (&rp)[C::CPW], int kt, int w, char *lds,
                                              f32x16 (&acc)[C::FM][C::FN], bf16x8 (&af)[2][C::FM],
                                              bf16x8 (&bfr)[2][C::FN])
{
    static_assert(C::NS == 2 && C::FM == 2 && C::FN == 4 && C::CPW == C::FM * C::FN, "step shape");
    static_assert(BASE + (C::CPW - 1) * STRIDE < (C::BK / 16) * C::FM * C::FN, "copies inside the step");
    constexpr int KK = C::BK / 16;
    const int lane = threadIdx.x & 63;
    const int wm = w >> 1, wn = w & 1;
    const char *st = lds + (kt & 1) * C::STAGE_BYTES;
    char *nst = lds + ((kt + 1) & 1) * C::STAGE_BYTES;
    // fragment f of group kk (0, 1: A rows of fragment m = f; 2..5: B rows of fragment n = f - 2)
    auto frag = [&](int kk, int f) -> bf16x8 {
        const int c = kk * 2 + (lane >> 5);
        const int r = (f < 2) ? (wm * C::FM + f) * 32 + (lane & 31) : (wn * C::FN + f - 2) * 32 + (lane & 31);
        const char *base = (f < 2) ? st : st + C::OPERAND_BYTES;
        return *reinterpret_cast<const bf16x8 *>(base + (r * C::CPR + big_swz_pos<C>(r, c)) * 16);
    };
    wait_vmcnt_c<0>();
    asm volatile("s_barrier" ::: "memory");            // see big_mainloop
#pragma unroll
    for (int f = 0; f < 6; ++f) {
        if (f < 2) af[0][f] = frag(0, f);
        else bfr[0][f - 2] = frag(0, f);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const int slot = kk & 1;
#pragma unroll
        for (int i = 0; i < C::FM * C::FN; ++i) {
            const int m = i / C::FN, n = i % C::FN;
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][m], bfr[slot][n], acc[m][n], 0, 0, 0);
            if (kk + 1 < KK && i < 6) {
                if (i < 2) af[slot ^ 1][i] = frag(kk + 1, i);
                else bfr[slot ^ 1][i - 2] = frag(kk + 1, i);
            }
            const int g = kk * C::FM * C::FN + i;        // MFMA index within the step
            if (MORE && g >= BASE && (g - BASE) % STRIDE == 0 && (g - BASE) / STRIDE < C::CPW) {
                const int j = (g - BASE) / STRIDE;        // copy j of stage kt + 1 (j < CPO: A rows, else B)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(rp[j] + (kt + 1) * C::BK),
                    (__attribute__((address_space(3))) void *)(nst + (j / C::CPO) * C::OPERAND_BYTES +
                                                               ((j % C::CPO) * 8 + w) * 1024),
                    16, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <class C, int BASE, int STRIDE>
__device__ __forceinline__ void big_full_loop(const uint16_t *const (&rp)[C::CPW], int nk, int w, char *lds,
                                              f32x16 (&acc)[C::FM][C::FN])
{
    bf16x8 af[2][C::FM], bfr[2][C::FN];
    for (int kt = 0; kt + 1 < nk; ++kt) big_full_step<C, true, BASE, STRIDE>(rp, kt, w, lds, acc, af, bfr);
    if (nk > 0) big_full_step<C, false, BASE, STRIDE>(rp, nk - 1, w, lds, acc, af, bfr);
}

// rp[j]: this lane's source for copy j at k = 0 (row big_copy_row(j, w),
// chunk big_copy_chunk(row) already applied; j < CPO: A, else B), readable
// for every k < K.  w = this wave (0..7), wm = w >> 1, wn = w & 1.  Full
// tiles (valid = BM) take big_full_loop.
template <class C, int NFW>
__device__ __forceinline__ void big_mainloop(const uint16_t *const (&rp)[C::CPW], int K, int valid, int w,
                                             char *lds, f32x16 (&acc)[C::FM][C::FN])
{
    const int lane = threadIdx.x & 63;
    const int wm = w >> 1, wn = w & 1;
    const int nk = K / C::BK;

#pragma unroll
    for (int m = 0; m < C::FM; ++m)
#pragma unroll
        for (int n = 0; n < C::FN; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;

#define COLI_BIG_ISSUE(kt_)                                                                    \
    do {                                                                                       \
        char *st_ = lds + ((kt_) % C::NS) * C::STAGE_BYTES;                                    \
        _Pragma("unroll") for (int j_ = 0; j_ < C::CPW; ++j_)                                  \
            if (C::NS > 2 || j_ >= C::CPO || ((j_ % C::CPO) * 8 + w) * C::RPI < valid)         \
            __builtin_amdgcn_global_load_lds(                                                  \
                (const __attribute__((address_space(1))) void *)(rp[j_] + (kt_) * C::BK),     \
                (__attribute__((address_space(3))) void *)(st_ + (j_ / C::CPO) * C::OPERAND_BYTES + \
                                                           ((j_ % C::CPO) * 8 + w) * 1024),    \
                16, 0, 0);                                                                     \
    } while (0)

    bf16x8 af[2][C::FM], bfr[2][C::FN];
#define COLI_BIG_LFRAG(st_, kk_, slot_)                                                        \
    do {                                                                                       \
        const int c_ = (kk_) * 2 + (lane >> 5);                                                \
        _Pragma("unroll") for (int m_ = 0; m_ < NFW; ++m_) {                                   \
            const int r_ = (wm * C::FM + m_) * 32 + (lane & 31);                               \
            af[slot_][m_] = *reinterpret_cast<const bf16x8 *>(                                 \
                (st_) + (r_ * C::CPR + big_swz_pos<C>(r_, c_)) * 16);                          \
        }                                                                                      \
        _Pragma("unroll") for (int n_ = 0; n_ < C::FN; ++n_) {                                 \
            const int r_ = (wn * C::FN + n_) * 32 + (lane & 31);                               \
            bfr[slot_][n_] = *reinterpret_cast<const bf16x8 *>(                                \
                (st_) + C::OPERAND_BYTES + (r_ * C::CPR + big_swz_pos<C>(r_, c_)) * 16);       \
        }                                                                                      \
    } while (0)

#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s)
        if (s < nk) COLI_BIG_ISSUE(s);
    if constexpr (C::NS == 2 && NFW == 2) {
        if (valid >= C::BM) {                          // a full tile: every copy is issued, every wave has NFW = 2
            if (w < 4) big_full_loop<C, 0, 1>(rp, nk, w, lds, acc);        // copies after MFMAs 0..7
            else big_full_loop<C, C::FM * C::FN, 1>(rp, nk, w, lds, acc);  // after MFMAs 8..15
            return;
        }
    }
    if constexpr (C::NS >= 3) {
        // With three or more stages the barrier of step kt comes before its
        // last MFMA group and also covers stage kt + 1 (issued two steps
        // earlier): its first fragments are then read while the last MFMAs
        // of stage kt run, so no step starts by waiting for LDS reads.
        constexpr int KK = C::BK / 16;
        big_wait_stages<C, C::NS - 2>(min(C::NS - 2, nk - 1));
        asm volatile("s_barrier" ::: "memory");
        if (NFW > 0) COLI_BIG_LFRAG(lds, 0, 0);
        for (int kt = 0; kt < nk; ++kt) {
            const char *st = lds + (kt % C::NS) * C::STAGE_BYTES;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int slot = kk & 1;          // KK is even: stage kt + 1 starts in slot 0
                if (kk + 1 < KK) {
                    if (NFW > 0) COLI_BIG_LFRAG(st, kk + 1, slot ^ 1);
                } else {
                    // stages issued after kt + 1 that may still be in flight
                    big_wait_stages<C, C::NS - 3>(max(min(C::NS - 3, nk - 2 - kt), 0));
                    asm volatile("s_barrier" ::: "memory");
                    if (kt + C::NS - 1 < nk) COLI_BIG_ISSUE(kt + C::NS - 1);
                    if (NFW > 0 && kt + 1 < nk)
                        COLI_BIG_LFRAG(lds + ((kt + 1) % C::NS) * C::STAGE_BYTES, 0, slot ^ 1);
                }
#pragma unroll
                for (int m = 0; m < NFW; ++m)
#pragma unroll
                    for (int n = 0; n < C::FN; ++n)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][m], bfr[slot][n],
                                                                            acc[m][n], 0, 0, 0);
            }
        }
        return;
    }
    for (int kt = 0; kt < nk; ++kt) {
        // stages issued after kt that may still be in flight
        big_wait_stages<C, C::NS - 2>(min(C::NS - 2, nk - 1 - kt));
        // A bare barrier: __syncthreads() would also wait for the copies
        // still in flight (its memory fence covers them).  Every LDS read of
        // the previous step has been consumed by an MFMA before this point,
        // and the memory clobber keeps the compiler from moving LDS accesses
        // across it.
        asm volatile("s_barrier" ::: "memory");
        if (kt + C::NS - 1 < nk) COLI_BIG_ISSUE(kt + C::NS - 1);
        if (NFW > 0) {
            const char *st = lds + (kt % C::NS) * C::STAGE_BYTES;
            COLI_BIG_LFRAG(st, 0, 0);
#pragma unroll
            for (int kk = 0; kk < C::BK / 16; ++kk) {
                const int slot = kk & 1;
                if (kk + 1 < C::BK / 16) COLI_BIG_LFRAG(st, kk + 1, slot ^ 1);
#pragma unroll
                for (int m = 0; m < NFW; ++m)
#pragma unroll
                    for (int n = 0; n < C::FN; ++n)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][m], bfr[slot][n],
                                                                            acc[m][n], 0, 0, 0);
            }
        }
    }
#undef COLI_BIG_ISSUE
#undef COLI_BIG_LFRAG
}

// ---------------------------------------------------------------------------
// Streaming mode of the large-tile engine, for tiles with at most 64 real
// rows (experts with few tokens).  Such a tile is a stream of its 256 weight
// rows with little arithmetic, so the LDS holds a deeper ring of small
// stages: 64 A rows + 256 B rows of 128 bytes (40 KB) per step, NS = 4
// stages, three in flight.  Each wave issues up to 5 copies per stage: one
// for A rows 8 w .. 8 w + 7 (skipped when they all lie past the tile's real
// rows), four for B rows as in big_mainloop.  The waves of the first two
// rows (w < 4) multiply, one 32-row fragment each (A rows 32 (w / 2) ..,
// skipped when that fragment has no real row), against B fragments
// 4 (w % 2) .. + 3; they issue their copies after their MFMAs, so the
// copy-issue queue (about 16 cycles per 1 KB copy instruction on a CU) never
// holds their matrix work, and the three-stage lead leaves the copies two
// steps to land (prefill gate+up 353 -> 348 us).
// ---------------------------------------------------------------------------
struct StreamCfg {
    static constexpr int BK = 64, NS = 4, A_ROWS = 64;
    static constexpr int A_BYTES = A_ROWS * BK * 2;
    static constexpr int B_BYTES = 256 * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = NS * STAGE_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Tile row of this lane's A copy (wave w).
__device__ __forceinline__ int stream_a_row(int w) { return w * 8 + ((threadIdx.x & 63) >> 3); }

// Wait until at most `pending` stages (0..2) of this wave's copies, cw per
// stage (4 or 5), are in flight.
__device__ __forceinline__ void stream_wait(int pending, int cw)
{
    if (pending == 0) wait_vmcnt_c<0>();
    else if (cw == 4) { if (pending == 1) wait_vmcnt_c<4>(); else wait_vmcnt_c<8>(); }
    else { if (pending == 1) wait_vmcnt_c<5>(); else wait_vmcnt_c<10>(); }
}

// ra: this lane's A source at k = 0 (row stream_a_row(w), chunk
// big_copy_chunk<BigCfgT<64, 2>>(row) applied); rb[j]: B sources as the last
// four entries of big_mainloop's rp; valid: real A rows of the tile (1..64).
// acc: this wave's fragment products (waves 0..3).
__device__ __forceinline__ void stream_mainloop(const uint16_t *ra, const uint16_t *const (&rb)[4], int K, int valid,
                                                int w, char *lds, f32x16 (&acc)[4])
{
    using C = StreamCfg;
    const int lane = threadIdx.x & 63;
    const int wn = w & 1;
    const bool mma = w < 4 && 32 * (w >> 1) < valid;   // a first-two-row wave with real rows
    const bool acopy = 8 * w < valid;                   // this wave's A rows are not all padding
    const int cw = acopy ? 5 : 4;
    const int nk = K / C::BK;

#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[n][i] = 0.f;

#define COLI_ST_ISSUE(kt_)                                                                     \
    do {                                                                                       \
        char *st_ = lds + ((kt_) % C::NS) * C::STAGE_BYTES;                                    \
        if (acopy)                                                                             \
            __builtin_amdgcn_global_load_lds(                                                  \
                (const __attribute__((address_space(1))) void *)(ra + (kt_) * C::BK),         \
                (__attribute__((address_space(3))) void *)(st_ + w * 1024), 16, 0, 0);        \
        _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_)                                       \
            __builtin_amdgcn_global_load_lds(                                                  \
                (const __attribute__((address_space(1))) void *)(rb[j_] + (kt_) * C::BK),     \
                (__attribute__((address_space(3))) void *)(st_ + C::A_BYTES + (j_ * 8 + w) * 1024), \
                16, 0, 0);                                                                     \
    } while (0)

#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s)
        if (s < nk) COLI_ST_ISSUE(s);
    const int ra_ = 32 * (w >> 1) + (lane & 31);
    for (int kt = 0; kt < nk; ++kt) {
        stream_wait(min(C::NS - 2, nk - 1 - kt), cw);     // stages after kt still in flight
        asm volatile("s_barrier" ::: "memory");               // see big_mainloop
        if (kt + C::NS - 1 < nk && w >= 4) COLI_ST_ISSUE(kt + C::NS - 1);
        if (mma) {
            const char *st = lds + (kt % C::NS) * C::STAGE_BYTES;
#pragma unroll
            for (int kk = 0; kk < C::BK / 16; ++kk) {
                const int c = kk * 2 + (lane >> 5);
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(st + swz(ra_, c) * 2);
                bf16x8 b[4];
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    const int rb_ = (wn * 4 + n) * 32 + (lane & 31);
                    b[n] = *reinterpret_cast<const bf16x8 *>(st + C::A_BYTES + swz(rb_, c) * 2);
                }
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[n], acc[n], 0, 0, 0);
            }
        }
        if (w < 4 && kt + C::NS - 1 < nk) COLI_ST_ISSUE(kt + C::NS - 1);   // after the MFMAs: see above
    }
#undef COLI_ST_ISSUE
}

// ---------------------------------------------------------------------------
// int4 engine (fp16 MFMA, fp32 accumulation)
//
// Weights: int4, element 2i in the low nibble of byte i, value (nibble - 8) *
// scale with one fp16 scale per `group` consecutive elements (offset-binary,
// "feat(glm53): add device-resident HIP backend for MI350P", section "Key
// changes"); the shared expert's weights are bf16.  The A operand (token
// rows of x, or rows of h) is fp16 already, written by the previous kernel
// in the permuted chunk order described below (exact for magnitudes in
// fp16's normal range).
//
// Order of K: inside every 8-element chunk the elements are held in the
// order 0,4,1,5,2,6,3,7 (dword j holds elements j and j + 4).  A dot product
// does not depend on that order, and it lets one AND/OR put two nibbles of a
// 32-bit word (bits 4j and 16 + 4j) under the fp16 exponent of 1024: the
// pair is then 1024 + n exactly, subtracting 1032 leaves n - 8 exactly, and
// one fp16 multiply by the scale rounds the exact product (n - 8) * scale
// once.  Inside a 64-element block, lane half h takes elements 32h .. 32h +
// 31 over four MFMA steps j (chunk 4h + j of A), eight per step: for int4
// that is exactly the 16-byte chunk 2 blk + h of the weight row's nibbles,
// one LDS read whose dword j holds the step's nibbles; the 32 elements lie
// inside one scale group (the group is a multiple of 32).
//
// Tile: BM token rows x 256 weight rows, four waves.  One stage covers KS =
// 128 elements of int4 weights (64 bytes of nibbles per row) or 32 of bf16
// weights (64 bytes per row as well), so a stage needs 26 KB (BM = 32) or
// 34 KB (BM = 64) of LDS and two or three workgroups share a CU.  Weight and
// token rows reach LDS by LDS-DMA copies (16 rows x 64 B or 8 rows x 128 B
// per instruction); 16-byte chunks are XOR-swizzled so that fragment reads
// are free of bank conflicts:
//   B: [256 rows][64 B], chunk ^ (row >> 2) & 3;
//   A (int4 tiles): [64-element block][BM rows][128 B], chunk ^ (row >> 1) & 7;
//   A (bf16 tiles): [BM rows][64 B], chunk ^ (row >> 2) & 3;
// and the stage's scales (at most 4 per weight row) with ordinary loads
// into S[256][4].
// ---------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 8 bf16 (elements 0..7) -> 8 fp16 in the chunk order 0,4,1,5,2,6,3,7
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v)
{
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t p = v[j >> 1], q = v[2 + (j >> 1)];
        const float a = __uint_as_float((j & 1) ? (p & 0xffff0000u) : (p << 16));
        const float b = __uint_as_float((j & 1) ? (q & 0xffff0000u) : (q << 16));
        r[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
    }
    return r;
}

// slot of element e (0..7) of a chunk in the order 0,4,1,5,2,6,3,7
__device__ __forceinline__ int f16_chunk_slot(int e) { return (e & 3) * 2 + (e >> 2); }

// 8 nibbles of w (element p in bits 4p..4p+3) -> 8 fp16 values
// (nibble - 8) * scale in the chunk order 0,4,1,5,2,6,3,7.  Pairs j = 0, 2
// take the nibbles from bits 0-3 (and 16-19) of w and of w >> 8: under the
// exponent of 1024 they read 1024 + n, and subtracting 1032 leaves n - 8.
// Pairs j = 1, 3 take them in place from bits 4-7: 1024 + 16 n, and
// (1024 + 16 n) / 16 - 72 = n - 8 (one fused multiply-add; every step is
// exact in fp16).  Either way n - 8 is exact and the one multiply by the
// scale rounds the exact product (n - 8) * scale, for every finite scale.
__device__ __forceinline__ uint32_t nibble_pair(uint32_t w, uint32_t mask, uint32_t magic)
{
    // (w & mask) | magic in one instruction (the compiler splits it in two
    // when both constants are literals); mask in an SGPR, magic in a VGPR
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
    return r;
}
__device__ __forceinline__ u32x4 int4x8_to_f16x8(uint32_t w, f16x2 scale2)
{
    const f16x2 off0 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const f16x2 off1 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t w8 = w >> 8;
    const uint32_t magic = 0x64006400u;
    auto lo = [&](uint32_t v) { return __builtin_bit_cast(f16x2, nibble_pair(v, 0x000F000Fu, magic)) - off0; };
    auto hi = [&](uint32_t v) {
        return __builtin_elementwise_fma(__builtin_bit_cast(f16x2, nibble_pair(v, 0x00F000F0u, magic)), sixteenth, off1);
    };
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, lo(w) * scale2);
    r[1] = __builtin_bit_cast(uint32_t, hi(w) * scale2);
    r[2] = __builtin_bit_cast(uint32_t, lo(w8) * scale2);
    r[3] = __builtin_bit_cast(uint32_t, hi(w8) * scale2);
    return r;
}

__device__ __forceinline__ f16x2 fp16_bits_splat(uint16_t h)
{
    return __builtin_bit_cast(f16x2, (uint32_t)h * 0x00010001u);
}

template <int BM_>
struct I4Cfg {
    static constexpr int BM = BM_, BN = 256, NT = 256;
    static constexpr int WAVES_M = BM / 32, WAVES_N = 4 / WAVES_M;
    static constexpr int FM = 1, FN = BN / (WAVES_N * 32);
    static constexpr int KS_I4 = 128, KS_BF = 32;   // reduction elements per stage
    static constexpr int B_BYTES = BN * 64;
    static constexpr int A_BYTES = BM * KS_I4 * 2;
    static constexpr int S_BYTES = BN * 8;
    static constexpr int STAGE_BYTES = B_BYTES + A_BYTES + S_BYTES;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static constexpr int AROWS = BM / 8;            // token rows per lane among the int4 A copy sources
    static constexpr int WAVES_PER_EU = (BM == 32) ? 3 : 2;   // workgroups per CU that the LDS allows
    static_assert(BM == 32 || BM == 64, "tile height");
};

// One tile.  I4: arow[u] is token row 8u + lane / 8 of the tile (element 0),
// brow[j] weight row (4w + j) * 16 + lane / 4 (byte 0), w = wave, srow the
// scales of weight row tid.  bf16 tiles (the shared expert): a0 + r * lda
// is token row r in bf16, natural order (the shared expert's rows are
// contiguous), brow as above, srow unused; the products run on bf16 MFMA as
// in the bf16 layer.  valid:
// token rows of the tile that are real (copies of row groups wholly past
// them are skipped; their results are dropped by the caller).
template <class C, bool I4>
__device__ __forceinline__ void i4_mainloop(const uint16_t *const (&arow)[C::AROWS], const uint16_t *a0,
                                            int lda, const char *const (&brow)[4], const uint16_t *srow,
                                            int group, int K, int valid, char *lds, f32x16 (&acc)[C::FN])
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w / C::WAVES_N, wn = w % C::WAVES_N;
    const int h = lane >> 5;
    constexpr int KS = I4 ? C::KS_I4 : C::KS_BF;
    const int nk = (K + KS - 1) / KS;
    auto dma = [](const void *src, char *dst) {
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    };
    // scales of stage kt for weight row tid: groups first .. last.  When the
    // row's scales fill at most one 128-byte line (group 32, K / 32 a
    // multiple of 8, at most 64), the whole row is loaded once per tile into
    // sv and each stage takes its four scales from the front (sv shifts by
    // one entry every second stage): a scale line is then fetched once per
    // tile instead of once per stage.
    uint2 sreg = make_uint2(0u, 0u);
    const bool sline = I4 && group == 32 && ((K / 32) & 7) == 0 && K / 32 <= 64;
    u32x4 sv[8];
    if (sline) {
        const int n16 = K / 256;                      // 16-byte pieces of the row's scales
#pragma unroll
        for (int i = 0; i < 8; ++i) sv[i] = *reinterpret_cast<const u32x4 *>(srow + 8 * min(i, n16 - 1));
    }
    auto load_scales = [&](int kt) {
        if (sline) {
            sreg = (kt & 1) ? make_uint2(sv[0][2], sv[0][3]) : make_uint2(sv[0][0], sv[0][1]);
            if (kt & 1) {
#pragma unroll
                for (int i = 0; i < 7; ++i) sv[i] = sv[i + 1];
            }
            return;
        }
        const int first = kt * KS / group, last = (min(K, kt * KS + KS) - 1) / group;
        const uint32_t s0 = srow[min(first, last)], s1 = srow[min(first + 1, last)];
        const uint32_t s2 = srow[min(first + 2, last)], s3 = srow[min(first + 3, last)];
        sreg = make_uint2(s0 | (s1 << 16), s2 | (s3 << 16));
    };
    auto issue = [&](int kt) {
        char *sb = lds + (kt & 1) * C::STAGE_BYTES, *sa = sb + C::B_BYTES;
#pragma unroll
        for (int j = 0; j < 4; ++j) {                 // B: 256 rows of 64 bytes, 16 rows per copy
            const int q = w * 4 + j;
            const int row = q * 16 + (lane >> 2);
            const int c = (lane & 3) ^ ((row >> 2) & 3);
            if (I4) {
                const int cs = (kt * KS + 32 * c < K) ? c : 0;      // past K: any valid chunk
                dma(brow[j] + kt * 64 + cs * 16, sb + q * 1024);
            } else {
                dma(brow[j] + (kt * KS + c * 8) * 2, sb + q * 1024);
            }
        }
        if (I4) {                                     // A: lines blk * BM + row of 128 bytes
            constexpr int AQ = C::BM * 2 / 8;
#pragma unroll
            for (int i = 0; i < AQ / 4; ++i) {
                const int q = w + 4 * i;
                const int blk = q / C::AROWS, u = q % C::AROWS;
                if (u * 8 < valid) {
                    const int row = u * 8 + (lane >> 3);
                    const int c = (lane & 7) ^ ((row >> 1) & 7);
                    const int bs = (kt * KS + blk * 64 < K) ? blk : 0;
                    dma(arow[u] + kt * KS + bs * 64 + c * 8, sa + q * 1024);
                }
            }
            load_scales(kt);
        } else {                                      // A: BM rows of 64 bytes, 16 rows per copy
            if (w < C::BM / 16 && w * 16 < valid) {
                const int row = w * 16 + (lane >> 2);
                const int c = (lane & 3) ^ ((row >> 2) & 3);
                dma(a0 + (size_t)min(row, valid - 1) * lda + kt * KS + c * 8, sa + w * 1024);
            }
        }
    };
    auto store_scales = [&](int kt) {
        if (I4)
            *reinterpret_cast<uint2 *>(lds + (kt & 1) * C::STAGE_BYTES + C::B_BYTES + C::A_BYTES + tid * 8) = sreg;
    };

#pragma unroll
    for (int n = 0; n < C::FN; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[n][i] = 0.f;
    const int ar = wm * 32 + (lane & 31);             // this lane's A fragment row
    int br[C::FN];                                    // and B fragment rows
#pragma unroll
    for (int n = 0; n < C::FN; ++n) br[n] = (wn * C::FN + n) * 32 + (lane & 31);

    issue(0);
    wait_vmcnt_c<0>();
    store_scales(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) issue(kt + 1);
        const char *sb = lds + (kt & 1) * C::STAGE_BYTES, *sa = sb + C::B_BYTES;
        if (I4) {
            const uint16_t *ss = reinterpret_cast<const uint16_t *>(sa + C::A_BYTES);
            const int nblk = min(KS / 64, (K - kt * KS) / 64);
            for (int blk = 0; blk < nblk; ++blk) {
                const int gi = (group == 32) ? 2 * blk + h
                                             : (kt * KS + 64 * blk + 32 * h) / group - kt * KS / group;
                u32x4 bq[C::FN];
                f16x2 sc[C::FN];
#pragma unroll
                for (int n = 0; n < C::FN; ++n) {
                    const int c = 2 * blk + h;
                    bq[n] = *reinterpret_cast<const u32x4 *>(sb + br[n] * 64 + ((c ^ ((br[n] >> 2) & 3)) * 16));
                    sc[n] = fp16_bits_splat(ss[br[n] * 4 + gi]);
                }
                f16x8 a[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int ca = 4 * h + j;
                    a[j] = *reinterpret_cast<const f16x8 *>(sa + (blk * C::BM + ar) * 128 + ((ca ^ ((ar >> 1) & 7)) * 16));
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int n = 0; n < C::FN; ++n)
                        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            a[j], __builtin_bit_cast(f16x8, int4x8_to_f16x8(bq[n][j], sc[n])), acc[n], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = 2 * h + j;
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sa + ar * 64 + ((c ^ ((ar >> 2) & 3)) * 16));
#pragma unroll
                for (int n = 0; n < C::FN; ++n) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8 *>(sb + br[n] * 64 + ((c ^ ((br[n] >> 2) & 3)) * 16));
                    acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[n], 0, 0, 0);
                }
            }
        }
        if (kt + 1 < nk) {
            wait_vmcnt_c<0>();
            store_scales(kt + 1);
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Narrow form of the int4 engine for tiles that hold few token rows
// (decode-sized batches).  An int4 pass multiplies 8 token rows: the A
// fragment rows repeat them (fragment row r reads token row r mod 8), so
// rows 0-7 of the results are the pass's rows and the rest are dropped; a
// tile with more real rows takes several passes over its weights.  The small
// A stage leaves LDS for stages of 256 reduction elements, i.e. whole
// 128-byte lines of every weight row per stage (a streaming probe of this
// tile's copies measured 5.9 TB/s with 128-byte pieces of 256 rows per
// stage against 4.7 TB/s with the 64-byte pieces of the staged engine).  The
// scales never pass through LDS: lane l of wave w holds the 64 scales of
// weight row 64 w + l in registers, which are exactly the rows of its wave's
// two B fragments, and v_permlane32_swap hands each lane the words of its
// fragments' rows (an LDS store after LDS-DMA copies would also make the
// compiler wait for every copy in flight).  bf16 tiles (the shared expert)
// keep all 32 rows with 64-element stages of the same size.  Scales must
// fill at most one 128-byte line per weight row (group 32, K a multiple of
// 256 and at most 2048: i4n_fits).
// LDS: B [256 rows][128 B], A int4 [4 blocks of 64][8 rows][128 B], A bf16
// [32 rows][128 B]; chunk c of row r sits in slot c ^ (r & 7).
// ---------------------------------------------------------------------------
struct I4NCfg {
    static constexpr int BM = 32, BN = 256, NT = 256;
    static constexpr int WAVES_M = 1, WAVES_N = 4, FM = 1, FN = 2;
    static constexpr int KS_I4 = 256, KS_BF = 64;    // reduction elements per stage
    static constexpr int AR = 8;                      // token rows of an int4 pass
    static constexpr int B_BYTES = BN * 128;
    static constexpr int A_BYTES = 4096;              // 8 rows x 256 fp16, or 32 rows x 64 bf16
    static constexpr int STAGE_BYTES = B_BYTES + A_BYTES;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static constexpr int WAVES_PER_EU = 2;
};
static_assert(I4NCfg::LDS_BYTES * 2 <= 160 * 1024, "two workgroups per CU");

// Whether the narrow engine can take a product of reduction width K: the
// scales of a row in one line, the reduction in whole stages.
__host__ __device__ inline bool i4n_fits(int K, int group)
{
    return group == 32 && K % 256 == 0 && K / 32 <= 64;
}

// fp16 bits in half h of a 32-bit word, in both halves of the result
__device__ __forceinline__ f16x2 half_splat(uint32_t word, int h)
{
    const uint32_t b = (word >> (16 * h)) & 0xffffu;
    return __builtin_bit_cast(f16x2, b * 0x00010001u);
}

// One pass of a tile.  brow[j]: weight row 64 w + 8 j + lane / 8 (byte 0).
// I4: ap = token row lane / 8 of the pass (element 0, fp16 in chunk order),
// srow = the scales of weight row tid.  bf16: a0 + r * lda = token row r
// (r < valid), srow unused.
template <bool I4>
__device__ __forceinline__ void i4n_mainloop(const uint16_t *ap, const uint16_t *a0, int lda,
                                             const char *const (&brow)[8], const uint16_t *srow, int K, int valid,
                                             char *lds, f32x16 (&acc)[I4NCfg::FN])
{
    using C = I4NCfg;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    constexpr int KS = I4 ? C::KS_I4 : C::KS_BF;
    const int nk = K / KS;
    auto dma = [](const void *src, char *dst) {
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    };
    u32x4 sv[8];                                      // scales of weight row tid: sv[i] = stage i's eight
    if (I4) {
        const int n16 = K / 256;
#pragma unroll
        for (int i = 0; i < 8; ++i) sv[i] = *reinterpret_cast<const u32x4 *>(srow + 8 * min(i, n16 - 1));
    }
    const int cr = lane >> 3, cp = lane & 7;          // a copy's row within its 8 and its slot
    const int ab = min(w * 8 + cr, valid - 1);        // bf16: this lane's A row
    auto issue = [&](int kt) {
        char *sb = lds + (kt & 1) * C::STAGE_BYTES, *sa = sb + C::B_BYTES;
#pragma unroll
        for (int j = 0; j < 8; ++j) {                 // B: 8 rows of 128 bytes per copy
            const int c = cp ^ cr;                    // rows 64 w + 8 j + cr: (row & 7) = cr
            if (I4) dma(brow[j] + kt * 128 + c * 16, sb + (w * 8 + j) * 1024);
            else dma(brow[j] + (kt * KS + c * 8) * 2, sb + (w * 8 + j) * 1024);
        }
        if (I4) dma(ap + kt * KS + w * 64 + (cp ^ cr) * 8, sa + w * 1024);        // block w, rows 0-7
        else dma(a0 + (size_t)ab * lda + kt * KS + (cp ^ cr) * 8, sa + w * 1024);  // rows 8 w .. 8 w + 7
    };

#pragma unroll
    for (int n = 0; n < C::FN; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[n][i] = 0.f;
    const int ar = lane & 31;                         // A fragment row
    const int arn = ar & 7;                           // its pass row (int4)
    int br[C::FN];                                    // B fragment rows: 64 w + 32 n + lane % 32
#pragma unroll
    for (int n = 0; n < C::FN; ++n) br[n] = (w * C::FN + n) * 32 + (lane & 31);

    issue(0);
    for (int kt = 0; kt < nk; ++kt) {
        wait_vmcnt_c<0>();                            // stage kt has landed
        // LDS-only barrier: every wave's copies of stage kt are visible, and
        // every wave is done with stage kt - 1, whose slot the next issue
        // overwrites
        __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (kt + 1 < nk) issue(kt + 1);
        const char *sb = lds + (kt & 1) * C::STAGE_BYTES, *sa = sb + C::B_BYTES;
        if (I4) {
            // stage kt's scales of rows 64 w + lane % 32 (n = 0) and
            // 64 w + 32 + lane % 32 (n = 1), from lanes lane % 32 and
            // 32 + lane % 32: word q holds groups 2 q (low) and 2 q + 1
            const u32x4 own = sv[0];
#pragma unroll
            for (int i = 0; i < 7; ++i) sv[i] = sv[i + 1];
            uint32_t sword[C::FN][4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const auto x = __builtin_amdgcn_permlane32_swap(own[q], own[q], false, false);
                sword[0][q] = x[0];
                sword[1][q] = x[1];
            }
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const int c = 2 * blk + h;            // 16-byte chunk = scale group 2 blk + h
                u32x4 bq[C::FN];
                f16x2 sc[C::FN];
#pragma unroll
                for (int n = 0; n < C::FN; ++n) {
                    bq[n] = *reinterpret_cast<const u32x4 *>(sb + br[n] * 128 + ((c ^ (br[n] & 7)) * 16));
                    sc[n] = half_splat(sword[n][blk], h);
                }
                f16x8 a[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int ca = 4 * h + j;
                    a[j] = *reinterpret_cast<const f16x8 *>(sa + (blk * 8 + arn) * 128 + ((ca ^ arn) * 16));
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int n = 0; n < C::FN; ++n)
                        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            a[j], __builtin_bit_cast(f16x8, int4x8_to_f16x8(bq[n][j], sc[n])), acc[n], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 2 * j + h;
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sa + ar * 128 + ((c ^ (ar & 7)) * 16));
#pragma unroll
                for (int n = 0; n < C::FN; ++n) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8 *>(sb + br[n] * 128 + ((c ^ (br[n] & 7)) * 16));
                    acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[n], 0, 0, 0);
                }
            }
        }
    }
    // the slots are reused by the next pass or tile: every wave is done
    // reading them
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
}

}  // namespace coli
