// device_common.h -- device helpers shared by the gfx950 kernels of the routed
// MoE FFN layer: bf16 conversions, the clamped SwiGLU, and the LDS-staged
// bf16 MFMA tile engine used by every matrix product of the layer.
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
// fp16 variant of the register-staged engine, for int4 weights
//
// Operands are fp16 in LDS and multiplied with v_mfma_f32_32x32x16_f16 (fp32
// accumulation).  A rows arrive in bf16 and are converted on the way into
// LDS (exact for magnitudes in fp16's normal range).  Each of the BN (= 256
// = threads) B rows is staged by one thread, one of two ways per tile:
//   int4: 32 bytes of nibbles per K step of 64, element 2i in the low nibble
//         of byte i, value (nibble - 8) * scale with one fp16 scale per
//         `group` consecutive elements (offset-binary, "feat(glm53): add
//         device-resident HIP backend for MI350P", section "Key changes");
//   bf16: converted like the A rows (the shared expert's dense weights).
//
// Both operands are stored with the same order of K inside every 16-byte
// chunk of 8 elements, 0,4,1,5,2,6,3,7: dword j holds elements j and j + 4.
// A dot product over the chunk does not depend on that order, and it lets
// one AND/OR put two nibbles of a 32-bit word (bits 4j and 16 + 4j) under the
// fp16 exponent of 1024: the pair is then 1024 + n exactly, subtracting 1032
// leaves n - 8 exactly, and one fp16 multiply by the scale rounds the exact
// product (n - 8) * scale once, as an fp32 product rounded to fp16 would.
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

// 8 nibbles of w (element p in bits 4p..4p+3) -> 8 fp16 values
// (nibble - 8) * scale in the chunk order 0,4,1,5,2,6,3,7
__device__ __forceinline__ u32x4 int4x8_to_f16x8(uint32_t w, f16x2 scale2)
{
    const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t d = ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
        const f16x2 v = (__builtin_bit_cast(f16x2, d) - off) * scale2;
        r[j] = __builtin_bit_cast(uint32_t, v);
    }
    return r;
}

__device__ __forceinline__ f16x2 fp16_bits_splat(uint16_t h)
{
    return __builtin_bit_cast(f16x2, (uint32_t)h * 0x00010001u);
}

// ap: A rows (bf16) as in mfma_mainloop.  B row of this thread (row tid):
// int4 when bq != nullptr (nibbles bq, fp16 scales bs, `group` elements per
// scale, a multiple of 32), else bf16 row bb.
template <class C>
__device__ __forceinline__ void mfma_mainloop_f16(const uint16_t *const (&ap)[C::A_PER_T],
                                                  const uint16_t *bb, const uint8_t *bq,
                                                  const uint16_t *bs, int group, int K, uint16_t *lds,
                                                  f32x16 (&acc)[C::FM][C::FN])
{
    static_assert(C::BN == C::NT, "one B row per thread");
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int ch0 = tid & 7;
    const bool i4 = bq != nullptr;

    u32x4 ra[C::A_PER_T];
    u32x4 rq[2];
    u32x4 rb[8];
    f16x2 s0 = {}, s1 = {};
#define COLI_GLOAD16(kt_)                                                                      \
    do {                                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < C::A_PER_T; ++i_) ra[i_] =                     \
            *reinterpret_cast<const u32x4 *>(ap[i_] + (kt_) * C::BK);                          \
        if (i4) {                                                                              \
            rq[0] = *reinterpret_cast<const u32x4 *>(bq + (kt_) * (C::BK / 2));                \
            rq[1] = *reinterpret_cast<const u32x4 *>(bq + (kt_) * (C::BK / 2) + 16);           \
            s0 = fp16_bits_splat(bs[((kt_) * C::BK) / group]);                                   \
            s1 = fp16_bits_splat(bs[((kt_) * C::BK + 32) / group]);                              \
        } else {                                                                               \
            _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) rb[j_] =                          \
                *reinterpret_cast<const u32x4 *>(bb + (kt_) * C::BK + 8 * j_);                 \
        }                                                                                      \
    } while (0)
#define COLI_SSTORE16(buf_)                                                                    \
    do {                                                                                       \
        uint16_t *sa_ = lds + (buf_) * C::STAGE;                                               \
        uint16_t *sb_ = sa_ + C::BM * C::BK;                                                   \
        _Pragma("unroll") for (int i_ = 0; i_ < C::A_PER_T; ++i_) {                            \
            const int c_ = tid + i_ * C::NT;                                                   \
            if (C::A_CHUNKS % C::NT == 0 || c_ < C::A_CHUNKS)                                  \
                *reinterpret_cast<u32x4 *>(sa_ + swz(c_ >> 3, ch0)) = bf16x8_to_f16x8(ra[i_]); \
        }                                                                                      \
        if (i4) {                                                                              \
            _Pragma("unroll") for (int c_ = 0; c_ < 8; ++c_)                                   \
                *reinterpret_cast<u32x4 *>(sb_ + swz(tid, c_)) =                               \
                    int4x8_to_f16x8(rq[c_ >> 2][c_ & 3], c_ < 4 ? s0 : s1);                    \
        } else {                                                                               \
            _Pragma("unroll") for (int c_ = 0; c_ < 8; ++c_)                                   \
                *reinterpret_cast<u32x4 *>(sb_ + swz(tid, c_)) = bf16x8_to_f16x8(rb[c_]);      \
        }                                                                                      \
    } while (0)

#pragma unroll
    for (int m = 0; m < C::FM; ++m)
#pragma unroll
        for (int n = 0; n < C::FN; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;

    f16x8 af[2][C::FM], bfr[2][C::FN];
#define COLI_LFRAG16(stage_, kk_, slot_)                                                       \
    do {                                                                                       \
        const uint16_t *sa_ = lds + (stage_) * C::STAGE;                                       \
        const uint16_t *sb_ = sa_ + C::BM * C::BK;                                             \
        const int ch_ = (kk_) * 2 + (lane >> 5);                                               \
        _Pragma("unroll") for (int m_ = 0; m_ < C::FM; ++m_) af[slot_][m_] =                   \
            *reinterpret_cast<const f16x8 *>(sa_ + swz((wm * C::FM + m_) * 32 + (lane & 31), ch_)); \
        _Pragma("unroll") for (int n_ = 0; n_ < C::FN; ++n_) bfr[slot_][n_] =                  \
            *reinterpret_cast<const f16x8 *>(sb_ + swz((wn * C::FN + n_) * 32 + (lane & 31), ch_)); \
    } while (0)

    const int nk = K / C::BK;
    COLI_GLOAD16(0);
    COLI_SSTORE16(0);
    __syncthreads();
    COLI_LFRAG16(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) COLI_GLOAD16(kt + 1);
#pragma unroll
        for (int kk = 0; kk < C::BK / 16; ++kk) {
            const int slot = kk & 1;
            if (kk + 1 < C::BK / 16) COLI_LFRAG16(cur, kk + 1, slot ^ 1);
#pragma unroll
            for (int m = 0; m < C::FM; ++m)
#pragma unroll
                for (int n = 0; n < C::FN; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[slot][m], bfr[slot][n],
                                                                       acc[m][n], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            COLI_SSTORE16(cur ^ 1);
            __syncthreads();
            COLI_LFRAG16(cur ^ 1, 0, 0);
        }
    }
#undef COLI_GLOAD16
#undef COLI_SSTORE16
#undef COLI_LFRAG16
}

// ---------------------------------------------------------------------------
// Direct-to-LDS tile engine (large tiles)
//
// Same contract as mfma_mainloop, but the tiles travel from global memory
// straight into LDS (global_load_lds_dwordx4: each lane's 16 bytes land at
// M0 + 16 * lane), so no VGPRs are spent on staging and NS stages of BK = 32
// can be in flight at once (a ring of NS LDS buffers).  A stage holds the
// BM A rows followed by the BN B rows, 64 bytes (4 chunks) per row; chunk c
// of row r sits at position c ^ ((r >> 2) & 3), which makes both the 1 KB
// DMA writes and the 16-rows-per-cycle fragment reads bank-conflict free.
// Load instruction j of wave w covers rows 16 (4 j + w) .. +15.
//
// `valid` = number of real A rows in the tile (1..BM).  A load instruction
// whose 16 rows are all past `valid` is skipped, and so are the MFMAs and
// LDS reads of a 32-row fragment past `valid`: a tile of a lightly loaded
// expert costs little more than streaming its weight rows.  The per-wave
// count of issued loads is uniform, so the vmcnt waits below stay exact.
//
// Per stage kt (frags of reduction step 0 already in registers):
//   read frags of step 1 | MFMAs of step 0 |
//   wait for stage kt+1 (own loads), barrier (everyone's loads landed and
//   everyone left stage kt-1), issue stage kt+NS-1 into kt-1's buffer,
//   read frags of stage kt+1 step 0 | MFMAs of step 1
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NS_>
struct DmaCfg {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NS = NS_;
    static constexpr int BK = 32;
    static constexpr int FM = BM / (WAVES_M * 32);
    static constexpr int FN = BN / (WAVES_N * 32);
    static constexpr int ROWS = BM + BN;
    static constexpr int LPW = ROWS / 64;               // load instructions per wave per stage
    static constexpr int STAGE_BYTES = ROWS * 64;
    static constexpr int LDS_BYTES = NS * STAGE_BYTES;
    static_assert(ROWS % 64 == 0 && BM % 16 == 0, "rows per stage");
    static_assert(NS >= 3 && (NS & (NS - 1)) == 0, "stages");
    static_assert(WAVES_M * WAVES_N == 4, "four waves");
    static_assert(FM >= 1 && FN >= 1, "tile shape");
};

// Tile row covered by this lane in load instruction j, and the source chunk
// it must fetch so that the DMA's lane-contiguous layout is the swizzled one.
template <class C>
__device__ __forceinline__ int dma_row(int j)
{
    return (j * 4 + (threadIdx.x >> 6)) * 16 + ((threadIdx.x & 63) >> 2);
}
__device__ __forceinline__ int dma_chunk(int row) { return (threadIdx.x & 3) ^ ((row >> 2) & 3); }

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt unconstrained (gfx9 encoding: vmcnt
// in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).  n <= 47.
__device__ __forceinline__ void wait_vmcnt(int n)
{
#define COLI_W(k) case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | 0x0F70); break;
    switch (n) {
        COLI_W(0) COLI_W(1) COLI_W(2) COLI_W(3) COLI_W(4) COLI_W(5) COLI_W(6) COLI_W(7)
        COLI_W(8) COLI_W(9) COLI_W(10) COLI_W(11) COLI_W(12) COLI_W(13) COLI_W(14) COLI_W(15)
        COLI_W(16) COLI_W(17) COLI_W(18) COLI_W(19) COLI_W(20) COLI_W(21) COLI_W(22) COLI_W(23)
        COLI_W(24) COLI_W(25) COLI_W(26) COLI_W(27) COLI_W(28) COLI_W(29) COLI_W(30) COLI_W(31)
        COLI_W(32) COLI_W(33) COLI_W(34) COLI_W(35) COLI_W(36) COLI_W(37) COLI_W(38) COLI_W(39)
        COLI_W(40) COLI_W(41) COLI_W(42) COLI_W(43) COLI_W(44) COLI_W(45) COLI_W(46) COLI_W(47)
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
#undef COLI_W
}

// rp[j]: this lane's source for load instruction j (its row, already offset
// by dma_chunk), a valid readable address even for padding rows.
template <class C>
__device__ __forceinline__ void dma_mainloop(const uint16_t *const (&rp)[C::LPW], int K, int valid,
                                             char *lds, f32x16 (&acc)[C::FM][C::FN])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int nk = K / C::BK;

    // load instructions this wave issues per stage (A instructions past
    // `valid` are skipped; B instructions always run)
    int nload = 0;
#pragma unroll
    for (int j = 0; j < C::LPW; ++j) {
        const int q = j * 4 + wave;
        nload += (q * 16 >= C::BM || q * 16 < valid) ? 1 : 0;
    }

#define COLI_ISSUE(kt_)                                                                          \
    do {                                                                                         \
        char *sb_ = lds + ((kt_) & (C::NS - 1)) * C::STAGE_BYTES;                               \
        _Pragma("unroll") for (int j_ = 0; j_ < C::LPW; ++j_) {                                 \
            const int q_ = j_ * 4 + wave;                                                        \
            if (q_ * 16 >= C::BM || q_ * 16 < valid)                                            \
                __builtin_amdgcn_global_load_lds(                                                \
                    (const __attribute__((address_space(1))) void *)(rp[j_] + (kt_) * C::BK),  \
                    (__attribute__((address_space(3))) void *)(sb_ + q_ * 1024), 16, 0, 0);     \
        }                                                                                        \
    } while (0)

    bf16x8 af[2][C::FM], bfr[2][C::FN];
#define COLI_LFRAG(kt_, kk_, slot_)                                                              \
    do {                                                                                         \
        const char *sa_ = lds + ((kt_) & (C::NS - 1)) * C::STAGE_BYTES;                         \
        const char *sbb_ = sa_ + C::BM * 64;                                                     \
        const int c_ = (kk_) * 2 + (lane >> 5);                                                 \
        _Pragma("unroll") for (int m_ = 0; m_ < C::FM; ++m_) {                                  \
            const int r_ = (wm * C::FM + m_) * 32 + (lane & 31);                                \
            if ((wm * C::FM + m_) * 32 < valid)                                                  \
                af[slot_][m_] = *reinterpret_cast<const bf16x8 *>(                               \
                    sa_ + r_ * 64 + ((c_ ^ ((r_ >> 2) & 3)) << 4));                              \
        }                                                                                        \
        _Pragma("unroll") for (int n_ = 0; n_ < C::FN; ++n_) {                                  \
            const int r_ = (wn * C::FN + n_) * 32 + (lane & 31);                                \
            bfr[slot_][n_] = *reinterpret_cast<const bf16x8 *>(                                  \
                sbb_ + r_ * 64 + ((c_ ^ ((r_ >> 2) & 3)) << 4));                                 \
        }                                                                                        \
    } while (0)
#define COLI_MMA(slot_)                                                                          \
    do {                                                                                         \
        _Pragma("unroll") for (int m_ = 0; m_ < C::FM; ++m_)                                    \
            if ((wm * C::FM + m_) * 32 < valid)                                                  \
                _Pragma("unroll") for (int n_ = 0; n_ < C::FN; ++n_)                            \
                    acc[m_][n_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                       \
                        af[slot_][m_], bfr[slot_][n_], acc[m_][n_], 0, 0, 0);                    \
    } while (0)

#pragma unroll
    for (int m = 0; m < C::FM; ++m)
#pragma unroll
        for (int n = 0; n < C::FN; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;
#pragma unroll
    for (int m = 0; m < C::FM; ++m)
#pragma unroll
        for (int i = 0; i < 8; ++i) af[0][m][i] = af[1][m][i] = (__bf16)0.f;

    // prologue: stages 0 .. NS-2 in flight; wait for stage 0
#pragma unroll
    for (int st = 0; st < C::NS - 1; ++st)
        if (st < nk) COLI_ISSUE(st);
    wait_vmcnt(min(C::NS - 2, nk - 1) * nload);
    __syncthreads();
    COLI_LFRAG(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        COLI_LFRAG(kt, 1, 1);
        COLI_MMA(0);
        if (kt + 1 < nk) {
            wait_vmcnt((min(kt + C::NS - 2, nk - 1) - (kt + 1)) * nload);
            __syncthreads();
            if (kt + C::NS - 1 < nk) COLI_ISSUE(kt + C::NS - 1);
            COLI_LFRAG(kt + 1, 0, 0);
        }
        COLI_MMA(1);
    }
    // leave LDS quiescent for the caller's epilogue
    __syncthreads();
#undef COLI_ISSUE
#undef COLI_LFRAG
#undef COLI_MMA
}

}  // namespace coli
