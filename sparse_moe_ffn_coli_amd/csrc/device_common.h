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
// bf16 MFMA tile engine
//
// A workgroup of 256 threads (4 waves of 64) computes a BM x BN block of
// C = A * B^T with A [BM][K] and B [BN][K] both K-contiguous (every matrix
// product of the layer has this form: activations times weight rows).  K is
// walked in steps of BK = 64: each step's A and B tiles are copied from
// global memory into LDS (16-byte chunks, one row = 8 chunks, chunk c of row
// r stored at position c ^ (r & 7) to spread MFMA operand reads over the
// banks), double-buffered so the global loads of step k+1 are in flight
// while step k runs on the matrix cores.  The waves form a WAVES_M x WAVES_N
// grid; each wave owns FM x FN fragments of 16x16 and issues
// v_mfma_f32_16x16x32_bf16 on them.
//
// Fragment layouts of v_mfma_f32_16x16x32_bf16 (lane l, i = 0..3):
//   A operand: row (l & 15), reduction slots 8*(l >> 4) .. +7
//   B operand: col (l & 15), the same reduction slots
//   result   : row 4*(l >> 4) + i, col (l & 15)
// A and B take the same slots from the same K positions, so the pairing of
// products is exact whatever the hardware's slot order.
//
// Rows are supplied as per-thread source pointers (gathered activation rows,
// expert weight rows), one per load chunk of the thread, including chunks
// past the tile (rows >= BM or >= BN), which are loaded and dropped.  Every
// pointer must be a readable row: a padding row
// (past an expert's last token, past the weight matrix's last row) points at
// any valid row instead.  Row m of the result depends only on row m of A and
// column n only on row n of B, so padding rows only reach results that the
// caller discards.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NT = 256;
    static constexpr int BK = 64;
    static constexpr int FM = BM / (WAVES_M * 16);
    static constexpr int FN = BN / (WAVES_N * 16);
    static constexpr int A_CHUNKS = BM * BK / 8;
    static constexpr int B_CHUNKS = BN * BK / 8;
    static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
    static constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
    static constexpr int STAGE = (BM + BN) * BK;      // bf16 elements per stage
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
    static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid");
    static_assert(BM % (WAVES_M * 16) == 0 && BN % (WAVES_N * 16) == 0, "tile shape");
};

// Index (in bf16 elements) of chunk `ch` of row `row` inside one tile region.
__device__ __forceinline__ int swz(int row, int ch)
{
    return (row * 8 + (ch ^ (row & 7))) * 8;
}

// Row of this thread's i-th load chunk (the chunk column is tid & 7 for all i).
template <class C>
__device__ __forceinline__ int a_chunk_row(int i) { return (threadIdx.x + i * C::NT) >> 3; }

template <class C>
__device__ __forceinline__ void mfma_mainloop(const uint16_t *const (&ap)[C::A_PER_T],
                                              const uint16_t *const (&bp)[C::B_PER_T], int K,
                                              uint16_t *lds, f32x4 (&acc)[C::FM][C::FN])
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
            acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / C::BK;
    COLI_GLOAD(0);
    COLI_SSTORE(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) COLI_GLOAD(kt + 1);
        const uint16_t *sa = lds + (kt & 1) * C::STAGE;
        const uint16_t *sb = sa + C::BM * C::BK;
#pragma unroll
        for (int kk = 0; kk < C::BK / 32; ++kk) {
            bf16x8 af[C::FM], bfr[C::FN];
            const int ch = kk * 4 + (lane >> 4);
#pragma unroll
            for (int m = 0; m < C::FM; ++m) {
                int row = (wm * C::FM + m) * 16 + (lane & 15);
                af[m] = *reinterpret_cast<const bf16x8 *>(sa + swz(row, ch));
            }
#pragma unroll
            for (int n = 0; n < C::FN; ++n) {
                int row = (wn * C::FN + n) * 16 + (lane & 15);
                bfr[n] = *reinterpret_cast<const bf16x8 *>(sb + swz(row, ch));
            }
#pragma unroll
            for (int m = 0; m < C::FM; ++m)
#pragma unroll
                for (int n = 0; n < C::FN; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bfr[n], acc[m][n],
                                                                        0, 0, 0);
        }
        if (kt + 1 < nk) COLI_SSTORE((kt + 1) & 1);
        __syncthreads();
    }
#undef COLI_GLOAD
#undef COLI_SSTORE
}

}  // namespace coli
