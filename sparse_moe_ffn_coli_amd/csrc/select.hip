// select.hip -- index selection of the sparse attention's IndexPool: per
// row, the k positions with the largest indexer scores, with the last `tail`
// positions always kept ("Add GLM-5.3-Flash (glm5next) support with ROCmFP
// mix qtypes (105/106)", section "MLA/DSA": top-k over the indexer scores
// with k = 2048, the last kpool tokens always selected).
//
// One workgroup of 16 waves per row.  Scores become order-preserving
// unsigned keys (-0 folded onto +0; the tail positions take the largest key),
// so "larger score first, lower position on ties" is "larger key first,
// lower position on ties".  The k-th largest key tau is found by a radix
// select over three digits (bits 31-21, 20-10, 9-0): an LDS histogram of the
// current digit among the keys that match the digits found so far, and a
// workgroup suffix scan over the bins to find the digit holding the k-th key.
// Every position whose key is above tau is selected, and of those equal to
// tau the lowest positions until k are reached.  The selected positions are
// written in ascending order by an ordered compaction: each wave owns a
// contiguous segment of the row, counts its keys above and equal to tau,
// takes its starting counts from a scan over the waves, and then walks its
// segment 64 positions at a time placing each selected position by ballot
// popcounts.  Integer work only: the result is unique and reproducible.
// Rows of up to SEL_CAP positions keep their keys in LDS after one read of
// the scores; longer rows re-read the scores (from L2) in each pass.
#include "device_common.h"
#include "kernels.h"

namespace coli {

constexpr int SEL_NT = 1024;             // threads per workgroup (16 waves)
constexpr int SEL_WAVES = SEL_NT / 64;

__device__ __forceinline__ uint32_t score_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;        // -0 ranks with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int CAP>
__global__ __launch_bounds__(SEL_NT) void index_topk_kernel(const float *__restrict__ scores, int L, long ld,
                                                            const int32_t *__restrict__ lens, int k, int tail,
                                                            int32_t *__restrict__ idx)
{
    __shared__ __attribute__((aligned(16))) uint32_t keys[CAP > 0 ? CAP : 1];
    __shared__ int32_t hist[2048];
    __shared__ int32_t ws[SEL_WAVES];
    __shared__ int32_t sel_s[2];
    __shared__ int32_t wave_gt[SEL_WAVES], wave_eq[SEL_WAVES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x;
    const int n = lens ? min(max(lens[r], 0), L) : L;
    int32_t *__restrict__ out = idx + (size_t)r * k;
    if (n <= k) {                                 // the whole row, then -1
        for (int j = tid; j < k; j += SEL_NT) out[j] = j < n ? j : -1;
        return;
    }
    const float *__restrict__ row = scores + (size_t)r * ld;
    const int tail0 = n - min(tail, k);           // positions >= tail0 are always kept
    const bool cached = n <= CAP;
    auto key_at = [&](int i) { return i >= tail0 ? 0xffffffffu : score_key(row[i]); };
    auto get = [&](int i) { return cached ? keys[i] : key_at(i); };

    for (int b = tid; b < 2048; b += SEL_NT) hist[b] = 0;
    __syncthreads();
    // digit 0 histogram; cached rows are read once here, four scores per load
    if (cached) {
        const int n4 = n & ~3;
        for (int i = 4 * tid; i < n4; i += 4 * SEL_NT) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(row + i);
            uint32_t q[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                q[c] = (i + c >= tail0) ? 0xffffffffu : score_key(v[c]);
                atomicAdd(&hist[q[c] >> 21], 1);
            }
            *reinterpret_cast<u32x4 *>(keys + i) = u32x4{q[0], q[1], q[2], q[3]};
        }
        for (int i = n4 + tid; i < n; i += SEL_NT) {
            const uint32_t q = key_at(i);
            keys[i] = q;
            atomicAdd(&hist[q >> 21], 1);
        }
    } else {
        for (int i = tid; i < n; i += SEL_NT) atomicAdd(&hist[key_at(i) >> 21], 1);
    }
    __syncthreads();

    // radix select: digits of 11, 11 and 10 bits, most significant first
    uint32_t prefix = 0;
    int need = k;                                 // keys still to take at or below the prefix
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
        const int nb = pass == 2 ? 1024 : 2048;
        if (pass > 0) {
            const uint32_t hi = 0xffffffffu << (shift + (pass == 2 ? 10 : 11));
            for (int i = tid; i < n; i += SEL_NT) {
                const uint32_t q = get(i);
                if ((q & hi) == prefix) atomicAdd(&hist[(q >> shift) & (nb - 1)], 1);
            }
            __syncthreads();
        }
        // thread t holds bins nb-1-2t and nb-2-2t: a scan in thread order is a
        // suffix scan over the bins; the digit is the bin where the count of
        // keys above it first reaches `need`
        const int b0 = nb - 1 - 2 * tid, b1 = b0 - 1;
        const int c0 = (b0 >= 0) ? hist[b0] : 0, c1 = (b1 >= 0) ? hist[b1] : 0;
        const int incl = block_scan_incl<SEL_WAVES>(c0 + c1, ws);
        const int above = incl - c0 - c1;
        if (above < need && above + c0 >= need) {
            sel_s[0] = b0;
            sel_s[1] = above;
        } else if (above + c0 < need && above + c0 + c1 >= need) {
            sel_s[0] = b1;
            sel_s[1] = above + c0;
        }
        __syncthreads();
        prefix |= (uint32_t)sel_s[0] << shift;
        need -= sel_s[1];
        __syncthreads();
        for (int b = tid; b < 2048; b += SEL_NT) hist[b] = 0;
        __syncthreads();
    }
    const uint32_t tau = prefix;                  // the k-th largest key; `need` keys equal to it are taken

    // ordered compaction: wave w owns positions [seg0, seg1)
    const int seg = ((n + SEL_WAVES - 1) / SEL_WAVES + 63) & ~63;
    const int seg0 = min(wave * seg, n), seg1 = min(seg0 + seg, n);
    int gt = 0, eq = 0;
    for (int i = seg0 + lane; i < seg1; i += 64) {
        const uint32_t q = get(i);
        gt += q > tau;
        eq += q == tau;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        gt += __shfl_xor(gt, off);
        eq += __shfl_xor(eq, off);
    }
    if (lane == 0) {
        wave_gt[wave] = gt;
        wave_eq[wave] = eq;
    }
    __syncthreads();
    int gt_b = 0, eq_b = 0;                       // keys above / equal to tau before this segment
    for (int w2 = 0; w2 < wave; ++w2) {
        gt_b += wave_gt[w2];
        eq_b += wave_eq[w2];
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i0 = seg0; i0 < seg1; i0 += 64) {
        const int i = i0 + lane;
        const uint32_t q = (i < seg1) ? get(i) : 0u;
        const bool g = (i < seg1) && q > tau, e = (i < seg1) && q == tau;
        const uint64_t mg = __ballot(g), me = __ballot(e);
        const int my_gt = gt_b + __popcll(mg & below), my_eq = eq_b + __popcll(me & below);
        if (g) out[my_gt + min(my_eq, need)] = i;
        else if (e && my_eq < need) out[my_gt + my_eq] = i;
        gt_b += __popcll(mg);
        eq_b += __popcll(me);
    }
}

int index_topk_cap(int L) { return L <= 8192 ? 8192 : 32768; }

hipError_t launch_index_topk(const float *scores, int rows, int L, long ld, const int32_t *lens, int k, int tail,
                             int32_t *idx, hipStream_t st)
{
    if (rows == 0) return hipSuccess;
    if (index_topk_cap(L) == 8192)
        index_topk_kernel<8192><<<rows, SEL_NT, 0, st>>>(scores, L, ld, lens, k, tail, idx);
    else
        index_topk_kernel<32768><<<rows, SEL_NT, 0, st>>>(scores, L, ld, lens, k, tail, idx);
    return hipGetLastError();
}

}  // namespace coli
