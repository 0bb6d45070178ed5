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
// the scores; longer rows re-read the scores (from L2) in each pass.  Each
// workgroup walks several rows and loads the next row's scores into
// registers while it selects the current one.
#include "device_common.h"
#include "kernels.h"

namespace coli {

constexpr int SEL_NT = 1024;             // threads per workgroup (16 waves)
constexpr int SEL_WAVES = SEL_NT / 64;
constexpr int SEL_BATCH = 8;             // positions per thread whose loads are in flight together

__device__ __forceinline__ uint32_t score_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;        // -0 ranks with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int SEL_CAP = 32768;           // positions whose keys a workgroup keeps in LDS (128 KB)
constexpr int SEL_PER = SEL_CAP / (4 * SEL_NT);   // 16-byte loads per thread for a cached row
constexpr int SEL_MAX_K = 4096;          // largest k

// Inclusive prefix sum over the 64 lanes of a wave on DPP lane moves: shifts
// by 1, 2, 4 and 8 inside each row of 16 lanes, then each row's total is
// added to the rows above it (row broadcasts of lanes 15 and 31).  Lanes
// whose source is outside the pattern add 0.
__device__ __forceinline__ int wave_scan_incl(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    return v;
}

// Barrier for LDS traffic only: every wave's LDS operations have completed
// (global loads in flight, such as the next row's prefetch, are not waited for).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
}

// Inclusive prefix sum over the workgroup in thread order (ws: SEL_WAVES ints).
__device__ __forceinline__ int block_scan_incl_dpp(int v, int32_t *ws)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_scan_incl(v);
    if (lane == 63) ws[wave] = v;
    lds_barrier();
    int before = 0;
#pragma unroll
    for (int w2 = 0; w2 < SEL_WAVES; ++w2) before += (w2 < wave) ? ws[w2] : 0;
    return v + before;
}

// ---- a cached row (n <= SEL_CAP): keys in LDS, thread t holding the groups
// of four positions 4 (j * SEL_NT + t) .. + 3 -------------------------------

// The scores of a row into registers (one 16-byte load per group; the groups
// past the last whole one reread it, their values unused).
__device__ __forceinline__ void load_row(const float *__restrict__ row, int n, f32x4 (&v)[SEL_PER])
{
    const int n4 = n & ~3;
#pragma unroll
    for (int j = 0; j < SEL_PER; ++j) {
        const int i = 4 * (j * SEL_NT + (int)threadIdx.x);
        v[j] = (n4 >= 4) ? *reinterpret_cast<const f32x4 *>(row + min(i, n4 - 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// keys[i] = key of position i, hist[d] = positions whose top 11 key bits are d
__device__ __forceinline__ void store_keys(const float *__restrict__ row, int n, int tail0, const f32x4 (&v)[SEL_PER],
                                           uint32_t *keys, int32_t *hist)
{
    const int n4 = n & ~3;
#pragma unroll
    for (int j = 0; j < SEL_PER; ++j) {
        const int i = 4 * (j * SEL_NT + (int)threadIdx.x);
        if (i < n4) {
            uint32_t q[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                q[c] = (i + c >= tail0) ? 0xffffffffu : score_key(v[j][c]);
                atomicAdd(&hist[q[c] >> 21], 1);
            }
            *reinterpret_cast<u32x4 *>(keys + i) = u32x4{q[0], q[1], q[2], q[3]};
        }
    }
    for (int i = n4 + (int)threadIdx.x; i < n; i += SEL_NT) {     // the last 0-3 positions
        const uint32_t q = (i >= tail0) ? 0xffffffffu : score_key(row[i]);
        keys[i] = q;
        atomicAdd(&hist[q >> 21], 1);
    }
}

// The digit holding the need-th largest key: thread t holds bins nb-1-2t and
// nb-2-2t, so a scan in thread order is a suffix scan over the bins.  Returns
// the bin; *above receives the keys in higher bins.  Clears hist afterwards.
__device__ __forceinline__ int pick_bin(int32_t *hist, int nb, int need, int32_t *ws, int32_t *sel_s, int *above_out)
{
    const int tid = threadIdx.x;
    const int b0 = nb - 1 - 2 * tid, b1 = b0 - 1;
    const int c0 = (b0 >= 0) ? hist[b0] : 0, c1 = (b1 >= 0) ? hist[b1] : 0;
    const int incl = block_scan_incl_dpp(c0 + c1, ws);
    const int above = incl - c0 - c1;
    if (above < need && above + c0 >= need) {
        sel_s[0] = b0;
        sel_s[1] = above;
    } else if (above + c0 < need && above + c0 + c1 >= need) {
        sel_s[0] = b1;
        sel_s[1] = above + c0;
    }
    if (b0 >= 0) hist[b0] = 0;                    // every bin is read above by its owner only
    if (b1 >= 0) hist[b1] = 0;
    for (int b = nb + tid; b < 2048; b += SEL_NT) hist[b] = 0;
    lds_barrier();
    const int bin = sel_s[0];
    *above_out = sel_s[1];
    lds_barrier();                                // sel_s and ws are free again
    return bin;
}

// Ordered compaction of a cached row: wave w owns positions [seg0, seg1)
// (whole groups of 256: four consecutive positions per lane), counts its keys
// above and equal to tau, takes its starting counts from the waves before it,
// and walks its segment 256 positions at a time: a lane's count of earlier
// selected positions in the wave comes from ballots of the four position
// slots and bit counts below the lane.  A slot is written only inside the
// row's k outputs.
__device__ __forceinline__ void compact_cached(const uint32_t *keys, int n, int k, uint32_t tau, int need,
                                               int32_t *wave_gt, int32_t *wave_eq, int32_t *staged)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = ((n + SEL_WAVES - 1) / SEL_WAVES + 255) & ~255;
    const int seg0 = min(wave * seg, n), seg1 = min(seg0 + seg, n);
    constexpr int MAXIT = SEL_CAP / SEL_WAVES / 256;  // 256-position steps of the longest segment
    // keys of the segment's step `it` for this lane (past seg1: masked by the caller)
    auto group = [&](int it) {
        return *reinterpret_cast<const u32x4 *>(keys + min(seg0 + 256 * it + 4 * lane, SEL_CAP - 4));
    };
    int gt = 0, eq = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {                 // half the steps' keys loaded at a time
        u32x4 q[MAXIT / 2];
#pragma unroll
        for (int j = 0; j < MAXIT / 2; ++j) q[j] = group(h * (MAXIT / 2) + j);
#pragma unroll
        for (int j = 0; j < MAXIT / 2; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool in = seg0 + 256 * (h * (MAXIT / 2) + j) + 4 * lane + c < seg1;
                gt += in && q[j][c] > tau;
                eq += in && q[j][c] == tau;
            }
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
    lds_barrier();
    int gt_b = 0, eq_b = 0;                       // keys above / equal to tau before this segment
#pragma unroll
    for (int w2 = 0; w2 < SEL_WAVES; ++w2) {
        gt_b += (w2 < wave) ? wave_gt[w2] : 0;
        eq_b += (w2 < wave) ? wave_eq[w2] : 0;
    }
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
        const int p0 = seg0 + 256 * it + 4 * lane;
        if (seg0 + 256 * it >= seg1) break;       // uniform over the wave
        const u32x4 q = group(it);
        bool g[4], e[4];
        uint64_t mg[4], me[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool in = p0 + c < seg1;
            g[c] = in && q[c] > tau;
            e[c] = in && q[c] == tau;
            mg[c] = __ballot(g[c]);
            me[c] = __ballot(e[c]);
        }
        // selected positions of this step before this lane's first
        int my_gt = gt_b, my_eq = eq_b;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            my_gt += __builtin_amdgcn_mbcnt_hi((uint32_t)(mg[c] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg[c], 0));
            my_eq += __builtin_amdgcn_mbcnt_hi((uint32_t)(me[c] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me[c], 0));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (g[c]) {
                const int slot = my_gt + min(my_eq, need);
                if (slot < k) staged[slot] = p0 + c;
                ++my_gt;
            } else if (e[c]) {
                if (my_eq < need) staged[my_gt + my_eq] = p0 + c;
                ++my_eq;
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            gt_b += __popcll(mg[c]);
            eq_b += __popcll(me[c]);
        }
    }
}

// ---- a row too long for LDS: every pass re-reads the scores -----------------
__device__ __forceinline__ void select_uncached(const float *__restrict__ row, int n, int tail0, int k, int32_t *hist,
                                                int32_t *ws, int32_t *sel_s, int32_t *wave_gt, int32_t *wave_eq,
                                                int32_t *__restrict__ out)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto key_at = [&](int i) { return i >= tail0 ? 0xffffffffu : score_key(row[i]); };
    // f(i, key) for every position, SEL_BATCH per thread with their loads in flight together
    auto for_each_key = [&](auto &&f) {
        for (int b0 = 0; b0 < n; b0 += SEL_BATCH * SEL_NT) {
            uint32_t q[SEL_BATCH];
#pragma unroll
            for (int j = 0; j < SEL_BATCH; ++j) q[j] = key_at(min(b0 + j * SEL_NT + tid, n - 1));
#pragma unroll
            for (int j = 0; j < SEL_BATCH; ++j)
                if (b0 + j * SEL_NT + tid < n) f(q[j]);
        }
    };
    uint32_t prefix = 0;
    int need = k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
        const int nb = pass == 2 ? 1024 : 2048;
        const uint32_t hi = pass == 0 ? 0u : 0xffffffffu << (shift + (pass == 2 ? 10 : 11));
        for_each_key([&](uint32_t q) {
            if ((q & hi) == prefix) atomicAdd(&hist[(q >> shift) & (nb - 1)], 1);
        });
        __syncthreads();
        int above;
        prefix |= (uint32_t)pick_bin(hist, nb, need, ws, sel_s, &above) << shift;
        need -= above;
    }
    const uint32_t tau = prefix;
    const int seg = ((n + SEL_WAVES - 1) / SEL_WAVES + 63) & ~63;
    const int seg0 = min(wave * seg, n), seg1 = min(seg0 + seg, n);
    int gt = 0, eq = 0;
    for (int i = seg0 + lane; i < seg1; i += 64) {
        const uint32_t q = key_at(i);
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
    int gt_b = 0, eq_b = 0;
    for (int w2 = 0; w2 < wave; ++w2) {
        gt_b += wave_gt[w2];
        eq_b += wave_eq[w2];
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i0 = seg0; i0 < seg1; i0 += 64) {
        const int i = i0 + lane;
        const uint32_t q = (i < seg1) ? key_at(i) : 0u;
        const bool g = (i < seg1) && q > tau, e = (i < seg1) && q == tau;
        const uint64_t mg = __ballot(g), me = __ballot(e);
        const int my_gt = gt_b + __popcll(mg & below), my_eq = eq_b + __popcll(me & below);
        if (g) out[my_gt + min(my_eq, need)] = i;
        else if (e && my_eq < need) out[my_gt + my_eq] = i;
        gt_b += __popcll(mg);
        eq_b += __popcll(me);
    }
}

// Persistent workgroups: workgroup b takes rows b, b + G, b + 2G, ...  While
// a cached row is being selected, the next row's scores are already loading
// into registers, so the row reads overlap the selection work.
__global__ __launch_bounds__(SEL_NT) void index_topk_kernel(const float *__restrict__ scores, int rows, int L,
                                                            long ld, const int32_t *__restrict__ lens, int k,
                                                            int tail, int32_t *__restrict__ idx)
{
    __shared__ __attribute__((aligned(16))) uint32_t keys[SEL_CAP];
    __shared__ int32_t hist[2048];
    __shared__ int32_t ws[SEL_WAVES];
    __shared__ int32_t sel_s[2];
    __shared__ int32_t wave_gt[SEL_WAVES], wave_eq[SEL_WAVES];
    __shared__ __attribute__((aligned(16))) int32_t staged[SEL_MAX_K];   // the output row
    const int tid = threadIdx.x;
    auto row_len = [&](int r) { return lens ? min(max(lens[r], 0), L) : L; };
    for (int b = tid; b < 2048; b += SEL_NT) hist[b] = 0;
    f32x4 v[SEL_PER];
    int have = -1;                                // the row whose scores are in v
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
        const int n = row_len(r);
        int32_t *__restrict__ out = idx + (size_t)r * k;
        if (n <= k) {                             // the whole row, then -1
            for (int j = tid; j < k; j += SEL_NT) out[j] = j < n ? j : -1;
            continue;
        }
        if (n > SEL_CAP) continue;                // index_topk_long_kernel's row
        const float *__restrict__ row = scores + (size_t)r * ld;
        const int tail0 = n - min(tail, k);       // positions >= tail0 are always kept
        __syncthreads();                          // the previous row is done with keys / hist
        if (have != r) load_row(row, n, v);
        store_keys(row, n, tail0, v, keys, hist);
        lds_barrier();
        // the next row of this workgroup starts loading now
        have = -1;
        const int rn = r + gridDim.x;
        if (rn < rows) {
            const int nn = row_len(rn);
            if (nn > k && nn <= SEL_CAP) {
                load_row(scores + (size_t)rn * ld, nn, v);
                have = rn;
            }
        }
        // radix select: digits of 11, 11 and 10 bits, most significant first
        uint32_t prefix = 0;
        int need = k, above;
        prefix = (uint32_t)pick_bin(hist, 2048, need, ws, sel_s, &above) << 21;
        need -= above;
#pragma unroll 1
        for (int pass = 1; pass < 3; ++pass) {
            const int shift = pass == 1 ? 10 : 0;
            const int nb = pass == 2 ? 1024 : 2048;
            const uint32_t hi = 0xffffffffu << (shift + (pass == 2 ? 10 : 11));
            // groups of four positions, half the thread's groups loaded at a time
            constexpr int HALF = SEL_PER / 2;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4 g[HALF];
#pragma unroll
                for (int j = 0; j < HALF; ++j)
                    g[j] = *reinterpret_cast<const u32x4 *>(keys + min(4 * ((h * HALF + j) * SEL_NT + tid), SEL_CAP - 4));
#pragma unroll
                for (int j = 0; j < HALF; ++j) {
                    const int i = 4 * ((h * HALF + j) * SEL_NT + tid);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (i + c < n && (g[j][c] & hi) == prefix) atomicAdd(&hist[(g[j][c] >> shift) & (nb - 1)], 1);
                }
            }
            lds_barrier();
            prefix |= (uint32_t)pick_bin(hist, nb, need, ws, sel_s, &above) << shift;
            need -= above;
        }
        compact_cached(keys, n, k, prefix, need, wave_gt, wave_eq, staged);
        lds_barrier();
        if ((k & 3) == 0) {
            for (int j = 4 * tid; j < k; j += 4 * SEL_NT)
                *reinterpret_cast<u32x4 *>(out + j) = *reinterpret_cast<const u32x4 *>(staged + j);
        } else {
            for (int j = tid; j < k; j += SEL_NT) out[j] = staged[j];
        }
    }
}

// Rows longer than SEL_CAP: one workgroup per row, every pass re-reading the
// scores; the other rows are left to index_topk_kernel.
__global__ __launch_bounds__(SEL_NT) void index_topk_long_kernel(const float *__restrict__ scores, int L, long ld,
                                                                 const int32_t *__restrict__ lens, int k, int tail,
                                                                 int32_t *__restrict__ idx)
{
    __shared__ int32_t hist[2048];
    __shared__ int32_t ws[SEL_WAVES];
    __shared__ int32_t sel_s[2];
    __shared__ int32_t wave_gt[SEL_WAVES], wave_eq[SEL_WAVES];
    const int r = blockIdx.x;
    const int n = lens ? min(max(lens[r], 0), L) : L;
    if (n <= SEL_CAP) return;
    for (int b = threadIdx.x; b < 2048; b += SEL_NT) hist[b] = 0;
    __syncthreads();
    select_uncached(scores + (size_t)r * ld, n, n - min(tail, k), k, hist, ws, sel_s, wave_gt, wave_eq,
                    idx + (size_t)r * k);
}

// ---- rows of up to SEL_CAP positions, keys held in registers ---------------
// For launches with more rows than CUs.  One workgroup of 8 waves per row,
// two workgroups per CU (two rows in flight, each with half the waves of a
// cached-row workgroup at its barriers, and no 128 KB key array in LDS).
// Thread t holds the groups of four positions 4 (j * SR_NT + t) .. + 3,
// j < SR_PER, as keys in registers, so the radix passes and the compaction
// read no keys from LDS.  Same selection as the cached kernel: the k-th
// largest key tau by three radix digits, every key above tau, and of those
// equal to tau the lowest positions; the output in ascending position order.
// (2048 rows of 30 721-32 768 scores: 179 -> 153 us.  With 1024 threads and
// 32 keys each the registers spill heavily (301 us); four histogram copies
// indexed by lane, against same-address atomics, measured the same.)
constexpr int SR_NT = 512;
constexpr int SEL_REG_MIN_ROWS = 256;    // larger launches run index_topk_reg_kernel
constexpr int SR_WAVES = SR_NT / 64;
constexpr int SR_PER = SEL_CAP / (4 * SR_NT);     // groups of four positions per thread
static_assert(SR_WAVES % 4 == 0 && 4 * SR_NT >= 2048, "wave totals in fours; four bins per thread");

// Inclusive prefix sum over the workgroup in thread order (ws: SR_WAVES ints).
__device__ __forceinline__ int sr_block_scan_incl(int v, int32_t *ws)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_scan_incl(v);
    if (lane == 63) ws[wave] = v;
    lds_barrier();
    int before = 0;
#pragma unroll
    for (int w2 = 0; w2 < SR_WAVES; ++w2) before += (w2 < wave) ? ws[w2] : 0;
    return v + before;
}

// The digit holding the need-th largest key among bins 0 .. nb - 1 (nb <=
// 4 * SR_NT): thread t holds bins nb-1-4t .. nb-4-4t, so a scan in thread
// order is a suffix scan over the bins.  Returns the bin; *above receives the
// keys in higher bins.  Clears the bins it read.  The caller's next write of
// ws or sel_s comes after another barrier.
__device__ __forceinline__ int sr_pick_bin(int32_t *hist, int nb, int need, int32_t *ws, int32_t *sel_s,
                                           int *above_out)
{
    const int tid = threadIdx.x;
    int c[4], sum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int b = nb - 1 - 4 * tid - u;
        c[u] = (b >= 0) ? hist[b] : 0;
        sum += c[u];
    }
    int acc = sr_block_scan_incl(sum, ws) - sum;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (acc < need && acc + c[u] >= need) {
            sel_s[0] = nb - 1 - 4 * tid - u;
            sel_s[1] = acc;
        }
        acc += c[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int b = nb - 1 - 4 * tid - u;
        if (b >= 0) hist[b] = 0;
    }
    lds_barrier();
    *above_out = sel_s[1];
    return sel_s[0];
}

__global__ __launch_bounds__(SR_NT) __attribute__((amdgpu_waves_per_eu(SR_NT / 128))) void index_topk_reg_kernel(
    const float *__restrict__ scores, int L, long ld, const int32_t *__restrict__ lens, int k, int tail,
    int32_t *__restrict__ idx)
{
    __shared__ int32_t hist[2048];
    __shared__ int32_t ws[SR_WAVES];
    __shared__ int32_t sel_s[2];
    __shared__ __attribute__((aligned(16))) int32_t tot[SR_PER][SR_WAVES];    // per group round, per wave
    __shared__ __attribute__((aligned(16))) int32_t staged[SEL_MAX_K];        // the output row
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lens ? min(max(lens[r], 0), L) : L;
    int32_t *__restrict__ out = idx + (size_t)r * k;
    if (n <= k) {                                 // the whole row, then -1
        for (int j = tid; j < k; j += SR_NT) out[j] = j < n ? j : -1;
        return;
    }
    if (n > SEL_CAP) return;                      // index_topk_long_kernel's row
    const float *__restrict__ row = scores + (size_t)r * ld;
    const int tail0 = n - min(tail, k);           // positions >= tail0 are always kept
    const int n4 = n & ~3;

    // the row's scores: 16-byte buffer loads of whole groups (the buffer
    // ends after the last whole group, so the loads past it return zeros and
    // need no clamped addresses), then the last 0-3 positions one by one
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row), 0, n4 * 4, 0x00020000);
    f32x4 v[SR_PER];
#pragma unroll
    for (int j = 0; j < SR_PER; ++j)
        v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * tid, 16 * j * SR_NT, 0));
    // the last 0-3 positions: group n4 / 4, i.e. round jt of thread tt
    const int g4 = n4 >> 2, jt = g4 / SR_NT, tt = g4 - jt * SR_NT;
    float ex[3] = {0.f, 0.f, 0.f};
    if (tid == tt) {
#pragma unroll
        for (int c = 0; c < 3; ++c)
            if (n4 + c < n) ex[c] = row[n4 + c];
    }
    for (int b = tid; b < 2048; b += SR_NT) hist[b] = 0;
    uint32_t q[SR_PER][4];
#pragma unroll
    for (int j = 0; j < SR_PER; ++j) {
        const int p0 = 4 * (j * SR_NT + tid);
        const bool last = j == jt && tid == tt;
#pragma unroll
        for (int c = 0; c < 3; ++c) v[j][c] = last ? ex[c] : v[j][c];
        // positions past the row take key 0, below every real key but one
        // that a real key can share: the histograms discount them (bin 0,
        // while the digits found so far are all 0), and as they follow every
        // real position the compaction never reaches them
#pragma unroll
        for (int c = 0; c < 4; ++c)
            q[j][c] = (p0 + c >= n) ? 0u : (p0 + c >= tail0) ? 0xffffffffu : score_key(v[j][c]);
    }
    const int pad = SEL_CAP - n;                  // positions past the row
    lds_barrier();                                // hist is clear

    // radix select: digits of 11, 11 and 10 bits, most significant first
#pragma unroll
    for (int j = 0; j < SR_PER; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) atomicAdd(&hist[q[j][c] >> 21], 1);
    if (tid == 0) atomicAdd(hist, -pad);
    lds_barrier();
    int need = k, above;
    uint32_t prefix = (uint32_t)sr_pick_bin(hist, 2048, need, ws, sel_s, &above) << 21;
    need -= above;
#pragma unroll 1
    for (int pass = 1; pass < 3; ++pass) {
        const int shift = pass == 1 ? 10 : 0;
        const int nb = pass == 2 ? 1024 : 2048;
        const uint32_t hi = 0xffffffffu << (shift + (pass == 2 ? 10 : 11));
#pragma unroll
        for (int j = 0; j < SR_PER; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if ((q[j][c] & hi) == prefix) atomicAdd(&hist[(q[j][c] >> shift) & (nb - 1)], 1);
        if (tid == 0 && prefix == 0u) atomicAdd(hist, -pad);
        lds_barrier();
        prefix |= (uint32_t)sr_pick_bin(hist, nb, need, ws, sel_s, &above) << shift;
        need -= above;
    }
    const uint32_t tau = prefix;

    // ordered compaction: per group round j, the keys above tau (low 16 bits)
    // and equal to tau (high 16 bits) of this thread, scanned over the wave;
    // the wave totals of every round go through LDS in one barrier
    // (packed sums stay below 2^32: at most SEL_CAP keys in each half; the
    // scans are recomputed after the barrier rather than kept in registers)
    auto round_count = [&](int j) {
        int cnt = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            cnt += (q[j][c] > tau) ? 1 : 0;
            cnt += (q[j][c] == tau) ? 0x10000 : 0;
        }
        return cnt;
    };
#pragma unroll
    for (int j = 0; j < SR_PER; ++j) {
        const int incl = wave_scan_incl(round_count(j));   // at most 256 per half
        if (lane == 63) tot[j][wave] = incl;
    }
    lds_barrier();
    uint32_t base = 0;                            // packed counts of all rounds before j
#pragma unroll
    for (int j = 0; j < SR_PER; ++j) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int w4 = 0; w4 < SR_WAVES; w4 += 4) {
            const int4 t4 = *reinterpret_cast<const int4 *>(&tot[j][w4]);
            const uint32_t tw[4] = {(uint32_t)t4.x, (uint32_t)t4.y, (uint32_t)t4.z, (uint32_t)t4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                before += (w4 + u < wave) ? tw[u] : 0u;
                all += tw[u];
            }
        }
        const int cnt = round_count(j);
        uint32_t my = base + before + (uint32_t)(wave_scan_incl(cnt) - cnt);
        const int p0 = 4 * (j * SR_NT + tid);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int gt = (int)(my & 0xffffu), eq = (int)(my >> 16);
            if (q[j][c] > tau) {
                staged[gt + min(eq, need)] = p0 + c;
                my += 1u;
            } else if (q[j][c] == tau) {
                if (eq < need) staged[gt + eq] = p0 + c;
                my += 0x10000u;
            }
        }
        base += all;
    }
    lds_barrier();
    if ((k & 3) == 0) {
        for (int j = 4 * tid; j < k; j += 4 * SR_NT)
            *reinterpret_cast<u32x4 *>(out + j) = *reinterpret_cast<const u32x4 *>(staged + j);
    } else {
        for (int j = tid; j < k; j += SR_NT) out[j] = staged[j];
    }
}

hipError_t launch_index_topk(const float *scores, int rows, int L, long ld, const int32_t *lens, int k, int tail,
                             int32_t *idx, hipStream_t st)
{
    if (rows == 0) return hipSuccess;
    // more rows than CUs: the register-key kernel; otherwise one workgroup
    // per CU (the key cache fills most of a CU's LDS), each walking its
    // share of the rows
    if (rows > SEL_REG_MIN_ROWS) {
        // two rows in flight per CU (64 rows: 28.2 us here against 24.4 us
        // for one cached-row workgroup per CU, each row's latency deciding)
        index_topk_reg_kernel<<<rows, SR_NT, 0, st>>>(scores, L, ld, lens, k, tail, idx);
    } else {
        const int grid = min(rows, 256);
        index_topk_kernel<<<grid, SEL_NT, 0, st>>>(scores, rows, L, ld, lens, k, tail, idx);
    }
    if (L > SEL_CAP && L > k) index_topk_long_kernel<<<rows, SEL_NT, 0, st>>>(scores, L, ld, lens, k, tail, idx);
    return hipGetLastError();
}

}  // namespace coli
