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
// bf16 path: two grouped MFMA GEMMs over a device-built list of
// (expert, first row) tiles -- no host synchronisation is needed to learn the
// per-expert row counts -- and an elementwise combine:
//   1. gate+up over the routed rows AND the shared expert (as expert E with
//      all T tokens), clamped SwiGLU in the epilogue, h in bf16;
//   2. down over the same rows: routed rows to o in bf16, the shared
//      expert's rows to sx in fp32;
//   3. per token and column, sx plus the routed rows of the token in one
//      fixed fmaf chain (no atomics: bitwise repeatable), plus the residual.
// fp32 path: the same steps with one thread per output value.
#include "device_common.h"
#include "kernels.h"

namespace coli {

// ---------------------------------------------------------------------------
// Tile order.  Every expert with rows is cut into ceil(count/BM) row tiles
// and, per GEMM, into n_nt column tiles: one workgroup per (expert, row tile,
// column tile).  The tiles are numbered expert by expert (routed experts in
// index order, then the shared expert: index E, all T tokens).  Within an
// expert the row tiles are taken in blocks of ROW_BLOCK, and a block's tiles
// are numbered column-tile major, row-tile minor: a block (ROW_BLOCK x n_nt
// tiles) runs together behind one L2 (see xcd_tile), so each weight tile is
// streamed once per block and shared by its row tiles, and each block of
// token rows is fetched once and shared by all column tiles.
//
// Each workgroup finds its own tile from the per-expert row counts (no list
// in memory, no extra launch): every wave scans the counts itself -- lane l
// sums the row tiles of a contiguous run of experts, a wave-wide inclusive
// scan of those sums locates the lane whose run holds the tile, and that
// run is walked -- with shuffles and a ballot only, so no LDS and no
// barrier.  All waves reach the same answer.
// ---------------------------------------------------------------------------
constexpr int ROW_BLOCK = 8;
constexpr int TILE_N = 256;          // columns of a tile in the 256 x 256 and int4 grouped kernels

// q / d for 0 <= q, d < 2^22 without an integer division (whose expansion
// is several times longer): the float quotient from the hardware
// reciprocal is within one of the exact one and is corrected.
__device__ __forceinline__ int small_div(int q, int d)
{
    int i = (int)((float)q * __builtin_amdgcn_rcpf((float)d));
    if (i * d > q) --i;
    else if ((i + 1) * d <= q) ++i;
    return i;
}

// Tile `local` of an expert with `mte` row tiles and `nnt` column tiles ->
// (row tile, column tile) in the block order described above.
__device__ __forceinline__ int2 block_order(int local, int mte, int nnt)
{
    const int per_block = ROW_BLOCK * nnt;
    const int blk = small_div(local, per_block), in = local - blk * per_block;
    const int rows = min(ROW_BLOCK, mte - blk * ROW_BLOCK);   // the last block may be short
    const int ct = small_div(in, rows);
    return make_int2(blk * ROW_BLOCK + in - ct * rows, ct);
}

// XCD-aware block -> tile map.  Workgroups are dispatched to the 8 XCDs
// round-robin (block b runs on XCD b % 8, the blocks of one XCD in order).
// The actual tile count (known only on the device) is split into 8
// contiguous ranges, and the blocks of XCD x take the tiles of range x in
// order, so tiles that share A rows (same rows, neighbouring columns) or B
// rows (same expert and columns, neighbouring rows) run at the same time
// behind the same L2.  The grid is an upper bound; surplus blocks return -1.
__device__ __forceinline__ int xcd_tile(int ntiles)
{
    const int x = blockIdx.x & 7, w = blockIdx.x >> 3;
    const int per = (ntiles + 7) >> 3;
    const int t = x * per + w;
    return (w < per && t < ntiles) ? t : -1;
}

static long xcd_grid(long max_items) { return ((max_items + 7) / 8) * 8; }

// A tile of a grouped kernel: expert e (E: the shared expert; e < 0: no
// tile), its first row m0, column tile ct, the expert's row count and the
// expert's first row in the h / o buffers.
struct ExpertTile {
    int e, m0, ct, cnt, base;
    bool shared;
};

constexpr int FIND_MAX_RUN = 16;     // experts per lane for E <= 1024

// Token of row r of a tile.  The shared expert's rows (and a dense layer's,
// which has no routed rows: R = 0) are the tokens in order; a routed row's
// token comes from the permutation.  Every lane loads its permutation entry
// (a clamped index for the shared expert) and the token is selected, not
// branched on, so the loads of all rows are in flight together.
__device__ __forceinline__ int tile_token(const ExpertTile &et, const int32_t *__restrict__ perm, int r, int R,
                                          int K)
{
    const int p = (R > 0) ? perm[min(et.base + r, R - 1)] : 0;
    return et.shared ? r : p / max(K, 1);
}

// Tile of this block for BM-row tiles and nnt column tiles.  The expert's row
// count and first row come from the same register copy of the counts as the
// search (the first row of expert e is the sum of the counts before it), so
// the tile is known after one round of loads.  R = T * K routed rows.
__device__ __forceinline__ ExpertTile find_tile(const int32_t *__restrict__ count, int E, int T, int R, int BM,
                                                int nnt)
{
    const int lane = threadIdx.x & 63;
    const int run = (E + 63) >> 6;                 // experts per lane
    // all counts are loaded at once (unconditional loads of a clamped index,
    // so no load waits for another); each lane keeps the counts and row
    // tiles of its run
    int cnt[FIND_MAX_RUN];
#pragma unroll
    for (int k = 0; k < FIND_MAX_RUN; ++k) cnt[k] = (E > 0) ? count[min(lane * run + k, E - 1)] : 0;
    int mtk[FIND_MAX_RUN];
    int local = 0, clocal = 0;
#pragma unroll
    for (int k = 0; k < FIND_MAX_RUN; ++k) {
        const int e = lane * run + k;
        if (!(k < run && e < E)) cnt[k] = 0;
        mtk[k] = (cnt[k] + BM - 1) / BM;
        local += mtk[k];
        clocal += cnt[k];
    }
    int incl = local, cincl = clocal;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off), c = __shfl_up(cincl, off);
        if (lane >= off) {
            incl += v;
            cincl += c;
        }
    }
    const int routed = __shfl(incl, 63);
    const int mt_sh = (T + BM - 1) / BM;
    const int t = xcd_tile((routed + mt_sh) * nnt);
    if (t < 0) return ExpertTile{-1, 0, 0, 0, 0, false};
    const int i = t / nnt;                         // row tile index over all experts
    int e = E, mte = mt_sh, first = routed, ecnt = T, base = R;
    if (i < routed) {
        // first lane whose run ends past i (uniform, so its registers are
        // read with readlane)
        const int L = __builtin_ctzll(__ballot(incl > i));
        first = __builtin_amdgcn_readlane(incl - local, L);
        base = __builtin_amdgcn_readlane(cincl - clocal, L);
#pragma unroll
        for (int k = 0; k < FIND_MAX_RUN; ++k) {
            const int m = __builtin_amdgcn_readlane(mtk[k], L);
            const int c = __builtin_amdgcn_readlane(cnt[k], L);
            if (first + m > i) {
                e = L * run + k;
                mte = m;
                ecnt = c;
                break;
            }
            first += m;
            base += c;
        }
    }
    const int2 mn = block_order(t - first * nnt, mte, nnt);
    return ExpertTile{e, mn.x * BM, mn.y, ecnt, base, e == E};
}

// The 256 x 256 kernels run one workgroup per CU, so nothing hides a
// per-tile search there: their tiles come from a list built beforehand by
// one small kernel in the same order.  Each list is cut into 8 contiguous
// per-XCD ranges of equal estimated cost -- a tile costs TILE_COST0 + its
// real rows (the fixed part is the weight stream every tile pays; a 32-row
// tile takes about half as long as a 256-row one) -- and the workgroups of
// XCD x walk range x.  n_items: [0] entries of the down list, [1] of the
// gate+up list, [2..10] gate+up range starts (x = 0..8), [11..19] down.
constexpr int TILE_COST0 = 208;

// Sets starts[0..8] (in LDS): entry q goes to XCD floor(8 * (cost of entries
// before q) / total).
template <class Cost>
__device__ __forceinline__ void xcd_split(int n, Cost &&cost, int32_t *starts)
{
    __shared__ int32_t csum[1024];
    __shared__ int32_t ws[16];
    const int tid = threadIdx.x;
    const int per = (n + 1023) / 1024;
    const int q0 = min(tid * per, n), q1 = min(q0 + per, n);
    int c = 0;
    for (int q = q0; q < q1; ++q) c += cost(q);
    csum[tid] = block_scan_incl_1024(c, ws);
    __syncthreads();
    const long tot = max((long)csum[1023], 1L);
    // floor(8 b / tot) >= x  <=>  b >= ceil(x tot / 8): the XCD of a cost
    // prefix b is the number of these thresholds it reaches (x = 1..7)
    long thr[8];
#pragma unroll
    for (int x = 1; x < 8; ++x) thr[x] = (x * tot + 7) >> 3;
    auto xcd_of = [&](long b) {
        int xq = 0;
#pragma unroll
        for (int x = 1; x < 8; ++x) xq += (b >= thr[x]) ? 1 : 0;
        return xq;
    };
    long before = csum[tid] - c;                  // cost of entries before q0
    // XCD of entry q0 - 1 (-1 for the first entry), so that a boundary on
    // this chunk's first entry is written by this thread
    int prev = -1;
    if (q0 > 0 && q0 < n) prev = xcd_of(before - cost(q0 - 1));
    for (int q = q0; q < q1; ++q) {
        const int xq = xcd_of(before);
        for (int xx = prev + 1; xx <= xq; ++xx) starts[xx] = q;    // first entry of XCD xx
        prev = xq;
        before += cost(q);
    }
    // the thread holding the last entry closes the ranges: XCDs after its
    // XCD are empty and every range ends at n
    if (q0 < q1 && q1 == n)
        for (int xx = prev + 1; xx <= 8; ++xx) starts[xx] = n;
    if (n == 0 && tid == 0)
        for (int xx = 0; xx <= 8; ++xx) starts[xx] = 0;
    __syncthreads();
}

// Two workgroups, one per list (both phases are bound by instruction issue on
// one CU, so the lists are built side by side).  Each reads the counts once;
// the owner of every row tile goes into an LDS table, so each list entry is
// computed from LDS alone, once for its cost, which stays in LDS for the
// split, and once more when it is written to its place after the split.
// Lists longer than the LDS tables recompute entries by binary search and
// keep list order.
constexpr int TILES_LDS_ROWS = 4096;     // row tiles with an owner entry in LDS
constexpr int TILES_LDS_COST = 8192;     // entries per list with a cost in LDS
// The last TAIL_Q entries of every XCD range (about 1.5 per CU) are placed
// in decreasing cost (ties in list order): an XCD's CUs take its range in
// order as they free up, so the range ends on its cheapest tiles instead of
// whichever full tiles the expert order put last (prefill gate+up 339 ->
// 326 us).  Only the tail is sorted: in list order the CUs of an XCD run
// weight-streaming (few-row) and MFMA-bound (full) tiles side by side,
// which keeps both HBM and the matrix cores busy.
constexpr int TAIL_Q = 48;

__global__ __launch_bounds__(1024) void ffn_tiles_kernel(const int32_t *__restrict__ count, int E, int T,
                                                         int R, int nnt_gu, int nnt_dn,
                                                         int4 *__restrict__ list_gu,
                                                         int4 *__restrict__ list_dn,
                                                         int32_t *__restrict__ n_items)
{
    // cnt[e]: rows of expert e; sc[e] = row tiles of routed experts 0..e
    // (inclusive scan); the shared expert's ceil(T/BM) row tiles follow them;
    // first[e]: first row of expert e in h / o (exclusive scan of the counts)
    __shared__ int32_t cnt[1024];
    __shared__ int32_t sc[1024];
    __shared__ int32_t first_s[1024];
    __shared__ int32_t ws[16];
    __shared__ int16_t owner_s[TILES_LDS_ROWS];
    __shared__ int16_t cost_s[TILES_LDS_COST];
    constexpr int BM = BigCfg::BM;
    const int tid = threadIdx.x;
    const int c = (tid < E) ? count[tid] : 0;
    cnt[tid] = c;
    const int mte_t = (c + BM - 1) / BM;
    sc[tid] = block_scan_incl_1024(mte_t, ws);
    __syncthreads();
    first_s[tid] = block_scan_incl_1024(c, ws) - c;
    __syncthreads();
    const int routed = sc[1023];
    const int mt_sh = (T + BM - 1) / BM;
    const bool table = routed <= TILES_LDS_ROWS;
    if (table && tid < E)
        for (int i = sc[tid] - mte_t; i < sc[tid]; ++i) owner_s[i] = (int16_t)tid;
    __syncthreads();
    // entry q of a list with nnt column tiles -> {expert | column tile << 16,
    // first row, rows of the expert, first row of the expert in h / o}
    auto entry = [&](int q, int nnt) {
        const int i = small_div(q, nnt);
        int e = E;
        if (i < routed) {
            if (table) {
                e = owner_s[i];
            } else {                              // the first e with sc[e] > i
                int lo = 0, hi = E - 1;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (sc[mid] > i) hi = mid; else lo = mid + 1;
                }
                e = lo;
            }
        }
        const int mte = (e == E) ? mt_sh : (cnt[e] + BM - 1) / BM;
        const int first = (e == E) ? routed : sc[e] - mte;
        const int2 mn = block_order(q - first * nnt, mte, nnt);
        return (e == E) ? make_int4(e | (mn.y << 16), mn.x * BM, T, R)
                        : make_int4(e | (mn.y << 16), mn.x * BM, cnt[e], first_s[e]);
    };
    auto cost_of = [&](const int4 &en) { return TILE_COST0 + min(BM, en.z - en.y); };
    // workgroup 0 builds the gate+up list, workgroup 1 the down list
    const bool gu = blockIdx.x == 0;
    const int nnt = gu ? nnt_gu : nnt_dn;
    int4 *__restrict__ list = gu ? list_gu : list_dn;
    const int n = (routed + mt_sh) * nnt;
    // every entry is written in list order first (the stores are in flight
    // during the split); a list whose costs all fit in LDS then has the tail
    // of every range rewritten in sorted order (the barriers in between
    // order the two stores of a place)
    const bool sort_tails = n <= TILES_LDS_COST;
    for (int q = tid; q < n; q += 1024) {
        const int4 en = entry(q, nnt);
        list[q] = en;
        if (q < TILES_LDS_COST) cost_s[q] = (int16_t)cost_of(en);
    }
    if (tid == 0) n_items[gu ? 1 : 0] = n;
    __syncthreads();
    __shared__ int32_t starts[9];
    xcd_split(n, [&](int q) { return q < TILES_LDS_COST ? (int)cost_s[q] : cost_of(entry(q, nnt)); }, starts);
    if (tid < 9) n_items[(gu ? 2 : 2 + 9) + tid] = starts[tid];
    if (!sort_tails) return;
    // one thread per tail place (range x = tid / TAIL_Q): the rank of the
    // tail's entry q among its tail -- costlier entries, then earlier equal
    // ones -- from the tail's TAIL_Q costs (the same for all threads of a
    // range, so the LDS reads are broadcasts), and the entry is rewritten
    // only if it moves.  (With every thread walking its own 2-3 list entries
    // the pass issued about 2300 LDS reads on the one CU: prefill list
    // stage 16.4 -> 13.2 us, A/B.)
    if (tid < 8 * TAIL_Q) {
        const int x = tid / TAIL_Q;
        const int s1 = starts[x + 1], s0 = max(starts[x], s1 - TAIL_Q);
        const int q = s1 - TAIL_Q + (tid - x * TAIL_Q);
        if (q >= s0) {
            const int c = cost_s[q];
            int rank = 0;
#pragma unroll
            for (int k = 0; k < TAIL_Q; ++k) {
                const int j = s1 - TAIL_Q + k;
                const int cj = cost_s[max(j, s0)];
                rank += (j >= s0 && (cj > c || (cj == c && j < q))) ? 1 : 0;
            }
            if (s0 + rank != q) list[s0 + rank] = entry(q, nnt);
        }
    }
}

// List entry of the 256 x 256 kernels: {e | ct << 16, m0, cnt, base}.
__device__ __forceinline__ ExpertTile list_tile(const int4 &en, int E)
{
    const int e = en.x & 0xffff;
    return ExpertTile{e, en.y, en.x >> 16, en.z, en.w, e == E};
}

// Gate/up B rows are interleaved in blocks of 32: block b of a 2*FC-row tile
// holds rows f0 + (b >> 1) * 32 .. +31 of gate (b even) or up (b odd), so a
// wave's fragment pair (2j, 2j+1) holds gate and up of the same columns.
// Rows past F (a ragged last tile) reread row F-1; their outputs are dropped.
__device__ __forceinline__ const uint16_t *gateup_b_row(const uint16_t *G, const uint16_t *U, int f0,
                                                        int b, int D, int F)
{
    const int blk = b >> 5;
    const int f = min(f0 + (blk >> 1) * 32 + (b & 31), F - 1);
    return ((blk & 1) ? U : G) + (size_t)f * D;
}
// The same in blocks of 16, for tiles whose waves hold one fragment each:
// rows f0 + (b >> 5) * 16 .. +15 of gate, then the same rows of up, so a
// fragment holds gate of 16 columns in lanes 0..15 and their up 16 lanes above.
__device__ __forceinline__ const uint16_t *gateup_b_row16(const uint16_t *G, const uint16_t *U, int f0,
                                                          int b, int D, int F)
{
    const int f = min(f0 + (b >> 5) * 16 + (b & 15), F - 1);
    return (((b >> 4) & 1) ? U : G) + (size_t)f * D;
}

// Epilogue of the grouped kernels: accumulator element (m, n, i) of a lane is
// tile row r0 + 32 m + 8 (i / 4) + i % 4 (r0 = the lane's first row: its
// wave's first row + 4 (lane / 32)) and column 32 n of the lane's column
// `out` points at.  Each real row's pointer is formed once and the FN values
// stored at immediate offsets.  out_row0: output row of the tile's row 0
// minus et.m0; cols: columns left from the lane's first (later fragments
// are dropped); val(m, n, i): the value to store.
template <int FM, int FN, class T, class Val>
__device__ __forceinline__ void frag_store_rows(const ExpertTile &et, T *out, size_t ld, int out_row0, int r0,
                                                int cols, Val val)
{
    const int rows = et.cnt - et.m0;
    T *const base = out + (size_t)(out_row0 + et.m0) * ld;
#pragma unroll
    for (int m = 0; m < FM; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = r0 + 32 * m + 8 * (i >> 2) + (i & 3);
            if (r < rows) {
                T *row = base + (size_t)r * ld;
#pragma unroll
                for (int n = 0; n < FN; ++n)
                    if (32 * n < cols) row[32 * n] = val(m, n, i);
            }
        }
}

// ---------------------------------------------------------------------------
// 1. gate+up grouped GEMM with the clamped SwiGLU in the epilogue, h in bf16.
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(256) void gateup_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gate, const uint16_t *__restrict__ up,
    const uint16_t *__restrict__ s_gate, const uint16_t *__restrict__ s_up,
    const int32_t *__restrict__ count, const int32_t *__restrict__ perm, int T, int D, int E, int K, int F,
    uint16_t *__restrict__ h)
{
    static_assert(C::FN % 2 == 0 || C::FN == 1, "gate/up fragment pairs, or gate/up halves of one fragment");
    __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_BYTES / 2];
    constexpr int FC = C::BN / 2;                 // output columns per tile
    const ExpertTile et = find_tile(count, E, T, T * K, C::BM, (F + FC - 1) / FC);
    if (et.e < 0) return;
    const int nt = et.ct;
    const uint16_t *G = et.shared ? s_gate : gate + (size_t)et.e * F * D;
    const uint16_t *U = et.shared ? s_up : up + (size_t)et.e * F * D;
    const int f0 = nt * FC;
    const int ch0 = threadIdx.x & 7;

    const uint16_t *ap[C::A_PER_T];
    const uint16_t *bp[C::B_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        // padding rows (past the expert's last row) reread its first row
        int r = et.m0 + a_chunk_row<C>(i);
        if (a_chunk_row<C>(i) >= C::BM || r >= et.cnt) r = et.m0;
        ap[i] = x + (size_t)tile_token(et, perm, r, T * K, K) * D + ch0 * 8;
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i)
        bp[i] = (C::FN == 1 ? gateup_b_row16(G, U, f0, a_chunk_row<C>(i), D, F)
                            : gateup_b_row(G, U, f0, a_chunk_row<C>(i), D, F)) + ch0 * 8;
    f32x16 acc[C::FM][C::FN];
    mfma_mainloop<C>(ap, bp, D, lds, acc);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave % C::WAVES_N, wm = wave / C::WAVES_N;
    if constexpr (C::FN == 1) {
        // lanes 0..15 (32..47) hold gate of h columns fl, the lanes 16 above their up
        float upv[C::FM][16];
#pragma unroll
        for (int m = 0; m < C::FM; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) upv[m][i] = __shfl_xor(acc[m][0][i], 16);
        const int fl = f0 + wn * 16 + (lane & 15);
        frag_store_rows<C::FM, 1>(et, h + fl, (size_t)F, et.base, wm * C::FM * 32 + 4 * (lane >> 5),
                                  (lane & 16) ? 0 : F - fl, [&](int m, int, int i) {
                                      return f32_to_bf16_bits(swiglu_clamped_fast(acc[m][0][i], upv[m][i]));
                                  });
        return;
    }
    // fragment pair (2p, 2p + 1) = gate and up of h columns fl + 32 p
    const int fl = f0 + wn * (C::FN / 2) * 32 + (lane & 31);
    frag_store_rows<C::FM, C::FN / 2>(et, h + fl, (size_t)F, et.base, wm * C::FM * 32 + 4 * (lane >> 5), F - fl,
                                      [&](int m, int p, int i) {
                                          return f32_to_bf16_bits(
                                              swiglu_clamped_fast(acc[m][2 * p][i], acc[m][2 * p + 1][i]));
                                      });
}

// ---------------------------------------------------------------------------
// 2. down grouped GEMM: o[row] = W_down[e] h[row] in bf16 for the routed rows,
//    sx[t] = S_down h[R + t] in fp32 for the shared expert's rows.
// ---------------------------------------------------------------------------

// ksplit > 1 (layers without routed rows only): the reduction over F is cut
// into ksplit equal parts, each a tile of its own, and part s of the shared
// rows' output goes to sx + s * T * D; the combine adds the parts in order.
template <class C>
__global__ __launch_bounds__(256) void down_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ down, const uint16_t *__restrict__ s_down,
    const int32_t *__restrict__ count, int T, int D, int E, int K, int F, int ksplit,
    uint16_t *__restrict__ o, float *__restrict__ sx)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_BYTES / 2];
    const int ncol = (D + C::BN - 1) / C::BN;
    const ExpertTile et = find_tile(count, E, T, T * K, C::BM, ncol * ksplit);
    if (et.e < 0) return;
    const uint16_t *W = et.shared ? s_down : down + (size_t)et.e * D * F;
    const int sp = et.ct / ncol;                     // reduction part (0 unless split)
    const int d0 = (et.ct - sp * ncol) * C::BN;      // the last column tile may be ragged
    const int kl = F / ksplit, k0 = sp * kl;
    const int ch0 = threadIdx.x & 7;

    const uint16_t *ap[C::A_PER_T];
    const uint16_t *bp[C::B_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        const int rr = a_chunk_row<C>(i);
        const int r = (rr < C::BM && et.m0 + rr < et.cnt) ? et.m0 + rr : et.m0;
        ap[i] = h + (size_t)(et.base + r) * F + k0 + ch0 * 8;
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        const int d = min(d0 + a_chunk_row<C>(i), D - 1);    // rows past D reread the last one
        bp[i] = W + (size_t)d * F + k0 + ch0 * 8;
    }
    f32x16 acc[C::FM][C::FN];
    mfma_mainloop<C>(ap, bp, kl, lds, acc);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave % C::WAVES_N, wm = wave / C::WAVES_N;
    const int dl = d0 + acc_col<C>(wn, 0, lane);
    const int r0 = wm * C::FM * 32 + 4 * (lane >> 5);
    if (et.shared)
        frag_store_rows<C::FM, C::FN>(et, sx + (size_t)sp * T * D + dl, (size_t)D, 0, r0, D - dl,
                                      [&](int m, int n, int i) { return acc[m][n][i]; });
    else
        frag_store_rows<C::FM, C::FN>(et, o + dl, (size_t)D, et.base, r0, D - dl,
                                      [&](int m, int n, int i) { return f32_to_bf16_bits(acc[m][n][i]); });
}

// ---------------------------------------------------------------------------
// 1/2 on the large-tile engine (row-heavy batches): 256 x 256 tiles, eight
// waves.  A tile with at most 64 real rows runs the engine's streaming mode;
// otherwise each wave runs the variant for its number of real 32-row
// fragments.
// ---------------------------------------------------------------------------
constexpr int BIG_LDS_BYTES = (BigCfg::LDS_BYTES > StreamCfg::LDS_BYTES) ? BigCfg::LDS_BYTES : StreamCfg::LDS_BYTES;
using StreamRows = BigCfgT<64, 2>;                // copy layout of the streaming mode's rows
__device__ __forceinline__ int big_wave_fragments(int rows, int wm)
{
    return min(max((rows - wm * 64 + 31) >> 5, 0), 2);
}

// Epilogue of the 256 x 256 down tiles: accumulator element (m, n, i) of a
// lane is tile row wm * 64 + m * 32 + 8 (i / 4) + 4 (lane / 32) + i % 4 and
// column 32 n of the lane's column `out` points at; each real row's pointer
// is formed once and its FN values stored at immediate offsets.  out_row0:
// the output row of the tile's first row minus et.m0; cols: columns left
// from the lane's first (fragments at or past it are dropped); full: every
// row and column of the tile real (the same for all lanes, so the wave takes
// one branch).
template <int NFW, class T, class Cvt>
__device__ __forceinline__ void big_store_rows(const f32x16 (&acc)[BigCfg::FM][BigCfg::FN], const ExpertTile &et,
                                               T *out, size_t ld, int out_row0, int cols, bool full, int w, Cvt cvt)
{
    const int lane = threadIdx.x & 63, wm = w >> 1;
    const int rows = et.cnt - et.m0;
    const int r0 = wm * 64 + 4 * (lane >> 5);
    T *const base = out + (size_t)(out_row0 + et.m0) * ld;
    if (full) {                                   // no checks
#pragma unroll
        for (int m = 0; m < NFW; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                T *row = base + (size_t)(r0 + m * 32 + 8 * (i >> 2) + (i & 3)) * ld;
#pragma unroll
                for (int n = 0; n < BigCfg::FN; ++n) row[32 * n] = cvt(acc[m][n][i]);
            }
        return;
    }
#pragma unroll
    for (int m = 0; m < NFW; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = r0 + m * 32 + 8 * (i >> 2) + (i & 3);
            if (r < rows) {
                T *row = base + (size_t)r * ld;
#pragma unroll
                for (int n = 0; n < BigCfg::FN; ++n)
                    if (32 * n < cols) row[32 * n] = cvt(acc[m][n][i]);
            }
        }
}

template <int NFW>
__device__ __forceinline__ void gateup_big_body(const uint16_t *const (&rp)[BigCfg::CPW], const ExpertTile &et,
                                                int f0, int D, int F, int w, char *lds,
                                                uint16_t *__restrict__ h)
{
    f32x16 acc[BigCfg::FM][BigCfg::FN];
    big_mainloop<BigCfg, NFW>(rp, D, min(et.cnt - et.m0, BigCfg::BM), w, lds, acc);
    const int lane = threadIdx.x & 63, wm = w >> 1, wn = w & 1;
    // fragment pair (n, n + 1) = gate and up of h columns fl + 16 n
    const int fl = f0 + wn * 64 + (lane & 31);
    const int rows = et.cnt - et.m0;
    const int r0 = wm * 64 + 4 * (lane >> 5);
#pragma unroll
    for (int m = 0; m < NFW; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = r0 + m * 32 + 8 * (i >> 2) + (i & 3);
            if (r < rows) {
                uint16_t *row = h + (size_t)(et.base + et.m0 + r) * F + fl;
#pragma unroll
                for (int n = 0; n < BigCfg::FN; n += 2)
                    if (16 * n < F - fl) row[16 * n] = f32_to_bf16_bits(swiglu_clamped_fast(acc[m][n][i], acc[m][n + 1][i]));
            }
        }
}

__device__ __forceinline__ void gateup_big_tile(
    const ExpertTile &et, const uint16_t *__restrict__ x, const uint16_t *__restrict__ gate,
    const uint16_t *__restrict__ up, const uint16_t *__restrict__ s_gate, const uint16_t *__restrict__ s_up,
    const int32_t *__restrict__ perm, int T, int D, int K, int F, char *lds, uint16_t *__restrict__ h)
{
    const int R = T * K;
    const uint16_t *G = et.shared ? s_gate : gate + (size_t)et.e * F * D;
    const uint16_t *U = et.shared ? s_up : up + (size_t)et.e * F * D;
    const int f0 = et.ct * (BigCfg::BN / 2);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (et.cnt - et.m0 <= StreamCfg::A_ROWS) {
        using S = StreamRows;
        const int row = stream_a_row(w);
        const int r = (et.m0 + row < et.cnt) ? et.m0 + row : et.m0;
        const uint16_t *ra = x + (size_t)tile_token(et, perm, r, R, K) * D + big_copy_chunk<S>(row) * 8;
        const uint16_t *rb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int br = big_copy_row<S>(j, w);
            rb[j] = gateup_b_row(G, U, f0, br, D, F) + big_copy_chunk<S>(br) * 8;
        }
        f32x16 acc[4];
        stream_mainloop(ra, rb, D, et.cnt - et.m0, w, lds, acc);
        if ((w >> 2) != 0) return;
        // fragment pair (2p, 2p + 1) = gate and up of h columns fl + 32 p
        const int fl = f0 + (w & 1) * 64 + (threadIdx.x & 31);
        frag_store_rows<1, 2>(et, h + fl, (size_t)F, et.base, 32 * (w >> 1) + 4 * ((threadIdx.x & 63) >> 5), F - fl,
                              [&](int, int p, int i) {
                                  return f32_to_bf16_bits(swiglu_clamped_fast(acc[2 * p][i], acc[2 * p + 1][i]));
                              });
        return;
    }
    const uint16_t *rp[BigCfg::CPW];
#pragma unroll
    for (int j = 0; j < BigCfg::CPO; ++j) {
        const int row = big_copy_row<BigCfg>(j, w);
        const int ch = big_copy_chunk<BigCfg>(row);
        int r = et.m0 + row;                      // padding rows reread the tile's first row
        if (r >= et.cnt) r = et.m0;
        rp[j] = x + (size_t)tile_token(et, perm, r, R, K) * D + ch * 8;
        rp[BigCfg::CPO + j] = gateup_b_row(G, U, f0, row, D, F) + ch * 8;
    }
    const int nfw = big_wave_fragments(et.cnt - et.m0, w >> 1);
    if (nfw == 2) gateup_big_body<2>(rp, et, f0, D, F, w, lds, h);
    else if (nfw == 1) gateup_big_body<1>(rp, et, f0, D, F, w, lds, h);
    else gateup_big_body<0>(rp, et, f0, D, F, w, lds, h);
}

template <int NFW>
__device__ __forceinline__ void down_big_body(const uint16_t *const (&rp)[BigCfg::CPW], const ExpertTile &et,
                                              int d0, int D, int kl, int w, char *lds,
                                              uint16_t *__restrict__ o, float *__restrict__ sx)
{
    f32x16 acc[BigCfg::FM][BigCfg::FN];
    big_mainloop<BigCfg, NFW>(rp, kl, min(et.cnt - et.m0, BigCfg::BM), w, lds, acc);
    const int lane = threadIdx.x & 63, wn = w & 1;
    const int dl = d0 + wn * BigCfg::FN * 32 + (lane & 31);   // column of fragment n: dl + 32 n
    const bool full = et.cnt - et.m0 >= BigCfg::BM && d0 + BigCfg::BN <= D;
    if (et.shared) big_store_rows<NFW>(acc, et, sx + dl, (size_t)D, 0, D - dl, full, w, [](float v) { return v; });
    else big_store_rows<NFW>(acc, et, o + dl, (size_t)D, et.base, D - dl, full, w,
                             [](float v) { return f32_to_bf16_bits(v); });
}

// k0, kl: the part of the reduction over F this tile covers (all of it but
// for layers without routed rows, whose parts write their own slices of sx).
__device__ __forceinline__ void down_big_tile(
    const ExpertTile &et, const uint16_t *__restrict__ h, const uint16_t *__restrict__ down,
    const uint16_t *__restrict__ s_down, int D, int F, int k0, int kl, char *lds, uint16_t *__restrict__ o,
    float *__restrict__ sx)
{
    const int d0 = et.ct * BigCfg::BN;
    const uint16_t *W = (et.shared ? s_down : down + (size_t)et.e * D * F) + k0;
    h += k0;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (et.cnt - et.m0 <= StreamCfg::A_ROWS) {
        using S = StreamRows;
        const int row = stream_a_row(w);
        const int r = (et.m0 + row < et.cnt) ? et.m0 + row : et.m0;
        const uint16_t *ra = h + (size_t)(et.base + r) * F + big_copy_chunk<S>(row) * 8;
        const uint16_t *rb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int br = big_copy_row<S>(j, w);
            rb[j] = W + (size_t)min(d0 + br, D - 1) * F + big_copy_chunk<S>(br) * 8;
        }
        f32x16 acc[4];
        stream_mainloop(ra, rb, kl, et.cnt - et.m0, w, lds, acc);
        if ((w >> 2) != 0) return;
        const int dl = d0 + (w & 1) * 128 + (threadIdx.x & 31);
        if (et.shared)
            frag_store_rows<1, 4>(et, sx + dl, (size_t)D, 0, 32 * (w >> 1) + 4 * ((threadIdx.x & 63) >> 5), D - dl,
                                  [&](int, int n, int i) { return acc[n][i]; });
        else
            frag_store_rows<1, 4>(et, o + dl, (size_t)D, et.base, 32 * (w >> 1) + 4 * ((threadIdx.x & 63) >> 5), D - dl,
                                  [&](int, int n, int i) { return f32_to_bf16_bits(acc[n][i]); });
        return;
    }
    const uint16_t *rp[BigCfg::CPW];
#pragma unroll
    for (int j = 0; j < BigCfg::CPO; ++j) {
        const int row = big_copy_row<BigCfg>(j, w);
        const int ch = big_copy_chunk<BigCfg>(row);
        int r = et.m0 + row;
        if (r >= et.cnt) r = et.m0;
        rp[j] = h + (size_t)(et.base + r) * F + ch * 8;
        const int d = min(d0 + row, D - 1);       // rows past D reread the last one
        rp[BigCfg::CPO + j] = W + (size_t)d * F + ch * 8;
    }
    const int nfw = big_wave_fragments(et.cnt - et.m0, w >> 1);
    if (nfw == 2) down_big_body<2>(rp, et, d0, D, kl, w, lds, o, sx);
    else if (nfw == 1) down_big_body<1>(rp, et, d0, D, kl, w, lds, o, sx);
    else down_big_body<0>(rp, et, d0, D, kl, w, lds, o, sx);
}

// Between two tiles of a workgroup: every wave has finished reading LDS
// (its LDS reads have returned) before any wave's copies of the next tile
// overwrite it.  The epilogue's global stores need not have completed, so
// this is a bare barrier rather than __syncthreads(), which also waits for
// them.
__device__ __forceinline__ void tile_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup (x = blockIdx % 8, its XCD) walks range x of the list with a
// stride of gridDim / 8 workgroups.
__global__ __launch_bounds__(512) void gateup_big_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gate, const uint16_t *__restrict__ up,
    const uint16_t *__restrict__ s_gate, const uint16_t *__restrict__ s_up, const int32_t *__restrict__ perm,
    const int4 *__restrict__ list, const int32_t *__restrict__ n_items, int T, int D, int E, int K, int F,
    uint16_t *__restrict__ h)
{
    __shared__ __attribute__((aligned(1024))) char lds[BIG_LDS_BYTES];
    const int xc = blockIdx.x & 7;
    const int beg = max(n_items[2 + xc], 0), end = min(n_items[2 + xc + 1], n_items[1]);
    for (int t = beg + (blockIdx.x >> 3); t < end; t += gridDim.x >> 3) {
        gateup_big_tile(list_tile(list[t], E), x, gate, up, s_gate, s_up, perm, T, D, K, F, lds, h);
        tile_barrier();
    }
}

// ksplit > 1 (layers without routed rows only): the list's column tiles run
// over ncol * ksplit, tile c covering columns (c % ncol) and part c / ncol of
// the reduction, whose sums go to slice c / ncol of sx.
__global__ __launch_bounds__(512) void down_big_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ down, const uint16_t *__restrict__ s_down,
    const int4 *__restrict__ list, const int32_t *__restrict__ n_items, int T, int D, int E, int F, int ksplit,
    uint16_t *__restrict__ o, float *__restrict__ sx)
{
    __shared__ __attribute__((aligned(1024))) char lds[BIG_LDS_BYTES];
    const int xc = blockIdx.x & 7;
    const int beg = max(n_items[11 + xc], 0), end = min(n_items[11 + xc + 1], n_items[0]);
    const int ncol = (D + BigCfg::BN - 1) / BigCfg::BN, kl = F / ksplit;
    for (int t = beg + (blockIdx.x >> 3); t < end; t += gridDim.x >> 3) {
        ExpertTile et = list_tile(list[t], E);
        const int sp = et.ct / ncol;
        et.ct -= sp * ncol;
        down_big_tile(et, h, down, s_down, D, F, sp * kl, kl, lds, o, sx + (size_t)sp * T * D);
        tile_barrier();
    }
}

// ---------------------------------------------------------------------------
// 1'/2'. int4 routed experts: the same grouped GEMMs on the int4 engine
// (weights dequantised from LDS as their fragments are read).  The shared
// expert (bf16) shares the launches: its tiles run the engine's bf16 mode on
// x and on its hidden rows in bf16, exactly the arithmetic of the bf16
// layer.  The routed experts' A operands are fp16 in the engine's chunk
// order: x16 (written by x_to_f16_kernel) and h16 (written by the gate+up
// kernel in that order; the shared expert's rows of the same buffer hold
// bf16 in natural order).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t *__restrict__ x, long n8,
                                                       uint16_t *__restrict__ x16)
{
    const long q = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n8) return;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(x + q * 8);
    *reinterpret_cast<u32x4 *>(x16 + q * 8) = bf16x8_to_f16x8(v);
}

template <class C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_EU))) void gateup_int4_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ x16, const uint8_t *__restrict__ gate_q, const uint16_t *__restrict__ gate_s,
    const uint8_t *__restrict__ up_q, const uint16_t *__restrict__ up_s, int group,
    const uint16_t *__restrict__ s_gate, const uint16_t *__restrict__ s_up,
    const int32_t *__restrict__ count, const int32_t *__restrict__ perm, int T, int D, int E, int K, int F,
    uint16_t *__restrict__ h16)
{
    static_assert(C::FN % 2 == 0, "gate/up fragment pairs");
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];
    constexpr int FC = C::BN / 2;
    const ExpertTile et = find_tile(count, E, T, T * K, C::BM, (F + TILE_N / 2 - 1) / (TILE_N / 2));
    if (et.e < 0) return;
    const int f0 = et.ct * FC;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int valid = min(et.cnt - et.m0, C::BM);

    // weight row tr of the tile: block tr / 32 holds gate (even) or up (odd)
    // rows f0 + (block / 2) * 32 ..; rows past F read row F - 1
    auto wrow = [&](int tr) { return min(f0 + ((tr >> 5) >> 1) * 32 + (tr & 31), F - 1); };
    const char *brow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tr = (w * 4 + j) * 16 + (lane >> 2);
        const bool upb = (tr >> 5) & 1;
        brow[j] = et.shared
            ? reinterpret_cast<const char *>((upb ? s_up : s_gate) + (size_t)wrow(tr) * D)
            : reinterpret_cast<const char *>((upb ? up_q : gate_q) + ((size_t)et.e * F + wrow(tr)) * (D / 2));
    }
    const uint16_t *arow[C::AROWS];
    f32x16 acc[C::FN];
    if (et.shared) {
#pragma unroll
        for (int u = 0; u < C::AROWS; ++u) arow[u] = x;
        i4_mainloop<C, false>(arow, x + (size_t)et.m0 * D, D, brow, nullptr, group, D, valid, lds, acc);
    } else {
#pragma unroll
        for (int u = 0; u < C::AROWS; ++u) {
            int r = et.m0 + u * 8 + (lane >> 3);      // padding rows read the tile's first row
            if (r >= et.cnt) r = et.m0;
            arow[u] = x16 + (size_t)(perm[et.base + r] / K) * D;
        }
        const int tr = threadIdx.x;
        const uint16_t *srow = (((tr >> 5) & 1) ? up_s : gate_s) + ((size_t)et.e * F + wrow(tr)) * (D / group);
        i4_mainloop<C, true>(arow, nullptr, 0, brow, srow, group, D, valid, lds, acc);
    }

    // routed rows: h16 in fp16, the engine's chunk order -- column f is stored
    // at (f & ~7) + slot(f & 7) (fragment pair (2p, 2p + 1) = columns fo + 32 p;
    // 32 p keeps the chunk slot); the shared expert's rows: bf16, natural order
    const int wn = w % C::WAVES_N, wm = w / C::WAVES_N;
    const int fo = f0 + wn * (C::FN / 2) * 32 + (lane & 31);
    const int r0 = wm * 32 + 4 * (lane >> 5);
    if (et.shared) {
        frag_store_rows<1, C::FN / 2>(et, h16 + fo, (size_t)F, et.base, r0, F - fo, [&](int, int p, int i) {
            return f32_to_bf16_bits(swiglu_clamped_fast(acc[2 * p][i], acc[2 * p + 1][i]));
        });
    } else {
        const int fs = (fo & ~7) + f16_chunk_slot(fo & 7);
        frag_store_rows<1, C::FN / 2>(et, h16 + fs, (size_t)F, et.base, r0, F - fo, [&](int, int p, int i) {
            return __builtin_bit_cast(uint16_t, (_Float16)swiglu_clamped_fast(acc[2 * p][i], acc[2 * p + 1][i]));
        });
    }
}

template <class C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_EU))) void down_int4_kernel(
    const uint16_t *__restrict__ h16, const uint8_t *__restrict__ down_q, const uint16_t *__restrict__ down_s,
    int group, const uint16_t *__restrict__ s_down, const int32_t *__restrict__ count, int T, int D, int E, int K,
    int F, uint16_t *__restrict__ o, float *__restrict__ sx)
{
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];
    const ExpertTile et = find_tile(count, E, T, T * K, C::BM, (D + TILE_N - 1) / TILE_N);
    if (et.e < 0) return;
    const int d0 = et.ct * C::BN;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int valid = min(et.cnt - et.m0, C::BM);

    const char *brow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int d = min(d0 + (w * 4 + j) * 16 + (lane >> 2), D - 1);
        brow[j] = et.shared ? reinterpret_cast<const char *>(s_down + (size_t)d * F)
                            : reinterpret_cast<const char *>(down_q + ((size_t)et.e * D + d) * (F / 2));
    }
    const uint16_t *arow[C::AROWS];
    f32x16 acc[C::FN];
    if (et.shared) {
#pragma unroll
        for (int u = 0; u < C::AROWS; ++u) arow[u] = h16;
        i4_mainloop<C, false>(arow, h16 + (size_t)(et.base + et.m0) * F, F, brow, nullptr, group, F, valid, lds,
                              acc);
    } else {
#pragma unroll
        for (int u = 0; u < C::AROWS; ++u) {
            int r = et.m0 + u * 8 + (lane >> 3);
            if (r >= et.cnt) r = et.m0;
            arow[u] = h16 + (size_t)(et.base + r) * F;
        }
        const int d = min(d0 + (int)threadIdx.x, D - 1);
        i4_mainloop<C, true>(arow, nullptr, 0, brow, down_s + ((size_t)et.e * D + d) * (F / group), group, F,
                             valid, lds, acc);
    }

    const int wn = w % C::WAVES_N, wm = w / C::WAVES_N;
    const int dl = d0 + wn * C::FN * 32 + (lane & 31);
    const int r0 = wm * 32 + 4 * (lane >> 5);
    if (et.shared)
        frag_store_rows<1, C::FN>(et, sx + dl, (size_t)D, 0, r0, D - dl, [&](int, int n, int i) { return acc[n][i]; });
    else
        frag_store_rows<1, C::FN>(et, o + dl, (size_t)D, et.base, r0, D - dl,
                                  [&](int, int n, int i) { return f32_to_bf16_bits(acc[n][i]); });
}

// The gate+up product on the narrow engine (few rows per expert tile): the
// tiles and outputs are those of gateup_int4_kernel; an int4 tile runs one
// pass per 8 of its real rows, and each pass stores its own rows.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(I4NCfg::WAVES_PER_EU))) void gateup_int4n_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ x16, const uint8_t *__restrict__ gate_q, const uint16_t *__restrict__ gate_s,
    const uint8_t *__restrict__ up_q, const uint16_t *__restrict__ up_s,
    const uint16_t *__restrict__ s_gate, const uint16_t *__restrict__ s_up,
    const int32_t *__restrict__ count, const int32_t *__restrict__ perm, int T, int D, int E, int K, int F,
    uint16_t *__restrict__ h16)
{
    using C = I4NCfg;
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];
    constexpr int FC = C::BN / 2;
    const ExpertTile et = find_tile(count, E, T, T * K, C::BM, (F + TILE_N / 2 - 1) / (TILE_N / 2));
    if (et.e < 0) return;
    const int f0 = et.ct * FC;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int valid = min(et.cnt - et.m0, C::BM);

    // weight row tr of the tile: block tr / 32 holds gate (even) or up (odd)
    // rows f0 + (block / 2) * 32 ..; rows past F read row F - 1
    auto wrow = [&](int tr) { return min(f0 + ((tr >> 5) >> 1) * 32 + (tr & 31), F - 1); };
    const char *brow[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int tr = w * 64 + j * 8 + (lane >> 3);
        const bool upb = (tr >> 5) & 1;
        brow[j] = et.shared
            ? reinterpret_cast<const char *>((upb ? s_up : s_gate) + (size_t)wrow(tr) * D)
            : reinterpret_cast<const char *>((upb ? up_q : gate_q) + ((size_t)et.e * F + wrow(tr)) * (D / 2));
    }
    const int fo = f0 + w * (C::FN / 2) * 32 + (lane & 31);
    const int r0 = 4 * (lane >> 5);
    f32x16 acc[C::FN];
    if (et.shared) {
        i4n_mainloop<false>(nullptr, x + (size_t)et.m0 * D, D, brow, nullptr, D, valid, lds, acc);
        frag_store_rows<1, C::FN / 2>(et, h16 + fo, (size_t)F, et.base, r0, F - fo, [&](int, int p, int i) {
            return f32_to_bf16_bits(swiglu_clamped_fast(acc[2 * p][i], acc[2 * p + 1][i]));
        });
        return;
    }
    const int tr = threadIdx.x;
    const uint16_t *srow = (((tr >> 5) & 1) ? up_s : gate_s) + ((size_t)et.e * F + wrow(tr)) * (D / 32);
    const int fs = (fo & ~7) + f16_chunk_slot(fo & 7);
    for (int p0 = 0; p0 < valid; p0 += C::AR) {
        int r = et.m0 + p0 + (lane >> 3);             // this lane's A row of the pass
        if (r >= et.cnt) r = et.m0 + p0;
        const uint16_t *ap = x16 + (size_t)(perm[et.base + r] / K) * D;
        i4n_mainloop<true>(ap, nullptr, 0, brow, srow, D, valid, lds, acc);
        ExpertTile ep = et;
        ep.m0 = et.m0 + p0;
        ep.cnt = min(et.cnt, ep.m0 + C::AR);
        frag_store_rows<1, C::FN / 2>(ep, h16 + fs, (size_t)F, et.base, r0, F - fo, [&](int, int p, int i) {
            return __builtin_bit_cast(uint16_t, (_Float16)swiglu_clamped_fast(acc[2 * p][i], acc[2 * p + 1][i]));
        });
    }
}

// ---------------------------------------------------------------------------
// 3. combine: per token t and column d,
//      v = sx[t][d]; v = fmaf(w_tj, o[inv(t,j)][d], v) for j = 0..K-1;
//      y = residual + v
//    Each thread owns 8 consecutive columns of one token (16-byte loads of
//    the routed rows); every routed row of the token is fetched before the
//    fixed-order sum.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ sx, int nsplit,
                                                      const uint16_t *__restrict__ o,
                                                      const float *__restrict__ w, const int32_t *__restrict__ inv,
                                                      const float *residual, int T, int D, int K, float *y,
                                                      uint16_t *__restrict__ y_bf16)
{
    const int per_row = D / 8;
    const long q = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= (long)T * per_row) return;
    const int t = (int)(q / per_row), d = (int)(q % per_row) * 8;
    // all K row indices and weights, then all K rows, each round of loads in
    // flight together: unconditional loads (slots past K reread slot K - 1;
    // they are not summed), and the empty asm statements take every loaded
    // value before any use, so the compiler cannot sink a load into a branch
    const size_t idx = (size_t)t * D + d;
    const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sx + idx);
    const f32x4 s1 = *reinterpret_cast<const f32x4 *>(sx + idx + 4);
    float v[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    for (int p = 1; p < nsplit; ++p) {            // parts of a split reduction, in order
        const f32x4 q0 = *reinterpret_cast<const f32x4 *>(sx + (size_t)p * T * D + idx);
        const f32x4 q1 = *reinterpret_cast<const f32x4 *>(sx + (size_t)p * T * D + idx + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] += q0[k];
            v[4 + k] += q1[k];
        }
    }
    if (K > 0) {                                  // K = 0: a dense layer, no routed rows
        float wj[8];
        int iv[8];
        u32x4 ov[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const size_t a = (size_t)t * K + min(j, K - 1);
            wj[j] = w[a];
            iv[j] = inv[a];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) ov[j] = *reinterpret_cast<const u32x4 *>(o + (size_t)iv[j] * D + d);
#pragma unroll
        for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(ov[j]));
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < K)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[2 * k] = fmaf(wj[j], __uint_as_float(ov[j][k] << 16), v[2 * k]);
                    v[2 * k + 1] = fmaf(wj[j], __uint_as_float(ov[j][k] & 0xffff0000u), v[2 * k + 1]);
                }
    }
    if (residual) {
        const f32x4 r0 = *reinterpret_cast<const f32x4 *>(residual + idx);
        const f32x4 r1 = *reinterpret_cast<const f32x4 *>(residual + idx + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = r0[k] + v[k];
            v[4 + k] = r1[k] + v[4 + k];
        }
    }
    *reinterpret_cast<f32x4 *>(y + idx) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(y + idx + 4) = f32x4{v[4], v[5], v[6], v[7]};
    if (y_bf16) {
        u32x4 pk;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            pk[k] = (uint32_t)f32_to_bf16_bits(v[2 * k]) | ((uint32_t)f32_to_bf16_bits(v[2 * k + 1]) << 16);
        *reinterpret_cast<u32x4 *>(y_bf16 + idx) = pk;
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
// row-light tiles: gate+up 32 rows x 256 weight rows (128 h columns, two
// workgroups per CU) for batches of at most GU_WIDE_MAX_T tokens that still
// give at least GU_WIDE_MIN_TILES tiles, else 32 x 128 (64 h columns, four
// per CU); down 32 x 128.  Measured A/B on one box, gate+up median: wide
// against narrow 167.0 / 170.9 us at T = 32, 246.8 / 248.3 at T = 64
// (decode), but 298.5 / 285.5 at T = 96, 304.5 / 294.1 at T = 128 and
// 313.9 / 306.1 at T = 256; with few tiles (a dense layer of 64 tokens: 108
// of them) the wide tile leaves CUs idle (dense decode 42 -> 46 us).  The
// same width for down, whose 12-step reductions leave fewer stages in
// flight per CU at two workgroups, was slower (129.8 -> 132.3 us at T = 64).
using SmallGuCfg = TileCfg<32, 128, 1, 4>;
using SmallGuWideCfg = TileCfg<32, 256, 1, 4>;
using SmallDownCfg = TileCfg<32, 128, 1, 4>;
constexpr long GU_WIDE_MIN_TILES = 1024;
constexpr int GU_WIDE_MAX_T = 64;
constexpr int SMALL_BM = SmallGuCfg::BM;
constexpr int I4N_MAX_T = 128;    // int4 batches up to this size run the narrow engine
constexpr int BIG_BM = BigCfg::BM;
static_assert(SmallDownCfg::BM == SMALL_BM && I4Cfg<32>::BM == SMALL_BM, "row-light paths share the tile height");
static_assert(I4Cfg<64>::BN == TILE_N && I4Cfg<32>::BN == TILE_N && BigCfg::BN == TILE_N,
              "the list-driven and int4 paths cut columns alike");

int ffn_tile_rows(int T, int E, int K, int int4)
{
    // a dense layer (K = 0: no experts, T rows of one weight set) takes the
    // 256-row tiles from 512 rows on; otherwise rows per expert on average
    // decides the tile height
    if (K == 0) return T >= 512 ? BIG_BM : SMALL_BM;
    const long R = (long)T * K;
    if (R <= 24L * E) return SMALL_BM;
    return int4 ? I4Cfg<64>::BM : BIG_BM;
}

// Parts of the down projection's reduction for a layer without routed rows
// (E = 0), each part a whole number of 64-wide steps.  Row-light tiles:
// enough tiles to occupy the GPU (up to 1024, four workgroups per CU).
// 256 x 256 tiles (one workgroup per CU): the fewest parts that give every
// CU a tile, since each part adds a T x D slice of fp32 partial sums (at
// most 8; the most parts below that when no count reaches every CU).
int ffn_down_splits(int T, int E, int D, int F, int bm)
{
    if (E != 0) return 1;
    if (bm == SMALL_BM) {
        const long tiles = (long)((T + SMALL_BM - 1) / SMALL_BM) * ((D + SmallDownCfg::BN - 1) / SmallDownCfg::BN);
        int best = 1;
        for (int s = 2; s <= 16; ++s)
            if ((F / 64) % s == 0 && tiles * s <= 1024) best = s;
        return best;
    }
    const long tiles = (long)((T + BIG_BM - 1) / BIG_BM) * ((D + TILE_N - 1) / TILE_N);
    int best = 1;
    for (int s = 1; s <= 8; ++s)
        if ((F / 64) % s == 0) {
            best = s;
            if (tiles * s >= 256) break;
        }
    return best;
}

long ffn_max_tiles(int T, int E, int K, int bm)
{
    const long R = (long)T * K;
    return R / bm + (R < E ? R : E) + (T + bm - 1) / bm;
}

int ffn_col_tiles_gu(int F) { return (F + TILE_N / 2 - 1) / (TILE_N / 2); }
int ffn_col_tiles_dn(int D) { return (D + TILE_N - 1) / TILE_N; }

static void launch_combine(const FfnLaunch &a, StageMarks &mk, hipStream_t st)
{
    const long n = (long)a.T * (a.D / 8);
    mk.mark(st);
    combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
        a.sx, max(a.ksplit, 1), (const uint16_t *)a.o, a.w, a.inv, a.residual, a.T, a.D, a.K, a.y,
        (uint16_t *)a.y_bf16);
    mk.mark(st);
}

template <class C, class CD>
static void launch_staged(const FfnLaunch &a, StageMarks &mk, hipStream_t st)
{
    const long mt = ffn_max_tiles(a.T, a.E, a.K, C::BM);
    const long grid_gu = xcd_grid(mt * ((a.F + C::BN / 2 - 1) / (C::BN / 2)));
    const int ks = max(a.ksplit, 1);
    const long grid_dn = xcd_grid(mt * ((a.D + CD::BN - 1) / CD::BN) * ks);
    mk.mark(st);
    gateup_kernel<C><<<(unsigned)grid_gu, 256, 0, st>>>(
        (const uint16_t *)a.x, (const uint16_t *)a.gate, (const uint16_t *)a.up,
        (const uint16_t *)a.s_gate, (const uint16_t *)a.s_up, a.count, a.perm,
        a.T, a.D, a.E, a.K, a.F, (uint16_t *)a.h);
    mk.mark(st);
    down_kernel<CD><<<(unsigned)grid_dn, 256, 0, st>>>(
        (const uint16_t *)a.h, (const uint16_t *)a.down, (const uint16_t *)a.s_down, a.count,
        a.T, a.D, a.E, a.K, a.F, ks, (uint16_t *)a.o, a.sx);
    launch_combine(a, mk, st);
}

static void launch_big(const FfnLaunch &a, StageMarks &mk, hipStream_t st)
{
    const long mt = ffn_max_tiles(a.T, a.E, a.K, BigCfg::BM);
    const long grid_gu = xcd_grid(mt * ffn_col_tiles_gu(a.F));
    const int ks = max(a.ksplit, 1);
    const long grid_dn = xcd_grid(mt * ffn_col_tiles_dn(a.D) * ks);
    ffn_tiles_kernel<<<2, 1024, 0, st>>>(a.count, a.E, a.T, a.T * a.K, ffn_col_tiles_gu(a.F),
                                         ffn_col_tiles_dn(a.D) * ks, a.list_gu, a.list_dn, a.n_items);
    mk.mark(st);                                     // the gate+up stage is its kernel alone
    gateup_big_kernel<<<(unsigned)grid_gu, BigCfg::NT, 0, st>>>(
        (const uint16_t *)a.x, (const uint16_t *)a.gate, (const uint16_t *)a.up,
        (const uint16_t *)a.s_gate, (const uint16_t *)a.s_up, a.perm, a.list_gu, a.n_items,
        a.T, a.D, a.E, a.K, a.F, (uint16_t *)a.h);
    mk.mark(st);
    down_big_kernel<<<(unsigned)grid_dn, BigCfg::NT, 0, st>>>(
        (const uint16_t *)a.h, (const uint16_t *)a.down, (const uint16_t *)a.s_down, a.list_dn,
        a.n_items, a.T, a.D, a.E, a.F, ks, (uint16_t *)a.o, a.sx);
    launch_combine(a, mk, st);
}

template <class C>
static void launch_staged_int4(const FfnLaunch &a, StageMarks &mk, hipStream_t st)
{
    const long mt = ffn_max_tiles(a.T, a.E, a.K, C::BM);
    const long grid_gu = xcd_grid(mt * ffn_col_tiles_gu(a.F));
    const long grid_dn = xcd_grid(mt * ffn_col_tiles_dn(a.D));
    const long n8 = (long)a.T * a.D / 8;
    x_to_f16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>((const uint16_t *)a.x, n8, a.x16);
    mk.mark(st);                                     // the gate+up stage is its kernel alone
    gateup_int4_kernel<C><<<(unsigned)grid_gu, 256, 0, st>>>(
        (const uint16_t *)a.x, a.x16, a.gate_q, a.gate_s, a.up_q, a.up_s, a.group,
        (const uint16_t *)a.s_gate, (const uint16_t *)a.s_up, a.count, a.perm,
        a.T, a.D, a.E, a.K, a.F, (uint16_t *)a.h);
    mk.mark(st);
    down_int4_kernel<C><<<(unsigned)grid_dn, 256, 0, st>>>(
        (const uint16_t *)a.h, a.down_q, a.down_s, a.group, (const uint16_t *)a.s_down, a.count,
        a.T, a.D, a.E, a.K, a.F, (uint16_t *)a.o, a.sx);
    launch_combine(a, mk, st);
}

static void launch_narrow_int4(const FfnLaunch &a, StageMarks &mk, hipStream_t st)
{
    using C = I4NCfg;
    static_assert(C::BM == I4Cfg<32>::BM, "the narrow gate+up and the staged down share the tiles");
    const long mt = ffn_max_tiles(a.T, a.E, a.K, C::BM);
    const long grid_gu = xcd_grid(mt * ffn_col_tiles_gu(a.F));
    const long grid_dn = xcd_grid(mt * ffn_col_tiles_dn(a.D));
    const long n8 = (long)a.T * a.D / 8;
    x_to_f16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>((const uint16_t *)a.x, n8, a.x16);
    mk.mark(st);                                     // the gate+up stage is its kernel alone
    gateup_int4n_kernel<<<(unsigned)grid_gu, 256, 0, st>>>(
        (const uint16_t *)a.x, a.x16, a.gate_q, a.gate_s, a.up_q, a.up_s,
        (const uint16_t *)a.s_gate, (const uint16_t *)a.s_up, a.count, a.perm,
        a.T, a.D, a.E, a.K, a.F, (uint16_t *)a.h);
    mk.mark(st);
    // the down product stays on the staged engine (same tiles, same h16
    // layout), which was measured as fast or faster for these batches
    down_int4_kernel<I4Cfg<32>><<<(unsigned)grid_dn, 256, 0, st>>>(
        (const uint16_t *)a.h, a.down_q, a.down_s, a.group, (const uint16_t *)a.s_down, a.count,
        a.T, a.D, a.E, a.K, a.F, (uint16_t *)a.o, a.sx);
    launch_combine(a, mk, st);
}

hipError_t launch_ffn(const FfnLaunch &a, hipStream_t st)
{
    const int T = a.T, D = a.D, K = a.K, F = a.F;
    const int R = T * K;
    StageMarks none;
    StageMarks &mk = a.marks ? *a.marks : none;
    if (a.bf16) {
        if (a.use_int4) {
            if (a.bm == SMALL_BM && a.T <= I4N_MAX_T && i4n_fits(a.D, a.group))
                launch_narrow_int4(a, mk, st);
            else if (a.bm == SMALL_BM)
                launch_staged_int4<I4Cfg<32>>(a, mk, st);
            else
                launch_staged_int4<I4Cfg<64>>(a, mk, st);
        } else if (a.bm == SMALL_BM) {
            // tile count bound: row tiles (at most) x column tiles of the wide tile
            const long wide_tiles = ffn_max_tiles(a.T, a.E, a.K, SMALL_BM) *
                                    ((a.F + SmallGuWideCfg::BN / 2 - 1) / (SmallGuWideCfg::BN / 2));
            if (a.T <= GU_WIDE_MAX_T && wide_tiles >= GU_WIDE_MIN_TILES)
                launch_staged<SmallGuWideCfg, SmallDownCfg>(a, mk, st);
            else launch_staged<SmallGuCfg, SmallDownCfg>(a, mk, st);
        } else {
            launch_big(a, mk, st);
        }
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
