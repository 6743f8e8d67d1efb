// layout.hip -- dispatch layout: counts, alignment-padded expert offsets and a
// stable expert-grouped row for every (token, k) routing entry.
//
// What is computed (Normal Mode API page, dispatch Parameters / Return
// Values; EPBatchManager page, ep_dispatch() Returns; CANN
// aclnnMoeDistributeDispatchV2 page, Constraint 1, results are deterministic):
//   c[e]        = number of entries with topk_idx == e
//   off[e]      = sum over e' < e of ceil(c[e'] / a) * a
//   row(t, k)   = off[e] + #{ (t', k') : idx[t', k'] == e, t'K + k' < tK + k }
//   recv_src    = inverse of row (-1 on padding / unused rows)
//   is_token_in_rank[t, r], num_tokens_per_rank[r]  with rank(e) = e / (E / R)
//
// Design (gfx950, wave64): a small batch (at most kSingleLayoutMaxEntries
// entries) is laid out by layout_single_kernel, one workgroup and one launch
// (below).  Larger batches are split into chunks of whole tokens, one
// workgroup per chunk, in two launches:
//   layout_count_kernel: each wave takes a contiguous run of the chunk's
//     entries in flat (token, k) order.  Lanes holding the same expert are
//     found with one ballot per key bit; the lowest of them writes the
//     group's size into the wave's LDS count for that expert (one writer, no
//     atomics).  The exclusive prefix of those counts over the waves gives
//     each wave's base, so base + position among equal keys (a masked
//     popcount) is the entry's stable rank within the chunk.  The kernel
//     stores it in token_row packed with the expert, (e << 16) | rank, and
//     writes the chunk's expert totals as one row of a [chunks][E] table.
//     The same pass marks token x rank membership in LDS and writes the
//     is_token_in_rank rows.
//   layout_rank_kernel: every workgroup re-derives the expert totals and its
//     own chunk base from the small [chunks][E] table, scans the aligned
//     totals in one wave, and turns each packed entry of its chunk into the
//     row off[e] + (entries of e in earlier chunks) + rank.  Ranks come from
//     prefix sums only (never from atomic return order), which makes the
//     result deterministic.
// When many ranks force many small chunks, the table is large (from
// kLayoutScanMinCells cells on) and layout_scan_kernel runs between the two:
// it forms the column prefix sums and the totals once, and each rank
// workgroup reads its own prefix row and the totals instead.
#include "device_common.h"
#include "launch.h"

#include "../../include/moe_dispatch_combine.h"

namespace moe {

constexpr int kRankThreads = 1024;
constexpr int kRankWaves = kRankThreads / kWave;
constexpr int kIdxPerThread = kMaxChunkEntries / 1024; // topk_idx entries prefetched per thread
constexpr int kRankCellsPerThread = 2; // per-chunk rank counts prefetched per thread
constexpr int kRankSumSlots = 512;     // ranks one workgroup can sum (R <= 512)
constexpr int kTabRows = 16;           // expert-table rows prefetched per thread

static_assert(kRankThreads == 1024, "prefetch sizes assume 1024 threads");

// Workgroup size of the count kernel for chunks of at most `ne_max` entries:
// one entry per thread up to 1024 entries (a wave per 64 entries, at least
// four waves), 1024 threads and several entries per thread beyond.  Extra
// idle waves only lengthen the launch of the 64-odd workgroups.
inline int count_threads(int ne_max)
{
    const int t = (ne_max + kWave - 1) / kWave * kWave;
    return t <= 256 ? 256 : t <= 512 ? 512 : 1024;
}
static_assert(kMaxChunkEntries <= 65536 && MOE_MAX_EXPERTS <= 32768,
              "packed (expert << 16 | rank) entries between the count and rank kernels");

// Issue this chunk's topk_idx loads (one per thread and pass of 1024 entries;
// the pass guard is uniform over the workgroup, the index clamped into range).
__device__ __forceinline__ void prefetch_idx(const int64_t *__restrict__ topk_idx, int64_t base,
                                             int ne, int64_t (&reg)[kIdxPerThread])
{
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u)
        reg[u] = u * 1024 < ne ? topk_idx[base + min((int)threadIdx.x + u * 1024, ne - 1)] : -1;
}

// Exclusive prefix over the 16 lanes of each lane group of 16 (width-16
// shuffles); returns the exclusive value, *total gets the group's sum.
__device__ __forceinline__ int exclusive_scan16(int v, int *total)
{
    int incl = v;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
        const int u = __shfl_up(incl, d, 16);
        if ((threadIdx.x & 15) >= d)
            incl += u;
    }
    *total = __shfl(incl, 15, 16);
    return incl - v;
}

template <int THREADS>
__global__ __launch_bounds__(THREADS) void layout_count_kernel(
    const int64_t *__restrict__ topk_idx, int T, int K, int E, int R, int L, int tpc, int nbits,
    int32_t *__restrict__ itr, int32_t *__restrict__ cnt_tab, int32_t *__restrict__ rank_tab,
    int32_t *__restrict__ flag_tab, int32_t *__restrict__ token_row)
{
    constexpr int kCountThreads = THREADS;
    constexpr int kCountWaves = THREADS / kWave;
    // a chunk's entries fit in kIdxPerThread vectors per wave (count_threads)
    __shared__ int s_w[kCountWaves * MOE_MAX_EXPERTS]; // [wave][e], row stride E
    __shared__ int s_rcnt[MOE_MAX_EXPERTS];
    __shared__ uint8_t s_flags[kMaxChunkFlags];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int chunk = blockIdx.x;
    const int t0 = chunk * tpc;
    const int nt = min(tpc, T - t0); // >= 1: chunks cover [0, T) and T > 0 on this path
    const int ne = nt * K;
    const int64_t base = (int64_t)t0 * K;

    // Each wave owns a contiguous run of entries in flat (token, k) order,
    // at most kIdxPerThread vectors of 64; the ids are loaded at once (index
    // clamped into the chunk, entries past the run masked afterwards).
    const int per_wave = ((ne + kCountThreads - 1) / kCountThreads) * kWave;
    const int w_lo = wave * per_wave;
    const int w_hi = min(ne, w_lo + per_wave);
    int64_t idx_reg[kIdxPerThread];
#pragma unroll
    for (int it = 0; it < kIdxPerThread; ++it)
        idx_reg[it] = it * kWave < per_wave ? topk_idx[base + min(w_lo + it * kWave + lane, ne - 1)] : -1;

    for (int i = tid; i < kCountWaves * E; i += kCountThreads)
        s_w[i] = 0;
    for (int i = tid; i < R; i += kCountThreads)
        s_rcnt[i] = 0;
    for (int i = tid; i < nt * R; i += kCountThreads)
        s_flags[i] = 0;
    if (tid == 0)
        s_bad = 0;
    __syncthreads();

    // per-wave expert counts: lanes holding the same expert are matched by
    // one ballot per key bit and the lowest of them adds the group's size
    // (one writer per (wave, expert) and vector; a wave's vectors are in
    // program order).  Each lane keeps its expert, its position among the
    // equal keys of its vector and their number (below | count << 8) in
    // registers for the ranking below.
    int e_reg[kIdxPerThread];
    int pos_reg[kIdxPerThread];
    int bad = 0;
#pragma unroll
    for (int it = 0; it < kIdxPerThread; ++it) {
        e_reg[it] = -1;
        pos_reg[it] = 0;
        if (it * kWave < per_wave) { // uniform: ballots below stay convergent
            const int j = w_lo + it * kWave + lane;
            int e = -1;
            if (j < w_hi) {
                const int64_t v = idx_reg[it];
                if (v < -1 || v >= E)
                    bad = 1;
                else
                    e = (int)v;
            }
            const bool has = e >= 0;
            const uint64_t same = match_same_key(e, has, nbits);
            const int below = count_below(same);
            const int n = __popcll(same);
            if (has) {
                if (below == 0)
                    s_w[wave * E + e] += n;
                s_flags[(j / K) * R + e / L] = 1;
            }
            e_reg[it] = e;
            pos_reg[it] = below | (n << 8);
        }
    }
    if (bad)
        atomicOr(&s_bad, 1);
    __syncthreads();

    // every expert's count over the chunk (one table row) and the exclusive
    // prefix of the per-wave counts in wave order: the base of each wave's
    // entries among the chunk's entries of that expert
    const int Ep = (E + 3) & ~3; // table rows padded to whole 16-byte vectors
    for (int e = tid; e < Ep; e += kCountThreads) {
        int run = 0;
        if (e < E) {
#pragma unroll
            for (int w = 0; w < kCountWaves; ++w) {
                const int v = s_w[w * E + e];
                s_w[w * E + e] = run;
                run += v;
            }
        }
        cnt_tab[(int64_t)chunk * Ep + e] = run;
    }

    // is_token_in_rank rows and per-rank token counts: thread (r, part) owns
    // rank r of tokens part, part + parts, ...; a wave's stores cover
    // consecutive (token, rank) cells, and each thread adds its count once
    {
        int32_t *itr_chunk = itr + (int64_t)t0 * R;
        if (R <= kCountThreads) {
            const int parts = kCountThreads / R;
            if (tid < parts * R) {
                const int r = tid % R;
                const int part = tid / R;
                int cnt = 0;
                for (int t = part; t < nt; t += parts) {
                    const int f = s_flags[t * R + r];
                    itr_chunk[t * R + r] = f;
                    cnt += f;
                }
                if (cnt)
                    atomicAdd(&s_rcnt[r], cnt);
            }
        } else { // more ranks than threads: thread tid owns ranks tid, tid + THREADS, ...
            for (int r = tid; r < R; r += kCountThreads) {
                int cnt = 0;
                for (int t = 0; t < nt; ++t) {
                    const int f = s_flags[t * R + r];
                    itr_chunk[t * R + r] = f;
                    cnt += f;
                }
                s_rcnt[r] = cnt;
            }
        }
    }
    __syncthreads();

    // stable rank of every entry among the chunk's entries of its expert
    // (wave base + position among the equal keys of its vector), stored in
    // token_row packed with the expert, (e << 16) | rank, for the rank kernel
    // to complete; dropped entries get their final -1 here
#pragma unroll
    for (int it = 0; it < kIdxPerThread; ++it) {
        if (it * kWave < per_wave) {
            const int j = w_lo + it * kWave + lane;
            const int e = e_reg[it];
            const int below = pos_reg[it] & 0xFF;
            if (e >= 0)
                token_row[base + j] = (e << 16) | (s_w[wave * E + e] + below);
            else if (j < w_hi)
                token_row[base + j] = -1;
            if (e >= 0 && below == 0) // after every lane of the wave has read the running count
                s_w[wave * E + e] += pos_reg[it] >> 8;
        }
    }

    for (int r = tid; r < R; r += kCountThreads)
        rank_tab[(int64_t)chunk * R + r] = s_rcnt[r];
    if (tid == 0)
        flag_tab[chunk] = s_bad;
}

// Column scan of the count table, for large tables only: cb_tab[c][e] =
// sum over chunks c' < c of cnt_tab[c'][e], and tot_tab[e] = the sum over all
// chunks.  One workgroup per 16 columns; its 64 groups of 16 lanes each own a
// contiguous run of chunks: they sum their run, take the exclusive prefix of
// the group sums from LDS, then walk the run again writing running prefixes.
constexpr int kScanCols = 16;
constexpr int kScanGroups = 1024 / kScanCols;

__global__ __launch_bounds__(1024) void layout_scan_kernel(const int32_t *__restrict__ cnt_tab,
                                                           int nchunks, int Ep,
                                                           int32_t *__restrict__ cb_tab,
                                                           int32_t *__restrict__ tot_tab)
{
    __shared__ int s_part[kScanGroups][kScanCols];
    const int c = threadIdx.x % kScanCols;
    const int g = threadIdx.x / kScanCols;
    const int col = blockIdx.x * kScanCols + c;
    const int per = (nchunks + kScanGroups - 1) / kScanGroups;
    const int r0 = min(nchunks, g * per);
    const int r1 = min(nchunks, r0 + per);
    int sum = 0;
    if (col < Ep)
        for (int r = r0; r < r1; ++r)
            sum += cnt_tab[(int64_t)r * Ep + col];
    s_part[g][c] = sum;
    __syncthreads();
    int base = 0;
    for (int h = 0; h < g; ++h)
        base += s_part[h][c];
    if (col < Ep) {
        if (g == kScanGroups - 1)
            tot_tab[col] = base + sum;
        int run = base;
        for (int r = r0; r < r1; ++r) {
            const int v = cnt_tab[(int64_t)r * Ep + col];
            cb_tab[(int64_t)r * Ep + col] = run;
            run += v;
        }
    }
}

__global__ __launch_bounds__(kRankThreads) void layout_rank_kernel(
    int T, int K, int E, int R, int a, int tpc, int nchunks, int64_t cap,
    const int32_t *__restrict__ cnt_tab, const int32_t *__restrict__ rank_tab,
    const int32_t *__restrict__ flag_tab, const int32_t *__restrict__ cb_tab,
    const int32_t *__restrict__ tot_tab, int32_t *__restrict__ ntpr, int32_t *__restrict__ ntpe,
    int32_t *__restrict__ nrtpe, int32_t *__restrict__ off, int32_t *__restrict__ token_row,
    int32_t *__restrict__ recv_src, int32_t *__restrict__ error_flag)
{
    __shared__ int s_tot[MOE_MAX_EXPERTS];
    __shared__ int s_cb[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_rsum[kRankSumSlots];
    __shared__ int s_flag;
    __shared__ int4 s_pall[kRankThreads]; // table threads' column sums, slot part * groups + g
    __shared__ int4 s_pbef[kRankThreads]; // the same over the rows before this chunk
    __shared__ int s_wsum[kRankWaves];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int chunk = blockIdx.x;
    const int nblocks = gridDim.x;
    const bool has_chunk = chunk < nchunks; // false only when T == 0 (one workgroup then)
    const int t0 = chunk * tpc;
    const int nt = has_chunk ? min(tpc, T - t0) : 0;
    const int ne = nt * K;
    const int64_t base = (int64_t)t0 * K;

    // (0) Every global load the workgroup needs is issued here, before the
    // first barrier (a barrier waits for all outstanding loads), so that the
    // kernel pays one memory round trip:
    //   - this chunk's entries as the count kernel left them in token_row,
    //     (expert << 16) | rank within the chunk, or -1;
    //   - the expert-count table [nchunks][Ep] (Ep = E rounded up to 4): a
    //     thread owns 4 adjacent columns (one 16-byte load per row) and up to
    //     kTabRows rows; rows beyond parts * kTabRows (very many chunks only)
    //     are read in later passes;
    //   - the per-chunk counts of the ranks this workgroup sums (ranks
    //     r = chunk, chunk + nblocks, ...), one (rank, chunk) cell per thread
    //     and pass;
    //   - in workgroup 0, the per-chunk error flags.
    int32_t ent_reg[kIdxPerThread];
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u)
        ent_reg[u] = u * kRankThreads < ne ? token_row[base + min(tid + u * kRankThreads, ne - 1)] : -1;

    const int groups = (E + 3) / 4; // <= 128
    const int parts = kRankThreads / groups; // >= 8
    const int g = tid % groups;
    const int part = tid / groups;
    const bool scanned = tot_tab != nullptr; // the scan launch left totals and this chunk's prefix row
    const bool tab_parts_ready = !scanned && nchunks > 0; // the partial sums below hold the table
    const bool tab_thread = tid < parts * groups && tab_parts_ready;
    const int rb = scanned ? 0 : min(kTabRows, (nchunks + parts - 1) / parts); // rows per thread and pass (uniform)
    const int4 *tab4 = (const int4 *)cnt_tab;
    int4 tab_reg[kTabRows];
#pragma unroll
    for (int u = 0; u < kTabRows; ++u) {
        tab_reg[u] = int4{0, 0, 0, 0};
        if (u < rb) // uniform
            tab_reg[u] = tab4[(int64_t)min(part * rb + u, nchunks - 1) * groups + g];
    }

    const int my_ranks = nchunks > 0 && chunk < R ? (R - 1 - chunk) / nblocks + 1 : 0;
    const int rank_cells = my_ranks * nchunks;
    int rank_reg[kRankCellsPerThread];
#pragma unroll
    for (int u = 0; u < kRankCellsPerThread; ++u) {
        rank_reg[u] = 0;
        if (u * kRankThreads < rank_cells) { // uniform
            const int cell = min(tid + u * kRankThreads, rank_cells - 1);
            rank_reg[u] = rank_tab[(int64_t)(cell % nchunks) * R + chunk + (cell / nchunks) * nblocks];
        }
    }
    int flag_reg = 0;
    if (chunk == 0)
        for (int c = tid; c < nchunks; c += kRankThreads)
            flag_reg |= flag_tab[c];
    int tot_reg = 0, cb_reg = 0; // scanned: expert tid's total and prefix (E <= 512 < 1024 threads)
    if (scanned && tid < E) {
        tot_reg = tot_tab[tid];
        cb_reg = has_chunk ? cb_tab[(int64_t)chunk * (4 * groups) + tid] : 0;
    }

    // (1) expert totals over all chunks, and the part of them in chunks
    // before this one: each table thread's sums of the rows it read (all of
    // them, and those before this chunk) go to LDS, and thread e then adds
    // the parts of expert e (no atomics: 16 parts per column at E = 256)
    for (int i = tid; i < kRankSumSlots; i += kRankThreads)
        s_rsum[i] = 0;
    if (tid == 0)
        s_flag = 0;
    if (tab_thread) {
        int4 all = int4{0, 0, 0, 0}, before = int4{0, 0, 0, 0};
        auto add_row = [&](int r, const int4 v) {
            const int keep = r < nchunks ? 1 : 0;
            const int early = r < chunk ? keep : 0;
            all.x += keep * v.x;
            all.y += keep * v.y;
            all.z += keep * v.z;
            all.w += keep * v.w;
            before.x += early * v.x;
            before.y += early * v.y;
            before.z += early * v.z;
            before.w += early * v.w;
        };
#pragma unroll
        for (int u = 0; u < kTabRows; ++u)
            if (u < rb)
                add_row(part * rb + u, tab_reg[u]);
        for (int r = parts * rb + part; r < nchunks; r += parts) // only for very many chunks
            add_row(r, tab4[(int64_t)r * groups + g]);
        s_pall[tid] = all; // slot part * groups + g
        s_pbef[tid] = before;
    }
    __syncthreads();

    // this workgroup's rank sums and the error flags
#pragma unroll
    for (int u = 0; u < kRankCellsPerThread; ++u) {
        const int cell = tid + u * kRankThreads;
        if (cell < rank_cells && rank_reg[u])
            atomicAdd(&s_rsum[cell / nchunks], rank_reg[u]);
    }
    for (int cell = tid + kRankCellsPerThread * kRankThreads; cell < rank_cells; cell += kRankThreads)
        atomicAdd(&s_rsum[cell / nchunks],
                  rank_tab[(int64_t)(cell % nchunks) * R + chunk + (cell / nchunks) * nblocks]);
    if (flag_reg)
        atomicOr(&s_flag, flag_reg);

    // (2) expert tid's total, its aligned count ("/" is integer division,
    // CANN page Constraint 11) and their exclusive prefix sum over the
    // experts: a shuffle scan in each wave, then the waves' totals through
    // LDS.  No overflow: the host checked T*K + E*(a-1) < 2^31.
    int tot = 0, ac = 0;
    if (tid < E) {
        int cb = 0;
        if (scanned) {
            tot = tot_reg;
            cb = cb_reg;
        } else if (tab_parts_ready) {
            const int *pa = (const int *)s_pall;
            const int *pb = (const int *)s_pbef;
            const int col = (tid >> 2) * 4 + (tid & 3);
            for (int p = 0; p < parts; ++p) {
                tot += pa[p * 4 * groups + col];
                cb += pb[p * 4 * groups + col];
            }
        }
        s_tot[tid] = tot;
        s_cb[tid] = cb;
        ac = a == 1 ? tot : ((tot + a - 1) / a) * a;
    }
    int incl = ac;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(incl, d, kWave);
        if (lane >= d)
            incl += v;
    }
    if (lane == kWave - 1)
        s_wsum[tid / kWave] = incl;
    __syncthreads();
    if (tid < E) {
        int run = 0;
        for (int w = 0; w < tid / kWave; ++w)
            run += s_wsum[w];
        s_off[tid] = run + incl - ac;
        if (tid == E - 1)
            s_off[E] = run + incl;
    }
    __syncthreads();

    // (3) the small outputs: per-expert ones and the error flag from workgroup
    // 0, each rank's token count from the workgroup that summed it
    if (chunk == 0) {
        for (int e = tid; e < E; e += kRankThreads) {
            ntpe[e] = s_tot[e];
            nrtpe[e] = s_off[e + 1] - s_off[e];
        }
        for (int e = tid; e <= E; e += kRankThreads)
            off[e] = s_off[e];
        if (tid == 0)
            *error_flag = s_flag;
    }
    for (int j = tid; j < my_ranks; j += kRankThreads)
        ntpr[chunk + j * nblocks] = s_rsum[j];
    if (nchunks == 0)
        for (int r = tid; r < R; r += kRankThreads)
            ntpr[r] = 0;

    // (4) rows holding no entry: alignment padding inside each expert, and
    // every row past the last expert up to the capacity
    for (int e = chunk; e < E; e += nblocks) {
        const int lo = s_off[e] + s_tot[e];
        const int hi = s_off[e + 1];
        for (int row = lo + tid; row < hi; row += kRankThreads)
            recv_src[row] = -1;
    }
    for (int64_t row = (int64_t)s_off[E] + (int64_t)chunk * kRankThreads + tid; row < cap;
         row += (int64_t)nblocks * kRankThreads)
        recv_src[row] = -1;

    if (!has_chunk)
        return;

    // (5) each entry's row: expert base + the expert's entries in earlier
    // chunks + its rank within this chunk (dropped entries are already -1)
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u) {
        const int i = tid + u * kRankThreads;
        const int v = ent_reg[u];
        if (i < ne && v >= 0) {
            const int e = v >> 16;
            const int row = s_off[e] + s_cb[e] + (v & 0xFFFF);
            token_row[base + i] = row;
            recv_src[row] = (int32_t)(base + i);
        }
    }
}

// n / d for 0 <= n < 2^24 and 1 <= d <= 2^24 without the integer division
// sequence: a float quotient is within one of the exact one, then fixed.
__device__ __forceinline__ int div_small(int n, int d)
{
    int q = (int)((float)n * __frcp_rn((float)d));
    q += (q + 1) * d <= n ? 1 : 0;
    q -= q * d > n ? 1 : 0;
    return q;
}

// One workgroup for a whole small batch (T*K <= kSingleLayoutMaxEntries
// entries and T*R <= kMaxChunkFlags token x rank cells): every entry lives in
// LDS, so the histogram, the aligned scan and the ranks need no count table
// and no second launch.  All the ballot matching runs on one CU, so its cost
// grows with the batch (about 1.3 ns per entry): measured as graph replays,
// 4.6 us for 128 x 2 entries and 7.2 us for 128 x 8, level with the
// two-launch layout (a flat ~10.2 us at these sizes) at 3072 entries and
// 1.5 us slower at 4096.  The per-wave expert counts are the histogram: their
// sum over the waves is the expert total, their exclusive prefix over the
// waves the wave's base, as in layout_count_kernel with a single chunk.
// Counts are held in 16 bits (at most kMaxChunkEntries entries per batch).
__global__ __launch_bounds__(kRankThreads) void layout_single_kernel(
    const int64_t *__restrict__ topk_idx, int T, int K, int E, int R, int L, int a, int nbits,
    int64_t cap, int32_t *__restrict__ itr, int32_t *__restrict__ ntpr, int32_t *__restrict__ ntpe,
    int32_t *__restrict__ nrtpe, int32_t *__restrict__ off, int32_t *__restrict__ token_row,
    int32_t *__restrict__ recv_src, int32_t *__restrict__ error_flag)
{
    static_assert(kMaxChunkEntries <= 32767, "16-bit per-wave counts");
    __shared__ int16_t s_e[kMaxChunkEntries];
    __shared__ uint8_t s_flags[kMaxChunkFlags];
    __shared__ int16_t s_w[kRankWaves][MOE_MAX_EXPERTS];
    __shared__ int s_tot[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_rcnt[MOE_MAX_EXPERTS];
    __shared__ int s_wsum[kRankWaves];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int ne = T * K;

    int64_t idx_reg[kIdxPerThread];
    prefetch_idx(topk_idx, 0, ne, idx_reg); // in flight while LDS is cleared

    for (int i = tid; i < kRankWaves * E; i += kRankThreads)
        s_w[i / E][i % E] = 0;
    for (int i = tid; i < R; i += kRankThreads)
        s_rcnt[i] = 0;
    for (int i = tid; i < T * R; i += kRankThreads)
        s_flags[i] = 0;
    if (tid == 0)
        s_bad = 0;
    __syncthreads();

    // ids into LDS (out-of-range ids become -1 and raise the error bit) and
    // token x rank membership
    int bad = 0;
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u) {
        const int i = tid + u * kRankThreads;
        if (i < ne) {
            const int64_t v = idx_reg[u];
            int e = -1;
            if (v < -1 || v >= E)
                bad = 1;
            else
                e = (int)v;
            s_e[i] = (int16_t)e;
            if (e >= 0)
                s_flags[div_small(i, K) * R + div_small(e, L)] = 1;
        }
    }
    if (bad)
        atomicOr(&s_bad, 1);
    __syncthreads();

    // per-wave expert counts; each wave owns a contiguous run of entries in
    // flat order.  The match masks and ids stay in registers for the ranking
    // pass below (at most kIdxPerThread iterations per wave; the iteration
    // guard is uniform over the workgroup, so the ballots stay convergent).
    const int per_wave = ((ne + kRankWaves * kWave - 1) / (kRankWaves * kWave)) * kWave;
    const int w_lo = wave * per_wave;
    const int w_hi = min(ne, w_lo + per_wave);
    uint64_t same_reg[kIdxPerThread];
    int e_reg[kIdxPerThread];
#pragma unroll
    for (int it = 0; it < kIdxPerThread; ++it) {
        same_reg[it] = 0;
        e_reg[it] = -1;
        if (it * kWave < per_wave) {
            const int j = w_lo + it * kWave + lane;
            const int e = (j < w_hi) ? (int)s_e[j] : -1;
            const bool has = e >= 0;
            const uint64_t same = match_same_key(e, has, nbits);
            same_reg[it] = same;
            e_reg[it] = e;
            if (has && count_below(same) == 0) // one writer per (wave, expert)
                s_w[wave][e] = (int16_t)(s_w[wave][e] + __popcll(same));
        }
    }
    // is_token_in_rank rows and per-rank token counts: thread (r, part) owns
    // rank r of tokens part, part + parts, ...
    {
        const int parts = kRankThreads / R;
        if (tid < parts * R) {
            const int r = tid % R;
            const int part = tid / R;
            int cnt = 0;
            for (int t = part; t < T; t += parts) {
                const int f = s_flags[t * R + r];
                itr[(int64_t)t * R + r] = f;
                cnt += f;
            }
            if (cnt)
                atomicAdd(&s_rcnt[r], cnt);
        }
    }
    __syncthreads();

    // expert totals and each wave's exclusive base, one thread per expert
    for (int e = tid; e < E; e += kRankThreads) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < kRankWaves; ++w) {
            const int v = s_w[w][e];
            s_w[w][e] = (int16_t)run;
            run += v;
        }
        s_tot[e] = run;
    }
    __syncthreads();

    // aligned counts and their exclusive prefix sum ("/" is integer division,
    // CANN page Constraint 11); E <= 512 < kRankThreads
    int ac = 0;
    if (tid < E) {
        const int c = s_tot[tid];
        ac = ((c + a - 1) / a) * a;
    }
    int incl = ac;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(incl, d, kWave);
        if (lane >= d)
            incl += v;
    }
    if (lane == kWave - 1)
        s_wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int total;
        const int v = lane < kRankWaves ? s_wsum[lane] : 0;
        const int ex = exclusive_scan16(v, &total);
        if (lane < kRankWaves)
            s_wsum[lane] = ex;
    }
    __syncthreads();
    if (tid < E)
        s_off[tid] = s_wsum[wave] + incl - ac;
    if (tid == E - 1)
        s_off[E] = s_wsum[wave] + incl;
    __syncthreads();

    // small outputs
    for (int e = tid; e < E; e += kRankThreads) {
        ntpe[e] = s_tot[e];
        nrtpe[e] = s_off[e + 1] - s_off[e];
    }
    for (int e = tid; e <= E; e += kRankThreads)
        off[e] = s_off[e];
    for (int r = tid; r < R; r += kRankThreads)
        ntpr[r] = s_rcnt[r];
    if (tid == 0)
        *error_flag = s_bad;

    // rows holding no entry: alignment padding inside each expert (wave w
    // takes experts w, w + 16, ...), then every row up to the capacity
    for (int e = wave; e < E; e += kRankWaves) {
        const int lo = s_off[e] + s_tot[e];
        const int hi = s_off[e + 1];
        for (int row = lo + lane; row < hi; row += kWave)
            recv_src[row] = -1;
    }
    for (int64_t row = (int64_t)s_off[E] + tid; row < cap; row += kRankThreads)
        recv_src[row] = -1;

    // ranks: expert base + this wave's base + position among equal keys
#pragma unroll
    for (int it = 0; it < kIdxPerThread; ++it) {
        if (it * kWave < per_wave) {
            const int j = w_lo + it * kWave + lane;
            const int e = e_reg[it];
            const uint64_t same = same_reg[it];
            const int below = count_below(same);
            if (e >= 0) {
                const int row = s_off[e] + s_w[wave][e] + below;
                token_row[j] = row;
                recv_src[row] = j;
            } else if (j < w_hi) {
                token_row[j] = -1;
            }
            if (e >= 0 && below == 0) // after every lane of the wave has read the running count
                s_w[wave][e] = (int16_t)(s_w[wave][e] + __popcll(same));
        }
    }
}

static int key_bits(int E)
{
    int b = 0;
    while ((1 << b) < E)
        ++b;
    return b;
}

hipError_t launch_layout(const LayoutArgs &A, const LayoutPlan &P, hipStream_t stream)
{
    const int L = A.E / A.R;
    const int nbits = key_bits(A.E);
    const int nchunks = P.num_chunks;
    if (P.single)
        return launch_kernel(layout_single_kernel, dim3(1), dim3(kRankThreads), 0, stream,
                             A.topk_idx, A.T, A.K, A.E, A.R, L, A.a, nbits, A.cap, A.itr, A.ntpr,
                             A.ntpe, A.nrtpe, A.off, A.token_row, A.recv_src, A.error_flag);
    const int Ep = (A.E + 3) & ~3;
    int32_t *cnt_tab = A.workspace;
    int32_t *rank_tab = cnt_tab ? cnt_tab + (size_t)nchunks * Ep : nullptr;
    int32_t *flag_tab = rank_tab ? rank_tab + (size_t)nchunks * A.R : nullptr;
    int32_t *cb_tab = P.scan ? flag_tab + nchunks : nullptr;
    int32_t *tot_tab = P.scan ? cb_tab + (size_t)nchunks * Ep : nullptr;
    if (nchunks > 0) {
        const int threads = count_threads(P.tokens_per_chunk * A.K);
        auto kern = threads == 256   ? layout_count_kernel<256>
                    : threads == 512 ? layout_count_kernel<512>
                                     : layout_count_kernel<1024>;
        hipError_t err = launch_kernel(kern, dim3(nchunks), dim3(threads), 0, stream, A.topk_idx,
                                       A.T, A.K, A.E, A.R, L, P.tokens_per_chunk, nbits, A.itr,
                                       cnt_tab, rank_tab, flag_tab, A.token_row);
        if (err != hipSuccess)
            return err;
        if (P.scan) {
            err = launch_kernel(layout_scan_kernel, dim3((Ep + kScanCols - 1) / kScanCols),
                                dim3(1024), 0, stream, (const int32_t *)cnt_tab, nchunks, Ep,
                                cb_tab, tot_tab);
            if (err != hipSuccess)
                return err;
        }
    }
    return launch_kernel(layout_rank_kernel, dim3(nchunks > 0 ? nchunks : 1), dim3(kRankThreads), 0,
                         stream, A.T, A.K, A.E, A.R, A.a, P.tokens_per_chunk, nchunks, A.cap,
                         cnt_tab, rank_tab, flag_tab, (const int32_t *)cb_tab,
                         (const int32_t *)tot_tab, A.ntpr, A.ntpe, A.nrtpe, A.off, A.token_row,
                         A.recv_src, A.error_flag);
}

} // namespace moe
