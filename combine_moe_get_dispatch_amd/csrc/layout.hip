// layout.hip -- dispatch layout: counts, alignment-padded expert offsets and a
// stable expert-grouped row for every (token, k) routing entry.
//
// What is computed (Normal Mode API page, dispatch Parameters / Return
// Values; EPBatchManager page, ep_dispatch() Returns; CANN
// aclnnMoeDistributeDispatchV2 page, Constraint 1 "deterministic"):
//   c[e]        = number of entries with topk_idx == e
//   off[e]      = sum over e' < e of ceil(c[e'] / a) * a
//   row(t, k)   = off[e] + #{ (t', k') : idx[t', k'] == e, t'K + k' < tK + k }
//   recv_src    = inverse of row (-1 on padding / unused rows)
//   is_token_in_rank[t, r], num_tokens_per_rank[r]  with rank(e) = e / (E / R)
//
// Design (gfx950, wave64): the T*K entries are split into chunks of whole
// tokens, one workgroup per chunk.
//   layout_count_kernel: per-chunk expert histogram.  Lanes of a wave holding
//     the same expert are found with one ballot per key bit; the lowest of them
//     adds the group's popcount to an LDS counter, so a hot expert costs one
//     LDS atomic per wave instead of one per lane.  The same pass marks
//     token x rank membership in LDS and writes is_token_in_rank rows.
//   layout_rank_kernel: every workgroup re-derives the expert totals and its
//     own chunk base from the small [chunks][E] table (L2 resident), scans the
//     aligned totals in LDS, then ranks its chunk: per-wave counts, an
//     exclusive scan over waves, and within a wave the position among equal
//     keys by masked popcount.  Ranks therefore come from prefix sums only
//     (never from atomic return order), which makes the result deterministic.
#include "device_common.h"
#include "launch.h"

#include "../../include/moe_dispatch_combine.h"

namespace moe {

constexpr int kCountThreads = 512;
constexpr int kRankThreads = 1024;
constexpr int kRankWaves = kRankThreads / kWave;

__global__ __launch_bounds__(kCountThreads) void layout_count_kernel(
    const int64_t *__restrict__ topk_idx, int T, int K, int E, int R, int L, int tpc, int nbits,
    int32_t *__restrict__ itr, int32_t *__restrict__ cnt_tab, int32_t *__restrict__ rank_tab,
    int32_t *__restrict__ flag_tab)
{
    __shared__ int s_hist[MOE_MAX_EXPERTS];
    __shared__ int s_rcnt[MOE_MAX_EXPERTS];
    __shared__ uint8_t s_flags[kMaxChunkFlags];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    const int t0 = chunk * tpc;
    const int nt = min(tpc, T - t0);
    const int ne = nt * K;
    const int64_t base = (int64_t)t0 * K;

    for (int i = tid; i < E; i += kCountThreads)
        s_hist[i] = 0;
    for (int i = tid; i < R; i += kCountThreads)
        s_rcnt[i] = 0;
    for (int i = tid; i < nt * R; i += kCountThreads)
        s_flags[i] = 0;
    if (tid == 0)
        s_bad = 0;
    __syncthreads();

    int bad = 0;
    for (int i0 = 0; i0 < ne; i0 += kCountThreads) { // uniform trip count: ballots stay convergent
        const int i = i0 + tid;
        int e = -1;
        if (i < ne) {
            const int64_t v = topk_idx[base + i];
            if (v < -1 || v >= E)
                bad = 1;
            else
                e = (int)v;
        }
        const bool has = e >= 0;
        const uint64_t same = match_same_key(e, has, nbits);
        if (has) {
            if (count_below(same) == 0)
                atomicAdd(&s_hist[e], __popcll(same));
            s_flags[(i / K) * R + e / L] = 1;
        }
    }
    if (bad)
        atomicOr(&s_bad, 1);
    __syncthreads();

    int32_t *itr_chunk = itr + (int64_t)t0 * R;
    for (int p = tid; p < nt * R; p += kCountThreads) {
        const int f = s_flags[p];
        itr_chunk[p] = f;
        if (f)
            atomicAdd(&s_rcnt[p % R], 1);
    }
    __syncthreads();

    for (int e = tid; e < E; e += kCountThreads)
        cnt_tab[(int64_t)chunk * E + e] = s_hist[e];
    for (int r = tid; r < R; r += kCountThreads)
        rank_tab[(int64_t)chunk * R + r] = s_rcnt[r];
    if (tid == 0)
        flag_tab[chunk] = s_bad;
}

// Column sums of a [nchunks][W] int32 table (W <= 512), spread over the whole
// workgroup: kRankThreads / W threads per column, each reading its share of
// the rows in batches of 8 independent loads (one L2 round trip per batch,
// instead of one per row).  Adds the full column sum to s_all[col] and, when
// s_before is given, the sum over rows < `row_end` to s_before[col].
__device__ __forceinline__ void column_sums(const int32_t *__restrict__ tab, int W, int nchunks,
                                            int row_end, int *s_all, int *s_before)
{
    constexpr int kBatch = 8;
    const int parts = kRankThreads / W;
    const int tid = threadIdx.x;
    if (tid >= parts * W || nchunks == 0)
        return;
    const int col = tid % W;
    const int part = tid / W;
    int all = 0, before = 0;
    for (int c0 = part * kBatch; c0 < nchunks; c0 += parts * kBatch) {
        int v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            v[u] = tab[(int64_t)min(c0 + u, nchunks - 1) * W + col]; // clamped: always in bounds
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int c = c0 + u;
            const int x = c < nchunks ? v[u] : 0;
            all += x;
            before += c < row_end ? x : 0;
        }
    }
    if (all)
        atomicAdd(&s_all[col], all);
    if (s_before && before)
        atomicAdd(&s_before[col], before);
}

__global__ __launch_bounds__(kRankThreads) void layout_rank_kernel(
    const int64_t *__restrict__ topk_idx, int T, int K, int E, int R, int a, int tpc, int nchunks,
    int nbits, int64_t cap, const int32_t *__restrict__ cnt_tab, const int32_t *__restrict__ rank_tab,
    const int32_t *__restrict__ flag_tab, int32_t *__restrict__ ntpr, int32_t *__restrict__ ntpe,
    int32_t *__restrict__ nrtpe, int32_t *__restrict__ off, int32_t *__restrict__ token_row,
    int32_t *__restrict__ recv_src, int32_t *__restrict__ error_flag)
{
    __shared__ int s_tot[MOE_MAX_EXPERTS];
    __shared__ int s_cb[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_rsum[MOE_MAX_EXPERTS];
    __shared__ int s_wsum[kRankWaves];
    __shared__ int s_w[kRankWaves][MOE_MAX_EXPERTS];
    __shared__ int16_t s_e[kMaxChunkEntries];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int chunk = blockIdx.x;
    const bool has_chunk = chunk < nchunks; // false only when T == 0 (one workgroup then)
    const int t0 = chunk * tpc;
    const int nt = has_chunk ? min(tpc, T - t0) : 0;
    const int ne = nt * K;
    const int64_t base = (int64_t)t0 * K;

    // (0) issue this chunk's topk_idx loads first, so that their latency
    // overlaps the table reads below (indices clamped: always in bounds)
    constexpr int kIdxPerThread = kMaxChunkEntries / kRankThreads;
    int64_t idx_reg[kIdxPerThread];
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u) // the guard is uniform over the workgroup
        idx_reg[u] = u * kRankThreads < ne ? topk_idx[base + min(tid + u * kRankThreads, ne - 1)] : -1;

    // (1) expert totals over all chunks, and the part of them in chunks before this one
    for (int e = tid; e < E; e += kRankThreads) {
        s_tot[e] = 0;
        s_cb[e] = 0;
    }
    for (int i = tid; i < kRankWaves * E; i += kRankThreads)
        s_w[i / E][i % E] = 0;
    __syncthreads();
    column_sums(cnt_tab, E, nchunks, chunk, s_tot, s_cb);
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u) {
        const int i = tid + u * kRankThreads;
        if (i < ne) {
            const int64_t v = idx_reg[u];
            s_e[i] = (v < 0 || v >= E) ? (int16_t)-1 : (int16_t)v;
        }
    }
    __syncthreads();

    // (2) aligned counts and their exclusive prefix sum ("/" is integer
    // division, CANN page Constraint 11).  No overflow: the host checked
    // T*K + E*(a-1) < 2^31.
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
    if (tid == 0) {
        int run = 0;
        for (int w = 0; w < kRankWaves; ++w) {
            const int v = s_wsum[w];
            s_wsum[w] = run;
            run += v;
        }
    }
    __syncthreads();
    if (tid < E)
        s_off[tid] = s_wsum[wave] + incl - ac;
    if (tid == E - 1)
        s_off[E] = s_wsum[wave] + incl;
    __syncthreads();

    // (3) the small per-expert / per-rank outputs, once
    if (chunk == 0) {
        for (int e = tid; e < E; e += kRankThreads) {
            ntpe[e] = s_tot[e];
            nrtpe[e] = s_off[e + 1] - s_off[e];
        }
        for (int e = tid; e <= E; e += kRankThreads)
            off[e] = s_off[e];
        for (int r = tid; r < R; r += kRankThreads)
            s_rsum[r] = 0;
        __syncthreads();
        column_sums(rank_tab, R, nchunks, 0, s_rsum, nullptr);
        __syncthreads();
        for (int r = tid; r < R; r += kRankThreads)
            ntpr[r] = s_rsum[r];
        if (wave == 0) {
            int f = 0;
            for (int c = lane; c < nchunks; c += kWave)
                f |= flag_tab[c];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
                f |= __shfl_xor(f, o, kWave);
            if (lane == 0)
                *error_flag = f;
        }
    }

    // (4) rows holding no entry: alignment padding inside each expert, and
    // every row past the last expert up to the capacity
    for (int e = chunk; e < E; e += gridDim.x) {
        const int lo = s_off[e] + s_tot[e];
        const int hi = s_off[e + 1];
        for (int row = lo + tid; row < hi; row += kRankThreads)
            recv_src[row] = -1;
    }
    for (int64_t row = (int64_t)s_off[E] + (int64_t)chunk * kRankThreads + tid; row < cap;
         row += (int64_t)gridDim.x * kRankThreads)
        recv_src[row] = -1;

    if (!has_chunk)
        return;

    // (5) rank this chunk's entries (ids already in s_e)
    // each wave owns a contiguous run of entries, in flat order
    const int per_wave = ((ne + kRankWaves * kWave - 1) / (kRankWaves * kWave)) * kWave;
    const int w_lo = wave * per_wave;
    const int w_hi = min(ne, w_lo + per_wave);

    for (int j0 = w_lo; j0 < w_lo + per_wave; j0 += kWave) {
        const int j = j0 + lane;
        const int e = (j < w_hi) ? (int)s_e[j] : -1;
        const bool has = e >= 0;
        const uint64_t same = match_same_key(e, has, nbits);
        if (has && count_below(same) == 0)
            s_w[wave][e] += __popcll(same); // one writer per (wave, expert)
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRankThreads) {
        int run = 0;
        for (int w = 0; w < kRankWaves; ++w) {
            const int v = s_w[w][e];
            s_w[w][e] = run;
            run += v;
        }
    }
    __syncthreads();

    for (int j0 = w_lo; j0 < w_lo + per_wave; j0 += kWave) {
        const int j = j0 + lane;
        const bool in = j < w_hi;
        const int e = in ? (int)s_e[j] : -1;
        const bool has = e >= 0;
        const uint64_t same = match_same_key(e, has, nbits);
        const int below = count_below(same);
        if (has) {
            const int row = s_off[e] + s_cb[e] + s_w[wave][e] + below;
            token_row[base + j] = row;
            recv_src[row] = (int32_t)(base + j);
        } else if (in) {
            token_row[base + j] = -1;
        }
        if (has && below == 0) // after every lane of the wave has read the running count
            s_w[wave][e] += __popcll(same);
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
    int32_t *cnt_tab = A.workspace;
    int32_t *rank_tab = cnt_tab ? cnt_tab + (size_t)nchunks * A.E : nullptr;
    int32_t *flag_tab = rank_tab ? rank_tab + (size_t)nchunks * A.R : nullptr;
    if (nchunks > 0) {
        const hipError_t err = launch_kernel(
            layout_count_kernel, dim3(nchunks), dim3(kCountThreads), 0, stream, A.topk_idx, A.T,
            A.K, A.E, A.R, L, P.tokens_per_chunk, nbits, A.itr, cnt_tab, rank_tab, flag_tab);
        if (err != hipSuccess)
            return err;
    }
    return launch_kernel(layout_rank_kernel, dim3(nchunks > 0 ? nchunks : 1), dim3(kRankThreads), 0,
                         stream, A.topk_idx, A.T, A.K, A.E, A.R, A.a, P.tokens_per_chunk, nchunks,
                         nbits, A.cap, cnt_tab, rank_tab, flag_tab, A.ntpr, A.ntpe, A.nrtpe, A.off,
                         A.token_row, A.recv_src, A.error_flag);
}

} // namespace moe
