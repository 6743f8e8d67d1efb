// small_batch.hip -- layout and bf16 dispatch of a decode-sized batch in one
// launch.
//
// What is computed: exactly what moe_get_dispatch_layout followed by
// moe_dispatch (no quantisation) compute (Normal Mode API page, dispatch
// Parameters / Return Values; EPBatchManager page, ep_dispatch(); CANN
// aclnnMoeDistributeDispatchV2 page, Constraint 1, deterministic):
//   c[e]        = number of entries with topk_idx == e
//   off[e]      = sum over e' < e of ceil(c[e'] / a) * a
//   row(t, k)   = off[e] + #{ j < tK : idx_j == e } + #{ k' < k : idx[t, k'] == e }
//   recv[row(t, k)] = x[t]
//
// Design (gfx950): at decode-sized batches the two-call form is bound by
// fixed costs -- two launches, the layout's store of token_row and the
// dispatch's reload of it.  Here one workgroup per token derives the whole
// (small) layout redundantly: every workgroup loads all T*K ids (at most
// three per thread, hits in L2 after the first workgroups), builds the
// expert totals with wave-aggregated LDS adds (keys matched by one ballot
// per key bit) and the aligned offsets (one wave, shuffle scan), and counts,
// for each of its own K entries, the entries before its token that hold the
// same expert.  It then writes its token's layout outputs and copies the
// token, whose 16-byte vectors were loaded at the start, to its rows with
// nontemporal stores.  Workgroups never wait for one another: all of them
// compute identical totals and offsets from the same ids.  Workgroup 0 also
// writes the per-expert and per-rank outputs and every is_token_in_rank row;
// the padding and unused rows of recv_src are spread over all workgroups.
// The redundant layout work grows as T * T*K, so the path is limited to
// small batches (kSmallMaxTokens tokens, kSmallMaxEntries entries).
#include "device_common.h"
#include "small_batch.h"

#include "../../include/moe_dispatch_combine.h"

namespace moe {

constexpr int kSmallThreads = 1024;
constexpr int kSmallIdsPerThread = kSmallMaxEntries / kSmallThreads;
static_assert(kSmallMaxEntries % kSmallThreads == 0, "ids per thread");
static_assert(kSmallMaxFlags <= kMaxChunkFlags, "membership bytes");

// n / d for 0 <= n < 2^24 and 1 <= d <= 2^24 without the integer division
// sequence: a float quotient is within one of the exact one, then fixed.
__device__ __forceinline__ int small_div(int n, int d)
{
    int q = (int)((float)n * __frcp_rn((float)d));
    q += (q + 1) * d <= n ? 1 : 0;
    q -= q * d > n ? 1 : 0;
    return q;
}

__global__ __launch_bounds__(kSmallThreads) void layout_dispatch_small_kernel(
    const int64_t *__restrict__ topk_idx, const u32x4 *__restrict__ x, int T, int K, int E, int R,
    int L, int a, int nbits, int nvec, int64_t cap, const float *__restrict__ topk_weights,
    int32_t *__restrict__ itr, int32_t *__restrict__ ntpr, int32_t *__restrict__ ntpe,
    int32_t *__restrict__ nrtpe, int32_t *__restrict__ off, int32_t *__restrict__ token_row,
    int32_t *__restrict__ recv_src, int32_t *__restrict__ error_flag, u32x4 *__restrict__ recv,
    float *__restrict__ recv_weights)
{
    __shared__ int s_tot[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_rcnt[MOE_MAX_EXPERTS];
    __shared__ uint8_t s_flags[kSmallMaxFlags];
    __shared__ int s_my[MOE_MAX_TOPK];     // this token's experts (-1: dropped)
    __shared__ int s_before[MOE_MAX_TOPK]; // entries before this token holding s_my[k]
    __shared__ int s_row[MOE_MAX_TOPK];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int b = blockIdx.x;
    const int nblocks = gridDim.x;
    const bool has_token = b < T; // false only when T == 0 (one workgroup then)
    const bool first = b == 0;
    const int ne = T * K;
    const int t = b;

    // every global load first: all ids (clamped), this token's row vector
    int64_t idx_reg[kSmallIdsPerThread];
#pragma unroll
    for (int u = 0; u < kSmallIdsPerThread; ++u)
        idx_reg[u] = u * kSmallThreads < ne ? topk_idx[min(tid + u * kSmallThreads, ne - 1)] : -1;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (has_token && tid < nvec)
        v = x[(int64_t)t * nvec + tid];

    for (int e = tid; e < E; e += kSmallThreads)
        s_tot[e] = 0;
    if (first) {
        for (int r = tid; r < R; r += kSmallThreads)
            s_rcnt[r] = 0;
        for (int i = tid; i < T * R; i += kSmallThreads)
            s_flags[i] = 0;
    }
    if (tid < MOE_MAX_TOPK) {
        int e = -1;
        if (has_token && tid < K) {
            const int64_t id = topk_idx[(int64_t)t * K + tid];
            e = (id < 0 || id >= E) ? -1 : (int)id;
        }
        s_my[tid] = e;
        s_before[tid] = 0;
    }
    if (tid == 0)
        s_bad = 0;
    __syncthreads();

    // expert totals; in workgroup 0 the token x rank membership; for this
    // token's entries, the earlier entries of the same expert
    int bad = 0;
#pragma unroll
    for (int u = 0; u < kSmallIdsPerThread; ++u) {
        if (u * kSmallThreads >= ne) // uniform: ballots below stay convergent
            break;
        const int j = tid + u * kSmallThreads;
        int e = -1;
        if (j < ne) {
            const int64_t id = idx_reg[u];
            if (id < -1 || id >= E)
                bad = 1;
            else
                e = (int)id;
        }
        const bool has = e >= 0;
        const uint64_t same = match_same_key(e, has, nbits);
        if (has) {
            if (count_below(same) == 0)
                atomicAdd(&s_tot[e], __popcll(same));
            if (first)
                s_flags[small_div(j, K) * R + small_div(e, L)] = 1;
            if (j < t * K)
                for (int k = 0; k < K; ++k)
                    if (s_my[k] == e)
                        atomicAdd(&s_before[k], 1);
        }
    }
    if (bad)
        atomicOr(&s_bad, 1);
    __syncthreads();

    // aligned counts and their exclusive prefix sum ("/" is integer
    // division, CANN page Constraint 11), by the first wave: lane l takes
    // experts [l * per, (l + 1) * per) and a shuffle scan gives its base
    if (tid < kWave) {
        const int per = (E + kWave - 1) / kWave; // <= 8
        const int e0 = lane * per;
        int sum = 0;
        for (int c = 0; c < per; ++c)
            if (e0 + c < E)
                sum += ((s_tot[e0 + c] + a - 1) / a) * a;
        int incl = sum;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int w = __shfl_up(incl, d, kWave);
            if (lane >= d)
                incl += w;
        }
        int run = incl - sum;
        for (int c = 0; c < per; ++c)
            if (e0 + c < E) {
                s_off[e0 + c] = run;
                run += ((s_tot[e0 + c] + a - 1) / a) * a;
            }
        if (lane == kWave - 1)
            s_off[E] = incl;
    }
    // workgroup 0: is_token_in_rank rows and tokens per rank (thread (r,
    // part) owns rank r of tokens part, part + parts, ...)
    if (first) {
        const int parts = kSmallThreads / R; // >= 2 (R <= 512)
        if (tid < parts * R) {
            const int r = tid % R;
            const int part = tid / R;
            int cnt = 0;
            for (int tt = part; tt < T; tt += parts) {
                const int f = s_flags[tt * R + r];
                itr[(int64_t)tt * R + r] = f;
                cnt += f;
            }
            if (cnt)
                atomicAdd(&s_rcnt[r], cnt);
        }
    }
    __syncthreads();

    // this token's rows: expert offset + earlier entries of the expert
    // (before the token, then among its own earlier k)
    if (has_token && tid < K) {
        const int e = s_my[tid];
        int row = -1;
        if (e >= 0) {
            int dup = 0;
            for (int k = 0; k < tid; ++k)
                dup += s_my[k] == e ? 1 : 0;
            row = s_off[e] + s_before[tid] + dup;
            recv_src[row] = t * K + tid;
            if (recv_weights)
                recv_weights[row] = topk_weights ? topk_weights[(int64_t)t * K + tid] : 1.0f;
        }
        token_row[(int64_t)t * K + tid] = row;
        s_row[tid] = row;
    }
    if (first) {
        for (int e = tid; e < E; e += kSmallThreads) {
            ntpe[e] = s_tot[e];
            nrtpe[e] = s_off[e + 1] - s_off[e];
        }
        for (int e = tid; e <= E; e += kSmallThreads)
            off[e] = s_off[e];
        for (int r = tid; r < R; r += kSmallThreads)
            ntpr[r] = s_rcnt[r];
        if (tid == 0)
            *error_flag = s_bad;
    }
    // rows holding no entry: padding inside experts b, b + nblocks, ...; then
    // every row past the last expert, strided over all workgroups
    for (int e = b; e < E; e += nblocks) {
        const int lo = s_off[e] + s_tot[e];
        const int hi = s_off[e + 1];
        for (int row = lo + tid; row < hi; row += kSmallThreads)
            recv_src[row] = -1;
    }
    for (int64_t row = (int64_t)s_off[E] + (int64_t)b * kSmallThreads + tid; row < cap;
         row += (int64_t)nblocks * kSmallThreads)
        recv_src[row] = -1;
    __syncthreads();

    // the token to its rows
    if (has_token && tid < nvec) {
        for (int k = 0; k < K; ++k) {
            const int row = s_row[k];
            if (row >= 0 && row < cap)
                __builtin_nontemporal_store(v, recv + (int64_t)row * nvec + tid);
        }
    }
}

static int small_key_bits(int E)
{
    int b = 0;
    while ((1 << b) < E)
        ++b;
    return b;
}

hipError_t launch_layout_dispatch_small(const LayoutArgs &A, const void *x, int H,
                                        const float *topk_weights, void *recv_x,
                                        float *recv_weights, hipStream_t stream)
{
    const int L = A.E / A.R;
    return launch_kernel(layout_dispatch_small_kernel, dim3(A.T > 0 ? A.T : 1), dim3(kSmallThreads), 0,
                         stream, A.topk_idx, (const u32x4 *)x, A.T, A.K, A.E, A.R, L, A.a,
                         small_key_bits(A.E), H / 8, A.cap, topk_weights, A.itr, A.ntpr, A.ntpe,
                         A.nrtpe, A.off, A.token_row, A.recv_src, A.error_flag, (u32x4 *)recv_x,
                         recv_weights);
}

} // namespace moe
