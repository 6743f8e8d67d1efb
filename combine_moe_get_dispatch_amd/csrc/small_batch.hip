// small_batch.hip -- layout and dispatch (bf16, or per-token int8 / FP8) of
// a decode-sized batch in one launch.
//
// What is computed: exactly what moe_get_dispatch_layout followed by
// moe_dispatch (unquantised, or with per-token quantisation) compute (Normal
// Mode API page, dispatch Parameters / Return Values; EPBatchManager page,
// ep_dispatch(); CANN aclnnMoeDistributeDispatchV2 page, Formula Case 3 and
// Constraint 1, deterministic):
//   c[e]        = number of entries with topk_idx == e
//   off[e]      = sum over e' < e of ceil(c[e'] / a) * a
//   row(t, k)   = off[e] + #{ j < tK : idx_j == e } + #{ k' < k : idx[t, k'] == e }
//   recv[row(t, k)] = x[t], or its per-token codes with their scale
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
// nontemporal stores (or, for the per-token modes, reduces the row maximum
// from per-wave maxima taken before the second barrier and stores the codes
// and the scale).  Workgroups never wait for one another: all of them
// compute identical totals and offsets from the same ids.  Workgroup 0 also
// writes the per-expert and per-rank outputs and every is_token_in_rank row;
// the padding and unused rows of recv_src are spread over all workgroups.
// The redundant layout work grows as T * T*K, so the path is limited to
// small batches (kSmallMaxTokens tokens, kSmallMaxEntries entries).
#include "device_common.h"
#include "element_codecs.h"
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

// QUANT: per-token dynamic quantisation to D (CANN page, Formula Case 3, as
// dispatch_pertoken_kernel computes it): the row maximum from per-wave
// maxima, dynamicScales = dstTypeMax / max in IEEE fp32, codes from one fp32
// product each, scale 1 / dynamicScales; codes 0 and scale 0 when
// dynamicScales is not finite.  Otherwise the bf16 row is copied.
template <bool QUANT, Dst D>
__global__ __launch_bounds__(kSmallThreads) void layout_dispatch_small_kernel(
    const int64_t *__restrict__ topk_idx, const u32x4 *__restrict__ x, int T, int K, int E, int R,
    int L, int a, int nbits, int nvec, int64_t cap, const float *__restrict__ topk_weights,
    int32_t *__restrict__ itr, int32_t *__restrict__ ntpr, int32_t *__restrict__ ntpe,
    int32_t *__restrict__ nrtpe, int32_t *__restrict__ off, int32_t *__restrict__ token_row,
    int32_t *__restrict__ recv_src, int32_t *__restrict__ error_flag, void *__restrict__ recv,
    float *__restrict__ recv_scales, float *__restrict__ recv_weights)
{
    __shared__ int s_tot[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_rcnt[MOE_MAX_EXPERTS];
    __shared__ uint8_t s_flags[kSmallMaxFlags];
    __shared__ int s_my[MOE_MAX_TOPK];     // this token's experts (-1: dropped)
    __shared__ int s_before[MOE_MAX_TOPK]; // entries before this token holding s_my[k]
    __shared__ int s_row[MOE_MAX_TOPK];
    __shared__ int s_bad;
    __shared__ float s_wmax[kSmallThreads / kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
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
    if (QUANT) { // this wave's share of the row maximum (lanes past the row hold zeros)
        float m = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            m = fmaxf(m, fabsf(bf16_lo(v[c])));
            m = fmaxf(m, fabsf(bf16_hi(v[c])));
        }
        m = wave_max(m);
        if (lane == 0)
            s_wmax[wave] = m;
    }
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
                sum += a == 1 ? s_tot[e0 + c] : ((s_tot[e0 + c] + a - 1) / a) * a;
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
                run += a == 1 ? s_tot[e0 + c] : ((s_tot[e0 + c] + a - 1) / a) * a;
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

    // the row's codes and scale
    float scale = 0.0f;
    u32x2 q = u32x2{0u, 0u};
    if (QUANT) {
        float m = s_wmax[0];
        for (int w = 1; w < kSmallThreads / kWave; ++w)
            m = fmaxf(m, s_wmax[w]);
        const float ds = DstTraits<D>::kMax / m; // IEEE division (correctly rounded fp32 divide)
        const bool degenerate = !(ds <= 3.402823466e38f);
        scale = 1.0f / ds;
        uint32_t wd[2] = {0u, 0u};
        if (!degenerate) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t lo = DstTraits<D>::code(bf16_lo(v[c]) * ds, sign_lo(v[c]));
                const uint32_t hi = DstTraits<D>::code(bf16_hi(v[c]) * ds, sign_hi(v[c]));
                wd[c >> 1] |= (lo | (hi << 8)) << (16 * (c & 1));
            }
        }
        q = u32x2{wd[0], wd[1]};
    }

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
        }
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

    // this token's layout entries, row weights and scales (stored after the
    // barrier, so that no wave waits for them before the copy)
    if (has_token && tid < K) {
        const int row = s_row[tid];
        token_row[(int64_t)t * K + tid] = row;
        if (row >= 0) {
            recv_src[row] = t * K + tid;
            if (QUANT)
                recv_scales[row] = scale;
            if (recv_weights)
                recv_weights[row] = topk_weights ? topk_weights[(int64_t)t * K + tid] : 1.0f;
        }
    }

    // the token (or its codes) to its rows
    if (has_token && tid < nvec) {
        for (int k = 0; k < K; ++k) {
            const int row = s_row[k];
            if (row < 0 || row >= cap)
                continue;
            if (QUANT)
                __builtin_nontemporal_store(q, (u32x2 *)recv + (int64_t)row * nvec + tid);
            else
                __builtin_nontemporal_store(v, (u32x4 *)recv + (int64_t)row * nvec + tid);
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
                                        const float *topk_weights, int quant_mode, void *recv_x,
                                        float *recv_scales, float *recv_weights, hipStream_t stream)
{
    const int L = A.E / A.R;
    auto go = [&](auto kernel) {
        return launch_kernel(kernel, dim3(A.T > 0 ? A.T : 1), dim3(kSmallThreads), 0, stream,
                             A.topk_idx, (const u32x4 *)x, A.T, A.K, A.E, A.R, L, A.a,
                             small_key_bits(A.E), H / 8, A.cap, topk_weights, A.itr, A.ntpr, A.ntpe,
                             A.nrtpe, A.off, A.token_row, A.recv_src, A.error_flag, recv_x,
                             recv_scales, recv_weights);
    };
    switch (quant_mode) {
    case MOE_QUANT_NONE:
        return go(layout_dispatch_small_kernel<false, Dst::Int8>);
    case MOE_QUANT_INT8_PER_TOKEN:
        return go(layout_dispatch_small_kernel<true, Dst::Int8>);
    case MOE_QUANT_FP8_E4M3_PER_TOKEN:
        return go(layout_dispatch_small_kernel<true, Dst::E4M3>);
    case MOE_QUANT_FP8_E5M2_PER_TOKEN:
        return go(layout_dispatch_small_kernel<true, Dst::E5M2>);
    default:
        return hipErrorInvalidValue;
    }
}

} // namespace moe
