// combine.hip -- top-k weighted sum of every token's expert-output rows.
//
// What is computed (Normal Mode API page, combine Description: the expert
// outputs are weighted and summed; EPBatchManager page, ep_combine(): output
// (num_local_tokens, hidden)):
//   out[t] = bf16( sum_k  w[t,k] * y[row(t,k)] )
// as an fp32 fused multiply-add chain in ascending k, rounded once to bf16
// (half to even).  Entries whose row is -1 (dropped) are skipped; no weights
// means weight 1.
//
// Design (gfx950): one single-wave workgroup per (token, 1 KiB slice of the
// row), one 16-byte vector (8 hidden elements) per lane: 14 workgroups per
// token at H = 7168.  A lane issues the loads of all K rows for its vector
// before the first FMA, so K independent 16-byte reads per lane are in
// flight (K <= 16 gives at most 64 VGPRs of staging).  The expanded rows are
// read exactly once; the rows of one token are scattered over the receive
// buffer, but each load instruction reads 1 KiB contiguous bytes of one row.
// Row indices and weights are uniform per workgroup and live in scalar
// registers.  One-wave workgroups let a CU hold its full 32 waves at any H
// (whole-row workgroups of 896 lanes stop at 28) and shorten the grid's tail.
// The row loads are nontemporal; the output is stored nontemporally when it
// is too large for the memory-side cache (see kCombineNtOutBytes).
//
// The epilogues named by the pages (EPBatchManager
// page, ep_combine(): shared expert outputs added to the reduced routed
// outputs; CANN page: the CombineAddRmsNorm companion): the shared-expert row
// and the residual row of the token are loaded with the expert rows and
// added to the fp32 sum (in the slice kernel when there is no
// normalisation), which is stored, and optionally normalised
// (combine_fused_kernel, one workgroup per token),
//   norm = s / sqrt(mean(s^2) + eps) * gamma,
// from the fp32 values (sum of squares: per lane, then wave shuffles, then
// the waves in order through LDS -- a fixed order, so results are
// deterministic).  This saves a full [T, H] read and write per epilogue.
#include "device_common.h"
#include "launch.h"

#include "../../include/moe_dispatch_combine.h"

namespace moe {

// One wave per (token, 64-vector slice of its row): 1 KiB of each of the
// token's K rows in, 1 KiB out.  Small one-wave workgroups let every CU hold
// its full complement of waves whatever H is (a whole-row workgroup of 896
// lanes at H = 7168 leaves a CU at 28 of 32 waves) and keep the tail of the
// grid short.  shared / residual (nullable) are the un-normalised epilogues.
// NT_OUT: nontemporal stores of `out`, chosen by the launcher for outputs
// too large for the 256 MB memory-side cache.  (A compile-time choice: with
// a runtime flag the compiler merges the two stores into one ordinary
// store.)
template <int KMAX, bool NT_OUT>
__global__ __launch_bounds__(kWave) void combine_slice_kernel(
    const u32x4 *__restrict__ y, int nvec, int nslices, int64_t nitems, int K,
    const int32_t *__restrict__ token_row, const float *__restrict__ topk_weights, int64_t cap,
    const u32x4 *__restrict__ shared, const u32x4 *__restrict__ residual,
    u32x4 *__restrict__ out)
{
    for (int64_t b = blockIdx.x; b < nitems; b += gridDim.x) {
        const int64_t t = b / nslices;
        const int i = (int)(b - t * nslices) * kWave + (int)threadIdx.x;
        int rows[KMAX];
        float wts[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            rows[k] = -1;
            wts[k] = 0.0f;
            if (k < K) {
                const int r = token_row[t * K + k];
                rows[k] = (r >= 0 && r < cap) ? r : -1;
                wts[k] = topk_weights ? topk_weights[t * K + k] : 1.0f;
            }
        }
        if (i >= nvec)
            continue;
        u32x4 yv[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (rows[k] >= 0)
                yv[k] = __builtin_nontemporal_load(y + (int64_t)rows[k] * nvec + i);
        u32x4 sv = u32x4{0u, 0u, 0u, 0u}, rv = u32x4{0u, 0u, 0u, 0u};
        if (shared)
            sv = shared[t * nvec + i];
        if (residual)
            rv = residual[t * nvec + i];
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (rows[k] < 0)
                continue;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[2 * c] = __builtin_fmaf(wts[k], bf16_lo(yv[k][c]), acc[2 * c]);
                acc[2 * c + 1] = __builtin_fmaf(wts[k], bf16_hi(yv[k][c]), acc[2 * c + 1]);
            }
        }
        if (shared)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[2 * c] += bf16_lo(sv[c]);
                acc[2 * c + 1] += bf16_hi(sv[c]);
            }
        if (residual)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[2 * c] += bf16_lo(rv[c]);
                acc[2 * c + 1] += bf16_hi(rv[c]);
            }
        u32x4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            o[c] = pack_bf16x2(acc[2 * c], acc[2 * c + 1]);
        if constexpr (NT_OUT)
            __builtin_nontemporal_store(o, out + t * nvec + i);
        else
            out[t * nvec + i] = o;
    }
}

// With RMS normalisation: one workgroup per token (the sum of squares spans
// the row).  Both outputs are stored nontemporally: with ordinary stores
// their 2 x 2H bytes per token stayed dirty in the caches, and writing them
// back slowed this kernel and the next dispatch (headline shape with shared
// output, residual and RMSNorm, whole steps: 240 -> 218 us; the kernel
// 121 -> 113 us).
template <int VPT, int KMAX>
__global__ __launch_bounds__(kRowMaxThreads) void combine_fused_kernel(
    const u32x4 *__restrict__ y, int nvec, int K, const int32_t *__restrict__ token_row,
    const float *__restrict__ topk_weights, int64_t cap, const u32x4 *__restrict__ shared,
    const u32x4 *__restrict__ residual, const u32x4 *__restrict__ gamma, float eps,
    u32x4 *__restrict__ out, u32x4 *__restrict__ out_norm)
{
    __shared__ float s_ss[kRowMaxThreads / kWave];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    int rows[KMAX];
    float wts[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        rows[k] = -1;
        wts[k] = 0.0f;
        if (k < K) {
            const int r = token_row[(int64_t)t * K + k];
            rows[k] = (r >= 0 && r < cap) ? r : -1;
            wts[k] = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;
        }
    }
    float acc[VPT][8];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int i = min(tid + j * nthr, nvec - 1); // clamped: always in bounds
        u32x4 yv[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (rows[k] >= 0)
                yv[k] = __builtin_nontemporal_load(y + (int64_t)rows[k] * nvec + i);
        u32x4 sv = u32x4{0u, 0u, 0u, 0u}, rv = u32x4{0u, 0u, 0u, 0u};
        if (shared)
            sv = shared[(int64_t)t * nvec + i];
        if (residual)
            rv = residual[(int64_t)t * nvec + i];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[j][e] = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (rows[k] < 0)
                continue;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[j][2 * c] = __builtin_fmaf(wts[k], bf16_lo(yv[k][c]), acc[j][2 * c]);
                acc[j][2 * c + 1] = __builtin_fmaf(wts[k], bf16_hi(yv[k][c]), acc[j][2 * c + 1]);
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (shared) {
                acc[j][2 * c] += bf16_lo(sv[c]);
                acc[j][2 * c + 1] += bf16_hi(sv[c]);
            }
            if (residual) {
                acc[j][2 * c] += bf16_lo(rv[c]);
                acc[j][2 * c + 1] += bf16_hi(rv[c]);
            }
        }
        if (tid + j * nthr < nvec) {
            u32x4 o;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                o[c] = pack_bf16x2(acc[j][2 * c], acc[j][2 * c + 1]);
            __builtin_nontemporal_store(o, out + (int64_t)t * nvec + tid + j * nthr);
        }
    }
    if (!out_norm)
        return;

    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        if (tid + j * nthr < nvec)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ss = __builtin_fmaf(acc[j][e], acc[j][e], ss);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        ss += __shfl_xor(ss, o, kWave);
    if ((tid & (kWave - 1)) == 0)
        s_ss[tid / kWave] = ss;
    __syncthreads();
    float total = 0.0f;
    for (int w = 0; w < nthr / kWave; ++w)
        total += s_ss[w];
    const float inv = 1.0f / sqrtf(total / (float)(nvec * 8) + eps);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int i = tid + j * nthr;
        if (i < nvec) {
            const u32x4 g = gamma[i];
            u32x4 o;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                o[c] = pack_bf16x2(acc[j][2 * c] * inv * bf16_lo(g[c]),
                                   acc[j][2 * c + 1] * inv * bf16_hi(g[c]));
            __builtin_nontemporal_store(o, out_norm + (int64_t)t * nvec + i);
        }
    }
}

// Outputs of at least this many bytes are stored nontemporally by the slice
// kernel.  Measured in whole steps (layout, dispatch, combine): at 32768
// tokens x 7168 (470 MB of output) the combine went 1419 -> 1389 us; at
// 4096 and 8192 tokens (59 and 117 MB, which the memory-side cache holds)
// nontemporal stores were level or 0.5 % slower.
constexpr int64_t kCombineNtOutBytes = int64_t(256) << 20;

template <bool NT>
static hipError_t launch_slices_k(int K, const SliceGrid &g, int nvec, hipStream_t stream,
                                  const u32x4 *y, const int32_t *token_row, const float *w,
                                  int64_t cap, const u32x4 *sh, const u32x4 *res, u32x4 *out)
{
    const dim3 grid(g.blocks), block(kWave);
    const int nslices = g.nslices;
    const int64_t nitems = g.nitems;
    if (K <= 1)
        return launch_kernel(combine_slice_kernel<1, NT>, grid, block, 0, stream, y, nvec, nslices, nitems, K, token_row, w, cap, sh, res, out);
    if (K <= 2)
        return launch_kernel(combine_slice_kernel<2, NT>, grid, block, 0, stream, y, nvec, nslices, nitems, K, token_row, w, cap, sh, res, out);
    if (K <= 4)
        return launch_kernel(combine_slice_kernel<4, NT>, grid, block, 0, stream, y, nvec, nslices, nitems, K, token_row, w, cap, sh, res, out);
    if (K <= 8)
        return launch_kernel(combine_slice_kernel<8, NT>, grid, block, 0, stream, y, nvec, nslices, nitems, K, token_row, w, cap, sh, res, out);
    return launch_kernel(combine_slice_kernel<16, NT>, grid, block, 0, stream, y, nvec, nslices, nitems, K, token_row, w, cap, sh, res, out);
}

static hipError_t launch_slices(int K, int64_t T, int nvec, hipStream_t stream, const u32x4 *y,
                                const int32_t *token_row, const float *w, int64_t cap,
                                const u32x4 *sh, const u32x4 *res, u32x4 *out)
{
    const SliceGrid g = slice_grid(T, nvec, 1);
    if (T * nvec * 16 >= kCombineNtOutBytes)
        return launch_slices_k<true>(K, g, nvec, stream, y, token_row, w, cap, sh, res, out);
    return launch_slices_k<false>(K, g, nvec, stream, y, token_row, w, cap, sh, res, out);
}

hipError_t launch_combine(const void *y, int64_t cap, int T, int H, int K,
                          const int32_t *token_row, const float *topk_weights, void *out,
                          hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    return launch_slices(K, T, H / 8, stream, (const u32x4 *)y, token_row, topk_weights, cap,
                         nullptr, nullptr, (u32x4 *)out);
}

template <int VPT>
static hipError_t launch_fused_k(int kmax, dim3 grid, dim3 block, hipStream_t stream,
                                 const u32x4 *y, int nvec, int K, const int32_t *token_row,
                                 const float *w, int64_t cap, const u32x4 *sh, const u32x4 *res,
                                 const u32x4 *g, float eps, u32x4 *out, u32x4 *norm)
{
    switch (kmax) {
    case 1:
        return launch_kernel(combine_fused_kernel<VPT, 1>, grid, block, 0, stream, y, nvec, K, token_row, w, cap, sh, res, g, eps, out, norm);
    case 2:
        return launch_kernel(combine_fused_kernel<VPT, 2>, grid, block, 0, stream, y, nvec, K, token_row, w, cap, sh, res, g, eps, out, norm);
    case 4:
        return launch_kernel(combine_fused_kernel<VPT, 4>, grid, block, 0, stream, y, nvec, K, token_row, w, cap, sh, res, g, eps, out, norm);
    case 8:
        return launch_kernel(combine_fused_kernel<VPT, 8>, grid, block, 0, stream, y, nvec, K, token_row, w, cap, sh, res, g, eps, out, norm);
    default:
        return launch_kernel(combine_fused_kernel<VPT, 16>, grid, block, 0, stream, y, nvec, K, token_row, w, cap, sh, res, g, eps, out, norm);
    }
}

hipError_t launch_combine_fused(const void *y, int64_t cap, int T, int H, int K,
                                const int32_t *token_row, const float *topk_weights,
                                const void *shared, const void *residual, const void *gamma,
                                float eps, void *out, void *out_norm, hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    const int nvec = H / 8;
    if (!out_norm) // no row-wide reduction: the slice kernel
        return launch_slices(K, T, nvec, stream, (const u32x4 *)y, token_row, topk_weights, cap,
                             (const u32x4 *)shared, (const u32x4 *)residual, (u32x4 *)out);
    const int threads = row_block_threads(nvec);
    const int vpt = (nvec + threads - 1) / threads;
    const int kmax = K <= 1 ? 1 : K <= 2 ? 2 : K <= 4 ? 4 : K <= 8 ? 8 : 16;
    const dim3 grid(T), block(threads);
    if (vpt == 1)
        return launch_fused_k<1>(kmax, grid, block, stream, (const u32x4 *)y, nvec, K, token_row,
                                 topk_weights, cap, (const u32x4 *)shared, (const u32x4 *)residual,
                                 (const u32x4 *)gamma, eps, (u32x4 *)out, (u32x4 *)out_norm);
    return launch_fused_k<2>(kmax, grid, block, stream, (const u32x4 *)y, nvec, K, token_row,
                             topk_weights, cap, (const u32x4 *)shared, (const u32x4 *)residual,
                             (const u32x4 *)gamma, eps, (u32x4 *)out, (u32x4 *)out_norm);
}

} // namespace moe
