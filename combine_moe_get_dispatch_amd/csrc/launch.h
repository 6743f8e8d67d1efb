// launch.h -- internal interface between the C ABI (moe_api.hip) and the
// kernel launchers.  Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace moe {

// Launch `kernel` and return the status of this launch alone.  (The
// hipGetLastError() idiom would also report an error some earlier, unrelated
// HIP call of the caller left pending.)  Arguments are converted to the
// kernel's parameter types and passed by address, as hipLaunchKernel expects.
template <typename... KArgs, typename Tuple, size_t... I>
hipError_t launch_with_tuple(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                             hipStream_t stream, Tuple &params, std::index_sequence<I...>)
{
    void *argv[] = {(void *)&std::get<I>(params)..., nullptr};
    return hipLaunchKernel((const void *)kernel, grid, block, argv, shmem, stream);
}

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, Args... args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> params(static_cast<KArgs>(args)...);
    return launch_with_tuple(kernel, grid, block, shmem, stream, params,
                             std::index_sequence_for<KArgs...>{});
}

// Launch shape of the row kernels (per-token dispatch, normalised combine):
// one workgroup per token, one 16-byte vector per lane; the workgroup covers
// the row with ceil(nvec / 64) waves (at most 16), and a lane takes a second
// vector only when the row has more than 1024 vectors (H > 8192).
constexpr int kRowMaxThreads = 1024;
// Upper bound on the grid of grid-stride kernels (work items beyond it are
// taken by the same workgroups in later iterations).  A test build lowers it
// so that the later iterations run at small sizes.
#ifndef MOE_MAX_GRID_LOG2
#define MOE_MAX_GRID_LOG2 24
#endif
constexpr int64_t kMaxGrid = int64_t(1) << MOE_MAX_GRID_LOG2;
inline int row_block_threads(int nvec)
{
    const int t = (nvec + 63) / 64 * 64;
    return t < kRowMaxThreads ? t : kRowMaxThreads;
}

// Launch shape of the slice kernels: one wave per (token, 64-vector slice of
// the row), `waves` such items per workgroup, at most kMaxGrid workgroups
// (grid-stride beyond).  Unquantised and pre-quantised dispatch use four
// waves per workgroup, combine one.
constexpr int kSliceWaves = 4;
struct SliceGrid {
    int nslices;    // slices per row
    int64_t nitems; // T * nslices
    unsigned blocks;
};
inline SliceGrid slice_grid(int64_t T, int nvec, int waves)
{
    SliceGrid g;
    g.nslices = (nvec + 63) / 64;
    g.nitems = T * g.nslices;
    const int64_t b = (g.nitems + waves - 1) / waves;
    g.blocks = (unsigned)(b < kMaxGrid ? b : kMaxGrid);
    return g;
}

// How the layout splits the T*K routing entries into chunks of whole tokens.
// Every chunk is handled by one workgroup in both layout kernels.  The
// limits keep one chunk's working set in LDS: its expert ids as int16
// (kMaxChunkEntries) and its token x rank membership bytes (kMaxChunkFlags).
constexpr int kLayoutTargetChunks = 64;
constexpr int kMaxChunkEntries = 8192;
constexpr int kMaxChunkFlags = 16384;
// Batches of at most this many routing entries (and T*R <= kMaxChunkFlags)
// are laid out by one workgroup in one launch.
constexpr int kSingleLayoutMaxEntries = 3072;

// From this many count-table cells (chunks x E rounded up to 4) on, a
// column-scan launch between the two kernels forms each chunk's prefix row
// and the expert totals once, so that a rank workgroup reads two rows
// instead of reducing the whole table itself (whose size grows as chunks x E
// when many ranks force small chunks).
constexpr int64_t kLayoutScanMinCells = 131072;

struct LayoutPlan {
    int tokens_per_chunk;
    int num_chunks;
    size_t workspace_bytes; // count table [chunks][Ep] + rank table [chunks][R] + flags [chunks]
                            // (+ prefix table [chunks][Ep] + totals [Ep] with scan), Ep = E rounded up to 4
    bool single;            // the whole batch in one workgroup (no workspace, one launch)
    bool scan;              // three launches: count, column scan, rank
};

inline LayoutPlan plan_layout(int T, int K, int E, int R)
{
    LayoutPlan p{0, 0, 0, false, false};
    if ((int64_t)T * K <= kSingleLayoutMaxEntries && (int64_t)T * R <= kMaxChunkFlags) {
        p.single = true; // includes T == 0
        p.tokens_per_chunk = T;
        p.num_chunks = T > 0 ? 1 : 0;
        return p;
    }
    int tpc = (T + kLayoutTargetChunks - 1) / kLayoutTargetChunks;
    if (tpc > kMaxChunkEntries / K)
        tpc = kMaxChunkEntries / K;
    if (tpc > kMaxChunkFlags / R)
        tpc = kMaxChunkFlags / R;
    if (tpc < 1)
        tpc = 1;
    p.tokens_per_chunk = tpc;
    p.num_chunks = (T + tpc - 1) / tpc;
    const size_t Ep = (size_t)((E + 3) & ~3);
    p.scan = (int64_t)p.num_chunks * (int64_t)Ep >= kLayoutScanMinCells;
    size_t cells = (size_t)p.num_chunks * (Ep + (size_t)R + 1);
    if (p.scan)
        cells += (size_t)p.num_chunks * Ep + Ep;
    p.workspace_bytes = cells * sizeof(int32_t);
    return p;
}

struct LayoutArgs {
    const int64_t *topk_idx;
    int T, K, E, R, a;
    int64_t cap;
    int32_t *ntpr, *ntpe, *itr, *nrtpe, *off, *token_row, *recv_src, *error_flag;
    int32_t *workspace;
};

hipError_t launch_layout(const LayoutArgs &args, const LayoutPlan &plan, hipStream_t stream);

hipError_t launch_dispatch(const void *x, int T, int H, int K, const int32_t *token_row,
                           const float *topk_weights, int64_t cap, int quant_mode, void *recv_x,
                           void *recv_scales, float *recv_weights, hipStream_t stream);

hipError_t launch_dispatch_static(const void *x, int T, int H, int K, const int32_t *token_row,
                                  const float *topk_weights, int64_t cap, const float *scales,
                                  int num_scales, void *recv_x, float *recv_weights,
                                  hipStream_t stream);

hipError_t launch_dispatch_static_expert(const void *x, int T, int H, int K, const int64_t *topk_idx,
                                         int E, const int32_t *token_row,
                                         const float *topk_weights, int64_t cap,
                                         const float *scales, void *recv_x, float *recv_weights,
                                         hipStream_t stream);

hipError_t launch_dispatch_rows(const void *data, int T, int row_bytes, const void *scales,
                                int scale_bytes, int K, const int32_t *token_row,
                                const float *topk_weights, int64_t cap, void *recv_data,
                                void *recv_scales, float *recv_weights, hipStream_t stream);

hipError_t launch_combine(const void *y, int64_t cap, int T, int H, int K,
                          const int32_t *token_row, const float *topk_weights, void *out,
                          hipStream_t stream);

hipError_t launch_combine_fused(const void *y, int64_t cap, int T, int H, int K,
                                const int32_t *token_row, const float *topk_weights,
                                const void *shared, const void *residual, const void *gamma,
                                float eps, void *out, void *out_norm, hipStream_t stream);

} // namespace moe
