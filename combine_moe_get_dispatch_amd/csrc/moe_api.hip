// moe_api.hip -- the C ABI declared in include/moe_dispatch_combine.h.
//
// Each entry point validates its arguments on the host first and returns a
// negative status without touching HIP when they are wrong; only then does it
// queue kernels on the caller's stream.  Nothing is allocated and nothing
// waits for the GPU.
#include "launch.h"
#include "small_batch.h"

#include "../../include/moe_dispatch_combine.h"

#include <climits>
#include <cmath>
#include <mutex>

using namespace moe;

// Layout workspace of moe_get_dispatch_layout_noalloc, for callers that
// cannot allocate.  One copy per GPU, held until the process ends; every
// call on a GPU shares it (calls that overlap on one GPU race).  The host
// name of the array is not a device address: kernels get the address that
// hipGetSymbolAddress reports for the GPU they run on.
static __device__ __align__(256) int32_t scratch[MOE_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices]; // device address of `scratch` per GPU, found on first use

// Device address of `scratch` on the GPU `stream` belongs to (NULL on a HIP
// error).  Looked up once per GPU, with that GPU current.
void *scratch_for_stream(hipStream_t stream)
{
    int dev = -1;
    if (stream == nullptr) {
        if (hipGetDevice(&dev) != hipSuccess)
            return nullptr;
    } else if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxScratchDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        int prev = -1;
        if (hipGetDevice(&prev) != hipSuccess)
            return nullptr;
        if (prev != dev && hipSetDevice(dev) != hipSuccess)
            return nullptr;
        void *p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (prev != dev && hipSetDevice(prev) != hipSuccess)
            return nullptr;
        if (err != hipSuccess || p == nullptr)
            return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_layout_sizes(int T, int K, int E, int R, int a, int64_t cap)
{
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS || R < 1 || R > E ||
        E % R != 0 || a < 1)
        return MOE_ERR_INVALID_ARG;
    const int64_t bound = (int64_t)T * K + (int64_t)E * (a - 1);
    if (bound > INT32_MAX)
        return MOE_ERR_INVALID_ARG;
    if (cap < bound || cap > INT32_MAX)
        return MOE_ERR_CAPACITY;
    return MOE_OK;
}

int check_rows_sizes(int T, int H, int K, int64_t cap, int quant_mode)
{
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK || H < MOE_HIDDEN_MULTIPLE || H > MOE_MAX_HIDDEN ||
        H % MOE_HIDDEN_MULTIPLE != 0 || cap < 0 || cap > INT32_MAX)
        return MOE_ERR_INVALID_ARG;
    if (quant_mode != MOE_QUANT_NONE && quant_mode != MOE_QUANT_INT8_PER_TOKEN &&
        quant_mode != MOE_QUANT_MXFP8_E4M3 && quant_mode != MOE_QUANT_FP8_E4M3_PER_TOKEN &&
        quant_mode != MOE_QUANT_FP8_E5M2_PER_TOKEN && quant_mode != MOE_QUANT_MXFP8_E5M2 &&
        quant_mode != MOE_QUANT_FP8_E4M3_PER_GROUP && quant_mode != MOE_QUANT_FP8_E5M2_PER_GROUP)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

bool fp32_scales(int quant_mode)
{
    return quant_mode == MOE_QUANT_INT8_PER_TOKEN || quant_mode == MOE_QUANT_FP8_E4M3_PER_TOKEN ||
           quant_mode == MOE_QUANT_FP8_E5M2_PER_TOKEN || quant_mode == MOE_QUANT_FP8_E4M3_PER_GROUP ||
           quant_mode == MOE_QUANT_FP8_E5M2_PER_GROUP;
}

int check_prequant_sizes(int T, int row_bytes, int scale_bytes, int K, int64_t cap)
{
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK || row_bytes < 16 || row_bytes > 32768 ||
        row_bytes % 16 != 0 || scale_bytes < 0 || scale_bytes > 4096 || cap < 0 || cap > INT32_MAX)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

} // namespace

extern "C" {

int64_t moe_recv_capacity_bound(int num_tokens, int num_topk, int num_experts, int expert_alignment)
{
    if (num_tokens < 0 || num_topk < 1 || num_experts < 1 || expert_alignment < 1)
        return -1;
    return (int64_t)num_tokens * num_topk + (int64_t)num_experts * (expert_alignment - 1);
}

size_t moe_layout_workspace_bytes(int num_tokens, int num_topk, int num_experts, int num_ranks)
{
    if (num_tokens < 0 || num_topk < 1 || num_topk > MOE_MAX_TOPK || num_experts < 1 ||
        num_experts > MOE_MAX_EXPERTS || num_ranks < 1 || num_ranks > num_experts ||
        num_experts % num_ranks != 0)
        return 0;
    return plan_layout(num_tokens, num_topk, num_experts, num_ranks).workspace_bytes;
}

int moe_get_dispatch_layout(const int64_t *topk_idx, int num_tokens, int num_topk,
                            int num_experts, int num_ranks, int expert_alignment,
                            int64_t recv_capacity, int32_t *num_tokens_per_rank,
                            int32_t *num_tokens_per_expert, int32_t *is_token_in_rank,
                            int32_t *num_recv_tokens_per_expert, int32_t *expert_offsets,
                            int32_t *token_row, int32_t *recv_src, int32_t *error_flag,
                            void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const int T = num_tokens, K = num_topk, E = num_experts, R = num_ranks, a = expert_alignment;
    int rc = check_layout_sizes(T, K, E, R, a, recv_capacity);
    if (rc != MOE_OK)
        return rc;
    if (!num_tokens_per_rank || !num_tokens_per_expert || !num_recv_tokens_per_expert ||
        !expert_offsets || !error_flag)
        return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !is_token_in_rank || !token_row))
        return MOE_ERR_INVALID_ARG;
    if (recv_capacity > 0 && !recv_src)
        return MOE_ERR_INVALID_ARG;
    const LayoutPlan plan = plan_layout(T, K, E, R);
    if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
        return MOE_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 15u) != 0)
        return MOE_ERR_WORKSPACE;

    LayoutArgs args;
    args.topk_idx = topk_idx;
    args.T = T;
    args.K = K;
    args.E = E;
    args.R = R;
    args.a = a;
    args.cap = recv_capacity;
    args.ntpr = num_tokens_per_rank;
    args.ntpe = num_tokens_per_expert;
    args.itr = is_token_in_rank;
    args.nrtpe = num_recv_tokens_per_expert;
    args.off = expert_offsets;
    args.token_row = token_row;
    args.recv_src = recv_src;
    args.error_flag = error_flag;
    args.workspace = (int32_t *)workspace;
    return launch_layout(args, plan, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_get_dispatch_layout_noalloc(const int64_t *topk_idx, int num_tokens, int num_topk,
                                    int num_experts, int num_ranks, int expert_alignment,
                                    int64_t recv_capacity, int32_t *num_tokens_per_rank,
                                    int32_t *num_tokens_per_expert, int32_t *is_token_in_rank,
                                    int32_t *num_recv_tokens_per_expert, int32_t *expert_offsets,
                                    int32_t *token_row, int32_t *recv_src, int32_t *error_flag,
                                    hipStream_t stream)
{
    const int T = num_tokens, K = num_topk, E = num_experts, R = num_ranks, a = expert_alignment;
    int rc = check_layout_sizes(T, K, E, R, a, recv_capacity);
    if (rc != MOE_OK)
        return rc;
    if (!num_tokens_per_rank || !num_tokens_per_expert || !num_recv_tokens_per_expert ||
        !expert_offsets || !error_flag)
        return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !is_token_in_rank || !token_row))
        return MOE_ERR_INVALID_ARG;
    if (recv_capacity > 0 && !recv_src)
        return MOE_ERR_INVALID_ARG;
    const LayoutPlan plan = plan_layout(T, K, E, R);
    if (plan.workspace_bytes > MOE_NOALLOC_SCRATCH_BYTES)
        return MOE_ERR_SCRATCH;
    void *ws = nullptr;
    if (plan.workspace_bytes > 0) {
        ws = scratch_for_stream(stream);
        if (ws == nullptr)
            return MOE_ERR_HIP;
    }

    LayoutArgs args;
    args.topk_idx = topk_idx;
    args.T = T;
    args.K = K;
    args.E = E;
    args.R = R;
    args.a = a;
    args.cap = recv_capacity;
    args.ntpr = num_tokens_per_rank;
    args.ntpe = num_tokens_per_expert;
    args.itr = is_token_in_rank;
    args.nrtpe = num_recv_tokens_per_expert;
    args.off = expert_offsets;
    args.token_row = token_row;
    args.recv_src = recv_src;
    args.error_flag = error_flag;
    args.workspace = (int32_t *)ws;
    return launch_layout(args, plan, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_layout_and_dispatch_fits(int num_tokens, int hidden, int num_topk, int num_ranks)
{
    return small_batch_fits(num_tokens, hidden, num_topk, num_ranks) ? 1 : 0;
}

int moe_layout_and_dispatch(const int64_t *topk_idx, const void *x, int num_tokens, int hidden,
                            int num_topk, int num_experts, int num_ranks, int expert_alignment,
                            int64_t recv_capacity, const float *topk_weights, int quant_mode,
                            int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                            int32_t *is_token_in_rank, int32_t *num_recv_tokens_per_expert,
                            int32_t *expert_offsets, int32_t *token_row, int32_t *recv_src,
                            int32_t *error_flag, void *recv_x, float *recv_scales,
                            float *recv_weights, hipStream_t stream)
{
    const int T = num_tokens, H = hidden, K = num_topk, E = num_experts, R = num_ranks,
              a = expert_alignment;
    int rc = check_layout_sizes(T, K, E, R, a, recv_capacity);
    if (rc != MOE_OK)
        return rc;
    rc = check_rows_sizes(T, H, K, recv_capacity, MOE_QUANT_NONE);
    if (rc != MOE_OK)
        return rc;
    if (!small_batch_fits(T, H, K, R))
        return MOE_ERR_INVALID_ARG;
    const bool per_token = quant_mode == MOE_QUANT_INT8_PER_TOKEN ||
                           quant_mode == MOE_QUANT_FP8_E4M3_PER_TOKEN ||
                           quant_mode == MOE_QUANT_FP8_E5M2_PER_TOKEN;
    if (quant_mode != MOE_QUANT_NONE && !per_token)
        return MOE_ERR_INVALID_ARG;
    if (T > 0 && per_token && !recv_scales)
        return MOE_ERR_INVALID_ARG;
    if (!num_tokens_per_rank || !num_tokens_per_expert || !num_recv_tokens_per_expert ||
        !expert_offsets || !error_flag)
        return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !is_token_in_rank || !token_row || !x || !recv_x ||
                  !aligned16(x) || !aligned16(recv_x)))
        return MOE_ERR_INVALID_ARG;
    if (recv_capacity > 0 && !recv_src)
        return MOE_ERR_INVALID_ARG;
    if (per_token && ((uintptr_t)recv_scales & 3u) != 0)
        return MOE_ERR_INVALID_ARG;
    if (recv_weights && ((uintptr_t)recv_weights & 3u) != 0)
        return MOE_ERR_INVALID_ARG;

    LayoutArgs args;
    args.topk_idx = topk_idx;
    args.T = T;
    args.K = K;
    args.E = E;
    args.R = R;
    args.a = a;
    args.cap = recv_capacity;
    args.ntpr = num_tokens_per_rank;
    args.ntpe = num_tokens_per_expert;
    args.itr = is_token_in_rank;
    args.nrtpe = num_recv_tokens_per_expert;
    args.off = expert_offsets;
    args.token_row = token_row;
    args.recv_src = recv_src;
    args.error_flag = error_flag;
    args.workspace = nullptr;
    return launch_layout_dispatch_small(args, x, H, topk_weights, quant_mode, recv_x, recv_scales,
                                        recv_weights, stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

int moe_dispatch(const void *x, int num_tokens, int hidden, int num_topk,
                 const int32_t *token_row, const float *topk_weights, int64_t recv_capacity,
                 int quant_mode, void *recv_x, void *recv_scales, float *recv_weights,
                 hipStream_t stream)
{
    const int T = num_tokens, H = hidden, K = num_topk;
    int rc = check_rows_sizes(T, H, K, recv_capacity, quant_mode);
    if (rc != MOE_OK)
        return rc;
    if (T == 0)
        return MOE_OK;
    if (!x || !token_row || !recv_x || !aligned16(x) || !aligned16(recv_x))
        return MOE_ERR_INVALID_ARG;
    if (quant_mode != MOE_QUANT_NONE && !recv_scales)
        return MOE_ERR_INVALID_ARG;
    if (fp32_scales(quant_mode) && ((uintptr_t)recv_scales & 3u) != 0)
        return MOE_ERR_INVALID_ARG;
    if (recv_weights && ((uintptr_t)recv_weights & 3u) != 0)
        return MOE_ERR_INVALID_ARG;
    return launch_dispatch(x, T, H, K, token_row, topk_weights, recv_capacity, quant_mode, recv_x,
                           recv_scales, recv_weights, stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

int moe_dispatch_static(const void *x, int num_tokens, int hidden, int num_topk,
                        const int32_t *token_row, const float *topk_weights,
                        int64_t recv_capacity, const float *scales, int num_scales, void *recv_x,
                        float *recv_weights, hipStream_t stream)
{
    const int T = num_tokens, H = hidden, K = num_topk;
    int rc = check_rows_sizes(T, H, K, recv_capacity, MOE_QUANT_NONE);
    if (rc != MOE_OK)
        return rc;
    if (num_scales != 1 && num_scales != H)
        return MOE_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_OK;
    if (!x || !token_row || !recv_x || !scales || !aligned16(x) || !aligned16(recv_x))
        return MOE_ERR_INVALID_ARG;
    if (((uintptr_t)scales & (num_scales == H ? 15u : 3u)) != 0)
        return MOE_ERR_INVALID_ARG;
    if (recv_weights && ((uintptr_t)recv_weights & 3u) != 0)
        return MOE_ERR_INVALID_ARG;
    return launch_dispatch_static(x, T, H, K, token_row, topk_weights, recv_capacity, scales,
                                  num_scales, recv_x, recv_weights, stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

int moe_dispatch_static_per_expert(const void *x, int num_tokens, int hidden, int num_topk,
                                   const int64_t *topk_idx, int num_experts,
                                   const int32_t *token_row, const float *topk_weights,
                                   int64_t recv_capacity, const float *scales, void *recv_x,
                                   float *recv_weights, hipStream_t stream)
{
    const int T = num_tokens, H = hidden, K = num_topk, E = num_experts;
    int rc = check_rows_sizes(T, H, K, recv_capacity, MOE_QUANT_NONE);
    if (rc != MOE_OK)
        return rc;
    if (E < 1 || E > MOE_MAX_EXPERTS)
        return MOE_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_OK;
    if (!x || !topk_idx || !token_row || !recv_x || !scales || !aligned16(x) ||
        !aligned16(recv_x) || !aligned16(scales))
        return MOE_ERR_INVALID_ARG;
    if (((uintptr_t)topk_idx & 7u) != 0)
        return MOE_ERR_INVALID_ARG;
    if (recv_weights && ((uintptr_t)recv_weights & 3u) != 0)
        return MOE_ERR_INVALID_ARG;
    return launch_dispatch_static_expert(x, T, H, K, topk_idx, E, token_row, topk_weights,
                                         recv_capacity, scales, recv_x, recv_weights,
                                         stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

int moe_dispatch_prequantized(const void *data, int num_tokens, int row_bytes, const void *scales,
                              int scale_bytes, int num_topk, const int32_t *token_row,
                              const float *topk_weights, int64_t recv_capacity, void *recv_data,
                              void *recv_scales, float *recv_weights, hipStream_t stream)
{
    const int T = num_tokens, K = num_topk;
    int rc = check_prequant_sizes(T, row_bytes, scale_bytes, K, recv_capacity);
    if (rc != MOE_OK)
        return rc;
    if (T == 0)
        return MOE_OK;
    if (!data || !token_row || !recv_data || !aligned16(data) || !aligned16(recv_data))
        return MOE_ERR_INVALID_ARG;
    if (scale_bytes > 0 && (!scales || !recv_scales))
        return MOE_ERR_INVALID_ARG;
    if (recv_weights && ((uintptr_t)recv_weights & 3u) != 0)
        return MOE_ERR_INVALID_ARG;
    return launch_dispatch_rows(data, T, row_bytes, scales, scale_bytes, K, token_row, topk_weights,
                                recv_capacity, recv_data, recv_scales, recv_weights,
                                stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

int moe_combine(const void *expert_out, int64_t recv_capacity, int num_tokens, int hidden,
                int num_topk, const int32_t *token_row, const float *topk_weights, void *out,
                hipStream_t stream)
{
    const int T = num_tokens, H = hidden, K = num_topk;
    int rc = check_rows_sizes(T, H, K, recv_capacity, MOE_QUANT_NONE);
    if (rc != MOE_OK)
        return rc;
    if (T == 0)
        return MOE_OK;
    if (!token_row || !out || !aligned16(out) || !aligned16(expert_out))
        return MOE_ERR_INVALID_ARG;
    if (recv_capacity > 0 && !expert_out)
        return MOE_ERR_INVALID_ARG;
    return launch_combine(expert_out, recv_capacity, T, H, K, token_row, topk_weights, out,
                          stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

int moe_combine_fused(const void *expert_out, int64_t recv_capacity, int num_tokens, int hidden,
                      int num_topk, const int32_t *token_row, const float *topk_weights,
                      const void *shared_out, const void *residual, const void *rms_weight,
                      float rms_eps, void *out, void *out_norm, hipStream_t stream)
{
    const int T = num_tokens, H = hidden, K = num_topk;
    int rc = check_rows_sizes(T, H, K, recv_capacity, MOE_QUANT_NONE);
    if (rc != MOE_OK)
        return rc;
    if (out_norm && (!rms_weight || !std::isfinite(rms_eps) || rms_eps < 0.0f))
        return MOE_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_OK;
    if (!token_row || !out || !aligned16(out) || !aligned16(expert_out) ||
        !aligned16(shared_out) || !aligned16(residual) || !aligned16(rms_weight) ||
        !aligned16(out_norm))
        return MOE_ERR_INVALID_ARG;
    if (recv_capacity > 0 && !expert_out)
        return MOE_ERR_INVALID_ARG;
    return launch_combine_fused(expert_out, recv_capacity, T, H, K, token_row, topk_weights,
                                shared_out, residual, rms_weight, rms_eps, out, out_norm,
                                stream) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

const char *moe_status_string(int status)
{
    switch (status) {
    case MOE_OK:
        return "ok";
    case MOE_ERR_INVALID_ARG:
        return "invalid argument";
    case MOE_ERR_CAPACITY:
        return "receive capacity below the worst-case row count (or not below 2^31)";
    case MOE_ERR_WORKSPACE:
        return "layout workspace missing, misaligned or too small";
    case MOE_ERR_HIP:
        return "HIP kernel launch failed";
    case MOE_ERR_SCRATCH:
        return "these sizes need more layout workspace than the built-in scratch buffer holds "
               "(MOE_NOALLOC_SCRATCH_BYTES); use moe_get_dispatch_layout with a workspace";
    default:
        return "unknown status";
    }
}

} // extern "C"
