// small_batch.h -- limits and launcher of the one-launch layout + dispatch
// for decode-sized batches (small_batch.hip).
#pragma once

#include "launch.h"

namespace moe {

// A batch takes the one-launch path when it has at most kSmallMaxTokens
// tokens, kSmallMaxEntries routing entries, kSmallMaxFlags token x rank
// cells and a hidden size of at most kSmallMaxHidden (one 16-byte vector
// per thread of a 1024-thread workgroup).
constexpr int kSmallMaxTokens = 512;
constexpr int kSmallMaxEntries = 3072;
constexpr int kSmallMaxFlags = 16384;
constexpr int kSmallMaxHidden = 8192;

inline bool small_batch_fits(int T, int H, int K, int R)
{
    return T >= 0 && T <= kSmallMaxTokens && (int64_t)T * K <= kSmallMaxEntries &&
           (int64_t)T * R <= kSmallMaxFlags && H <= kSmallMaxHidden;
}

// Layout outputs as in launch_layout (no workspace), plus recv_x [cap, H]
// (bf16, or int8 / FP8 codes), recv_scales fp32 [cap] for the per-token
// modes and the optional recv_weights [cap].  quant_mode: MOE_QUANT_NONE or
// one of the per-token modes.
hipError_t launch_layout_dispatch_small(const LayoutArgs &args, const void *x, int H,
                                        const float *topk_weights, int quant_mode, void *recv_x,
                                        float *recv_scales, float *recv_weights, hipStream_t stream);

} // namespace moe
