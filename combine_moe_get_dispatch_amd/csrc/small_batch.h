// small_batch.h -- limits and launcher of the one-launch layout + bf16
// dispatch for decode-sized batches (small_batch.hip).
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
// bf16 and the optional recv_weights [cap].
hipError_t launch_layout_dispatch_small(const LayoutArgs &args, const void *x, int H,
                                        const float *topk_weights, void *recv_x,
                                        float *recv_weights, hipStream_t stream);

} // namespace moe
