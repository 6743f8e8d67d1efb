// dispatch.hip -- copy every token into the rows of its selected experts,
// optionally quantised once per token.
//
// What is computed (Normal Mode API page, dispatch and Return Values recv_x;
// CANN aclnnMoeDistributeDispatchV2 page, Formula Cases 1, 3 and 5):
//   bf16 : recv[row(t,k)] = x[t]
//   int8 : dynamicScales = 127 / max|x[t]| (fp32), q = rint(x * dynamicScales),
//          scale = 1 / dynamicScales; codes 0 and scale 0 when dynamicScales
//          is not finite
//   MXFP8: per 32 elements sharedExp = max(floor(log2 max|x|) - 8, -127),
//          q = e4m3fn(x / 2^sharedExp) (ties to even, saturated to 448),
//          e8m0 byte = sharedExp + 127
//
// Design (gfx950): one workgroup per token, one 16-byte vector per lane
// (896 lanes for H = 7168; two vectors per lane above H = 8192).  The token
// row is read from HBM exactly once and held in VGPRs; it is quantised there
// once; then each of the
// K copies is written with 16-byte (bf16) or 8-byte (int8 / e4m3) stores, one
// contiguous row per wave instruction group.  The stores are nontemporal:
// every expanded row is written once and only read again by the next stage,
// so it should not evict the routing tables from L2.  Row offsets are 64-bit
// (the largest receive buffers exceed 4 GiB).
#include "device_common.h"
#include "launch.h"

#include "../../include/moe_dispatch_combine.h"

namespace moe {

// --------------------------------------------------------------------------- bf16

template <int VPT>
__global__ __launch_bounds__(kRowMaxThreads) void dispatch_bf16_kernel(
    const u32x4 *__restrict__ x, int nvec, int K, const int32_t *__restrict__ token_row,
    const float *__restrict__ topk_weights, int64_t cap, u32x4 *__restrict__ recv,
    float *__restrict__ recv_weights)
{
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const u32x4 *xt = x + (int64_t)t * nvec;
    u32x4 v[VPT];
    // branch-free loads (index clamped into the row) keep all VPT loads in flight
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        v[j] = xt[min(tid + j * nthr, nvec - 1)];
    for (int k = 0; k < K; ++k) {
        const int row = token_row[(int64_t)t * K + k];
        if (row < 0 || row >= cap)
            continue;
        u32x4 *dst = recv + (int64_t)row * nvec;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int i = tid + j * nthr;
            if (i < nvec)
                __builtin_nontemporal_store(v[j], dst + i);
        }
    }
    if (recv_weights && tid < K) {
        const int row = token_row[(int64_t)t * K + tid];
        if (row >= 0 && row < cap)
            recv_weights[row] = topk_weights ? topk_weights[(int64_t)t * K + tid] : 1.0f;
    }
}

// --------------------------------------------------------------------------- int8

__device__ __forceinline__ uint32_t q8(float f, float ds)
{
    // one fp32 multiply, then round half to even; |f * ds| <= 127 (plus one
    // rounding), so the integer always fits int8
    return (uint32_t)((int)__builtin_rintf(f * ds)) & 0xFFu;
}

template <int VPT>
__global__ __launch_bounds__(kRowMaxThreads) void dispatch_int8_kernel(
    const u32x4 *__restrict__ x, int nvec, int K, const int32_t *__restrict__ token_row,
    const float *__restrict__ topk_weights, int64_t cap, u32x2 *__restrict__ recv,
    float *__restrict__ recv_scales, float *__restrict__ recv_weights)
{
    __shared__ float s_wmax[kRowMaxThreads / kWave];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const u32x4 *xt = x + (int64_t)t * nvec;
    u32x4 v[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        v[j] = xt[min(tid + j * nthr, nvec - 1)]; // clamped: always in bounds
    float m = 0.0f; // a clamped duplicate of a real element cannot change the maximum
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            m = fmaxf(m, fabsf(bf16_lo(v[j][c])));
            m = fmaxf(m, fabsf(bf16_hi(v[j][c])));
        }
    }
    m = wave_max(m);
    if ((tid & (kWave - 1)) == 0)
        s_wmax[tid / kWave] = m;
    __syncthreads();
    m = s_wmax[0];
    for (int w = 1; w < nthr / kWave; ++w)
        m = fmaxf(m, s_wmax[w]);

    const float ds = 127.0f / m; // IEEE division (built with correctly rounded fp32 divide)
    const bool degenerate = !(ds <= 3.402823466e38f);
    const float scale = 1.0f / ds;

    u32x2 q[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        uint32_t w[2] = {0u, 0u};
        if (!degenerate) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t lo = q8(bf16_lo(v[j][c]), ds);
                const uint32_t hi = q8(bf16_hi(v[j][c]), ds);
                w[c >> 1] |= (lo | (hi << 8)) << (16 * (c & 1));
            }
        }
        q[j] = u32x2{w[0], w[1]};
    }

    for (int k = 0; k < K; ++k) {
        const int row = token_row[(int64_t)t * K + k];
        if (row < 0 || row >= cap)
            continue;
        u32x2 *dst = recv + (int64_t)row * nvec;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int i = tid + j * nthr;
            if (i < nvec)
                __builtin_nontemporal_store(q[j], dst + i);
        }
        if (tid == 0)
            recv_scales[row] = scale;
    }
    if (recv_weights && tid < K) {
        const int row = token_row[(int64_t)t * K + tid];
        if (row >= 0 && row < cap)
            recv_weights[row] = topk_weights ? topk_weights[(int64_t)t * K + tid] : 1.0f;
    }
}

// --------------------------------------------------------------------------- MXFP8 e4m3

// e4m3fn code of v (an exact multiple of a power of two, from a bf16 times
// 2^-sharedExp).  Magnitude saturated to 448; below 2^-6 the code is the
// number of 2^-9 steps, rounded half to even; otherwise exponent field
// (e + 7) and the top 3 mantissa bits, rounded half to even on the 20 bits
// below them (a carry out of the mantissa moves into the exponent field by
// the plain integer add).  `sign` is taken from the source element so that
// -0 and negative values that round to zero keep their sign.
__device__ __forceinline__ uint32_t e4m3fn_code(float v, uint32_t sign)
{
    const float a = fminf(fabsf(v), 448.0f);
    uint32_t code;
    if (a < 0x1p-6f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        const uint32_t b = __float_as_uint(a);
        const uint32_t base = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
        const uint32_t rem = b & 0xFFFFFu;
        code = base + ((rem > 0x80000u) || (rem == 0x80000u && (base & 1u)) ? 1u : 0u);
    }
    return code | sign;
}

template <int VPT>
__global__ __launch_bounds__(kRowMaxThreads) void dispatch_mxfp8_kernel(
    const u32x4 *__restrict__ x, int nvec, int K, const int32_t *__restrict__ token_row,
    const float *__restrict__ topk_weights, int64_t cap, u32x2 *__restrict__ recv,
    uint8_t *__restrict__ recv_scales, float *__restrict__ recv_weights)
{
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int nblk = nvec / 4; // 32-element blocks per row; 4 lanes (8 elements each) per block
    const u32x4 *xt = x + (int64_t)t * nvec;
    u32x4 xin[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        xin[j] = xt[min(tid + j * nthr, nvec - 1)]; // clamped: always in bounds
    u32x2 q[VPT];
    uint32_t sbyte[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        // lanes past the row end hold a copy of the row's last vector; since
        // nvec % 4 == 0 a 4-lane block is entirely real or entirely such copies
        const u32x4 xv = xin[j];
        float m = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            m = fmaxf(m, fabsf(bf16_lo(xv[c])));
            m = fmaxf(m, fabsf(bf16_hi(xv[c])));
        }
        m = fmaxf(m, __shfl_xor(m, 1, kWave));
        m = fmaxf(m, __shfl_xor(m, 2, kWave));
        const int ebits = (int)((__float_as_uint(m) >> 23) & 0xFFu);
        const int se = max(ebits - 127 - 8, -127); // floor(log2 m) - emax, emax(e4m3fn) = 8
        const float inv = __uint_as_float((uint32_t)(127 - se) << 23); // 2^-se, normal for se in [-127, 119]
        sbyte[j] = (uint32_t)(se + 127);
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t lo = e4m3fn_code(bf16_lo(xv[c]) * inv, (xv[c] >> 8) & 0x80u);
            const uint32_t hi = e4m3fn_code(bf16_hi(xv[c]) * inv, (xv[c] >> 24) & 0x80u);
            w[c >> 1] |= (lo | (hi << 8)) << (16 * (c & 1));
        }
        q[j] = u32x2{w[0], w[1]};
    }

    for (int k = 0; k < K; ++k) {
        const int row = token_row[(int64_t)t * K + k];
        if (row < 0 || row >= cap)
            continue;
        u32x2 *dst = recv + (int64_t)row * nvec;
        uint8_t *sdst = recv_scales + (int64_t)row * nblk;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int i = tid + j * nthr;
            if (i < nvec) {
                __builtin_nontemporal_store(q[j], dst + i);
                if ((i & 3) == 0)
                    sdst[i >> 2] = (uint8_t)sbyte[j];
            }
        }
    }
    if (recv_weights && tid < K) {
        const int row = token_row[(int64_t)t * K + tid];
        if (row >= 0 && row < cap)
            recv_weights[row] = topk_weights ? topk_weights[(int64_t)t * K + tid] : 1.0f;
    }
}

// --------------------------------------------------------------------------- launch

hipError_t launch_dispatch(const void *x, int T, int H, int K, const int32_t *token_row,
                           const float *topk_weights, int64_t cap, int quant_mode, void *recv_x,
                           void *recv_scales, float *recv_weights, hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    const int nvec = H / 8; // 16-byte vectors of bf16 per row
    const int threads = row_block_threads(nvec);
    const int vpt = (nvec + threads - 1) / threads; // 1 or 2 (H <= 16384)
    const dim3 grid(T), block(threads);
    const u32x4 *xv = (const u32x4 *)x;

#define MOE_DISPATCH_CASE(V)                                                                       \
    case V:                                                                                        \
        if (quant_mode == MOE_QUANT_NONE)                                                          \
            return launch_kernel(dispatch_bf16_kernel<V>, grid, block, 0, stream, xv, nvec, K,    \
                                 token_row, topk_weights, cap, (u32x4 *)recv_x, recv_weights);     \
        if (quant_mode == MOE_QUANT_INT8_PER_TOKEN)                                                \
            return launch_kernel(dispatch_int8_kernel<V>, grid, block, 0, stream, xv, nvec, K,    \
                                 token_row, topk_weights, cap, (u32x2 *)recv_x,                   \
                                 (float *)recv_scales, recv_weights);                              \
        return launch_kernel(dispatch_mxfp8_kernel<V>, grid, block, 0, stream, xv, nvec, K,       \
                             token_row, topk_weights, cap, (u32x2 *)recv_x,                       \
                             (uint8_t *)recv_scales, recv_weights);

    switch (vpt) {
        MOE_DISPATCH_CASE(1)
        MOE_DISPATCH_CASE(2)
    }
#undef MOE_DISPATCH_CASE
    return hipErrorInvalidValue;
}

} // namespace moe
