// device_common.h -- small CDNA helpers shared by the kernels of this library.
//
// Wave size is 64 on gfx950; every helper below assumes a full 64-lane wave
// executes it (no divergence around ballots or cross-lane moves).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// Native vector types (clang ext vectors), so that the nontemporal builtins
// and 16-byte global memory instructions apply to them directly.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id()
{
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int count_below(uint64_t mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Lanes of the wave that are `active` and hold the same `key` as the calling
// lane (meaningful for active lanes only).  `nbits` = bits needed for the
// largest key; one ballot per bit.
__device__ __forceinline__ uint64_t match_same_key(int key, bool active, int nbits)
{
    uint64_t m = ballot(active);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t ones = ballot(active && bit);
        m &= bit ? ones : ~ones;
    }
    return m;
}

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest, ties to even
// (finite inputs; an overflow rounds to infinity).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

} // namespace moe
