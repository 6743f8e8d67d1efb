// element_codecs.h -- 8-bit destination encoders shared by the dispatch
// kernels: int8 (round half to even) and the FP8 formats e4m3fn / e5m2
// (integer round-half-to-even encoders with saturation), with each format's
// dstTypeMax (CANN aclnnMoeDistributeDispatchV2 page, Formula Cases 3 to 5,
// and Constraint 8 for the destination types).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum class Dst { Int8, E4M3, E5M2 };

// e4m3fn code of an fp32 value: magnitude saturated to 448; below 2^-6 the
// code is the number of 2^-9 steps, rounded half to even (a * 2^9 is exact);
// otherwise exponent field (e + 7) and the top 3 mantissa bits, rounded half
// to even on the 20 bits below them (a carry out of the mantissa moves into
// the exponent field through the plain integer add).  `sign` (0 or 0x80)
// comes from the source element so that -0 and negative values that round
// to zero keep their sign.  Infinities saturate like any value above 448; a
// NaN gives the NaN code 0x7F whatever its sign (fminf alone would turn it
// into 448).
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
    return v == v ? code | sign : 0x7Fu;
}

// e5m2 code of an fp32 value: magnitude saturated to 57344; below 2^-14 the
// number of 2^-16 steps; otherwise exponent field (e + 15) and the top 2
// mantissa bits, rounded half to even on the 21 bits below them.  NaN gives
// 0x7F, as for e4m3fn.
__device__ __forceinline__ uint32_t e5m2_code(float v, uint32_t sign)
{
    const float a = fminf(fabsf(v), 57344.0f);
    uint32_t code;
    if (a < 0x1p-14f) {
        code = (uint32_t)__builtin_rintf(a * 65536.0f);
    } else {
        const uint32_t b = __float_as_uint(a);
        const uint32_t base = (((b >> 23) - 112u) << 2) | ((b >> 21) & 3u);
        const uint32_t rem = b & 0x1FFFFFu;
        code = base + ((rem > 0x100000u) || (rem == 0x100000u && (base & 1u)) ? 1u : 0u);
    }
    return v == v ? code | sign : 0x7Fu;
}

template <Dst D> struct DstTraits;
template <> struct DstTraits<Dst::Int8> {
    static constexpr float kMax = 127.0f;
    // the product is within +-127 (plus one rounding): the integer fits int8;
    // a NaN product (an infinite or NaN element) gives code 0
    __device__ static uint32_t code(float p, uint32_t)
    {
        return p == p ? (uint32_t)((int)__builtin_rintf(p)) & 0xFFu : 0u;
    }
};
template <> struct DstTraits<Dst::E4M3> {
    static constexpr float kMax = 448.0f;
    static constexpr int kEmax = 8;
    __device__ static uint32_t code(float p, uint32_t sign) { return e4m3fn_code(p, sign); }
};
template <> struct DstTraits<Dst::E5M2> {
    static constexpr float kMax = 57344.0f;
    static constexpr int kEmax = 15;
    __device__ static uint32_t code(float p, uint32_t sign) { return e5m2_code(p, sign); }
};

// sign bits (0 or 0x80) of the two bf16 elements of a 32-bit word
__device__ __forceinline__ uint32_t sign_lo(uint32_t w) { return (w >> 8) & 0x80u; }
__device__ __forceinline__ uint32_t sign_hi(uint32_t w) { return (w >> 24) & 0x80u; }

} // namespace moe
