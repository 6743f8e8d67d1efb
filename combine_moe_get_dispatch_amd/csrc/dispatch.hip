// dispatch.hip -- copy every token into the rows of its selected experts,
// optionally quantised once per token.
//
// What is computed (Normal Mode API page, dispatch and Return Values recv_x;
// CANN aclnnMoeDistributeDispatchV2 page, Formula Cases 1, 3 and 5 and
// Constraint 8 for the destination types):
//   bf16      : recv[row(t,k)] = x[t]
//   per-token : dynamicScales = dstTypeMax / max|x[t]| (fp32),
//               q = cast(x * dynamicScales) with the product in fp32,
//               scale = 1 / dynamicScales; codes 0 and scale 0 when
//               dynamicScales is not finite.  dstTypeMax / cast:
//               int8 127 / round half to even; e4m3fn 448 and e5m2 57344 /
//               round half to even, saturated to dstTypeMax
//   MX        : per 32 elements sharedExp = max(floor(log2 max|x|) - emax, -127)
//               (emax 8 for e4m3fn, 15 for e5m2), q = cast(x / 2^sharedExp),
//               e8m0 byte = sharedExp + 127
//   per-group : the per-token formula applied to each group of 128 elements
//               (Formula Case 4; FP8 destinations), one fp32 scale per group
//   static    : q = int8_sat(rint(x * scale)) with the caller's scale(s)
//               (Formula Case 2: one coefficient, one per channel, or one
//               row per expert, Constraint 8 -- then each copy uses the
//               row of its own expert)
//   pre-quantised rows (the Normal Mode API page's (data, scale) tuple input):
//               data row and scale row copied unchanged
//
// Design (gfx950): every 16-byte vector of x (8 bf16 elements) is read from
// HBM exactly once, held in a VGPR, quantised there once, and then written
// to each of the token's K rows with 16-byte (bf16) or 8-byte (1-byte codes)
// stores.  Two launch shapes:
//   - slices (bf16, static int8, pre-quantised rows): one wave per (token,
//     64-vector slice of its row), four waves per workgroup, so each wave
//     reads 1 KiB of x and writes 1 KiB (or 512 bytes) to each row;
//   - one workgroup per token (per-token scales, which need the maximum over
//     the whole row, and MX and per-group scales, measured faster so): one
//     vector per lane, 896 lanes at H = 7168, two vectors per lane above
//     H = 8192;
//   - static int8 with one scale row per expert, whose copies of a token
//     differ: one workgroup per (column slice, 256-token block) with every
//     expert's scales for the slice staged in LDS, each copy encoded
//     separately (dispatch_static_expert_lds_kernel).
// The stores are nontemporal: every expanded row is written once and read
// only by a later stage.  Ordinary stores finish this kernel sooner but
// leave up to a few hundred MB dirty in the L2s and the memory-side cache,
// and the write-back then slows the kernels that follow by more than was
// gained (measured over whole steps).  Row offsets are 64-bit (the largest
// receive buffers exceed 4 GiB).
#include "device_common.h"
#include "element_codecs.h"
#include "launch.h"

#include "../../include/moe_dispatch_combine.h"

namespace moe {

// recv_weights[row(t, k)] = topk_weights[t, k] (1 without weights), written by
// thread `tid` == k of the token's workgroup or wave
__device__ __forceinline__ void write_row_weight(const int32_t *__restrict__ token_row,
                                                 const float *__restrict__ topk_weights,
                                                 float *__restrict__ recv_weights, int64_t t, int K,
                                                 int64_t cap, int tid = (int)threadIdx.x)
{
    if (recv_weights && tid < K) {
        const int row = token_row[t * K + tid];
        if (row >= 0 && row < cap)
            recv_weights[row] = topk_weights ? topk_weights[t * K + tid] : 1.0f;
    }
}

// --------------------------------------------------------------------------- bf16 (slices)

// Rows copied unchanged need no row-wide value, so they are cut finer: one
// wave per (token, 64-vector slice of its row), kSliceWaves waves per
// workgroup, grid-stride beyond kMaxGrid workgroups.  A wave reads 1 KiB of
// the token's row once and writes it to each of the K rows.  Small
// workgroups give every CU its full 32 waves and many short-lived
// independent items, which hides the latency of reading x from HBM:
// measured against one 896-lane workgroup per token, equal at 4096 tokens
// with x in the memory-side cache, 7-11 % faster at 4096-8192 tokens after
// a cache flush, and 5-9 % faster at 32768 tokens (x beyond the cache).
// The item index is left in vector registers on purpose: made wave-uniform
// (readfirstlane), it turns the K token_row reads into scalar loads that
// each stall the store loop, 6 % slower at 32768 tokens x top-16.
__global__ __launch_bounds__(kSliceWaves * kWave) void dispatch_bf16_slice_kernel(
    const u32x4 *__restrict__ x, int nvec, int nslices, int64_t nitems, int K,
    const int32_t *__restrict__ token_row, const float *__restrict__ topk_weights, int64_t cap,
    u32x4 *__restrict__ recv, float *__restrict__ recv_weights)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)threadIdx.x / kWave;
    for (int64_t b = (int64_t)blockIdx.x * kSliceWaves + wave; b < nitems;
         b += (int64_t)gridDim.x * kSliceWaves) {
        const int64_t t = b / nslices;
        const int s = (int)(b - t * nslices);
        const int i = s * kWave + lane;
        const u32x4 v = x[t * nvec + min(i, nvec - 1)]; // clamped: always in bounds
        for (int k = 0; k < K; ++k) {
            const int row = token_row[t * K + k];
            if (row < 0 || row >= cap)
                continue;
            if (i < nvec)
                __builtin_nontemporal_store(v, recv + (int64_t)row * nvec + i);
        }
        if (s == 0)
            write_row_weight(token_row, topk_weights, recv_weights, t, K, cap, lane);
    }
}

// --------------------------------------------------------------------------- per-token dynamic

template <int VPT, Dst D>
__global__ __launch_bounds__(kRowMaxThreads) void dispatch_pertoken_kernel(
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

    const float ds = DstTraits<D>::kMax / m; // IEEE division (built with correctly rounded fp32 divide)
    const bool degenerate = !(ds <= 3.402823466e38f);
    const float scale = 1.0f / ds;

    u32x2 q[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        uint32_t w[2] = {0u, 0u};
        if (!degenerate) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t lo = DstTraits<D>::code(bf16_lo(v[j][c]) * ds, sign_lo(v[j][c]));
                const uint32_t hi = DstTraits<D>::code(bf16_hi(v[j][c]) * ds, sign_hi(v[j][c]));
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
    write_row_weight(token_row, topk_weights, recv_weights, t, K, cap);
}

// --------------------------------------------------------------------------- element-wise codecs

// MX, per-group and static quantisation need no value wider than 128
// elements.  Each lane encodes its 8 elements once into 8 code bytes plus,
// where the format has one, its share of the scale row; the codes are then
// stored to each of the K rows.  A codec provides
//   encode(xv, i, aux) -> the lane's 8 codes (i = clamped vector index,
//                         aux = the lane's scale payload)
//   store_scale(row, i, aux)  -> its scale bytes for one destination row
// and runs in one of two launch forms, chosen by measurement inside whole
// steps, with x in the memory-side cache and after flushing it by a 1 GiB
// fill and by a 1 GiB read:
//   - static int8 in the slice form of the bf16 copy (one wave per token and
//     64-vector slice): equal warm, 7-14 % faster cold;
//   - MX and per group in the one-workgroup-per-token form: the slice form
//     was equal warm but 8-20 % slower after the read flush (per group 10 %
//     faster after the fill flush).

// MX (32-element blocks, one e8m0 byte each): a block is 4 lanes of 8
// elements.  Lanes past the row end hold a copy of the row's last vector;
// since nvec % 4 == 0 a 4-lane block is entirely real or entirely such
// copies.
template <Dst D> struct MxCodec {
    uint8_t *__restrict__ scales; // [cap, nvec / 4]
    int nblk;
    __device__ u32x2 encode(const u32x4 xv, int, uint32_t &aux) const
    {
        float m = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            m = fmaxf(m, fabsf(bf16_lo(xv[c])));
            m = fmaxf(m, fabsf(bf16_hi(xv[c])));
        }
        m = fmaxf(m, __shfl_xor(m, 1, kWave));
        m = fmaxf(m, __shfl_xor(m, 2, kWave));
        // floor(log2 m) is the fp32 exponent field - 127 (any m below 2^-119,
        // subnormals and 0 included, ends up at the -127 clamp).  NaN elements
        // take no part in the maximum (fmaxf); a block whose maximum is +inf
        // (exponent field 255) has sharedExp = +inf: scale byte 0xFF and every
        // element divided by +inf, i.e. multiplied by 0 (finite ones give
        // signed zeros, infinite and NaN ones NaN)
        const int ebits = (int)((__float_as_uint(m) >> 23) & 0xFFu);
        const int se = max(ebits - 127 - DstTraits<D>::kEmax, -127);
        const bool inf_block = ebits == 255;
        const float inv = inf_block ? 0.0f : __uint_as_float((uint32_t)(127 - se) << 23); // 2^-se, normal for se in [-127, 119]
        aux = inf_block ? 0xFFu : (uint32_t)(se + 127);
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // x * 2^-se is exact: a bf16 scaled by a power of two (results
            // that would be fp32-subnormal are far below the fp8 rounding step)
            const uint32_t lo = DstTraits<D>::code(bf16_lo(xv[c]) * inv, sign_lo(xv[c]));
            const uint32_t hi = DstTraits<D>::code(bf16_hi(xv[c]) * inv, sign_hi(xv[c]));
            w[c >> 1] |= (lo | (hi << 8)) << (16 * (c & 1));
        }
        return u32x2{w[0], w[1]};
    }
    __device__ void store_scale(int64_t row, int i, uint32_t aux) const
    {
        if ((i & 3) == 0)
            scales[row * nblk + (i >> 2)] = (uint8_t)aux;
    }
};

// Per group of 128 elements (16 lanes x 8 elements; 16-lane groups are
// aligned inside the wave, and every wave starts at a multiple of 64
// vectors of the row):
// the per-token formula on each group, one fp32 scale per group.  Lanes
// past the row end hold copies of the row's last vector, which belongs to
// the row's last (possibly partial) group, so they cannot change any
// group's maximum.
template <Dst D> struct GroupCodec {
    float *__restrict__ scales; // [cap, ceil(nvec / 16)]
    int ngroups;
    __device__ u32x2 encode(const u32x4 xv, int, uint32_t &aux) const
    {
        float m = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            m = fmaxf(m, fabsf(bf16_lo(xv[c])));
            m = fmaxf(m, fabsf(bf16_hi(xv[c])));
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1)
            m = fmaxf(m, __shfl_xor(m, o, kWave));
        const float ds = DstTraits<D>::kMax / m; // IEEE division
        const bool degenerate = !(ds <= 3.402823466e38f);
        aux = __float_as_uint(1.0f / ds);
        uint32_t w[2] = {0u, 0u};
        if (!degenerate) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t lo = DstTraits<D>::code(bf16_lo(xv[c]) * ds, sign_lo(xv[c]));
                const uint32_t hi = DstTraits<D>::code(bf16_hi(xv[c]) * ds, sign_hi(xv[c]));
                w[c >> 1] |= (lo | (hi << 8)) << (16 * (c & 1));
            }
        }
        return u32x2{w[0], w[1]};
    }
    __device__ void store_scale(int64_t row, int i, uint32_t aux) const
    {
        if ((i & 15) == 0)
            scales[row * ngroups + (i >> 4)] = __uint_as_float(aux);
    }
};

// Static int8 code of one fp32 product: round half to even, then
// v_cvt_i32_f32, which gives 0 for NaN and saturates out-of-range values
// and infinities, then an integer clamp to [-128, 127].  (A float clamp
// before the conversion would turn NaN into -128: the min/max instructions
// return the non-NaN operand.)  The conversion is written as one VALU
// instruction because a C++ float-to-int cast of an out-of-range value is
// undefined.
__device__ __forceinline__ int cvt_i32_saturating(float r)
{
    int i;
    asm("v_cvt_i32_f32 %0, %1" : "=v"(i) : "v"(r));
    return i;
}
struct StaticInt8Code {
    __device__ __forceinline__ uint32_t operator()(float p) const
    {
        return (uint32_t)min(max(cvt_i32_saturating(__builtin_rintf(p)), -128), 127);
    }
};

// The same code for a product that is not NaN (finite or infinite), in two
// instructions instead of four: clamp to [-128, 127] in fp32 (v_med3_f32),
// then add 1.5 * 2^23.  The sum lies in [2^23, 2^24), where the fp32 spacing
// is 1, so the addition rounds the clamped value to an integer, half to
// even (the constant is even), and the sum's bits are 0x4B400000 plus that
// integer: its low byte is the two's-complement code.  Clamping before
// rounding gives the same code as rounding before clamping, since the bounds
// are integers.  Only the low byte of the result is meaningful.
struct StaticInt8CodeNotNan {
    __device__ __forceinline__ uint32_t operator()(float p) const
    {
        return __float_as_uint(__builtin_amdgcn_fmed3f(p, -128.0f, 127.0f) + 12582912.0f);
    }
};

// True when one of the 8 bf16 elements is infinite or NaN (exponent field
// all ones).  Per 16-bit half, (h & 0x7F80) + 0x80 reaches bit 15 exactly
// when the exponent field is 0xFF, and never carries into the next half.
__device__ __forceinline__ bool bf16x8_nonfinite(const u32x4 v)
{
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        m |= (v[c] & 0x7F807F80u) + 0x00800080u;
    return (m & 0x80008000u) != 0;
}

// Static int8 codes of 8 bf16 elements with their 8 scales (s_lo: elements
// 0-3, s_hi: 4-7): one fp32 multiply each, the code, and the low bytes
// packed with three byte permutes per 4 codes.  With StaticInt8Code that is
// about 5 VALU instructions per code, which matters where every copy of a
// token is encoded separately (per-expert scales); StaticInt8CodeNotNan
// saves one.
template <class Code = StaticInt8Code>
__device__ __forceinline__ u32x2 static_int8_codes(const u32x4 xv, const float4 s_lo,
                                                   const float4 s_hi, const Code code = Code())
{
    const float sv[8] = {s_lo.x, s_lo.y, s_lo.z, s_lo.w, s_hi.x, s_hi.y, s_hi.z, s_hi.w};
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t c0 = code(bf16_lo(xv[2 * h]) * sv[4 * h]);
        const uint32_t c1 = code(bf16_hi(xv[2 * h]) * sv[4 * h + 1]);
        const uint32_t c2 = code(bf16_lo(xv[2 * h + 1]) * sv[4 * h + 2]);
        const uint32_t c3 = code(bf16_hi(xv[2 * h + 1]) * sv[4 * h + 3]);
        const uint32_t c01 = __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u); // bytes c0, c1, 0, 0
        const uint32_t c23 = __builtin_amdgcn_perm(c3, c2, 0x0c0c0400u);
        w[h] = __builtin_amdgcn_perm(c23, c01, 0x05040100u);              // c0, c1, c2, c3
    }
    return u32x2{w[0], w[1]};
}

// Static int8 with the caller's scales: one coefficient, or one per channel
// (the 8 channel scales of vector i as two 16-byte loads).  No scale output.
struct StaticCodec {
    const float *__restrict__ scales; // [1] or [H], 16-byte aligned when [H]
    int per_channel;
    __device__ u32x2 encode(const u32x4 xv, int i, uint32_t &) const
    {
        float4 s_lo, s_hi;
        if (per_channel) { // uniform
            const float4 *sc4 = (const float4 *)scales;
            s_lo = sc4[2 * i];
            s_hi = sc4[2 * i + 1];
        } else {
            const float s0 = scales[0];
            s_lo = float4{s0, s0, s0, s0};
            s_hi = s_lo;
        }
        return static_int8_codes(xv, s_lo, s_hi);
    }
    __device__ void store_scale(int64_t, int, uint32_t) const {}
};

// The same codecs in the one-workgroup-per-token form (VPT vectors per lane).
template <int VPT, class Codec>
__global__ __launch_bounds__(kRowMaxThreads) void dispatch_codec_row_kernel(
    const u32x4 *__restrict__ x, int nvec, int K, const int32_t *__restrict__ token_row,
    const float *__restrict__ topk_weights, int64_t cap, u32x2 *__restrict__ recv,
    float *__restrict__ recv_weights, const Codec codec)
{
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const u32x4 *xt = x + (int64_t)t * nvec;
    u32x4 xin[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        xin[j] = xt[min(tid + j * nthr, nvec - 1)]; // clamped: always in bounds
    u32x2 q[VPT];
    uint32_t aux[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        q[j] = codec.encode(xin[j], min(tid + j * nthr, nvec - 1), aux[j]);
    for (int k = 0; k < K; ++k) {
        const int row = token_row[(int64_t)t * K + k];
        if (row < 0 || row >= cap)
            continue;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int i = tid + j * nthr;
            if (i < nvec) {
                __builtin_nontemporal_store(q[j], recv + (int64_t)row * nvec + i);
                codec.store_scale(row, i, aux[j]);
            }
        }
    }
    write_row_weight(token_row, topk_weights, recv_weights, t, K, cap);
}

template <class Codec>
__global__ __launch_bounds__(kSliceWaves * kWave) void dispatch_codec_slice_kernel(
    const u32x4 *__restrict__ x, int nvec, int nslices, int64_t nitems, int K,
    const int32_t *__restrict__ token_row, const float *__restrict__ topk_weights, int64_t cap,
    u32x2 *__restrict__ recv, float *__restrict__ recv_weights, const Codec codec)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)threadIdx.x / kWave; // kept in vector registers, as in the bf16 kernel
    for (int64_t b = (int64_t)blockIdx.x * kSliceWaves + wave; b < nitems;
         b += (int64_t)gridDim.x * kSliceWaves) {
        const int64_t t = b / nslices;
        const int s = (int)(b - t * nslices);
        const int i = s * kWave + lane;
        const int ic = min(i, nvec - 1); // clamped: always in bounds
        uint32_t aux = 0u;
        const u32x2 q = codec.encode(x[t * nvec + ic], ic, aux);
        for (int k = 0; k < K; ++k) {
            const int row = token_row[t * K + k];
            if (row < 0 || row >= cap)
                continue;
            if (i < nvec) {
                __builtin_nontemporal_store(q, recv + (int64_t)row * nvec + i);
                codec.store_scale(row, i, aux);
            }
        }
        if (s == 0)
            write_row_weight(token_row, topk_weights, recv_weights, t, K, cap, lane);
    }
}

// --------------------------------------------------------------------------- static, per expert

// Static int8 with one scale row per expert (scales [E, H]): a copy's codes
// depend on the expert it goes to, so every copy is encoded separately, and
// every code byte needs its own 4-byte scale.  Loading each copy's scale
// slice from the table (16 KiB of loads per 1 KiB slice of x at top-8) made
// the vector memory path the limit (~160 us at 8192 x 7168 top-8 over 256
// experts, against ~89 us for one static scale).  Here the table is staged
// in LDS instead.  A workgroup owns one column slice of 128 channels (64
// beyond 256 experts) and a block of up to 256 tokens.  It copies that slice
// of every expert's scale row into LDS (at most 128 KiB), and the block's
// row numbers and expert ids beside them ([token][KMAX], unused entries -1,
// so that a token's entries come in a few vector reads); then every copy of
// every token in the block is encoded from LDS.  Each scale leaves the table
// once per (slice, block) instead of once per copy: at 8192 x 7168 top-8
// that is ~0.24 GB of table reads instead of ~1.9 GB.  Sixteen lanes cover a
// token's 128 channels (8 per lane), so a wave handles four tokens at a time
// and writes 128-byte pieces of four rows per store (eight tokens and
// 64-byte pieces with 64-channel slices).  An entry whose row is -1 or whose
// id is outside [0, E) is skipped (the layout drops such ids).  Workgroups
// are numbered block-major: the slices of one token block run side by side
// on neighbouring CUs, so each receive row is written piece by piece within
// a short time.  Scales sit in LDS as [expert][half][lane][4]: lane j's two
// 16-byte reads (channels 8j..8j+3, then 8j+4..8j+7) each cover 256
// contiguous bytes over its 16 lanes.
// The 128 KiB tile allows one workgroup (16 waves) per CU.  Measured at
// 8192 x 7168 top-8 Zipf over 256 experts (warm / after a 1 GiB read, us):
// ~110 / ~137 against ~160 / ~215 for per-copy scale loads; blocks of 128 or
// 512 tokens were slower (168 / 162 warm), and the same kernel without any
// arithmetic (codes replaced by copied bits) takes ~103 / ~137, so what is
// left above that is the arithmetic that 4 waves per SIMD cannot fully hide
// behind the stores.  Hence the short conversion (StaticInt8CodeNotNan)
// wherever no product can be NaN, that is unless an element of the lane's
// vector or a staged scale is NaN or infinite: 118 us warm with the exact
// conversion for every code, 110 with the short one (105.6 against 113.8 at
// 128 experts; level at 512 experts, where the 64-channel slices' stores
// are the limit).
constexpr int kStaticLdsTile = 8192;  // float4 of scales in LDS (128 KiB)
constexpr int kStaticLdsThreads = 1024;
// Experts whose slices fit the tile: 2 * VECS float4 per expert (256 at
// VECS = 16, 512 at VECS = 8).
constexpr int static_lds_experts(int vecs) { return kStaticLdsTile / (2 * vecs); }
constexpr int kStaticLdsGroup = 4; // copies encoded between two rounds of stores
// Tokens per workgroup.  The block's row numbers and ids (5 bytes an entry,
// 256 x 16 entries at K = 16) take at most 20 KiB of LDS beside the 128 KiB
// of scales.
constexpr int kStaticLdsTokens = 256;

// VECS: 16-byte vectors of x per column slice, 16 (128 channels, up to 256
// experts in the tile) or 8 (64 channels, up to 512 experts).
template <int KMAX, int VECS>
__global__ __launch_bounds__(kStaticLdsThreads) void dispatch_static_expert_lds_kernel(
    const u32x4 *__restrict__ x, int nvec, int T, int K, int E,
    const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ token_row,
    const float *__restrict__ topk_weights, int64_t cap, const float4 *__restrict__ scales,
    int ncols, int64_t nitems, u32x2 *__restrict__ recv, float *__restrict__ recv_weights)
{
    __shared__ float4 s_sc[kStaticLdsTile];
    constexpr int kTokens = kStaticLdsTokens;
    constexpr int kTpw = kWave / VECS; // tokens per wave and pass
    __shared__ int s_row[kTokens * KMAX];
    __shared__ uint16_t s_e[kTokens * KMAX];
    // The number of the last item (in this workgroup's order) whose staged
    // scales held an infinity or a NaN: written during staging, compared
    // after the barrier, so it never needs clearing.
    __shared__ int s_nonfinite_item;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int nwaves = kStaticLdsThreads / kWave;
    const int sub = lane & (VECS - 1); // vector of the token's VECS in this slice
    const int grp = lane / VECS;       // token of the wave's kTpw
    const int nsc4 = nvec * 2;                   // float4 per scale row
    if (tid == 0)
        s_nonfinite_item = -1;
    int n_item = 0;
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x, ++n_item) {
        const int64_t blk = item / ncols;
        const int c = (int)(item - blk * ncols);
        const int64_t t0 = blk * kTokens;
        const int nt = (int)min((int64_t)kTokens, (int64_t)T - t0);
        const int col = c * VECS + sub; // this lane's vector in the row
        const bool col_ok = col < nvec;
        // x of all the wave's token groups (four), loaded together before the
        // staging barrier: after a cache flush their latency then overlaps the
        // staging instead of stalling each group (139 against 151 us after a
        // 1 GiB read, level warm, against loading each group's x one group
        // ahead).
        constexpr int kPasses = kTokens / (kStaticLdsThreads / kWave * kTpw);
        u32x4 xs[kPasses];
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const int tl = p * nwaves * kTpw + wave * kTpw + grp;
            xs[p] = u32x4{0u, 0u, 0u, 0u};
            if (tl < nt && col_ok)
                xs[p] = x[(t0 + tl) * nvec + col];
        }
        __syncthreads(); // the previous item's LDS reads are done
        // (the launcher passes E <= static_lds_experts(VECS); the bound keeps
        // the staging inside the tile regardless)
        for (int q = tid; q < min(E, static_lds_experts(VECS)) * 2 * VECS; q += kStaticLdsThreads) {
            const int e = q / (2 * VECS);
            const int h = (q / VECS) & 1;
            const int j = q & (VECS - 1);
            const int v = c * VECS + j;
            const float4 s = v < nvec ? scales[(int64_t)e * nsc4 + 2 * v + h] : float4{0.f, 0.f, 0.f, 0.f};
            s_sc[q] = s;
            if (!(__builtin_isfinite(s.x) && __builtin_isfinite(s.y) && __builtin_isfinite(s.z) &&
                  __builtin_isfinite(s.w)))
                s_nonfinite_item = n_item;
        }
        for (int q = tid; q < nt * KMAX; q += kStaticLdsThreads) { // entry (q / KMAX, q % KMAX)
            const int qt = q / KMAX, qk = q & (KMAX - 1);
            bool ok = false;
            int r = -1;
            int64_t e = 0, g = 0;
            if (qk < K) {
                g = (t0 + qt) * K + qk;
                r = token_row[g];
                e = topk_idx[g];
                ok = r >= 0 && r < cap && e >= 0 && e < E;
            }
            s_row[q] = ok ? r : -1;
            s_e[q] = ok ? (uint16_t)e : 0;
            if (ok && c == 0 && recv_weights)
                recv_weights[r] = topk_weights ? topk_weights[g] : 1.0f;
        }
        __syncthreads();
        const bool scales_nonfinite = s_nonfinite_item == n_item; // uniform over the workgroup
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const int tl = p * nwaves * kTpw + wave * kTpw + grp;
            const u32x4 xv = xs[p];
            if (tl < nt) {
                int rows[KMAX];
                uint32_t eo[KMAX];
#pragma unroll
                for (int k = 0; k < KMAX; ++k) {
                    rows[k] = s_row[tl * KMAX + k];
                    eo[k] = s_e[tl * KMAX + k];
                }
                // A product is NaN only when an element or a scale is NaN or
                // infinite; otherwise the shorter conversion gives the same
                // codes.
                const bool exact = scales_nonfinite || bf16x8_nonfinite(xv);
                // Groups of kStaticLdsGroup copies: scale reads and codes with
                // no branch between them, then the stores of the valid ones.
                constexpr int G = KMAX < kStaticLdsGroup ? KMAX : kStaticLdsGroup;
#pragma unroll
                for (int k0 = 0; k0 < KMAX; k0 += G) {
                    u32x2 qv[G];
#pragma unroll
                    for (int k = 0; k < G; ++k) {
                        const float4 *sc = s_sc + eo[k0 + k] * (2 * VECS) + sub;
                        qv[k] = static_int8_codes(xv, sc[0], sc[VECS], StaticInt8CodeNotNan());
                    }
                    if (exact) {
#pragma unroll
                        for (int k = 0; k < G; ++k) {
                            const float4 *sc = s_sc + eo[k0 + k] * (2 * VECS) + sub;
                            qv[k] = static_int8_codes(xv, sc[0], sc[VECS]);
                        }
                    }
#pragma unroll
                    for (int k = 0; k < G; ++k)
                        if (rows[k0 + k] >= 0 && col_ok)
                            __builtin_nontemporal_store(
                                qv[k], recv + (uint64_t)(uint32_t)rows[k0 + k] * (uint32_t)nvec + col);
                }
            }
        }
    }
}

// --------------------------------------------------------------------------- pre-quantised rows

// As the bf16 slices: one wave per (token, 64-vector slice of the data row);
// the scale row's bytes are spread over the token's slices, one byte per
// lane (H/32 bytes for MX data: 224 at H = 7168).
__global__ __launch_bounds__(kSliceWaves * kWave) void dispatch_rows_slice_kernel(
    const u32x4 *__restrict__ data, int nvec, int nslices, int64_t nitems,
    const uint8_t *__restrict__ scales, int scale_bytes, int K,
    const int32_t *__restrict__ token_row, const float *__restrict__ topk_weights, int64_t cap,
    u32x4 *__restrict__ recv_data, uint8_t *__restrict__ recv_scales,
    float *__restrict__ recv_weights)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)threadIdx.x / kWave;
    for (int64_t b = (int64_t)blockIdx.x * kSliceWaves + wave; b < nitems;
         b += (int64_t)gridDim.x * kSliceWaves) {
        const int64_t t = b / nslices;
        const int s = (int)(b - t * nslices);
        const int i = s * kWave + lane;
        const u32x4 v = data[t * nvec + min(i, nvec - 1)]; // clamped: always in bounds
        for (int k = 0; k < K; ++k) {
            const int row = token_row[t * K + k];
            if (row < 0 || row >= cap)
                continue;
            if (i < nvec)
                __builtin_nontemporal_store(v, recv_data + (int64_t)row * nvec + i);
            // the scale row is small: re-read from cache per copy
            for (int j = i; j < scale_bytes; j += nslices * kWave)
                recv_scales[(int64_t)row * scale_bytes + j] = scales[t * scale_bytes + j];
        }
        if (s == 0)
            write_row_weight(token_row, topk_weights, recv_weights, t, K, cap, lane);
    }
}

// --------------------------------------------------------------------------- launch

template <class Codec>
static hipError_t launch_codec(const Codec &codec, const SliceGrid &g, hipStream_t stream,
                               const u32x4 *x, int nvec, int K, const int32_t *token_row,
                               const float *topk_weights, int64_t cap, u32x2 *recv,
                               float *recv_weights)
{
    return launch_kernel(dispatch_codec_slice_kernel<Codec>, dim3(g.blocks),
                         dim3(kSliceWaves * kWave), 0, stream, x, nvec, g.nslices, g.nitems, K,
                         token_row, topk_weights, cap, recv, recv_weights, codec);
}

template <class Codec>
static hipError_t launch_codec_rows(const Codec &codec, int T, int nvec, hipStream_t stream,
                                    const u32x4 *x, int K, const int32_t *token_row,
                                    const float *topk_weights, int64_t cap, u32x2 *recv,
                                    float *recv_weights)
{
    const int threads = row_block_threads(nvec);
    const dim3 grid(T), block(threads);
    if (nvec <= threads)
        return launch_kernel(dispatch_codec_row_kernel<1, Codec>, grid, block, 0, stream, x, nvec,
                             K, token_row, topk_weights, cap, recv, recv_weights, codec);
    return launch_kernel(dispatch_codec_row_kernel<2, Codec>, grid, block, 0, stream, x, nvec, K,
                         token_row, topk_weights, cap, recv, recv_weights, codec);
}

template <int V>
static hipError_t launch_dispatch_v(dim3 grid, dim3 block, hipStream_t stream, const u32x4 *xv,
                                    int nvec, int K, const int32_t *token_row,
                                    const float *topk_weights, int64_t cap, int quant_mode,
                                    void *recv_x, void *recv_scales, float *recv_weights)
{
    switch (quant_mode) {
    case MOE_QUANT_INT8_PER_TOKEN:
        return launch_kernel(dispatch_pertoken_kernel<V, Dst::Int8>, grid, block, 0, stream, xv,
                             nvec, K, token_row, topk_weights, cap, (u32x2 *)recv_x,
                             (float *)recv_scales, recv_weights);
    case MOE_QUANT_FP8_E4M3_PER_TOKEN:
        return launch_kernel(dispatch_pertoken_kernel<V, Dst::E4M3>, grid, block, 0, stream, xv,
                             nvec, K, token_row, topk_weights, cap, (u32x2 *)recv_x,
                             (float *)recv_scales, recv_weights);
    case MOE_QUANT_FP8_E5M2_PER_TOKEN:
        return launch_kernel(dispatch_pertoken_kernel<V, Dst::E5M2>, grid, block, 0, stream, xv,
                             nvec, K, token_row, topk_weights, cap, (u32x2 *)recv_x,
                             (float *)recv_scales, recv_weights);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_dispatch(const void *x, int T, int H, int K, const int32_t *token_row,
                           const float *topk_weights, int64_t cap, int quant_mode, void *recv_x,
                           void *recv_scales, float *recv_weights, hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    const int nvec = H / 8; // 16-byte vectors of bf16 per row
    const SliceGrid g = slice_grid(T, nvec, kSliceWaves);
    const dim3 sgrid(g.blocks), sblock(kSliceWaves * kWave);
    const u32x4 *xs = (const u32x4 *)x;
    u32x2 *rq = (u32x2 *)recv_x;
    switch (quant_mode) {
    case MOE_QUANT_NONE:
        return launch_kernel(dispatch_bf16_slice_kernel, sgrid, sblock, 0, stream, xs, nvec,
                             g.nslices, g.nitems, K, token_row, topk_weights, cap,
                             (u32x4 *)recv_x, recv_weights);
    case MOE_QUANT_MXFP8_E4M3:
        return launch_codec_rows(MxCodec<Dst::E4M3>{(uint8_t *)recv_scales, nvec / 4}, T, nvec,
                                 stream, xs, K, token_row, topk_weights, cap, rq, recv_weights);
    case MOE_QUANT_MXFP8_E5M2:
        return launch_codec_rows(MxCodec<Dst::E5M2>{(uint8_t *)recv_scales, nvec / 4}, T, nvec,
                                 stream, xs, K, token_row, topk_weights, cap, rq, recv_weights);
    case MOE_QUANT_FP8_E4M3_PER_GROUP:
        return launch_codec_rows(GroupCodec<Dst::E4M3>{(float *)recv_scales, (nvec + 15) / 16}, T,
                                 nvec, stream, xs, K, token_row, topk_weights, cap, rq,
                                 recv_weights);
    case MOE_QUANT_FP8_E5M2_PER_GROUP:
        return launch_codec_rows(GroupCodec<Dst::E5M2>{(float *)recv_scales, (nvec + 15) / 16}, T,
                                 nvec, stream, xs, K, token_row, topk_weights, cap, rq,
                                 recv_weights);
    default: // per token: one workgroup per token (below)
        break;
    }
    const int threads = row_block_threads(nvec);
    const int vpt = (nvec + threads - 1) / threads; // 1 or 2 (H <= 16384)
    const dim3 grid(T), block(threads);
    const u32x4 *xv = (const u32x4 *)x;
    if (vpt == 1)
        return launch_dispatch_v<1>(grid, block, stream, xv, nvec, K, token_row, topk_weights, cap,
                                    quant_mode, recv_x, recv_scales, recv_weights);
    return launch_dispatch_v<2>(grid, block, stream, xv, nvec, K, token_row, topk_weights, cap,
                                quant_mode, recv_x, recv_scales, recv_weights);
}

hipError_t launch_dispatch_static(const void *x, int T, int H, int K, const int32_t *token_row,
                                  const float *topk_weights, int64_t cap, const float *scales,
                                  int num_scales, void *recv_x, float *recv_weights,
                                  hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    const int nvec = H / 8;
    const SliceGrid g = slice_grid(T, nvec, kSliceWaves);
    return launch_codec(StaticCodec{scales, num_scales == H ? 1 : 0}, g, stream, (const u32x4 *)x,
                        nvec, K, token_row, topk_weights, cap, (u32x2 *)recv_x, recv_weights);
}

template <int VECS>
static hipError_t launch_static_expert_lds(int K, int T, int nvec, int E, hipStream_t stream,
                                           const u32x4 *xs, const int64_t *topk_idx,
                                           const int32_t *token_row, const float *topk_weights,
                                           int64_t cap, const float4 *sc, u32x2 *rq,
                                           float *recv_weights)
{
    const int ncols = (nvec + VECS - 1) / VECS;
    const int64_t nitems = ((int64_t)T + kStaticLdsTokens - 1) / kStaticLdsTokens * ncols;
    const dim3 grid((unsigned)min(nitems, kMaxGrid)), block(kStaticLdsThreads);
    if (K <= 1)
        return launch_kernel(dispatch_static_expert_lds_kernel<1, VECS>, grid, block, 0, stream, xs, nvec, T, K, E, topk_idx, token_row, topk_weights, cap, sc, ncols, nitems, rq, recv_weights);
    if (K <= 2)
        return launch_kernel(dispatch_static_expert_lds_kernel<2, VECS>, grid, block, 0, stream, xs, nvec, T, K, E, topk_idx, token_row, topk_weights, cap, sc, ncols, nitems, rq, recv_weights);
    if (K <= 4)
        return launch_kernel(dispatch_static_expert_lds_kernel<4, VECS>, grid, block, 0, stream, xs, nvec, T, K, E, topk_idx, token_row, topk_weights, cap, sc, ncols, nitems, rq, recv_weights);
    if (K <= 8)
        return launch_kernel(dispatch_static_expert_lds_kernel<8, VECS>, grid, block, 0, stream, xs, nvec, T, K, E, topk_idx, token_row, topk_weights, cap, sc, ncols, nitems, rq, recv_weights);
    return launch_kernel(dispatch_static_expert_lds_kernel<16, VECS>, grid, block, 0, stream, xs, nvec, T, K, E, topk_idx, token_row, topk_weights, cap, sc, ncols, nitems, rq, recv_weights);
}

hipError_t launch_dispatch_static_expert(const void *x, int T, int H, int K, const int64_t *topk_idx,
                                         int E, const int32_t *token_row,
                                         const float *topk_weights, int64_t cap,
                                         const float *scales, void *recv_x, float *recv_weights,
                                         hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    const int nvec = H / 8;
    const u32x4 *xs = (const u32x4 *)x;
    const float4 *sc = (const float4 *)scales;
    u32x2 *rq = (u32x2 *)recv_x;
    if (E <= static_lds_experts(16)) // 128-channel slices: 512 bytes of scales per expert
        return launch_static_expert_lds<16>(K, T, nvec, E, stream, xs, topk_idx, token_row,
                                            topk_weights, cap, sc, rq, recv_weights);
    if (E <= static_lds_experts(8)) // 64-channel slices
        return launch_static_expert_lds<8>(K, T, nvec, E, stream, xs, topk_idx, token_row,
                                           topk_weights, cap, sc, rq, recv_weights);
    return hipErrorInvalidValue; // E > 512: rejected by the API before this
}

hipError_t launch_dispatch_rows(const void *data, int T, int row_bytes, const void *scales,
                                int scale_bytes, int K, const int32_t *token_row,
                                const float *topk_weights, int64_t cap, void *recv_data,
                                void *recv_scales, float *recv_weights, hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    const int nvec = row_bytes / 16;
    const SliceGrid g = slice_grid(T, nvec, kSliceWaves);
    return launch_kernel(dispatch_rows_slice_kernel, dim3(g.blocks), dim3(kSliceWaves * kWave), 0,
                         stream, (const u32x4 *)data, nvec, g.nslices, g.nitems,
                         (const uint8_t *)scales, scale_bytes, K, token_row, topk_weights, cap,
                         (u32x4 *)recv_data, (uint8_t *)recv_scales, recv_weights);
}

} // namespace moe
