/*
 * moe_oracle.c -- plain CPU oracle for MoE token dispatch and combine.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this file.  It shares no code, header,
 * table or constant generator with the HIP library, and includes nothing
 * from it.  It is deliberately slow and literal: every step is the plain
 * definition of what the pages describe, in the order they describe it.
 *
 * Sources (cited by page title and section):
 *   [NMA]  sgl-kernel-npu deep_ep "Normal Mode API" page: dispatch
 *          Parameters / Internal Logic / Return Values / Constraints,
 *          and the combine section.
 *   [CANN] Huawei CANN "aclnnMoeDistributeDispatchV2" page: Formula
 *          Cases 1, 3 and 5, and the numbered Constraints.
 *   [EPBM] Modular MAX "EPBatchManager" page: ep_dispatch() and
 *          ep_combine().
 *
 * Precision: the quantisers run in fp32 because [CANN] Formula Case 3 fixes
 * the working type (xFp32 = CastToFp32(X)); the MX step is exact power-of-two
 * scaling followed by an fp8 cast.  The combine sum is not given a precision
 * by any page, so the oracle forms it in fp64 and returns fp64.
 *
 * Pinning: every function here is pinned by CPU tests against closed forms,
 * invariants, brute force on tiny inputs and library routines (tests named
 * test_oracle_*).  No function is "parity unpinned".
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * OpenMP only splits the independent per-token loops; results do not depend
 * on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Status codes.  Same numbering as the library's public header, written out
 * again here on purpose (the oracle includes nothing from the library). */
enum {
    ORC_OK = 0,
    ORC_ERR_INVALID_ARG = -1,
    ORC_ERR_CAPACITY = -2,
};

/* Quantisation modes.  The low 4 bits are the quantMode of [CANN] Formula
 * (0 none, 2 per-token dynamic, 4 MX); the next 4 bits select the
 * destination type where the page allows more than one ([CANN] Constraint 8,
 * Ascend 950: quantMode 2 may write INT8, FLOAT8_E4M3FN or FLOAT8_E5M2;
 * quantMode 4 FLOAT8_E4M3FN or FLOAT8_E5M2): 0 = the default (int8 for mode
 * 2, e4m3fn for mode 4), 1 = e4m3fn, 2 = e5m2. */
enum {
    ORC_QUANT_NONE = 0,
    ORC_QUANT_INT8 = 2,
    ORC_QUANT_MXFP8 = 4,
    ORC_QUANT_FP8_E4M3_PT = 0x12,
    ORC_QUANT_FP8_E5M2_PT = 0x22,
    ORC_QUANT_MXFP8_E5M2 = 0x24,
    ORC_QUANT_FP8_E4M3_PG = 0x13,
    ORC_QUANT_FP8_E5M2_PG = 0x23,
};

/* Group size of the per-group dynamic quantisation (quantMode 3).  The page
 * gives none; its buffer sizing for this mode aligns H to 128 ([CANN]
 * Constraint 9, Ascend 950: alignedH = Align128(H)), read as the group. */
enum { ORC_GROUP = 128 };

/* 8-bit float element formats. */
enum { FMT_E4M3FN = 1, FMT_E5M2 = 2 };

/* ------------------------------------------------------------------------- */
/* Argument rules (host-side validation the library must reproduce).          */
/* ------------------------------------------------------------------------- */

/* Worst-case number of expert-grouped receive rows: every (t, k) entry valid
 * (T*K rows) and every expert padded by at most alignment-1 rows.  This is
 * the single-GPU form of the receive capacity "A" of [CANN] Constraint 7.
 * Returns -1 on invalid arguments. */
int64_t oracle_recv_capacity_bound(int T, int K, int E, int a)
{
    if (T < 0 || K < 1 || E < 1 || a < 1)
        return -1;
    return (int64_t)T * K + (int64_t)E * (a - 1);
}

/* Layout arguments.  Ranges: top-k in (0, 16] and experts in (0, 512]
 * ([NMA] Constraints; [CANN] Constraint 7 "K"); experts divide evenly over
 * ranks ([CANN] Constraint 7 "localExpertNum"); T >= 0; alignment >= 1;
 * row indices must fit int32. */
int oracle_check_layout_args(int T, int K, int E, int R, int a, int64_t cap)
{
    if (T < 0 || K < 1 || K > 16 || E < 1 || E > 512 || R < 1 || R > E || E % R != 0 ||
        a < 1)
        return ORC_ERR_INVALID_ARG;
    int64_t bound = oracle_recv_capacity_bound(T, K, E, a);
    if (bound > INT32_MAX)
        return ORC_ERR_INVALID_ARG;
    if (cap < bound || cap > INT32_MAX)
        return ORC_ERR_CAPACITY;
    return ORC_OK;
}

/* Dispatch / combine arguments.  H a positive multiple of 32 ([CANN]
 * Constraint 7 "H"; 32 is also the MX block, [NMA] Return Values) and at
 * most 16384. */
int oracle_check_rows_args(int T, int H, int K, int64_t cap, int quant_mode)
{
    if (T < 0 || K < 1 || K > 16 || H < 32 || H > 16384 || H % 32 != 0 || cap < 0 ||
        cap > INT32_MAX)
        return ORC_ERR_INVALID_ARG;
    if (quant_mode != ORC_QUANT_NONE && quant_mode != ORC_QUANT_INT8 &&
        quant_mode != ORC_QUANT_MXFP8 && quant_mode != ORC_QUANT_FP8_E4M3_PT &&
        quant_mode != ORC_QUANT_FP8_E5M2_PT && quant_mode != ORC_QUANT_MXFP8_E5M2 &&
        quant_mode != ORC_QUANT_FP8_E4M3_PG && quant_mode != ORC_QUANT_FP8_E5M2_PG)
        return ORC_ERR_INVALID_ARG;
    return ORC_OK;
}

/* Static quantisation arguments: the dispatch sizes plus 1 or H scales. */
int oracle_check_static_args(int T, int H, int K, int64_t cap, int num_scales)
{
    int rc = oracle_check_rows_args(T, H, K, cap, ORC_QUANT_NONE);
    if (rc != ORC_OK)
        return rc;
    if (num_scales != 1 && num_scales != H)
        return ORC_ERR_INVALID_ARG;
    return ORC_OK;
}

/* Static quantisation with one scale row per expert ([CANN] Constraint 8,
 * Ascend 950, quantMode 1, INT8: the scales fold each expert's smoothing
 * weight into its quantisation coefficient, shape (moeExpertNum, H)): the
 * dispatch sizes plus 1 <= E <= 512 experts. */
int oracle_check_static_expert_args(int T, int H, int K, int E, int64_t cap)
{
    int rc = oracle_check_rows_args(T, H, K, cap, ORC_QUANT_NONE);
    if (rc != ORC_OK)
        return rc;
    if (E < 1 || E > 512)
        return ORC_ERR_INVALID_ARG;
    return ORC_OK;
}

/* Pre-quantised rows ([NMA] dispatch Parameters x: a (data, scale) tuple for
 * MXFP8 / MXFP4; Quantization Constraints: data [T, H] or [T, H/2], scales
 * [T, H/32]): row_bytes a positive multiple of 16 up to 32768, scale_bytes
 * 0..4096. */
int oracle_check_prequant_args(int T, int row_bytes, int scale_bytes, int K, int64_t cap)
{
    if (T < 0 || K < 1 || K > 16 || row_bytes < 16 || row_bytes > 32768 || row_bytes % 16 != 0 ||
        scale_bytes < 0 || scale_bytes > 4096 || cap < 0 || cap > INT32_MAX)
        return ORC_ERR_INVALID_ARG;
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Layout: per-rank / per-expert counts, aligned expert offsets, stable rows  */
/* ------------------------------------------------------------------------- */

/*
 * [NMA] dispatch Parameters: num_tokens_per_rank [R] int32 (tokens each rank
 * receives), is_token_in_rank [T, R], num_tokens_per_expert [E], topk_idx
 * [T, K] int64 with -1 = no expert, expert_alignment; [NMA] Return Values:
 * num_recv_tokens_per_expert_list, aligned.  [EPBM] ep_dispatch() Returns:
 * expert_start_indices, row offsets of an expert-grouped buffer.  [CANN]
 * Constraint 1: deterministic.
 *
 * Readings: rank(e) = e / (E / R); an entry outside [-1, E) is an error,
 * flagged in bit 0 of *error_flag and treated as -1; rows within an expert
 * follow ascending t*K + k; every expert's row count is rounded up to a
 * multiple of the alignment (an empty expert keeps zero rows); recv_src of a
 * row is the flat index t*K + k it holds, or -1 for a padding / unused row.
 *
 * Outputs (caller-allocated):
 *   ntpr[R], ntpe[E] (entries per expert), itr[T*R] (0/1), nrtpe[E] (aligned),
 *   off[E+1], token_row[T*K] (-1 invalid), recv_src[cap], error_flag[1].
 */
int oracle_layout(const int64_t *topk_idx, int T, int K, int E, int R, int a, int64_t cap,
                  int32_t *ntpr, int32_t *ntpe, int32_t *itr, int32_t *nrtpe, int32_t *off,
                  int32_t *token_row, int32_t *recv_src, int32_t *error_flag)
{
    int rc = oracle_check_layout_args(T, K, E, R, a, cap);
    if (rc != ORC_OK)
        return rc;
    const int L = E / R; /* localExpertNum, [CANN] Constraint 7 */
    const int64_t M = (int64_t)T * K;
    int32_t flag = 0;

    /* expert id of each entry after range checking */
    int32_t *eid = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M > 0 ? M : 1));
    if (!eid)
        return ORC_ERR_INVALID_ARG;
    for (int64_t i = 0; i < M; ++i) {
        int64_t e = topk_idx[i];
        if (e < -1 || e >= E) {
            flag |= 1;
            e = -1;
        }
        eid[i] = (int32_t)e;
    }

    /* count entries per expert */
    for (int e = 0; e < E; ++e)
        ntpe[e] = 0;
    for (int64_t i = 0; i < M; ++i)
        if (eid[i] >= 0)
            ntpe[eid[i]] += 1;

    /* is_token_in_rank and tokens per rank */
    for (int r = 0; r < R; ++r)
        ntpr[r] = 0;
    for (int t = 0; t < T; ++t) {
        for (int r = 0; r < R; ++r)
            itr[(int64_t)t * R + r] = 0;
        for (int k = 0; k < K; ++k) {
            int e = eid[(int64_t)t * K + k];
            if (e >= 0)
                itr[(int64_t)t * R + e / L] = 1;
        }
        for (int r = 0; r < R; ++r)
            ntpr[r] += itr[(int64_t)t * R + r];
    }

    /* aligned counts ("/" is integer division, [CANN] Constraint 11) and
     * their exclusive prefix sum */
    off[0] = 0;
    for (int e = 0; e < E; ++e) {
        nrtpe[e] = ((ntpe[e] + a - 1) / a) * a;
        off[e + 1] = off[e] + nrtpe[e];
    }

    /* stable counting sort of the entries into the expert segments */
    for (int64_t row = 0; row < cap; ++row)
        recv_src[row] = -1;
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) {
        free(eid);
        return ORC_ERR_INVALID_ARG;
    }
    for (int e = 0; e < E; ++e)
        cursor[e] = off[e];
    for (int64_t i = 0; i < M; ++i) {
        int e = eid[i];
        if (e < 0) {
            token_row[i] = -1;
            continue;
        }
        int32_t row = cursor[e]++;
        token_row[i] = row;
        recv_src[row] = (int32_t)i;
    }
    free(cursor);
    free(eid);
    *error_flag = flag;
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Element codecs                                                             */
/* ------------------------------------------------------------------------- */

/* CastToFp32 of a bf16 value: the 16 bits are the top half of an fp32. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* CastToFp8 for float8_e4m3fn ([NMA] Return Values names the type; [CANN]
 * Formula Case 5 the cast).  e4m3fn: 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, 0x7F/0xFF are NaN, largest finite value
 * 1.75 * 2^8 = 448, smallest normal 2^-6, subnormals are multiples of 2^-9.
 * Rounding is to nearest, ties to even (the default IEEE mode); magnitudes
 * above 448 saturate to 448 (the "fn" format has no infinity), infinities
 * included.  The sign of zero is kept.  A NaN input gives the format's NaN
 * code 0x7F, whatever its sign bit (reading: the pages do not cover NaN; the
 * sign of a NaN that arithmetic produces is not defined).  Computed in
 * double, where every step below is exact except the one explicit rounding. */
uint8_t oracle_cast_to_fp8_e4m3fn(double v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a > 448.0)
        a = 448.0;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: a = q * 2^-9 with q in 0..8 (q = 8 is 2^-6, the
         * smallest normal, whose code is also 8) */
        double q = nearbyint(a * 512.0);
        return (uint8_t)(sign | (uint8_t)q);
    }
    int e2;
    double f = frexp(a, &e2);            /* a = f * 2^e2, f in [0.5, 1) */
    int exponent = e2 - 1;               /* a = (1 + m/8) * 2^exponent   */
    double m = nearbyint((2.0 * f - 1.0) * 8.0);
    if (m == 8.0) {                      /* mantissa rounded up into the next binade */
        m = 0.0;
        exponent += 1;
    }
    return (uint8_t)(sign | (uint8_t)(((exponent + 7) << 3) | (int)m));
}

/* Encode n values (test hook for the exhaustive encoder pin). */
void oracle_cast_to_fp8_e4m3fn_array(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_cast_to_fp8_e4m3fn((double)v[i]);
}

/* CastToFp8 for float8_e5m2 ([CANN] Constraint 8 lists FLOAT8_E5M2 as a
 * destination of quantModes 2 and 4).  e5m2: 1 sign bit, 5 exponent bits with
 * bias 15, 2 mantissa bits; largest finite value 1.75 * 2^15 = 57344,
 * smallest normal 2^-14, subnormals are multiples of 2^-16.  Round to
 * nearest, ties to even.  The format has infinities, but a quantiser that
 * sends a finite input to infinity loses it, so magnitudes above 57344
 * saturate to 57344, as for e4m3fn (reading), infinities included.  Zero
 * keeps its sign; NaN gives the NaN code 0x7F, as for e4m3fn. */
uint8_t oracle_cast_to_fp8_e5m2(double v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a > 57344.0)
        a = 57344.0;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: a = q * 2^-16 with q in 0..4 (q = 4 is 2^-14, the
         * smallest normal, whose code is also 4) */
        double q = nearbyint(a * 65536.0);
        return (uint8_t)(sign | (uint8_t)q);
    }
    int e2;
    double f = frexp(a, &e2);            /* a = f * 2^e2, f in [0.5, 1) */
    int exponent = e2 - 1;               /* a = (1 + m/4) * 2^exponent   */
    double m = nearbyint((2.0 * f - 1.0) * 4.0);
    if (m == 4.0) {
        m = 0.0;
        exponent += 1;
    }
    return (uint8_t)(sign | (uint8_t)(((exponent + 15) << 2) | (int)m));
}

void oracle_cast_to_fp8_e5m2_array(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_cast_to_fp8_e5m2((double)v[i]);
}

static uint8_t cast_to_fp8(int fmt, double v)
{
    return fmt == FMT_E5M2 ? oracle_cast_to_fp8_e5m2(v) : oracle_cast_to_fp8_e4m3fn(v);
}

/* Largest finite value and the exponent of the largest normal ("emax",
 * [CANN] Formula Case 5) of each 8-bit float format. */
static double fp8_max(int fmt) { return fmt == FMT_E5M2 ? 57344.0 : 448.0; }
static int fp8_emax(int fmt) { return fmt == FMT_E5M2 ? 15 : 8; }

/* [CANN] Formula Case 3 (quantMode 2, per-token dynamic quantisation), for
 * one token row, without smoothing scales:
 *   xFp32         = CastToFp32(X)
 *   dynamicScales = dstTypeMax / Max(Abs(xFp32))       dstTypeMax = 127 (int8)
 *   quantOut      = CastToInt8(xFp32 * dynamicScales)  round half to even
 *   scale out     = 1.0 / dynamicScales
 * all in fp32.  Reading for the degenerate row: when dynamicScales is not
 * finite (an all-zero row, or a maximum so small that 127/max overflows) the
 * codes are 0 and the scale is 1.0/dynamicScales = 0.
 * Readings for non-finite inputs (the pages do not cover them): IEEE fp32
 * arithmetic is carried through.  NaN elements take no part in the maximum
 * (as fmaxf), and CastToInt8 of NaN is 0.  A row holding an infinity has
 * maximum +inf, dynamicScales 0, scale +inf, and codes 0 (finite * 0 = 0,
 * inf * 0 = NaN). */
static void quant_int8_row(const uint16_t *x, int H, int8_t *quantOut, float *scale_out)
{
    float maxabs = 0.0f;
    for (int h = 0; h < H; ++h) {
        float xFp32 = bf16_to_f32(x[h]);
        float ab = fabsf(xFp32);
        if (ab > maxabs)
            maxabs = ab;
    }
    const float dstTypeMax = 127.0f;
    float dynamicScales = dstTypeMax / maxabs;
    if (!isfinite(dynamicScales)) {
        for (int h = 0; h < H; ++h)
            quantOut[h] = 0;
    } else {
        for (int h = 0; h < H; ++h) {
            float xFp32 = bf16_to_f32(x[h]);
            float prod = xFp32 * dynamicScales; /* one fp32 multiply */
            float q = rintf(prod);              /* ties to even */
            quantOut[h] = isnan(q) ? 0 : (int8_t)q;
        }
    }
    *scale_out = 1.0f / dynamicScales;
}

/* [CANN] Formula Case 5 (quantMode 4, MXFP8), for one token row, per block of
 * 32 consecutive elements (the block size of [NMA] Return Values):
 *   sharedExp     = Floor(log2(max(|x|))) - emax      emax = 8 for e4m3fn (448 = 1.75*2^8),
 *                                                     15 for e5m2 (57344 = 1.75*2^15)
 *   dynamicScales = 2^sharedExp
 *   quantOut      = CastToFp8(X / dynamicScales)
 * Readings: the block maximum is taken of |x|; sharedExp is clamped below at
 * -127, the smallest exponent an e8m0 byte holds, and an all-zero block uses
 * -127; the stored float8_e8m0fnu scale is 2^sharedExp, i.e. the byte
 * sharedExp + 127, so that x ~= code * 2^sharedExp.
 * Non-finite inputs (readings): NaN elements take no part in the maximum; a
 * block whose maximum is +inf has sharedExp = +inf, stored as the e8m0 NaN
 * byte 0xFF, and its elements are divided by 2^+inf = +inf (finite ones give
 * signed zeros, infinite ones NaN).  The casts then apply (NaN -> 0x7F). */
static void quant_mx_row(const uint16_t *x, int H, int fmt, uint8_t *quantOut, uint8_t *scales_out)
{
    const int emax = fp8_emax(fmt);
    for (int blk = 0; blk < H / 32; ++blk) {
        const uint16_t *xb = x + 32 * blk;
        double maxabs = 0.0;
        for (int j = 0; j < 32; ++j) {
            double ab = fabs((double)bf16_to_f32(xb[j]));
            if (ab > maxabs)
                maxabs = ab;
        }
        if (isinf(maxabs)) {
            for (int j = 0; j < 32; ++j)
                quantOut[32 * blk + j] = cast_to_fp8(fmt, (double)bf16_to_f32(xb[j]) / INFINITY);
            scales_out[blk] = 0xFF;
            continue;
        }
        int sharedExp = -127;
        if (maxabs > 0.0) {
            sharedExp = (int)floor(log2(maxabs)) - emax;
            if (sharedExp < -127)
                sharedExp = -127;
        }
        double dynamicScales = ldexp(1.0, sharedExp);
        for (int j = 0; j < 32; ++j)
            quantOut[32 * blk + j] = cast_to_fp8(fmt, (double)bf16_to_f32(xb[j]) / dynamicScales);
        scales_out[blk] = (uint8_t)(sharedExp + 127);
    }
}

/* [CANN] Formula Case 3 with an 8-bit float destination ([CANN] Constraint 8,
 * Ascend 950: quantMode 2 may write FLOAT8_E4M3FN or FLOAT8_E5M2; the
 * "pertoken_fp8_e4m3" mode of [NMA] Quantization Selection Priority):
 *   dynamicScales = dstTypeMax / Max(Abs(xFp32))     dstTypeMax = 448 or 57344
 *   quantOut      = CastToFp8(xFp32 * dynamicScales) (the product in fp32)
 *   scale out     = 1.0 / dynamicScales
 * Degenerate rows as for int8: codes 0 and scale 0 when dynamicScales is not
 * finite. */
static void quant_fp8_pertoken_row(const uint16_t *x, int H, int fmt, uint8_t *quantOut,
                                   float *scale_out)
{
    float maxabs = 0.0f;
    for (int h = 0; h < H; ++h) {
        float ab = fabsf(bf16_to_f32(x[h]));
        if (ab > maxabs)
            maxabs = ab;
    }
    const float dstTypeMax = (float)fp8_max(fmt);
    float dynamicScales = dstTypeMax / maxabs;
    if (!isfinite(dynamicScales)) {
        for (int h = 0; h < H; ++h)
            quantOut[h] = 0;
    } else {
        for (int h = 0; h < H; ++h) {
            float prod = bf16_to_f32(x[h]) * dynamicScales; /* one fp32 multiply */
            quantOut[h] = cast_to_fp8(fmt, (double)prod);
        }
    }
    *scale_out = 1.0f / dynamicScales;
}

/* [CANN] Formula Case 4 (quantMode 3, per-group dynamic quantisation; the
 * page prints the Case 3 formula for it, and Constraint 8 (Ascend 950) gives
 * FLOAT8_E4M3FN or FLOAT8_E5M2 as the destination): Case 3 applied to each
 * group of ORC_GROUP consecutive elements of the row (the last group holds
 * the H % 128 remaining elements when H is not a multiple of 128):
 *   dynamicScales_g = dstTypeMax / Max(Abs(xFp32 over g))
 *   quantOut        = CastToFp8(xFp32 * dynamicScales_g)   (product in fp32)
 *   scale out g     = 1.0 / dynamicScales_g                (fp32, ceil(H/128) per row)
 * A group whose dynamicScales is not finite gets codes 0 and scale 0. */
static void quant_fp8_pergroup_row(const uint16_t *x, int H, int fmt, uint8_t *quantOut,
                                   float *scales_out)
{
    const float dstTypeMax = (float)fp8_max(fmt);
    for (int g0 = 0, g = 0; g0 < H; g0 += ORC_GROUP, ++g) {
        const int n = H - g0 < ORC_GROUP ? H - g0 : ORC_GROUP;
        float maxabs = 0.0f;
        for (int h = g0; h < g0 + n; ++h) {
            float ab = fabsf(bf16_to_f32(x[h]));
            if (ab > maxabs)
                maxabs = ab;
        }
        float dynamicScales = dstTypeMax / maxabs;
        for (int h = g0; h < g0 + n; ++h)
            quantOut[h] = isfinite(dynamicScales)
                              ? cast_to_fp8(fmt, (double)(bf16_to_f32(x[h]) * dynamicScales))
                              : 0;
        scales_out[g] = 1.0f / dynamicScales;
    }
}

/* [CANN] Formula Case 2 (quantMode 1, static quantisation) with an INT8
 * destination ([CANN] Constraint 8, Ascend 950: the input scales are one
 * quantisation coefficient, shape (1,), a smoothing vector shared by all
 * experts, shape (H,), or one coefficient row per expert, shape (E, H), of
 * which the row of the copy's expert is passed here):
 *   xFp32    = CastToFp32(X) * scales     (fp32 multiply)
 *   quantOut = Cast(xFp32, INT8)
 * Reading: the cast rounds half to even and saturates to [-128, 127] (a
 * static scale does not bound the product as the dynamic modes do); a NaN
 * product casts to 0, as in the dynamic modes. */
static void quant_static_int8_row(const uint16_t *x, int H, const float *scales, int num_scales,
                                  int8_t *quantOut)
{
    for (int h = 0; h < H; ++h) {
        float xFp32 = bf16_to_f32(x[h]) * scales[num_scales == 1 ? 0 : h];
        float r = rintf(xFp32);
        if (isnan(r))
            r = 0.0f;
        if (r > 127.0f)
            r = 127.0f;
        if (r < -128.0f)
            r = -128.0f;
        quantOut[h] = (int8_t)r;
    }
}

/* ------------------------------------------------------------------------- */
/* Dispatch                                                                   */
/* ------------------------------------------------------------------------- */

/*
 * Dispatch copies every token to each of its selected experts' rows of the
 * expert-grouped receive buffer ([NMA] dispatch description; [CANN]
 * Description and Formula Case 1: expandXOut holds the tokens; [EPBM]
 * ep_dispatch(): output_tokens grouped by expert for a grouped matmul).  Quantisation,
 * when asked for, is applied to the source token once and the same codes and
 * scale go to all of its rows ([CANN] Formula: quantOut is formed from X
 * before the exchange).
 *
 * x: bf16 bits [T, H].  token_row: [T*K] from oracle_layout.  topk_weights:
 * [T*K] or NULL.  recv_x: [cap, H] of uint16 (bf16), int8 or uint8 (fp8)
 * elements.  recv_scales: NULL (bf16), float [cap] (per-token modes), float
 * [cap * ceil(H/128)] (per-group modes) or uint8 [cap * H/32] (MX modes),
 * row-major.  recv_weights: [cap] or NULL; receives the
 * weight of the (t, k) entry a row holds.  Rows not named by token_row are
 * left untouched.
 */
int oracle_dispatch(const uint16_t *x, int T, int H, int K, const int32_t *token_row,
                    const float *topk_weights, int64_t cap, int quant_mode, void *recv_x,
                    void *recv_scales, float *recv_weights)
{
    int rc = oracle_check_rows_args(T, H, K, cap, quant_mode);
    if (rc != ORC_OK)
        return rc;
    if (T > 0 && (!x || !token_row || !recv_x))
        return ORC_ERR_INVALID_ARG;
    if (T > 0 && quant_mode != ORC_QUANT_NONE && !recv_scales)
        return ORC_ERR_INVALID_ARG;

    const int per_token_scale = quant_mode == ORC_QUANT_INT8 || quant_mode == ORC_QUANT_FP8_E4M3_PT ||
                                quant_mode == ORC_QUANT_FP8_E5M2_PT;
    const int per_group = quant_mode == ORC_QUANT_FP8_E4M3_PG || quant_mode == ORC_QUANT_FP8_E5M2_PG;
    const int G = (H + ORC_GROUP - 1) / ORC_GROUP;
    const int fmt = (quant_mode >> 4) == 2 ? FMT_E5M2 : FMT_E4M3FN;
#pragma omp parallel
    {
        uint8_t *q = (uint8_t *)malloc((size_t)H);
        uint8_t *sc8 = (uint8_t *)malloc((size_t)H / 32);
        float *scg = (float *)malloc(sizeof(float) * (size_t)G);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            const uint16_t *xt = x + (int64_t)t * H;
            float s_row = 0.0f;
            if (quant_mode == ORC_QUANT_INT8)
                quant_int8_row(xt, H, (int8_t *)q, &s_row);
            else if (quant_mode == ORC_QUANT_FP8_E4M3_PT || quant_mode == ORC_QUANT_FP8_E5M2_PT)
                quant_fp8_pertoken_row(xt, H, fmt, q, &s_row);
            else if (quant_mode == ORC_QUANT_MXFP8 || quant_mode == ORC_QUANT_MXFP8_E5M2)
                quant_mx_row(xt, H, fmt, q, sc8);
            else if (per_group)
                quant_fp8_pergroup_row(xt, H, fmt, q, scg);
            for (int k = 0; k < K; ++k) {
                int32_t row = token_row[(int64_t)t * K + k];
                if (row < 0 || row >= cap)
                    continue;
                if (quant_mode == ORC_QUANT_NONE) {
                    memcpy((uint16_t *)recv_x + (int64_t)row * H, xt, sizeof(uint16_t) * (size_t)H);
                } else {
                    memcpy((uint8_t *)recv_x + (int64_t)row * H, q, (size_t)H);
                    if (per_token_scale)
                        ((float *)recv_scales)[row] = s_row;
                    else if (per_group)
                        memcpy((float *)recv_scales + (int64_t)row * G, scg, sizeof(float) * (size_t)G);
                    else
                        memcpy((uint8_t *)recv_scales + (int64_t)row * (H / 32), sc8, (size_t)H / 32);
                }
                if (recv_weights)
                    recv_weights[row] = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;
            }
        }
        free(q);
        free(sc8);
        free(scg);
    }
    return ORC_OK;
}

/*
 * Dispatch with static int8 quantisation ([CANN] Formula Case 2, quantMode
 * 1): every token is quantised once with the caller's scales (1 value, or H
 * values applied per channel) and copied to its rows; no scales are output
 * (they are the caller's).  recv_x: int8 [cap, H].
 */
int oracle_dispatch_static(const uint16_t *x, int T, int H, int K, const int32_t *token_row,
                           const float *topk_weights, int64_t cap, const float *scales,
                           int num_scales, int8_t *recv_x, float *recv_weights)
{
    int rc = oracle_check_static_args(T, H, K, cap, num_scales);
    if (rc != ORC_OK)
        return rc;
    if (T > 0 && (!x || !token_row || !recv_x || !scales))
        return ORC_ERR_INVALID_ARG;
#pragma omp parallel
    {
        int8_t *q = (int8_t *)malloc((size_t)H);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            quant_static_int8_row(x + (int64_t)t * H, H, scales, num_scales, q);
            for (int k = 0; k < K; ++k) {
                int32_t row = token_row[(int64_t)t * K + k];
                if (row < 0 || row >= cap)
                    continue;
                memcpy(recv_x + (int64_t)row * H, q, (size_t)H);
                if (recv_weights)
                    recv_weights[row] = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;
            }
        }
        free(q);
    }
    return ORC_OK;
}

/*
 * Dispatch with static int8 quantisation and one scale row per expert
 * ([CANN] Formula Case 2, quantMode 1, with the (moeExpertNum, H) scale shape
 * of Constraint 8, Ascend 950).  The page quantises before the exchange;
 * with a scale row per destination expert the codes depend on where a copy
 * goes, so the entry (t, k) sent to expert e = topk_idx[t, k] holds
 *   recv_x[row(t, k), h] = Cast(CastToFp32(x[t, h]) * scales[e, h], INT8)
 * (the same cast as the other static shapes), and the K copies of a token
 * differ wherever their experts' scales do.  scales: fp32 [E, H], row-major.
 * Entries the layout dropped (row -1) are skipped; so is an entry whose id is
 * outside [0, E) (the layout drops those too).  recv_x: int8 [cap, H].
 */
int oracle_dispatch_static_expert(const uint16_t *x, int T, int H, int K, const int64_t *topk_idx,
                                  int E, const int32_t *token_row, const float *topk_weights,
                                  int64_t cap, const float *scales, int8_t *recv_x,
                                  float *recv_weights)
{
    int rc = oracle_check_static_expert_args(T, H, K, E, cap);
    if (rc != ORC_OK)
        return rc;
    if (T > 0 && (!x || !topk_idx || !token_row || !recv_x || !scales))
        return ORC_ERR_INVALID_ARG;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int32_t row = token_row[(int64_t)t * K + k];
            int64_t e = topk_idx[(int64_t)t * K + k];
            if (row < 0 || row >= cap || e < 0 || e >= E)
                continue;
            quant_static_int8_row(x + (int64_t)t * H, H, scales + e * H, H,
                                  recv_x + (int64_t)row * H);
            if (recv_weights)
                recv_weights[row] = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;
        }
    }
    return ORC_OK;
}

/*
 * Dispatch of pre-quantised tokens ([NMA] dispatch Parameters x: for MXFP8 /
 * MXFP4 per-block quantisation x is a tuple (data, scale); Return Values: the
 * received rows keep that format).  Each token's data row (row_bytes) and
 * scale row (scale_bytes) are copied unchanged to every row the layout gives
 * it.  data: [T, row_bytes]; scales: [T, scale_bytes] or NULL when
 * scale_bytes is 0; recv_data: [cap, row_bytes]; recv_scales:
 * [cap, scale_bytes].
 */
int oracle_dispatch_prequantized(const uint8_t *data, int T, int row_bytes, const uint8_t *scales,
                                 int scale_bytes, int K, const int32_t *token_row,
                                 const float *topk_weights, int64_t cap, uint8_t *recv_data,
                                 uint8_t *recv_scales, float *recv_weights)
{
    int rc = oracle_check_prequant_args(T, row_bytes, scale_bytes, K, cap);
    if (rc != ORC_OK)
        return rc;
    if (T > 0 && (!data || !token_row || !recv_data))
        return ORC_ERR_INVALID_ARG;
    if (T > 0 && scale_bytes > 0 && (!scales || !recv_scales))
        return ORC_ERR_INVALID_ARG;
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int32_t row = token_row[(int64_t)t * K + k];
            if (row < 0 || row >= cap)
                continue;
            memcpy(recv_data + (int64_t)row * row_bytes, data + (int64_t)t * row_bytes,
                   (size_t)row_bytes);
            if (scale_bytes > 0)
                memcpy(recv_scales + (int64_t)row * scale_bytes, scales + (int64_t)t * scale_bytes,
                       (size_t)scale_bytes);
            if (recv_weights)
                recv_weights[row] = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;
        }
    }
    return ORC_OK;
}

/* Test hooks: the per-token quantisers on their own. */
void oracle_quant_int8_rows(const uint16_t *x, int T, int H, int8_t *q, float *scales)
{
    for (int t = 0; t < T; ++t)
        quant_int8_row(x + (int64_t)t * H, H, q + (int64_t)t * H, scales + t);
}

void oracle_quant_mxfp8_rows(const uint16_t *x, int T, int H, uint8_t *q, uint8_t *scales)
{
    for (int t = 0; t < T; ++t)
        quant_mx_row(x + (int64_t)t * H, H, FMT_E4M3FN, q + (int64_t)t * H,
                     scales + (int64_t)t * (H / 32));
}

void oracle_quant_mx_e5m2_rows(const uint16_t *x, int T, int H, uint8_t *q, uint8_t *scales)
{
    for (int t = 0; t < T; ++t)
        quant_mx_row(x + (int64_t)t * H, H, FMT_E5M2, q + (int64_t)t * H,
                     scales + (int64_t)t * (H / 32));
}

/* fmt: 1 = e4m3fn, 2 = e5m2; scales [T, ceil(H/128)] */
void oracle_quant_fp8_pergroup_rows(const uint16_t *x, int T, int H, int fmt, uint8_t *q,
                                    float *scales)
{
    const int G = (H + ORC_GROUP - 1) / ORC_GROUP;
    for (int t = 0; t < T; ++t)
        quant_fp8_pergroup_row(x + (int64_t)t * H, H, fmt, q + (int64_t)t * H,
                               scales + (int64_t)t * G);
}

void oracle_quant_static_int8_rows(const uint16_t *x, int T, int H, const float *scales,
                                   int num_scales, int8_t *q)
{
    for (int t = 0; t < T; ++t)
        quant_static_int8_row(x + (int64_t)t * H, H, scales, num_scales, q + (int64_t)t * H);
}

/* fmt: 1 = e4m3fn, 2 = e5m2 */
void oracle_quant_fp8_pertoken_rows(const uint16_t *x, int T, int H, int fmt, uint8_t *q,
                                    float *scales)
{
    for (int t = 0; t < T; ++t)
        quant_fp8_pertoken_row(x + (int64_t)t * H, H, fmt, q + (int64_t)t * H, scales + t);
}

/* ------------------------------------------------------------------------- */
/* Combine                                                                    */
/* ------------------------------------------------------------------------- */

/*
 * Combine brings each token's expert outputs back and takes their weighted
 * sum ([NMA] combine Description: the expert outputs are weighted and summed; [EPBM]
 * ep_combine(): weighted sum of routed expert outputs, result
 * (num_local_tokens, hidden)):
 *   out[t, h] = sum over valid k of  w[t, k] * y[token_row[t, k], h]
 * with w = 1 when no weights are given ([NMA] combine Parameters:
 * topk_weights is optional).  Formed in fp64, k ascending; a token with no
 * valid entry gets 0.  y: bf16 bits [cap, H]; out: double [T, H].
 */
int oracle_combine(const uint16_t *y, int64_t cap, int T, int H, int K, const int32_t *token_row,
                   const float *topk_weights, double *out)
{
    int rc = oracle_check_rows_args(T, H, K, cap, ORC_QUANT_NONE);
    if (rc != ORC_OK)
        return rc;
    if (T > 0 && (!y || !token_row || !out))
        return ORC_ERR_INVALID_ARG;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double *o = out + (int64_t)t * H;
        for (int h = 0; h < H; ++h)
            o[h] = 0.0;
        for (int k = 0; k < K; ++k) {
            int32_t row = token_row[(int64_t)t * K + k];
            if (row < 0 || row >= cap)
                continue;
            double w = topk_weights ? (double)topk_weights[(int64_t)t * K + k] : 1.0;
            const uint16_t *yr = y + (int64_t)row * H;
            for (int h = 0; h < H; ++h)
                o[h] += w * (double)bf16_to_f32(yr[h]);
        }
    }
    return ORC_OK;
}

/*
 * Combine with the epilogues the pages name ([EPBM] ep_combine(): in fused
 * shared-expert mode the shared expert's outputs are added to the reduced
 * routed outputs; [CANN] Description names aclnnMoeDistributeCombineAddRmsNorm,
 * a combine followed by a residual add and an RMS normalisation).  Reading:
 *   s[t, h]    = sum_k w[t,k] * y[row(t,k), h]  +  shared[t, h]  +  residual[t, h]
 *   out[t, h]  = s[t, h]
 *   norm[t, h] = s[t, h] / sqrt(mean_h(s[t, :]^2) + eps) * gamma[h]
 * with shared, residual and gamma optional (NULL: absent / no
 * normalisation).  shared, residual: bf16 bits [T, H]; gamma: bf16 bits [H];
 * out, norm: double [T, H] (norm may be NULL).  All in fp64.
 */
int oracle_combine_fused(const uint16_t *y, int64_t cap, int T, int H, int K,
                         const int32_t *token_row, const float *topk_weights,
                         const uint16_t *shared, const uint16_t *residual, const uint16_t *gamma,
                         double eps, double *out, double *norm)
{
    int rc = oracle_combine(y, cap, T, H, K, token_row, topk_weights, out);
    if (rc != ORC_OK)
        return rc;
    if (norm && (!gamma || !(eps >= 0.0)))
        return ORC_ERR_INVALID_ARG;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double *o = out + (int64_t)t * H;
        for (int h = 0; h < H; ++h) {
            if (shared)
                o[h] += (double)bf16_to_f32(shared[(int64_t)t * H + h]);
            if (residual)
                o[h] += (double)bf16_to_f32(residual[(int64_t)t * H + h]);
        }
        if (norm) {
            double ss = 0.0;
            for (int h = 0; h < H; ++h)
                ss += o[h] * o[h];
            const double rms = sqrt(ss / H + eps);
            for (int h = 0; h < H; ++h)
                norm[(int64_t)t * H + h] = o[h] / rms * (double)bf16_to_f32(gamma[h]);
        }
    }
    return ORC_OK;
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
