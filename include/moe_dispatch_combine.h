/*
 * moe_dispatch_combine.h -- C ABI of the MoE token dispatch / combine library
 * for AMD Instinct MI355X (gfx950).  Library: libmoe_dispatch_combine.so.
 *
 * One step of a Mixture-of-Experts layer's token routing on one GPU:
 *
 *   moe_get_dispatch_layout    counts and a stable expert-grouped row for every
 *                              (token, k) routing entry
 *   moe_dispatch               copy every token into the rows of its selected
 *                              experts, optionally quantised once per token
 *                              (int8, FP8 per token or per group of 128, MX)
 *   moe_dispatch_static        the same with int8 and caller-given scales
 *   moe_dispatch_static_per_expert  the same with one scale row per expert
 *                              (each copy quantised for its own expert)
 *   moe_dispatch_prequantized  the same for rows the caller has quantised
 *                              (data and scale bytes moved unchanged)
 *   moe_combine                top-k weighted sum of every token's expert rows
 *   moe_combine_fused          the same plus shared-expert and residual adds
 *                              and an optional RMS normalisation
 *   moe_layout_and_dispatch    moe_get_dispatch_layout and moe_dispatch (bf16
 *                              or per-token int8 / FP8) in one launch, for
 *                              decode-sized batches (moe_layout_and_dispatch_fits)
 *   moe_get_dispatch_layout_noalloc  the layout without a workspace argument,
 *                              for callers that cannot allocate
 * plus the size queries moe_recv_capacity_bound and moe_layout_workspace_bytes.
 *
 * Sources, by page title and section:
 *   sgl-kernel-npu deep_ep "Normal Mode API": dispatch Parameters, Return
 *     Values, Constraints and Quantization Selection Priority; combine
 *     Description / Parameters.
 *   Huawei CANN "aclnnMoeDistributeDispatchV2": Formula Cases 1 to 5;
 *     Constraints 1 (deterministic), 7 (shapes), 8 and 9 (destination types,
 *     per-group sizing), 11 (integer division); the companion combine with
 *     residual add and RMS normalisation; the two-phase calling pattern (query
 *     the workspace size, then run).
 *   Modular MAX "EPBatchManager": ep_dispatch() and ep_combine() Returns, and
 *     the shared-expert mode of ep_combine().
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must point to GPU memory that the
 *     caller owns and keeps alive until the work queued on `stream` is done.
 *     The library allocates no memory and keeps no state between calls, with
 *     one exception: moe_get_dispatch_layout_noalloc keeps its workspace in
 *     a scratch array built into the library, one per GPU (see there).
 *   - All work is queued on `stream` (NULL = the default stream); no call
 *     waits for the GPU.
 *   - Return value: MOE_OK, or a negative MOE_ERR_* code.  Argument errors are
 *     detected on the host before any HIP call, so nothing is queued when an
 *     error is returned.  MOE_ERR_HIP reports a failed kernel launch.
 *   - Row indices are int32; byte offsets inside the library are 64-bit, so a
 *     receive buffer may exceed 4 GiB.
 *   - Everything is deterministic: the same inputs give bit-identical outputs
 *     (CANN page, Constraint 1).
 *   - NaN and infinite values (the pages do not cover them) follow IEEE fp32
 *     arithmetic, with each cast given a defined result: a row, group or
 *     block maximum ignores NaN elements; an int8 code of NaN is 0 and
 *     +-inf saturates to 127 / -128; an FP8 code of NaN is 0x7F whatever
 *     its sign, and +-inf saturates like any value above the largest finite
 *     one.  A dynamic maximum of +inf gives the scale +inf (per token, per
 *     group) or the e8m0 byte 0xFF (MX block); the elements of that row,
 *     group or block are then multiplied by 0 (or divided by 2^+inf), so
 *     finite ones give zero codes and infinite ones NaN (int8 0, FP8 0x7F).
 *     Scales passed in by the caller may be non-finite too; their products
 *     follow the same rules.
 */
#ifndef MOE_DISPATCH_COMBINE_H
#define MOE_DISPATCH_COMBINE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* a size, range or pointer argument is invalid */
#define MOE_ERR_CAPACITY (-2)    /* recv_capacity below moe_recv_capacity_bound()  */
#define MOE_ERR_WORKSPACE (-3)   /* workspace missing, misaligned or too small      */
#define MOE_ERR_HIP (-4)         /* a HIP launch failed                            */
#define MOE_ERR_SCRATCH (-5)     /* sizes beyond moe_get_dispatch_layout_noalloc's scratch */

/* Quantisation modes.  The low 4 bits are quantMode of the CANN page's Formula
 * (0 none, 2 per-token dynamic, 4 MX); bits 4-7 select the destination type
 * where the page allows several (CANN page, Constraint 8, Ascend 950):
 * 0 = default (int8 for 2, e4m3fn for 4), 1 = float8_e4m3fn, 2 = float8_e5m2. */
#define MOE_QUANT_NONE 0                  /* bf16 rows (Formula Case 1)                         */
#define MOE_QUANT_INT8_PER_TOKEN 2        /* int8 rows + fp32 scale per row (Case 3)             */
#define MOE_QUANT_MXFP8_E4M3 4            /* e4m3fn rows + e8m0 byte per 32 elements (Case 5)    */
#define MOE_QUANT_FP8_E4M3_PER_TOKEN 0x12 /* e4m3fn rows + fp32 scale per row (Case 3, max 448)  */
#define MOE_QUANT_FP8_E5M2_PER_TOKEN 0x22 /* e5m2 rows + fp32 scale per row (Case 3, max 57344)  */
#define MOE_QUANT_MXFP8_E5M2 0x24         /* e5m2 rows + e8m0 byte per 32 elements (Case 5)      */
#define MOE_QUANT_FP8_E4M3_PER_GROUP 0x13 /* e4m3fn rows + fp32 scale per 128 elements (Case 4) */
#define MOE_QUANT_FP8_E5M2_PER_GROUP 0x23 /* e5m2 rows + fp32 scale per 128 elements (Case 4)   */

/* Group size of the per-group modes.  The CANN page gives none; its buffer
 * sizing for per-group quantisation aligns H to 128 (Constraint 9). */
#define MOE_QUANT_GROUP 128

/* Bits of the device error flag written by moe_get_dispatch_layout. */
#define MOE_FLAG_BAD_EXPERT_ID 1 /* some topk_idx entry was outside [-1, num_experts) */

/* Limits.  Top-k and expert counts are the ranges of the Normal Mode API page
 * (Constraints: num_topk in (0, 16], num_experts in (0, 512]); hidden must be
 * a multiple of 32 (CANN page, Constraint 7 "H"; also the MX block).  The
 * hidden size is at most 16384, a limit of this library: the kernels that
 * keep one workgroup per token (per-token, MX and per-group scales, the RMS
 * normalisation) hold the row in one 1024-lane workgroup, at most two
 * 16-byte vectors per lane. */
#define MOE_MAX_TOPK 16
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_HIDDEN 16384
#define MOE_HIDDEN_MULTIPLE 32
#define MOE_MX_BLOCK 32

/*
 * Worst-case number of receive rows: T*K entries plus at most
 * expert_alignment-1 padding rows for each of the E experts.  It is the
 * single-GPU form of the receive capacity "A" (CANN page, Constraint 7).
 * Returns -1 if an argument is out of range (T < 0, K < 1, E < 1, a < 1).
 */
int64_t moe_recv_capacity_bound(int num_tokens, int num_topk, int num_experts,
                                int expert_alignment);

/*
 * Bytes of device workspace moe_get_dispatch_layout needs for these sizes
 * (first phase of the CANN page's two-phase pattern).  0 if the arguments are
 * invalid, and 0 when no workspace is needed: num_tokens is 0, or the batch is
 * small enough (num_tokens*num_topk <= 3072 and num_tokens*num_ranks <= 16384)
 * to be laid out by one workgroup in one launch.  Then workspace may be NULL.
 * The workspace needs no initialisation; its contents after the call are
 * unspecified.
 */
size_t moe_layout_workspace_bytes(int num_tokens, int num_topk, int num_experts, int num_ranks);

/*
 * Dispatch layout (Normal Mode API page, dispatch Parameters and Return
 * Values; EPBatchManager page, ep_dispatch() Returns).
 *
 * Input (device): topk_idx int64 [T, K], row-major; -1 = no expert.
 * Sizes: T >= 0, 1 <= K <= 16, 1 <= E <= 512, 1 <= R <= E with E % R == 0
 *   (experts are split into R virtual ranks of L = E / R consecutive experts;
 *   expert e belongs to rank e / L), expert_alignment a >= 1,
 *   recv_capacity >= moe_recv_capacity_bound(T, K, E, a) and < 2^31.
 * Outputs (device, all overwritten):
 *   num_tokens_per_rank        int32 [R]    distinct tokens with an entry in rank r
 *   num_tokens_per_expert      int32 [E]    valid entries routed to expert e
 *   is_token_in_rank           int32 [T, R] 1 if token t has an entry in rank r, else 0
 *   num_recv_tokens_per_expert int32 [E]    num_tokens_per_expert rounded up to a
 *                                           multiple of a (0 stays 0)
 *   expert_offsets             int32 [E+1]  exclusive prefix sum of the aligned counts;
 *                                           expert e owns rows [off[e], off[e+1])
 *   token_row                  int32 [T, K] row of entry (t, k), or -1 if dropped
 *   recv_src                   int32 [recv_capacity]  t*K + k of the entry a row holds,
 *                                           -1 for padding rows and unused rows
 *   error_flag                 int32 [1]    MOE_FLAG_* bits; 0 if all ids were valid
 * Within an expert, rows follow ascending t*K + k.  An id outside [-1, E) sets
 * MOE_FLAG_BAD_EXPERT_ID and the entry is treated as -1.
 * Workspace: device, 16-byte aligned, >= moe_layout_workspace_bytes(T, K, E, R)
 * bytes (may be NULL when that is 0).  Must not be shared by calls that may
 * run at the same time.
 * Errors: MOE_ERR_INVALID_ARG (ranges, NULL outputs), MOE_ERR_CAPACITY,
 * MOE_ERR_WORKSPACE, MOE_ERR_HIP.
 */
int moe_get_dispatch_layout(const int64_t *topk_idx, int num_tokens, int num_topk,
                            int num_experts, int num_ranks, int expert_alignment,
                            int64_t recv_capacity, int32_t *num_tokens_per_rank,
                            int32_t *num_tokens_per_expert, int32_t *is_token_in_rank,
                            int32_t *num_recv_tokens_per_expert, int32_t *expert_offsets,
                            int32_t *token_row, int32_t *recv_src, int32_t *error_flag,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dispatch (Normal Mode API page, dispatch; CANN page, Formula Cases 1, 3, 5;
 * EPBatchManager page, ep_dispatch()).
 *
 * For every entry (t, k) with row = token_row[t, k] in [0, recv_capacity):
 *   MOE_QUANT_NONE:           recv_x[row, :] = x[t, :]                 (bf16 bits)
 *   MOE_QUANT_INT8_PER_TOKEN: dynamicScales = 127 / max|x[t, :]| in fp32,
 *                             recv_x[row, h] = round_half_even(x[t, h] * dynamicScales)
 *                             recv_scales[row] = 1.0f / dynamicScales  (fp32)
 *                             (a row whose dynamicScales is not finite gets codes 0
 *                             and scale 0)
 *   MOE_QUANT_FP8_E4M3_PER_TOKEN / MOE_QUANT_FP8_E5M2_PER_TOKEN: as the int8
 *                             mode with dstTypeMax 448 / 57344 and the product
 *                             cast to e4m3fn / e5m2 (half to even, saturated to
 *                             dstTypeMax); recv_scales[row] = 1.0f / dynamicScales
 *   MOE_QUANT_FP8_E4M3_PER_GROUP / MOE_QUANT_FP8_E5M2_PER_GROUP: the per-token
 *                             FP8 formula applied to each group g of 128 elements
 *                             (the last group holds H % 128 elements when H is not
 *                             a multiple of 128); recv_scales[row * G + g] =
 *                             1.0f / dynamicScales_g, G = ceil(H / 128)
 *   MOE_QUANT_MXFP8_E4M3 / MOE_QUANT_MXFP8_E5M2: per 32-element block j:
 *                             sharedExp = max(floor(log2 max|x|) - emax, -127)
 *                             (emax 8 / 15; -127 for a zero block),
 *                             recv_x[row, h] = fp8(x[t, h] / 2^sharedExp), rounded
 *                             half to even and saturated to +-448 / +-57344,
 *                             recv_scales[row * H/32 + j] = sharedExp + 127 (e8m0)
 *   recv_weights[row] = topk_weights[t, k] (1.0f if topk_weights is NULL), when
 *   recv_weights is not NULL.
 * Quantisation is done once per token; all copies share codes and scales.
 * Rows no entry names (padding, unused) are not written.
 * Inputs (device): x bf16 [T, H]; token_row int32 [T, K] from
 *   moe_get_dispatch_layout; topk_weights fp32 [T, K] or NULL.
 * Outputs (device): recv_x [recv_capacity, H] of bf16 / int8 / fp8;
 *   recv_scales NULL (bf16) / fp32 [recv_capacity] (per-token modes) /
 *   fp32 [recv_capacity, ceil(H/128)] (per-group modes) /
 *   uint8 [recv_capacity, H/32] (MX modes);
 *   recv_weights fp32 [recv_capacity] or NULL.
 * Sizes: T >= 0, 32 <= H <= 16384 with H % 32 == 0, 1 <= K <= 16,
 *   0 <= recv_capacity < 2^31.
 * Alignment: x and recv_x 16 bytes; fp32 recv_scales and recv_weights 4
 *   bytes (MX scale bytes need none).
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP.
 */
int moe_dispatch(const void *x, int num_tokens, int hidden, int num_topk,
                 const int32_t *token_row, const float *topk_weights, int64_t recv_capacity,
                 int quant_mode, void *recv_x, void *recv_scales, float *recv_weights,
                 hipStream_t stream);

/*
 * Dispatch with static int8 quantisation (CANN page, Formula Case 2, quantMode
 * 1; Constraint 8: the scales are one quantisation coefficient, shape (1,),
 * or one smoothing value per channel, shape (H,); the third shape, one row
 * per expert, is moe_dispatch_static_per_expert).
 *
 * For every entry (t, k) with row = token_row[t, k] in [0, recv_capacity):
 *   recv_x[row, h] = saturate_int8(round_half_even(x[t, h] * scales[h or 0]))
 * with the product in fp32 and saturation to [-128, 127]; no scales are
 * written (they are the caller's).  recv_weights as for moe_dispatch.
 * Inputs (device): x bf16 [T, H]; token_row int32 [T, K]; topk_weights fp32
 *   [T, K] or NULL; scales fp32 [num_scales], num_scales 1 or H (16-byte
 *   aligned when H).
 * Output (device): recv_x int8 [recv_capacity, H].
 * Sizes and alignment as for moe_dispatch.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP.
 */
int moe_dispatch_static(const void *x, int num_tokens, int hidden, int num_topk,
                        const int32_t *token_row, const float *topk_weights,
                        int64_t recv_capacity, const float *scales, int num_scales, void *recv_x,
                        float *recv_weights, hipStream_t stream);

/*
 * Dispatch with static int8 quantisation and one scale row per expert (CANN
 * page, Formula Case 2, quantMode 1; Constraint 8, Ascend 950: the scales are
 * each expert's quantisation coefficient with its smoothing weight folded
 * in, shape (moeExpertNum, H)).
 *
 * For every entry (t, k) with row = token_row[t, k] in [0, recv_capacity) and
 * e = topk_idx[t, k] in [0, num_experts):
 *   recv_x[row, h] = saturate_int8(round_half_even(x[t, h] * scales[e, h]))
 * with the product in fp32 and saturation to [-128, 127].  Unlike the other
 * modes the codes depend on the destination: the K copies of a token differ
 * wherever their experts' scale rows do.  Entries with row -1 are skipped, and
 * so are entries whose id is outside [0, num_experts) (the layout drops them).
 * No scales are written; recv_weights as for moe_dispatch.
 * Inputs (device): x bf16 [T, H]; topk_idx int64 [T, K], the ids the layout was
 *   made from; token_row int32 [T, K]; topk_weights fp32 [T, K] or NULL;
 *   scales fp32 [num_experts, H], row-major.
 * Output (device): recv_x int8 [recv_capacity, H].
 * Sizes: as for moe_dispatch, and 1 <= num_experts <= 512.
 * Alignment: x, recv_x and scales 16 bytes; topk_idx 8 bytes; recv_weights
 *   4 bytes.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP.
 */
int moe_dispatch_static_per_expert(const void *x, int num_tokens, int hidden, int num_topk,
                                   const int64_t *topk_idx, int num_experts,
                                   const int32_t *token_row, const float *topk_weights,
                                   int64_t recv_capacity, const float *scales, void *recv_x,
                                   float *recv_weights, hipStream_t stream);

/*
 * Dispatch of pre-quantised tokens (Normal Mode API page, dispatch Parameters
 * x and Quantization Constraints: for MXFP8 / MXFP4 per-block quantisation x
 * is a (data, scale) tuple, data [T, H] float8 or [T, H/2] float4_e2m1fn_x2,
 * scales [T, H/32] float8_e8m0fnu; the received rows keep that format).
 *
 * For every entry (t, k) with row = token_row[t, k] in [0, recv_capacity):
 *   recv_data[row, :] = data[t, :] and recv_scales[row, :] = scales[t, :]
 * byte for byte; recv_weights[row] as for moe_dispatch.
 * Inputs (device): data [T, row_bytes]; scales [T, scale_bytes] (NULL when
 *   scale_bytes is 0); token_row int32 [T, K]; topk_weights fp32 [T, K] or NULL.
 * Outputs (device): recv_data [recv_capacity, row_bytes]; recv_scales
 *   [recv_capacity, scale_bytes]; recv_weights fp32 [recv_capacity] or NULL.
 * Sizes: T >= 0, 16 <= row_bytes <= 32768 with row_bytes % 16 == 0,
 *   0 <= scale_bytes <= 4096, 1 <= K <= 16, 0 <= recv_capacity < 2^31.
 * data and recv_data must be 16-byte aligned.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP.
 */
int moe_dispatch_prequantized(const void *data, int num_tokens, int row_bytes, const void *scales,
                              int scale_bytes, int num_topk, const int32_t *token_row,
                              const float *topk_weights, int64_t recv_capacity, void *recv_data,
                              void *recv_scales, float *recv_weights, hipStream_t stream);

/*
 * Combine (Normal Mode API page, combine Description: expert outputs weighted
 * and summed;
 * EPBatchManager page, ep_combine(): output (num_local_tokens, hidden)).
 *
 *   out[t, :] = bf16( sum over k with 0 <= token_row[t, k] < recv_capacity of
 *                     topk_weights[t, k] * expert_out[token_row[t, k], :] )
 * The sum is an fp32 fused multiply-add chain in ascending k, rounded once to
 * bf16 (half to even); weights are 1 when topk_weights is NULL; a token with
 * no valid entry gets +0.
 * Inputs (device): expert_out bf16 [recv_capacity, H]; token_row int32 [T, K];
 *   topk_weights fp32 [T, K] or NULL.
 * Output (device): out bf16 [T, H].
 * Sizes and alignment as for moe_dispatch (expert_out and out 16-byte aligned).
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP.
 */
int moe_combine(const void *expert_out, int64_t recv_capacity, int num_tokens, int hidden,
                int num_topk, const int32_t *token_row, const float *topk_weights, void *out,
                hipStream_t stream);

/*
 * Combine with epilogues (EPBatchManager page, ep_combine(): in fused
 * shared-expert mode the shared expert's outputs are added to the reduced
 * routed outputs; CANN page: the aclnnMoeDistributeCombineAddRmsNorm
 * companion of dispatch, a combine followed by a residual add and an RMS
 * normalisation).
 *
 *   s[t, :]        = sum_k w[t, k] * expert_out[token_row[t, k], :]     (as moe_combine)
 *                    + shared_out[t, :]  (if not NULL)  + residual[t, :]  (if not NULL)
 *   out[t, :]      = bf16(s[t, :])
 *   out_norm[t, :] = bf16(s[t, :] / sqrt(mean(s[t, :]^2) + rms_eps) * rms_weight[:])
 *                    (only if out_norm is not NULL)
 * All in fp32 from the fp32 sum (the fma chain of moe_combine, then the
 * shared and residual adds in that order); the sum of squares is reduced in
 * a fixed order.  A caller whose buffer holds the shared expert's rows first
 * ([T rows of shared output][routed rows], as the EPBatchManager page
 * describes) passes shared_out = that buffer and expert_out = buffer + T rows.
 * Inputs (device): as moe_combine, plus shared_out / residual bf16 [T, H] or
 *   NULL, rms_weight bf16 [H] (required with out_norm).
 * Outputs (device): out bf16 [T, H]; out_norm bf16 [T, H] or NULL.
 * rms_eps: finite and >= 0.  All row buffers 16-byte aligned.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP.
 */
int moe_combine_fused(const void *expert_out, int64_t recv_capacity, int num_tokens, int hidden,
                      int num_topk, const int32_t *token_row, const float *topk_weights,
                      const void *shared_out, const void *residual, const void *rms_weight,
                      float rms_eps, void *out, void *out_norm, hipStream_t stream);

/*
 * moe_get_dispatch_layout without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, allocation-free serving loops, harnesses that forbid
 * hipMalloc).  The layout's workspace is a scratch array built into the
 * library, MOE_NOALLOC_SCRATCH_BYTES (8 MiB) per GPU, held from the first call
 * on a GPU until the process ends.  Sizes whose workspace
 * (moe_layout_workspace_bytes) exceeds it return MOE_ERR_SCRATCH before any
 * HIP call.  Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (different streams, or different host threads) race
 * and give wrong results; serialise them, or use moe_get_dispatch_layout
 * with a workspace each.  The array needs no clearing between calls.
 * Arguments, outputs and other errors as for moe_get_dispatch_layout; the
 * outputs are bit-identical to it.  MOE_ERR_HIP also reports a failure to
 * find the array's device address on the stream's GPU.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_get_dispatch_layout_noalloc(const int64_t *topk_idx, int num_tokens, int num_topk,
                                    int num_experts, int num_ranks, int expert_alignment,
                                    int64_t recv_capacity, int32_t *num_tokens_per_rank,
                                    int32_t *num_tokens_per_expert, int32_t *is_token_in_rank,
                                    int32_t *num_recv_tokens_per_expert, int32_t *expert_offsets,
                                    int32_t *token_row, int32_t *recv_src, int32_t *error_flag,
                                    hipStream_t stream);

/*
 * 1 if moe_layout_and_dispatch takes a batch of these sizes, else 0:
 * 0 <= num_tokens <= 512, num_tokens*num_topk <= 3072,
 * num_tokens*num_ranks <= 16384 and hidden <= 8192 (the remaining argument
 * rules are those of moe_get_dispatch_layout and moe_dispatch).  Larger
 * batches use the two calls.
 */
int moe_layout_and_dispatch_fits(int num_tokens, int hidden, int num_topk, int num_ranks);

/*
 * moe_get_dispatch_layout followed by moe_dispatch, in one launch, for
 * decode-sized batches (the same pages and definitions as those two calls).
 * quant_mode: MOE_QUANT_NONE or one of the per-token modes
 * (MOE_QUANT_INT8_PER_TOKEN, MOE_QUANT_FP8_E4M3_PER_TOKEN,
 * MOE_QUANT_FP8_E5M2_PER_TOKEN).  At such sizes the two-call form is bound by
 * fixed costs: two launches, and the layout's store of token_row that
 * dispatch reads back.  Here one workgroup per token derives the whole small
 * layout itself (every workgroup computes the same expert totals and offsets
 * from the same ids, so none waits for another) and copies or quantises its
 * token into its rows.
 *
 * Every output equals, bit for bit, what moe_get_dispatch_layout and
 * moe_dispatch (same quant_mode, topk_weights and recv_weights) write: the
 * layout arrays, recv_src with -1 on padding and unused rows, the rows or
 * codes, the per-row scales, the row weights.  Rows holding no entry are not
 * written.
 * Inputs (device): topk_idx int64 [T, K]; x bf16 [T, H], 16-byte aligned;
 *   topk_weights fp32 [T, K] or NULL (only read for recv_weights).
 * Outputs (device): as moe_get_dispatch_layout (no workspace is needed);
 *   recv_x [recv_capacity, H] of bf16, int8 or FP8 codes, 16-byte aligned;
 *   recv_scales fp32 [recv_capacity], 4-byte aligned, for the per-token modes
 *   (else unused); recv_weights fp32 [recv_capacity], 4-byte aligned, or NULL.
 * Errors: MOE_ERR_INVALID_ARG (including sizes that
 *   moe_layout_and_dispatch_fits rejects and other quant modes),
 *   MOE_ERR_CAPACITY, MOE_ERR_HIP; out-of-range expert ids set bit 0 of
 *   *error_flag, as in the layout call.
 */
int moe_layout_and_dispatch(const int64_t *topk_idx, const void *x, int num_tokens, int hidden,
                            int num_topk, int num_experts, int num_ranks, int expert_alignment,
                            int64_t recv_capacity, const float *topk_weights, int quant_mode,
                            int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                            int32_t *is_token_in_rank, int32_t *num_recv_tokens_per_expert,
                            int32_t *expert_offsets, int32_t *token_row, int32_t *recv_src,
                            int32_t *error_flag, void *recv_x, float *recv_scales,
                            float *recv_weights, hipStream_t stream);

/* Static text for a status code. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DISPATCH_COMBINE_H */
