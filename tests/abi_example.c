/*
 * The C ABI used from plain C: device buffers from hipMalloc, one stream, no
 * Python and no torch.  Runs layout -> dispatch (bf16) -> combine on a small
 * seeded batch and checks what holds without a reference implementation:
 *   - every valid entry has a row inside its expert's range, rows of one
 *     expert follow ascending t*K + k, and recv_src inverts token_row;
 *   - every dispatched row equals its source token bit for bit;
 *   - with the receive buffer as the expert output (identity experts) and no
 *     weights, out[t] = bf16(c_t * x[t]) exactly, c_t = valid entries of t
 *     (c_t <= 8 copies of one bf16 value add exactly in fp32).
 * Then the first 96 tokens go through moe_layout_and_dispatch (one launch, per-token
 * FP8 e4m3fn codes) and through the two calls with the same mode: every layout
 * array, code row and scale must be identical.
 * Prints "abi example: ok" and exits 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_dispatch_combine.h"

#define HIP_CHECK(call)                                                            \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
            return 2;                                                              \
        }                                                                          \
    } while (0)

#define MOE_CHECK(call)                                                            \
    do {                                                                           \
        int s_ = (call);                                                           \
        if (s_ != MOE_OK) {                                                        \
            fprintf(stderr, "%s: %s\n", #call, moe_status_string(s_));             \
            return 3;                                                              \
        }                                                                          \
    } while (0)

static uint32_t s_rng = 12345u;
static uint32_t next_u32(void)
{
    s_rng = s_rng * 1664525u + 1013904223u;
    return s_rng;
}

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* layout and receive buffers of one batch, receive rows and scales zeroed */
typedef struct {
    int32_t *ntpr, *ntpe, *itr, *nrtpe, *off, *row, *src, *flag;
    uint8_t *recv;
    float *scales;
} Bufs;

static int alloc_bufs(Bufs *b, int T, int H, int K, int E, int R, int64_t cap)
{
    HIP_CHECK(hipMalloc((void **)&b->ntpr, sizeof(int32_t) * R));
    HIP_CHECK(hipMalloc((void **)&b->ntpe, sizeof(int32_t) * E));
    HIP_CHECK(hipMalloc((void **)&b->itr, sizeof(int32_t) * T * R));
    HIP_CHECK(hipMalloc((void **)&b->nrtpe, sizeof(int32_t) * E));
    HIP_CHECK(hipMalloc((void **)&b->off, sizeof(int32_t) * (E + 1)));
    HIP_CHECK(hipMalloc((void **)&b->row, sizeof(int32_t) * T * K));
    HIP_CHECK(hipMalloc((void **)&b->src, sizeof(int32_t) * cap));
    HIP_CHECK(hipMalloc((void **)&b->flag, sizeof(int32_t)));
    HIP_CHECK(hipMalloc((void **)&b->recv, (size_t)cap * H));
    HIP_CHECK(hipMalloc((void **)&b->scales, sizeof(float) * cap));
    HIP_CHECK(hipMemset(b->recv, 0, (size_t)cap * H));
    HIP_CHECK(hipMemset(b->scales, 0, sizeof(float) * cap));
    return 0;
}

/* 1 if the n bytes at device pointers p and q differ */
static int differ(const void *p, const void *q, size_t n)
{
    void *a = malloc(n), *b = malloc(n);
    int d = 1;
    if (a && b && hipMemcpy(a, p, n, hipMemcpyDeviceToHost) == hipSuccess &&
        hipMemcpy(b, q, n, hipMemcpyDeviceToHost) == hipSuccess)
        d = memcmp(a, b, n) != 0;
    free(a);
    free(b);
    return d;
}

int main(void)
{
    const int T = 700, H = 1024, K = 8, E = 64, R = 8, a = 4;
    const int64_t cap = moe_recv_capacity_bound(T, K, E, a);
    const size_t ws_bytes = moe_layout_workspace_bytes(T, K, E, R);

    int64_t *idx = malloc(sizeof(int64_t) * T * K);
    uint16_t *x = malloc(sizeof(uint16_t) * T * H);
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int e;
            int dup;
            do { /* distinct experts per token, some entries dropped */
                e = (int)(next_u32() % E);
                dup = 0;
                for (int j = 0; j < k; ++j)
                    dup |= idx[t * K + j] == e;
            } while (dup);
            idx[t * K + k] = (next_u32() % 10 == 0) ? -1 : e;
        }
        for (int h = 0; h < H; ++h) /* finite bf16: exponent 120..134 */
            x[(int64_t)t * H + h] = (uint16_t)((next_u32() & 0x807Fu) | ((120u + next_u32() % 15u) << 7));
    }

    hipStream_t st;
    HIP_CHECK(hipStreamCreate(&st));
    int64_t *d_idx;
    uint16_t *d_x, *d_recv, *d_out;
    int32_t *d_ntpr, *d_ntpe, *d_itr, *d_nrtpe, *d_off, *d_row, *d_src, *d_flag;
    void *d_ws = NULL;
    HIP_CHECK(hipMalloc((void **)&d_idx, sizeof(int64_t) * T * K));
    HIP_CHECK(hipMalloc((void **)&d_x, sizeof(uint16_t) * T * H));
    HIP_CHECK(hipMalloc((void **)&d_recv, sizeof(uint16_t) * cap * H));
    HIP_CHECK(hipMalloc((void **)&d_out, sizeof(uint16_t) * T * H));
    HIP_CHECK(hipMalloc((void **)&d_ntpr, sizeof(int32_t) * R));
    HIP_CHECK(hipMalloc((void **)&d_ntpe, sizeof(int32_t) * E));
    HIP_CHECK(hipMalloc((void **)&d_itr, sizeof(int32_t) * T * R));
    HIP_CHECK(hipMalloc((void **)&d_nrtpe, sizeof(int32_t) * E));
    HIP_CHECK(hipMalloc((void **)&d_off, sizeof(int32_t) * (E + 1)));
    HIP_CHECK(hipMalloc((void **)&d_row, sizeof(int32_t) * T * K));
    HIP_CHECK(hipMalloc((void **)&d_src, sizeof(int32_t) * cap));
    HIP_CHECK(hipMalloc((void **)&d_flag, sizeof(int32_t)));
    if (ws_bytes > 0)
        HIP_CHECK(hipMalloc(&d_ws, ws_bytes));
    HIP_CHECK(hipMemcpy(d_idx, idx, sizeof(int64_t) * T * K, hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(d_x, x, sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));

    MOE_CHECK(moe_get_dispatch_layout(d_idx, T, K, E, R, a, cap, d_ntpr, d_ntpe, d_itr, d_nrtpe, d_off,
                                      d_row, d_src, d_flag, d_ws, ws_bytes, st));
    MOE_CHECK(moe_dispatch(d_x, T, H, K, d_row, NULL, cap, MOE_QUANT_NONE, d_recv, NULL, NULL, st));
    MOE_CHECK(moe_combine(d_recv, cap, T, H, K, d_row, NULL, d_out, st));
    HIP_CHECK(hipStreamSynchronize(st));

    int32_t *row = malloc(sizeof(int32_t) * T * K), *src = malloc(sizeof(int32_t) * cap);
    int32_t *off = malloc(sizeof(int32_t) * (E + 1)), flag = -1;
    uint16_t *recv = malloc(sizeof(uint16_t) * cap * H), *out = malloc(sizeof(uint16_t) * T * H);
    HIP_CHECK(hipMemcpy(row, d_row, sizeof(int32_t) * T * K, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(src, d_src, sizeof(int32_t) * cap, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(off, d_off, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(&flag, d_flag, sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(recv, d_recv, sizeof(uint16_t) * cap * H, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(out, d_out, sizeof(uint16_t) * T * H, hipMemcpyDeviceToHost));

    int bad = flag != 0;
    int *last = malloc(sizeof(int) * E);
    for (int e = 0; e < E; ++e)
        last[e] = -1;
    for (int i = 0; i < T * K && !bad; ++i) {
        const int64_t e = idx[i];
        const int r = row[i];
        if (e < 0) {
            bad |= r != -1;
            continue;
        }
        bad |= r < off[e] || r >= off[e + 1] || r <= last[e] || src[r] != i;
        last[e] = r;
        bad |= memcmp(recv + (int64_t)r * H, x + (int64_t)(i / K) * H, sizeof(uint16_t) * H) != 0;
    }
    for (int t = 0; t < T && !bad; ++t) {
        int c = 0;
        for (int k = 0; k < K; ++k)
            c += idx[t * K + k] >= 0;
        for (int h = 0; h < H; ++h) {
            const uint16_t want = c ? f32_to_bf16_rne((float)c * bf16_to_f32(x[(int64_t)t * H + h])) : 0;
            bad |= out[(int64_t)t * H + h] != want;
        }
    }
    if (bad) {
        fprintf(stderr, "abi example: mismatch\n");
        return 1;
    }

    /* the first T1 tokens: one launch against the two calls, per-token FP8 */
    const int T1 = 96, q = MOE_QUANT_FP8_E4M3_PER_TOKEN;
    const int64_t cap1 = moe_recv_capacity_bound(T1, K, E, a);
    const size_t ws1 = moe_layout_workspace_bytes(T1, K, E, R);
    void *d_ws1 = NULL;
    Bufs A, B;
    if (!moe_layout_and_dispatch_fits(T1, H, K, R) || alloc_bufs(&A, T1, H, K, E, R, cap1) ||
        alloc_bufs(&B, T1, H, K, E, R, cap1)) {
        fprintf(stderr, "abi example: one-launch setup failed\n");
        return 1;
    }
    if (ws1 > 0)
        HIP_CHECK(hipMalloc(&d_ws1, ws1));
    MOE_CHECK(moe_layout_and_dispatch(d_idx, d_x, T1, H, K, E, R, a, cap1, NULL, q, A.ntpr, A.ntpe, A.itr,
                                      A.nrtpe, A.off, A.row, A.src, A.flag, A.recv, A.scales, NULL, st));
    MOE_CHECK(moe_get_dispatch_layout(d_idx, T1, K, E, R, a, cap1, B.ntpr, B.ntpe, B.itr, B.nrtpe, B.off,
                                      B.row, B.src, B.flag, d_ws1, ws1, st));
    MOE_CHECK(moe_dispatch(d_x, T1, H, K, B.row, NULL, cap1, q, B.recv, B.scales, NULL, st));
    HIP_CHECK(hipStreamSynchronize(st));
    bad = differ(A.ntpr, B.ntpr, sizeof(int32_t) * R) || differ(A.ntpe, B.ntpe, sizeof(int32_t) * E) ||
          differ(A.itr, B.itr, sizeof(int32_t) * T1 * R) || differ(A.nrtpe, B.nrtpe, sizeof(int32_t) * E) ||
          differ(A.off, B.off, sizeof(int32_t) * (E + 1)) || differ(A.row, B.row, sizeof(int32_t) * T1 * K) ||
          differ(A.src, B.src, sizeof(int32_t) * cap1) || differ(A.flag, B.flag, sizeof(int32_t)) ||
          differ(A.recv, B.recv, (size_t)cap1 * H) || differ(A.scales, B.scales, sizeof(float) * cap1);
    if (bad) {
        fprintf(stderr, "abi example: one launch and two calls differ\n");
        return 1;
    }
    printf("abi example: ok (T=%d H=%d K=%d E=%d, %lld receive rows, %zu workspace bytes)\n", T, H, K, E,
           (long long)off[E], ws_bytes);
    HIP_CHECK(hipStreamDestroy(st));
    return 0;
}
