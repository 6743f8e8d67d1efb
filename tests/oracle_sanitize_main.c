/*
 * Host program that runs every oracle entry point on small seeded inputs with
 * exactly sized heap buffers, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_oracle_sanitize.py: an access
 * outside a buffer or undefined arithmetic in the oracle aborts the run.
 * Input generation only (xorshift); the results are checked by the other
 * oracle tests, here only the return codes are.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

int64_t oracle_recv_capacity_bound(int T, int K, int E, int a);
int oracle_layout(const int64_t *topk_idx, int T, int K, int E, int R, int a, int64_t cap,
                  int32_t *ntpr, int32_t *ntpe, int32_t *itr, int32_t *nrtpe, int32_t *off,
                  int32_t *token_row, int32_t *recv_src, int32_t *error_flag);
int oracle_dispatch(const uint16_t *x, int T, int H, int K, const int32_t *token_row,
                    const float *topk_weights, int64_t cap, int quant_mode, void *recv_x,
                    void *recv_scales, float *recv_weights);
int oracle_dispatch_static(const uint16_t *x, int T, int H, int K, const int32_t *token_row,
                           const float *topk_weights, int64_t cap, const float *scales,
                           int num_scales, int8_t *recv_x, float *recv_weights);
int oracle_dispatch_static_expert(const uint16_t *x, int T, int H, int K, const int64_t *topk_idx,
                                  int E, const int32_t *token_row, const float *topk_weights,
                                  int64_t cap, const float *scales, int8_t *recv_x,
                                  float *recv_weights);
int oracle_dispatch_prequantized(const uint8_t *data, int T, int row_bytes, const uint8_t *scales,
                                 int scale_bytes, int K, const int32_t *token_row,
                                 const float *topk_weights, int64_t cap, uint8_t *recv_data,
                                 uint8_t *recv_scales, float *recv_weights);
int oracle_combine(const uint16_t *y, int64_t cap, int T, int H, int K, const int32_t *token_row,
                   const float *topk_weights, double *out);
int oracle_combine_fused(const uint16_t *y, int64_t cap, int T, int H, int K,
                         const int32_t *token_row, const float *topk_weights,
                         const uint16_t *shared, const uint16_t *residual, const uint16_t *gamma,
                         double eps, double *out, double *norm);

static uint64_t s_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)
{
    s_state ^= s_state << 13;
    s_state ^= s_state >> 7;
    s_state ^= s_state << 17;
    return s_state;
}

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* finite bf16: random sign / mantissa, exponent field 0..254 with a bias to moderate values */
static uint16_t rand_bf16(void)
{
    uint64_t r = next_u64();
    unsigned e = (r & 7) == 0 ? (unsigned)((r >> 3) % 255) : 120u + (unsigned)((r >> 3) % 14);
    return (uint16_t)(((r >> 16) & 0x8000u) | (e << 7) | ((r >> 24) & 0x7Fu));
}

#define CHECK(call)                                                                     \
    do {                                                                                \
        int rc_ = (call);                                                               \
        if (rc_ != 0) {                                                                 \
            fprintf(stderr, "%s failed with %d (T=%d K=%d E=%d H=%d)\n", #call, rc_, T, K, E, H); \
            exit(1);                                                                    \
        }                                                                               \
    } while (0)

static void run_case(int T, int K, int E, int R, int a, int H)
{
    const int64_t cap = oracle_recv_capacity_bound(T, K, E, a);
    int64_t *idx = xmalloc(sizeof(int64_t) * (size_t)T * K);
    float *w = xmalloc(sizeof(float) * (size_t)T * K);
    for (int64_t i = 0; i < (int64_t)T * K; ++i) {
        uint64_t r = next_u64();
        idx[i] = (r % 17 == 0) ? -1 : (r % 31 == 0 ? (int64_t)E + (int64_t)(r % 5) : (int64_t)(r % E));
        w[i] = (float)((r >> 20) % 1000) / 1000.0f;
    }
    int32_t *ntpr = xmalloc(4 * (size_t)R), *ntpe = xmalloc(4 * (size_t)E);
    int32_t *itr = xmalloc(4 * (size_t)T * R), *nrtpe = xmalloc(4 * (size_t)E);
    int32_t *off = xmalloc(4 * (size_t)(E + 1)), *row = xmalloc(4 * (size_t)T * K);
    int32_t *src = xmalloc(4 * (size_t)cap), flag = 0;
    CHECK(oracle_layout(idx, T, K, E, R, a, cap, ntpr, ntpe, itr, nrtpe, off, row, src, &flag));

    uint16_t *x = xmalloc(2 * (size_t)T * H);
    for (int64_t i = 0; i < (int64_t)T * H; ++i)
        x[i] = rand_bf16();
    if (T > 0)
        memset(x, 0, 2 * (size_t)H); /* an all-zero row */
    if (T > 3) { /* non-finite elements: NaN with a finite maximum, +-inf, an all-NaN row */
        x[(size_t)H + 1] = 0x7FC0;
        x[2 * (size_t)H + 3] = 0x7F80;
        x[2 * (size_t)H + 4] = 0xFFC1;
        x[3 * (size_t)H] = 0xFF80;
        for (int h = 0; h < H; ++h)
            x[(size_t)(T - 1) * H + h] = 0x7FC0;
    }
    const int modes[] = {0, 2, 4, 0x12, 0x22, 0x24, 0x13, 0x23};
    for (size_t m = 0; m < sizeof modes / sizeof modes[0]; ++m) {
        const int q = modes[m];
        size_t sbytes = 0;
        if (q == 2 || q == 0x12 || q == 0x22)
            sbytes = 4 * (size_t)cap;
        else if (q == 4 || q == 0x24)
            sbytes = (size_t)cap * (H / 32);
        else if (q == 0x13 || q == 0x23)
            sbytes = 4 * (size_t)cap * ((H + 127) / 128);
        void *rx = xmalloc((size_t)cap * H * (q == 0 ? 2 : 1));
        void *rs = sbytes ? xmalloc(sbytes) : NULL;
        float *rw = xmalloc(4 * (size_t)cap);
        CHECK(oracle_dispatch(x, T, H, K, row, w, cap, q, rx, rs, rw));
        free(rx);
        free(rs);
        free(rw);
    }
    for (int ns = 1; ns <= H; ns += H - 1) {
        float *sc = xmalloc(4 * (size_t)ns);
        for (int i = 0; i < ns; ++i)
            sc[i] = 0.5f + (float)(next_u64() % 100);
        int8_t *rx = xmalloc((size_t)cap * H);
        CHECK(oracle_dispatch_static(x, T, H, K, row, NULL, cap, sc, ns, rx, NULL));
        free(rx);
        free(sc);
        if (H == 1)
            break;
    }
    {
        float *sc = xmalloc(4 * (size_t)E * H);
        for (int64_t i = 0; i < (int64_t)E * H; ++i)
            sc[i] = 0.25f + (float)(next_u64() % 200);
        int8_t *rx = xmalloc((size_t)cap * H);
        float *rw = xmalloc(4 * (size_t)cap);
        CHECK(oracle_dispatch_static_expert(x, T, H, K, idx, E, row, w, cap, sc, rx, rw));
        /* non-finite and overflowing scales: every product is cast through the clamp */
        const float odd[5] = {INFINITY, -INFINITY, NAN, 0.0f, 3e38f};
        for (int64_t i = 0; i < (int64_t)E * H; ++i)
            sc[i] = odd[next_u64() % 5];
        CHECK(oracle_dispatch_static_expert(x, T, H, K, idx, E, row, w, cap, sc, rx, rw));
        CHECK(oracle_dispatch_static(x, T, H, K, row, NULL, cap, sc, H, rx, NULL));
        free(rx);
        free(rw);
        free(sc);
    }
    {
        const int rb = H, sb = H / 32;
        uint8_t *d = xmalloc((size_t)T * rb), *s = xmalloc((size_t)T * sb);
        for (int64_t i = 0; i < (int64_t)T * rb; ++i)
            d[i] = (uint8_t)next_u64();
        for (int64_t i = 0; i < (int64_t)T * sb; ++i)
            s[i] = (uint8_t)next_u64();
        uint8_t *rd = xmalloc((size_t)cap * rb), *rs = xmalloc((size_t)cap * sb);
        float *rw = xmalloc(4 * (size_t)cap);
        CHECK(oracle_dispatch_prequantized(d, T, rb, s, sb, K, row, w, cap, rd, rs, rw));
        free(d);
        free(s);
        free(rd);
        free(rs);
        free(rw);
    }
    {
        uint16_t *y = xmalloc(2 * (size_t)cap * H);
        for (int64_t i = 0; i < cap * H; ++i)
            y[i] = (uint16_t)(0x3C00u | (next_u64() & 0x80FFu));
        uint16_t *sh = xmalloc(2 * (size_t)T * H), *res = xmalloc(2 * (size_t)T * H);
        uint16_t *g = xmalloc(2 * (size_t)H);
        for (int64_t i = 0; i < (int64_t)T * H; ++i) {
            sh[i] = (uint16_t)(0x3E00u | (next_u64() & 0x80FFu));
            res[i] = (uint16_t)(0x3D00u | (next_u64() & 0x80FFu));
        }
        for (int i = 0; i < H; ++i)
            g[i] = 0x3F80;
        double *out = xmalloc(8 * (size_t)T * H), *nrm = xmalloc(8 * (size_t)T * H);
        CHECK(oracle_combine(y, cap, T, H, K, row, w, out));
        CHECK(oracle_combine(y, cap, T, H, K, row, NULL, out));
        CHECK(oracle_combine_fused(y, cap, T, H, K, row, w, sh, res, g, 1e-6, out, nrm));
        CHECK(oracle_combine_fused(y, cap, T, H, K, row, NULL, NULL, res, g, 0.0, out, nrm));
        CHECK(oracle_combine_fused(y, cap, T, H, K, row, w, sh, NULL, NULL, 0.0, out, NULL));
        free(y);
        free(sh);
        free(res);
        free(g);
        free(out);
        free(nrm);
    }
    free(x);
    free(idx);
    free(w);
    free(ntpr);
    free(ntpe);
    free(itr);
    free(nrtpe);
    free(off);
    free(row);
    free(src);
}

int main(void)
{
    /* T, K, E, R, a, H */
    const int cases[][6] = {
        {0, 4, 8, 2, 4, 64},     {1, 1, 1, 1, 1, 32},      {37, 3, 16, 4, 3, 160},
        {130, 16, 512, 64, 128, 96}, {64, 8, 256, 8, 1, 1056}, {33, 2, 4, 4, 200, 32},
        {9, 16, 4, 2, 2, 256},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i)
        run_case(cases[i][0], cases[i][1], cases[i][2], cases[i][3], cases[i][4], cases[i][5]);
    printf("oracle sanitizer run: ok\n");
    return 0;
}
