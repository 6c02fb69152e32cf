/*
 * Drives every entry point of qlin_oracle.c on small and edge-case inputs, so
 * that a build with AddressSanitizer and UndefinedBehaviorSanitizer checks the
 * oracle's own memory accesses and arithmetic (test infrastructure only; it is
 * compiled together with qlin_oracle.c by the CPU test suite and computes
 * nothing the tests compare).  Exit status 0 means every call returned the
 * status it should; the sanitizers abort on any finding.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_threads(void);
float orc_hadamard_scale(int b);
int orc_hadamard(const void *x, int dtype, int64_t rows, int64_t cols, int b, float *y);
int orc_dequantize_weight(const int8_t *qw, const float *sw, int64_t N, int64_t K, int b,
                          float *w);
int orc_quantize_rows(const void *x, int dtype, int64_t rows, int64_t cols,
                      const float *prescale, int had_block, int8_t *q, float *s);
int orc_quantize_cols(const void *x, int dtype, int64_t rows, int64_t cols,
                      const float *prescale, int8_t *q, float *s, float *col_sum);
int orc_gemm_s32(int op, const int8_t *a, const int8_t *b, int64_t M, int64_t N, int64_t K,
                 int32_t *c);
int orc_gemm_s32_at(int op, const int8_t *a, const int8_t *b, int64_t M, int64_t N, int64_t K,
                    const int64_t *ii, const int64_t *jj, int64_t count, int32_t *out);
int orc_fwd(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
            const float *bias, int64_t M, int64_t N, int64_t K, float *y);
int orc_bwd_dx(const int8_t *qg1, const float *sg1, const int8_t *qw, int64_t M, int64_t N,
               int64_t K, float *dx);
int orc_bwd_dw(const int8_t *qg2, const float *sg2, const int8_t *qx, int64_t M, int64_t N,
               int64_t K, float *dw);
int orc_bwd_dw_rows(const int8_t *qg2, const float *sg2, const int8_t *qx, int64_t M,
                    int64_t N, int64_t K, const int64_t *rows, int64_t count, float *out);
int orc_op_at(int op, const int8_t *a, const float *srow, const int8_t *b, const float *scol,
              const float *bias, int64_t M, int64_t N, int64_t K, const int64_t *ii,
              const int64_t *jj, int64_t count, float *out);
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);
uint32_t orc_sr_bits16(uint64_t seed, uint64_t step, uint64_t i);
int orc_sgd_requant(int8_t *qw, float *sw, const float *dw, int64_t N, int64_t K, float lr,
                    uint64_t seed, uint64_t step, float *bias, const float *db,
                    const int64_t *row_ids);
int orc_wn_init(const int8_t *q, const float *s, int64_t N, int64_t K, float *g, float *sw);
int orc_wn_grads(const int8_t *q, const float *s, const float *g, const float *dw, int64_t N,
                 int64_t K, float *dg, float *dv);
int orc_wn_sgd_requant(int8_t *q, float *s, float *g, float *sw, const float *dw, int64_t N,
                       int64_t K, float lr, uint64_t seed, uint64_t step, float *bias,
                       const float *db, const int64_t *row_ids);
void orc_adamw_constants(float lr, float b1, float b2, float wd, uint64_t t, float k[5]);
int orc_adamw_update(const int8_t *qw, const float *sw, const float *dw, float *m, float *v,
                     int64_t N, int64_t K, float lr, float b1, float b2, float eps, float wd,
                     uint64_t t, float *w);
int orc_adamw_requant(int8_t *qw, float *sw, const float *dw, float *m, float *v, int64_t N,
                      int64_t K, float lr, float b1, float b2, float eps, float wd,
                      uint64_t seed, uint64_t t, float *bias, const float *db, float *bm,
                      float *bv, const int64_t *row_ids);
int orc_gemm_s64_at(int op, const int8_t *a, const int8_t *b, int64_t M, int64_t N, int64_t K,
                    const int64_t *ii, const int64_t *jj, int64_t count, int64_t *out);
int orc_op_at_long(int op, const int8_t *a, const float *srow, const int8_t *b,
                   const float *scol, const float *bias, int64_t M, int64_t N, int64_t K,
                   const int64_t *ii, const int64_t *jj, int64_t count, float *out);

static int failures = 0;

static void expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        failures++;
    }
}

/* Exactly sized heap arrays, so that any access past an end is reported. */
static void *arr(size_t n) { return malloc(n ? n : 1); }

static uint32_t lcg = 12345u;
static uint32_t next_u32(void)
{
    lcg = lcg * 1664525u + 1013904223u;
    return lcg;
}
static float randf(void) { return (float)(int)(next_u32() % 2001u - 1000) * 0.001f; }

static float *rand_f32(size_t n)
{
    float *p = arr(n * sizeof(float));
    for (size_t i = 0; i < n; i++)
        p[i] = randf();
    return p;
}
/* One shape of the whole layer: quantizers, products, updates. */
static void run_shape(int64_t M, int64_t N, int64_t K, int had)
{
    float *x = rand_f32((size_t)(M * K)), *w = rand_f32((size_t)(N * K));
    float *dy = rand_f32((size_t)(M * N)), *bias = rand_f32((size_t)N);
    uint16_t *xb = arr((size_t)(M * K) * 2);
    for (int64_t i = 0; i < M * K; i++) {
        uint32_t u;
        memcpy(&u, &x[i], 4);
        xb[i] = (uint16_t)(u >> 16);
    }
    int8_t *qx = arr((size_t)(M * K)), *qw = arr((size_t)(N * K));
    int8_t *qg1 = arr((size_t)(M * N)), *qg2 = arr((size_t)(M * N));
    float *sx = arr((size_t)M * 4), *sw = arr((size_t)N * 4), *sg1 = arr((size_t)M * 4);
    float *sg2 = arr((size_t)N * 4), *db = arr((size_t)N * 4);
    float *rot = arr((size_t)(M * K) * 4);

    if (had) {
        expect(orc_hadamard(x, 0, M, K, had, rot), 0, "hadamard f32");
        expect(orc_hadamard(xb, 1, M, K, had, rot), 0, "hadamard bf16");
    }
    expect(orc_quantize_rows(w, 0, N, K, NULL, had, qw, sw), 0, "quantize weight");
    expect(orc_quantize_rows(xb, 1, M, K, NULL, had, qx, sx), 0, "quantize x");
    expect(orc_quantize_rows(dy, 0, M, N, sw, 0, qg1, sg1), 0, "quantize dy rows");
    expect(orc_quantize_cols(dy, 0, M, N, sx, qg2, sg2, db), 0, "quantize dy cols");

    float *y = arr((size_t)(M * N) * 4), *dx = arr((size_t)(M * K) * 4);
    float *dw = arr((size_t)(N * K) * 4);
    int32_t *c = arr((size_t)(M * (N > K ? N : K) + N * K) * 4);
    expect(orc_fwd(qx, sx, qw, sw, bias, M, N, K, y), 0, "fwd");
    expect(orc_bwd_dx(qg1, sg1, qw, M, N, K, dx), 0, "bwd_dx");
    expect(orc_bwd_dw(qg2, sg2, qx, M, N, K, dw), 0, "bwd_dw");
    expect(orc_gemm_s32(0, qx, qw, M, N, K, c), 0, "gemm fwd");
    expect(orc_gemm_s32(1, qg1, qw, M, N, K, c), 0, "gemm dx");
    expect(orc_gemm_s32(2, qg2, qx, M, N, K, c), 0, "gemm dw");

    enum { S = 5 };
    int64_t ii[S], jj[S], rows[S];
    int32_t o32[S];
    int64_t o64[S];
    float of[S], orows[S * 64];
    for (int op = 0; op < 3; op++) {
        const int64_t R = op == 2 ? N : M, C = op == 0 ? N : K;
        for (int t = 0; t < S; t++) {
            ii[t] = R ? (int64_t)(next_u32() % (uint32_t)R) : 0;
            jj[t] = (int64_t)(next_u32() % (uint32_t)C);
        }
        const int8_t *a = op == 0 ? qx : (op == 1 ? qg1 : qg2);
        const int8_t *b = op == 2 ? qx : qw;
        const float *sr = op == 0 ? sx : (op == 1 ? sg1 : sg2);
        const int n = R ? S : 0;
        expect(orc_gemm_s32_at(op, a, b, M, N, K, ii, jj, n, o32), 0, "gemm_s32_at");
        expect(orc_gemm_s64_at(op, a, b, M, N, K, ii, jj, n, o64), 0, "gemm_s64_at");
        expect(orc_op_at(op, a, sr, b, op == 0 ? sw : NULL, op == 0 ? bias : NULL, M, N, K, ii,
                         jj, n, of),
               0, "op_at");
        expect(orc_op_at_long(op, a, sr, b, op == 0 ? sw : NULL, op == 0 ? bias : NULL, M, N, K,
                              ii, jj, n, of),
               0, "op_at_long");
    }
    if (K <= 64) {
        for (int t = 0; t < S; t++)
            rows[t] = (int64_t)(next_u32() % (uint32_t)N);
        expect(orc_bwd_dw_rows(qg2, sg2, qx, M, N, K, rows, S, orows), 0, "bwd_dw_rows");
    }
    float *wexp = arr((size_t)(N * K) * 4);
    expect(orc_dequantize_weight(qw, sw, N, K, had, wexp), 0, "dequantize weight");
    free(wexp);

    int64_t *ids = arr((size_t)N * 8);
    for (int64_t n = 0; n < N; n++)
        ids[n] = 3 * n + 1;
    expect(orc_sgd_requant(qw, sw, dw, N, K, 1e-3f, 7, 2, bias, db, ids), 0, "sgd");
    float *m = arr((size_t)(N * K) * 4), *v = arr((size_t)(N * K) * 4), *wo = arr((size_t)(N * K) * 4);
    memset(m, 0, (size_t)(N * K) * 4);
    memset(v, 0, (size_t)(N * K) * 4);
    float *bm = arr((size_t)N * 4), *bv = arr((size_t)N * 4);
    memset(bm, 0, (size_t)N * 4);
    memset(bv, 0, (size_t)N * 4);
    expect(orc_adamw_update(qw, sw, dw, m, v, N, K, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 1, wo), 0,
           "adamw update");
    expect(orc_adamw_requant(qw, sw, dw, m, v, N, K, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 5, 1, bias,
                             db, bm, bv, NULL),
           0, "adamw requant");
    float *g = arr((size_t)N * 4), *swn = arr((size_t)N * 4), *dg = arr((size_t)N * 4);
    float *dv = arr((size_t)(N * K) * 4);
    if (orc_wn_init(qw, sw, N, K, g, swn) == 0) {
        expect(orc_wn_grads(qw, sw, g, dw, N, K, dg, dv), 0, "wn grads");
        expect(orc_wn_sgd_requant(qw, sw, g, swn, dw, N, K, 1e-3f, 3, 1, bias, db, NULL), 0,
               "wn sgd");
    }

    free(x); free(w); free(dy); free(bias); free(xb); free(qx); free(qw); free(qg1); free(qg2);
    free(sx); free(sw); free(sg1); free(sg2); free(db); free(rot); free(y); free(dx); free(dw);
    free(c); free(ids); free(m); free(v); free(wo); free(bm); free(bv); free(g); free(swn);
    free(dg); free(dv);
}

int main(void)
{
    run_shape(17, 48, 32, 0);
    run_shape(5, 16, 256, 128);
    run_shape(1, 32, 512, 512);
    run_shape(33, 64, 64, 2);
    run_shape(0, 16, 16, 0);          /* no tokens */

    /* All-zero rows and columns. */
    float z[4 * 16] = {0};
    int8_t q[4 * 16];
    float s[16], cs[16];
    expect(orc_quantize_rows(z, 0, 4, 16, NULL, 0, q, s), 0, "zero rows");
    expect(orc_quantize_cols(z, 0, 4, 16, NULL, q, s, cs), 0, "zero cols");

    /* Rejections. */
    expect(orc_hadamard(z, 0, 1, 16, 3, cs), 1, "bad block");
    expect(orc_quantize_rows(z, 0, 1, 48, NULL, 32, q, s), 1, "block does not divide");
    int8_t one[16] = {1};
    int32_t c1[1];
    expect(orc_gemm_s32(0, one, one, 1, 16, 131072, c1), 2, "contraction bound");
    expect(orc_gemm_s32(3, one, one, 1, 16, 16, c1), 1, "unknown op");

    /* Generators and constants. */
    uint32_t c32[4] = {1, 2, 3, 4}, k32[2] = {5, 6}, o32[4];
    uint64_t c64[4] = {1, 2, 3, 4}, k64[2] = {5, 6}, o64[4];
    orc_philox4x32_10(c32, k32, o32);
    orc_philox4x64_10(c64, k64, o64);
    uint32_t acc = 0;
    for (uint64_t i = 0; i < 64; i++)
        acc ^= orc_sr_bits16(0xFFFFFFFFFFFFFFFFull, 0xFFFFFFFFFFFFFFFFull, i * 0x123456789ull);
    float kk[5];
    orc_adamw_constants(1e-3f, 0.9f, 0.999f, 0.01f, 1000000, kk);
    if (orc_threads() < 1 || orc_hadamard_scale(128) <= 0.0f)
        failures++;
    printf("sanitized oracle driver: %d failures (%u)\n", failures, acc & 1u);
    return failures != 0;
}
