/*
 * CPU oracle for the INT8 W8A8 linear layer used in quantized training.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the package smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no source, header, table or
 * constant generator with the HIP library.
 *
 * Sources (the pages this implements):
 *  - mini_trainer, "quantized-training" guide: INT8 weights with a floating
 *    magnitude per output row, saved INT8 Linear inputs, integer forward and
 *    backward products, no float master weight, stochastic requantization of
 *    represented weights on update, and a bound of 131,071 on the contraction
 *    length for exact int32 partial dot products (feature table; update and
 *    arithmetic paragraphs).
 *  - OneTrainer PR #1681 "Int8 conv rot": a block-Hadamard rotation along the
 *    contraction dimension applied to the activations, per-row activation
 *    quantization on every call, int8 x int8 -> int32 matrix products, and an
 *    orthogonal rotation buffer (summary; commit notes 1 and 2).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - Rotation: Sylvester (natural order) Hadamard, normalised by 1/sqrt(b),
 *    applied as an in-place butterfly with stages h = 1, 2, 4, ... ascending,
 *    then one multiply by c_b = fl32(1/sqrt(b)).
 *  - Quantization: symmetric absmax, s = fl(amax / 127), q = clamp(rne(fl(g /
 *    s)), -127, 127); an all-zero row gives s = 0 and q = 0.
 *  - Dequant epilogues: fl(fl(fl32(acc) * s_row) * s_col) + bias, in that order.
 *  - Gradient scales sit on non-contraction axes only: dY is prescaled by s_w
 *    and quantized per row for dX, prescaled by s_x and quantized per column
 *    for dW.
 *  - SGD stochastic requant: w = fl(fl(s*q) - fl(lr*dw)), new per-row absmax
 *    scale, then q' = floor(y) + (u < frac(y)) with y = fl(w / s') and u a
 *    16-bit uniform from Philox4x32-10 keyed by (seed) with counter
 *    (element_index >> 3, step).
 *  - AdamW stochastic requant (the guide lists AdamW among the update paths
 *    with coverage on INT8 weights; its arithmetic is not given): the
 *    published decoupled-weight-decay algorithm with bias-corrected moments,
 *    in fp32 with host constants rounded once from double:
 *      m' = fl(fl(b1*m) + fl(a1*g)), v' = fl(fl(b2*v) + fl(fl(a2*g)*g)),
 *      d = fl(fl(sqrt(v')*c2) + eps), w = fl(fl(fl(s*q)*decay) - fl(c1*fl(m'/d)))
 *    with a1 = 1-b1, a2 = 1-b2, c1 = lr/(1-b1^t), c2 = 1/sqrt(1-b2^t),
 *    decay = 1-lr*wd, then the same row requant as SGD with Philox step t.
 *  - Row weight normalization (the guide's feature table: an INT8 direction
 *    and a floating magnitude per output row): W[n, :] = g[n] v[n, :] /
 *    ||v[n, :]|| with the direction v = s q held as INT8 codes q and a row
 *    scale s, and g trained as its own parameter.  ||q|| = fl32(sqrt(sum q^2))
 *    with the integer sum exact and the square root in double.  The products'
 *    column scale is fl(g / ||q||).  Backward from dW (the gradient of the
 *    represented weight): dot = fl32 of the pairwise (zero-padded to a power
 *    of two, adjacent pairs first) double sum of dW_k q_k; dg = fl(dot /
 *    ||q||); dv_k = fl(fl(g / fl(s ||q||)) * fl(dW_k - fl(fl(dg / ||q||) *
 *    q_k))).  SGD: g' = fl(g - fl(lr dg)), w_k = fl(fl(s q_k) - fl(lr dv_k)),
 *    then the row requant of SGD.  At preparation g = fl(s ||q||), so the
 *    represented weight starts as the absmax one.
 *  - fp32 arithmetic: IEEE binary32, round to nearest even, no FMA
 *    contraction (built with -ffp-contract=off), IEEE division.
 *
 * Parity is pinned by tests against scipy's Hadamard matrix, brute-force
 * integer and float64 matrix products, exactly quantizable inputs, numpy's
 * Philox4x64-10, Triton's Philox4x32-10 (run by its CPU interpreter),
 * statistical properties of the stochastic rounding, and numpy float32
 * replicas of every fp32 step above (rotation stage order, the quantizer's
 * division, the epilogue order, the SGD update and its rounding comparison),
 * compared bit for bit.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_EUNSUPPORTED 2

#define ORC_F32 0
#define ORC_BF16 1

/* Longest contraction whose int32 dot product of int8 values cannot overflow:
 * 131071 * 128 * 128 < 2^31 (mini_trainer guide, arithmetic paragraph on
 * contractions above 131,071). */
#define ORC_MAX_CONTRACTION 131071

/* Threads the parallel loops use (OMP_NUM_THREADS or all cores). */
int orc_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- helpers */

static float bf16_bits_to_f32(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16; /* bf16 is the top half of binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float load_elem(const void *x, int dtype, int64_t idx)
{
    if (dtype == ORC_BF16)
        return bf16_bits_to_f32(((const uint16_t *)x)[idx]);
    return ((const float *)x)[idx];
}

static int is_pow2(int64_t b) { return b > 0 && (b & (b - 1)) == 0; }

/* Normalisation of the b-point Hadamard: the double 1/sqrt(b), rounded once. */
float orc_hadamard_scale(int b) { return (float)(1.0 / sqrt((double)b)); }

/* Round half to even on a float, returned as float. */
static float rne(float v) { return nearbyintf(v); }

/* ----------------------------------------------------- Hadamard rotation */

/* Normalised Walsh-Hadamard transform of one block of length b, in place.
 * Stage h pairs element i with element i + h for every i whose bit h is clear
 * and replaces them by their sum and difference.  Afterwards every element is
 * multiplied by c_b.  The result is x * H_b / sqrt(b) with H_b the Sylvester
 * Hadamard matrix, which is symmetric, so the map is its own inverse
 * (OneTrainer PR #1681: rotation along the contraction dimension; the buffer
 * is orthogonal). */
static void fwht_block(float *y, int b)
{
    for (int h = 1; h < b; h <<= 1) {
        for (int i = 0; i < b; i++) {
            if ((i & h) == 0) {
                float lo = y[i];
                float hi = y[i + h];
                y[i] = lo + hi;
                y[i + h] = lo - hi;
            }
        }
    }
    float cb = orc_hadamard_scale(b);
    for (int j = 0; j < b; j++)
        y[j] = y[j] * cb;
}

int orc_check_block(int64_t cols, int b)
{
    if (b < 2 || b > 512 || !is_pow2(b))
        return ORC_EINVAL;
    if (cols % b != 0)
        return ORC_EINVAL;
    return ORC_OK;
}

/* y[rows, cols] (fp32) = block-Hadamard rotation of x along each row. */
int orc_hadamard(const void *x, int dtype, int64_t rows, int64_t cols, int b, float *y)
{
    if (orc_check_block(cols, b) != ORC_OK)
        return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float *row = y + r * cols;
        for (int64_t c = 0; c < cols; c++)
            row[c] = load_elem(x, dtype, r * cols + c);
        for (int64_t c0 = 0; c0 < cols; c0 += b)
            fwht_block(row + c0, b);
    }
    return ORC_OK;
}

/* The represented weight in the original basis (OneTrainer PR #1681, commit
 * note 2: callers that need the unquantized weight, such as LoRA, offload or
 * export, un-rotate it): w = fl(s[n] * q[n, k]) per row, then, when b != 0,
 * the rotation of each block (its own inverse).  w is [N, K] fp32. */
int orc_dequantize_weight(const int8_t *qw, const float *sw, int64_t N, int64_t K, int b,
                          float *w)
{
    if (N < 0 || K < 1 || (b != 0 && orc_check_block(K, b) != ORC_OK))
        return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        float *row = w + n * K;
        for (int64_t k = 0; k < K; k++)
            row[k] = sw[n] * (float)qw[n * K + k];
        if (b != 0)
            for (int64_t c0 = 0; c0 < K; c0 += b)
                fwht_block(row + c0, b);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------ quantizers */

/* Symmetric absmax quantization of one vector g[0..n) with element stride
 * 'qstride' in the output (OneTrainer PR #1681: per-row activation
 * quantization; mini_trainer guide: INT8 direction times a floating
 * magnitude). */
static float quant_vec(const float *g, int64_t n, int8_t *q, int64_t qstride)
{
    float amax = 0.0f;
    for (int64_t j = 0; j < n; j++) {
        float a = fabsf(g[j]);
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0f) {
        for (int64_t j = 0; j < n; j++)
            q[j * qstride] = 0;
        return 0.0f;
    }
    float s = amax / 127.0f;
    for (int64_t j = 0; j < n; j++) {
        float v = rne(g[j] / s);
        if (v > 127.0f)
            v = 127.0f;
        if (v < -127.0f)
            v = -127.0f;
        q[j * qstride] = (int8_t)v;
    }
    return s;
}

/* Per-row quantization of x[rows, cols]: optional block-Hadamard rotation of
 * each row (b = had_block, 0 = none), then an optional per-column prescale,
 * then absmax quantization of the row.  q[rows, cols], s[rows]. */
int orc_quantize_rows(const void *x, int dtype, int64_t rows, int64_t cols,
                      const float *prescale, int had_block, int8_t *q, float *s)
{
    if (rows < 0 || cols < 1)
        return ORC_EINVAL;
    if (had_block != 0 && orc_check_block(cols, had_block) != ORC_OK)
        return ORC_EINVAL;
#pragma omp parallel
    {
        float *g = (float *)malloc((size_t)cols * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; r++) {
            for (int64_t c = 0; c < cols; c++)
                g[c] = load_elem(x, dtype, r * cols + c);
            if (had_block)
                for (int64_t c0 = 0; c0 < cols; c0 += had_block)
                    fwht_block(g + c0, had_block);
            if (prescale)
                for (int64_t c = 0; c < cols; c++)
                    g[c] = g[c] * prescale[c];
            s[r] = quant_vec(g, cols, q + r * cols, 1);
        }
        free(g);
    }
    return ORC_OK;
}

/* Per-column quantization of x[rows, cols]: g[r, c] = x[r, c] * prescale[r]
 * (prescale optional), then absmax quantization of each column.  q keeps the
 * layout of x; s[cols].  col_sum[c] (optional) = sum over r of the raw x[r, c],
 * accumulated in fp32 in increasing r. */
int orc_quantize_cols(const void *x, int dtype, int64_t rows, int64_t cols,
                      const float *prescale, int8_t *q, float *s, float *col_sum)
{
    if (rows < 0 || cols < 1)
        return ORC_EINVAL;
#pragma omp parallel
    {
        float *g = (float *)malloc((size_t)(rows > 0 ? rows : 1) * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t c = 0; c < cols; c++) {
            float sum = 0.0f;
            for (int64_t r = 0; r < rows; r++) {
                float v = load_elem(x, dtype, r * cols + c);
                sum = sum + v;
                g[r] = prescale ? v * prescale[r] : v;
            }
            s[c] = quant_vec(g, rows, q + c, cols);
            if (col_sum)
                col_sum[c] = sum;
        }
        free(g);
    }
    return ORC_OK;
}

/* ------------------------------------------------ integer matrix products */

/* The three contractions of the layer (mini_trainer guide: integer forward and
 * backward matrix products over INT8 weights and saved INT8 inputs):
 *   op 0, forward : acc[m, n] = sum_k qx[m, k]  * qw[n, k]   a = qx [M,K], b = qw [N,K]
 *   op 1, dX      : acc[m, k] = sum_n qg1[m, n] * qw[n, k]   a = qg1[M,N], b = qw [N,K]
 *   op 2, dW      : acc[n, k] = sum_m qg2[m, n] * qx[m, k]   a = qg2[M,N], b = qx [M,K]
 * Each is a plain dot product accumulated in int64 and checked to fit int32. */
static int64_t dot_op(int op, const int8_t *a, const int8_t *b, int64_t M, int64_t N,
                      int64_t K, int64_t i, int64_t j)
{
    int64_t acc = 0;
    if (op == 0) { /* i = m, j = n */
        for (int64_t k = 0; k < K; k++)
            acc += (int64_t)a[i * K + k] * (int64_t)b[j * K + k];
    } else if (op == 1) { /* i = m, j = k */
        for (int64_t n = 0; n < N; n++)
            acc += (int64_t)a[i * N + n] * (int64_t)b[n * K + j];
    } else { /* i = n, j = k */
        for (int64_t m = 0; m < M; m++)
            acc += (int64_t)a[m * N + i] * (int64_t)b[m * K + j];
    }
    return acc;
}

static void op_shape(int op, int64_t M, int64_t N, int64_t K, int64_t *rows,
                     int64_t *cols, int64_t *contraction)
{
    if (op == 0) { *rows = M; *cols = N; *contraction = K; }
    else if (op == 1) { *rows = M; *cols = K; *contraction = N; }
    else { *rows = N; *cols = K; *contraction = M; }
}

static int check_op(int op, int64_t M, int64_t N, int64_t K)
{
    if (op < 0 || op > 2 || M < 0 || N < 1 || K < 1)
        return ORC_EINVAL;
    int64_t R, C, T;
    op_shape(op, M, N, K, &R, &C, &T);
    if (T > ORC_MAX_CONTRACTION)
        return ORC_EUNSUPPORTED;
    return ORC_OK;
}

/* Raw int32 accumulators of one product, full matrix [rows, cols]. */
int orc_gemm_s32(int op, const int8_t *a, const int8_t *b, int64_t M, int64_t N,
                 int64_t K, int32_t *c)
{
    int st = check_op(op, M, N, K);
    if (st != ORC_OK)
        return st;
    int64_t R, C, T;
    op_shape(op, M, N, K, &R, &C, &T);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; i++)
        for (int64_t j = 0; j < C; j++)
            c[i * C + j] = (int32_t)dot_op(op, a, b, M, N, K, i, j);
    return ORC_OK;
}

/* Raw int32 accumulators at sampled positions (ii[t], jj[t]). */
int orc_gemm_s32_at(int op, const int8_t *a, const int8_t *b, int64_t M, int64_t N,
                    int64_t K, const int64_t *ii, const int64_t *jj, int64_t count,
                    int32_t *out)
{
    int st = check_op(op, M, N, K);
    if (st != ORC_OK)
        return st;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; t++)
        out[t] = (int32_t)dot_op(op, a, b, M, N, K, ii[t], jj[t]);
    return ORC_OK;
}

/* Dequantized value of one output element of a product.
 *   forward: y  = fl(fl(fl32(acc) * sx[m]) * sw[n]) + bias[n]   (bias optional)
 *   dX     : dx = fl(fl32(acc) * sg1[m])        (rotated basis)
 *   dW     : dw = fl(fl32(acc) * sg2[n])
 * srow is the scale of the output row (sx, sg1 or sg2), scol the scale of the
 * output column (sw for the forward product, unused otherwise). */
static float dequant_f(int op, float v, const float *srow, const float *scol,
                       const float *bias, int64_t i, int64_t j)
{
    v = v * srow[i];
    if (op == 0) {
        v = v * scol[j];
        if (bias)
            v = v + bias[j];
    }
    return v;
}

static float dequant(int op, int64_t acc, const float *srow, const float *scol,
                     const float *bias, int64_t i, int64_t j)
{
    return dequant_f(op, (float)(int32_t)acc, srow, scol, bias, i, j);
}

/* Forward: y[M, N] from (qx, sx) and (qw, sw), optional bias. */
int orc_fwd(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
            const float *bias, int64_t M, int64_t N, int64_t K, float *y)
{
    int st = check_op(0, M, N, K);
    if (st != ORC_OK)
        return st;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = dequant(0, dot_op(0, qx, qw, M, N, K, m, n), sx, sw, bias, m, n);
    return ORC_OK;
}

/* dX in the rotated basis: dx[M, K] from (qg1, sg1) and qw. */
int orc_bwd_dx(const int8_t *qg1, const float *sg1, const int8_t *qw, int64_t M,
               int64_t N, int64_t K, float *dx)
{
    int st = check_op(1, M, N, K);
    if (st != ORC_OK)
        return st;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < K; k++)
            dx[m * K + k] = dequant(1, dot_op(1, qg1, qw, M, N, K, m, k), sg1, NULL, NULL, m, k);
    return ORC_OK;
}

/* One row of dW: out[k] = fl(fl32(sum_m qg2[m, n] * qx[m, k]) * sg2[n]) for all
 * k, accumulated over m with the saved-input rows streamed in order. */
static void dw_row(const int8_t *qg2, const float *sg2, const int8_t *qx, int64_t M,
                   int64_t N, int64_t K, int64_t n, int64_t *acc, float *out)
{
    for (int64_t k = 0; k < K; k++)
        acc[k] = 0;
    for (int64_t m = 0; m < M; m++) {
        int64_t g = qg2[m * N + n];
        if (g == 0)
            continue;
        for (int64_t k = 0; k < K; k++)
            acc[k] += g * (int64_t)qx[m * K + k];
    }
    for (int64_t k = 0; k < K; k++)
        out[k] = dequant(2, acc[k], sg2, NULL, NULL, n, k);
}

/* dW: dw[N, K] from (qg2, sg2) (qg2 [M, N] with per-column scales) and the
 * saved qx [M, K]. */
int orc_bwd_dw(const int8_t *qg2, const float *sg2, const int8_t *qx, int64_t M,
               int64_t N, int64_t K, float *dw)
{
    int st = check_op(2, M, N, K);
    if (st != ORC_OK)
        return st;
#pragma omp parallel
    {
        int64_t *acc = (int64_t *)malloc((size_t)K * sizeof(int64_t));
#pragma omp for schedule(dynamic)
        for (int64_t n = 0; n < N; n++)
            dw_row(qg2, sg2, qx, M, N, K, n, acc, dw + n * K);
        free(acc);
    }
    return ORC_OK;
}

/* Selected rows of dW: out[t, :] = dw[rows[t], :]. */
int orc_bwd_dw_rows(const int8_t *qg2, const float *sg2, const int8_t *qx, int64_t M,
                    int64_t N, int64_t K, const int64_t *rows, int64_t count, float *out)
{
    int st = check_op(2, M, N, K);
    if (st != ORC_OK)
        return st;
#pragma omp parallel
    {
        int64_t *acc = (int64_t *)malloc((size_t)K * sizeof(int64_t));
#pragma omp for schedule(dynamic)
        for (int64_t t = 0; t < count; t++)
            dw_row(qg2, sg2, qx, M, N, K, rows[t], acc, out + t * K);
        free(acc);
    }
    return ORC_OK;
}

/* Dequantized outputs of one product at sampled positions. */
int orc_op_at(int op, const int8_t *a, const float *srow, const int8_t *b,
              const float *scol, const float *bias, int64_t M, int64_t N, int64_t K,
              const int64_t *ii, const int64_t *jj, int64_t count, float *out)
{
    int st = check_op(op, M, N, K);
    if (st != ORC_OK)
        return st;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; t++)
        out[t] = dequant(op, dot_op(op, a, b, M, N, K, ii[t], jj[t]), srow, scol, bias,
                         ii[t], jj[t]);
    return ORC_OK;
}

/* ------------------------------------------------------------- Philox */

/* Philox-4xW-10 counter-based generator (Salmon, Moraes, Dror, Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC'11).  One round multiplies counter
 * words 0 and 2 by the round multipliers, keeps the full double-width
 * products, and forms the next counter as
 *   (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0));
 * between rounds the key is bumped by the Weyl constants.  Ten rounds, the
 * first with the unbumped key.  The word size is a parameter so the 64-bit
 * instance can be checked against an independent implementation and the
 * 32-bit instance used for the stochastic rounding. */
#define PHILOX_ROUNDS 10

/* One definition for both word sizes: WORD is the counter/key word, WIDE holds
 * a full product of two words, SHIFT is the word size in bits. */
#define DEFINE_PHILOX4(NAME, WORD, WIDE, SHIFT, M0, M1, W0, W1)                   \
    void NAME(const WORD ctr_in[4], const WORD key_in[2], WORD out[4])             \
    {                                                                              \
        WORD c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];       \
        WORD k0 = key_in[0], k1 = key_in[1];                                       \
        for (int r = 0; r < PHILOX_ROUNDS; r++) {                                  \
            if (r > 0) {                                                           \
                k0 += (WORD)(W0);                                                  \
                k1 += (WORD)(W1);                                                  \
            }                                                                      \
            WIDE p0 = (WIDE)(WORD)(M0) * (WIDE)c0;                                 \
            WIDE p1 = (WIDE)(WORD)(M1) * (WIDE)c2;                                 \
            WORD hi0 = (WORD)(p0 >> SHIFT), lo0 = (WORD)p0;                        \
            WORD hi1 = (WORD)(p1 >> SHIFT), lo1 = (WORD)p1;                        \
            WORD n0 = hi1 ^ c1 ^ k0;                                               \
            WORD n1 = lo1;                                                         \
            WORD n2 = hi0 ^ c3 ^ k1;                                               \
            WORD n3 = lo0;                                                         \
            c0 = n0; c1 = n1; c2 = n2; c3 = n3;                                    \
        }                                                                          \
        out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;                        \
    }

/* Round multipliers and Weyl key increments from the paper's tables. */
DEFINE_PHILOX4(orc_philox4x32_10, uint32_t, uint64_t, 32,
               0xD2511F53u, 0xCD9E8D57u, 0x9E3779B9u, 0xBB67AE85u)
DEFINE_PHILOX4(orc_philox4x64_10, uint64_t, unsigned __int128, 64,
               0xD2E7470EE14C6C93ull, 0xCA5A826395121157ull,
               0x9E3779B97F4A7C15ull, 0xBB67AE8584CAA73Bull)

/* The 16-bit uniform used to round element i (its index in the row-major
 * weight matrix) at optimizer step 'step' with seed 'seed'.  One Philox block
 * serves eight consecutive elements: counter = (lo(i>>3), hi(i>>3), lo(step),
 * hi(step)), key = (lo(seed), hi(seed)); element i takes 16-bit half (i & 1) of
 * output word (i & 7) >> 1. */
uint32_t orc_sr_bits16(uint64_t seed, uint64_t step, uint64_t i)
{
    uint64_t blk = i >> 3;
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)step,
                       (uint32_t)(step >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t x[4];
    orc_philox4x32_10(ctr, key, x);
    uint32_t word = x[(i & 7) >> 1];
    return (word >> (16 * (i & 1))) & 0xFFFFu;
}

/* Stochastic requant of one updated row w [K] (the tail shared by the SGD and
 * AdamW updates): s' = fl(amax / 127) (0 for an all-zero row), y = fl(w / s'),
 * q' = clamp(floor(y) + (u < y - floor(y)), -127, 127) with u the 16-bit
 * Philox uniform of global element index grow * K + j. */
static float requant_row(const float *w, int64_t K, int64_t grow, uint64_t seed,
                         uint64_t step, int8_t *q)
{
    float amax = 0.0f;
    for (int64_t j = 0; j < K; j++) {
        float a = fabsf(w[j]);
        if (a > amax)
            amax = a;
    }
    float s_new = amax == 0.0f ? 0.0f : amax / 127.0f;
    for (int64_t j = 0; j < K; j++) {
        int8_t code = 0;
        if (s_new != 0.0f) {
            float y = w[j] / s_new;
            float f = floorf(y);
            float frac = y - f;
            float u = (float)orc_sr_bits16(seed, step, (uint64_t)(grow * K + j)) *
                      (1.0f / 65536.0f);
            float v = f + (u < frac ? 1.0f : 0.0f);
            if (v > 127.0f)
                v = 127.0f;
            if (v < -127.0f)
                v = -127.0f;
            code = (int8_t)v;
        }
        q[j] = code;
    }
    return s_new;
}

/* --------------------------------------- SGD with stochastic requantization */

/* One plain SGD step on the represented weight, then stochastic requant of
 * each row (mini_trainer guide: updates stochastically requantize represented
 * weights, no floating master weight is kept).  In place on qw [N, K] and
 * sw [N]; bias -= lr * db when both are given.  row_ids (optional) gives the
 * row index of each local row in the full weight matrix, which keys the
 * random stream; without it local row n is row n. */
int orc_sgd_requant(int8_t *qw, float *sw, const float *dw, int64_t N, int64_t K,
                    float lr, uint64_t seed, uint64_t step, float *bias, const float *db,
                    const int64_t *row_ids)
{
    if (N < 0 || K < 1)
        return ORC_EINVAL;
#pragma omp parallel
    {
        float *w = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; n++) {
            float s = sw[n];
            for (int64_t j = 0; j < K; j++) {
                float cur = s * (float)qw[n * K + j];
                float upd = lr * dw[n * K + j];
                w[j] = cur - upd;
            }
            sw[n] = requant_row(w, K, row_ids ? row_ids[n] : n, seed, step, qw + n * K);
        }
        free(w);
    }
    if (bias && db)
        for (int64_t n = 0; n < N; n++)
            bias[n] = bias[n] - lr * db[n];
    return ORC_OK;
}

/* ------------------------------------------ row weight normalization */

/* ||q|| of one row of codes: the exact integer sum of squares, square root
 * in double, rounded once to fp32. */
static float code_norm(const int8_t *q, int64_t K)
{
    int64_t n2 = 0;
    for (int64_t k = 0; k < K; k++)
        n2 += (int64_t)q[k] * q[k];
    return (float)sqrt((double)n2);
}

/* Pairwise sum of x[lo .. lo + len) (len a power of two) where positions at
 * or past n read as zero: the two halves are summed first, then added. */
static double pairwise(const double *x, int64_t n, int64_t lo, int64_t len)
{
    if (len == 1)
        return lo < n ? x[lo] : 0.0;
    return pairwise(x, n, lo, len / 2) + pairwise(x, n, lo + len / 2, len / 2);
}

/* Gradients of one row for the magnitude (dg) and the direction (dv [K]),
 * from dW [K] (the gradient of the represented weight g v / ||v||, v = s q):
 *   dL/dg = <dW, v> / ||v|| = <dW, q> / ||q||,
 *   dL/dv = (g / ||v||) (dW - (dL/dg) v / ||v||)
 *         = (g / (s ||q||)) (dW - (dL/dg / ||q||) q).
 * A row whose codes are all zero has no direction: both gradients are zero. */
static void wn_row_grads(const int8_t *q, float s, float g, const float *dw, int64_t K,
                         double *tmp, float *dg, float *dv)
{
    const float nrm = code_norm(q, K);
    if (nrm == 0.0f) {
        *dg = 0.0f;
        for (int64_t k = 0; k < K; k++)
            dv[k] = 0.0f;
        return;
    }
    for (int64_t k = 0; k < K; k++)
        tmp[k] = (double)dw[k] * (double)q[k];     /* exact */
    int64_t len = 1;
    while (len < K)
        len *= 2;
    const float dot = (float)pairwise(tmp, K, 0, len);
    const float d = dot / nrm;
    const float a = g / (s * nrm);
    const float b = d / nrm;
    for (int64_t k = 0; k < K; k++)
        dv[k] = a * (dw[k] - b * (float)q[k]);
    *dg = d;
}

/* Magnitude and column scale of a weight-normalized layer at preparation,
 * from its direction codes and row scales: g = fl(s ||q||), sw = fl(g /
 * ||q||).  An all-zero direction is rejected (mini_trainer guide: initial zero
 * directions are rejected). */
int orc_wn_init(const int8_t *q, const float *s, int64_t N, int64_t K, float *g, float *sw)
{
    if (N < 0 || K < 1)
        return ORC_EINVAL;
    for (int64_t n = 0; n < N; n++)
        if (code_norm(q + n * K, K) == 0.0f)
            return ORC_EINVAL;
    for (int64_t n = 0; n < N; n++) {
        const float nrm = code_norm(q + n * K, K);
        g[n] = s[n] * nrm;
        sw[n] = g[n] / nrm;
    }
    return ORC_OK;
}

/* The float gradients of every row (dg [N], dv [N, K]), without an update. */
int orc_wn_grads(const int8_t *q, const float *s, const float *g, const float *dw, int64_t N,
                 int64_t K, float *dg, float *dv)
{
    if (N < 0 || K < 1)
        return ORC_EINVAL;
#pragma omp parallel
    {
        double *tmp = (double *)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; n++)
            wn_row_grads(q + n * K, s[n], g[n], dw + n * K, K, tmp, dg + n, dv + n * K);
        free(tmp);
    }
    return ORC_OK;
}

/* One SGD step of a weight-normalized layer, in place on q [N, K], s, g and
 * sw [N]: g' = fl(g - fl(lr dg)); the direction w = fl(fl(s q) - fl(lr dv))
 * is requantized exactly as in SGD (new absmax scale, Philox stochastic
 * rounding keyed by the element index); sw' = fl(g' / ||q'||), or 0 when the
 * new codes are all zero.  bias -= lr * db when both are given. */
int orc_wn_sgd_requant(int8_t *q, float *s, float *g, float *sw, const float *dw, int64_t N,
                       int64_t K, float lr, uint64_t seed, uint64_t step, float *bias,
                       const float *db, const int64_t *row_ids)
{
    if (N < 0 || K < 1)
        return ORC_EINVAL;
#pragma omp parallel
    {
        double *tmp = (double *)malloc((size_t)K * sizeof(double));
        float *dv = (float *)malloc((size_t)K * sizeof(float));
        float *w = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; n++) {
            int8_t *qn = q + n * K;
            float dg;
            wn_row_grads(qn, s[n], g[n], dw + n * K, K, tmp, &dg, dv);
            for (int64_t k = 0; k < K; k++) {
                float cur = s[n] * (float)qn[k];
                float upd = lr * dv[k];
                w[k] = cur - upd;
            }
            g[n] = g[n] - lr * dg;
            s[n] = requant_row(w, K, row_ids ? row_ids[n] : n, seed, step, qn);
            const float nrm = code_norm(qn, K);
            sw[n] = nrm == 0.0f ? 0.0f : g[n] / nrm;
        }
        free(tmp);
        free(dv);
        free(w);
    }
    if (bias && db)
        for (int64_t n = 0; n < N; n++)
            bias[n] = bias[n] - lr * db[n];
    return ORC_OK;
}

/* ------------------------------------- AdamW with stochastic requantization */

/* Step-dependent constants of AdamW, each computed in double from the fp32
 * hyperparameters and rounded once to fp32 (t >= 1):
 * k[0] = a1 = 1 - b1, k[1] = a2 = 1 - b2, k[2] = c1 = lr / (1 - b1^t),
 * k[3] = c2 = 1 / sqrt(1 - b2^t), k[4] = decay = 1 - lr * wd. */
void orc_adamw_constants(float lr, float b1, float b2, float wd, uint64_t t, float k[5])
{
    double db1 = b1, db2 = b2, dt = (double)t;
    k[0] = (float)(1.0 - db1);
    k[1] = (float)(1.0 - db2);
    k[2] = (float)((double)lr / (1.0 - pow(db1, dt)));
    k[3] = (float)(1.0 / sqrt(1.0 - pow(db2, dt)));
    k[4] = (float)(1.0 - (double)lr * (double)wd);
}

/* One AdamW update of n float parameters p (in place), with moments m, v (in
 * place) and gradient g, in the order given in the header. */
static void adamw_elems(float *p, float *m, float *v, const float *g, int64_t n, float b1,
                        float b2, float eps, const float k[5])
{
    for (int64_t j = 0; j < n; j++) {
        float mj = b1 * m[j] + k[0] * g[j];
        float vj = b2 * v[j] + (k[1] * g[j]) * g[j];
        float d = sqrtf(vj) * k[3] + eps;
        p[j] = p[j] * k[4] - k[2] * (mj / d);
        m[j] = mj;
        v[j] = vj;
    }
}

/* The float update alone on the represented weight w = fl(s * q): writes the
 * updated w [N, K] and moments (test hook for pinning against a reference
 * AdamW on the same starting point). */
int orc_adamw_update(const int8_t *qw, const float *sw, const float *dw, float *m, float *v,
                     int64_t N, int64_t K, float lr, float b1, float b2, float eps, float wd,
                     uint64_t t, float *w)
{
    if (N < 0 || K < 1 || t < 1)
        return ORC_EINVAL;
    float k[5];
    orc_adamw_constants(lr, b1, b2, wd, t, k);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t j = 0; j < K; j++)
            w[n * K + j] = sw[n] * (float)qw[n * K + j];
        adamw_elems(w + n * K, m + n * K, v + n * K, dw + n * K, K, b1, b2, eps, k);
    }
    return ORC_OK;
}

/* AdamW step on the represented weight, then the stochastic requant of each
 * row (Philox step = t).  In place on qw, sw, m, v; the float bias, when
 * given with db and its moments bm, bv, takes the same float update. */
int orc_adamw_requant(int8_t *qw, float *sw, const float *dw, float *m, float *v, int64_t N,
                      int64_t K, float lr, float b1, float b2, float eps, float wd,
                      uint64_t seed, uint64_t t, float *bias, const float *db, float *bm,
                      float *bv, const int64_t *row_ids)
{
    if (N < 0 || K < 1 || t < 1)
        return ORC_EINVAL;
    float k[5];
    orc_adamw_constants(lr, b1, b2, wd, t, k);
#pragma omp parallel
    {
        float *w = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; n++) {
            for (int64_t j = 0; j < K; j++)
                w[j] = sw[n] * (float)qw[n * K + j];
            adamw_elems(w, m + n * K, v + n * K, dw + n * K, K, b1, b2, eps, k);
            sw[n] = requant_row(w, K, row_ids ? row_ids[n] : n, seed, t, qw + n * K);
        }
        free(w);
    }
    if (bias && db && bm && bv)
        adamw_elems(bias, bm, bv, db, N, b1, b2, eps, k);
    return ORC_OK;
}

/* ------------------------------------------- contractions above 131,071 */

/* The guide's rule for contractions above 131,071: bounded int32 partial dot
 * products (each over at most 131,071 terms, so exact) are combined in int64
 * before scaling.  Integer addition is exact and associative, so the result
 * is the exact dot product whatever the chunking; it is converted to fp32
 * once (round to nearest even) and then dequantized as usual.  These entry
 * points take any contraction length. */
int orc_gemm_s64_at(int op, const int8_t *a, const int8_t *b, int64_t M, int64_t N,
                    int64_t K, const int64_t *ii, const int64_t *jj, int64_t count,
                    int64_t *out)
{
    if (op < 0 || op > 2 || M < 0 || N < 1 || K < 1)
        return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; t++)
        out[t] = dot_op(op, a, b, M, N, K, ii[t], jj[t]);
    return ORC_OK;
}

int orc_op_at_long(int op, const int8_t *a, const float *srow, const int8_t *b,
                   const float *scol, const float *bias, int64_t M, int64_t N, int64_t K,
                   const int64_t *ii, const int64_t *jj, int64_t count, float *out)
{
    if (op < 0 || op > 2 || M < 0 || N < 1 || K < 1)
        return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; t++)
        out[t] = dequant_f(op, (float)dot_op(op, a, b, M, N, K, ii[t], jj[t]), srow, scol,
                           bias, ii[t], jj[t]);
    return ORC_OK;
}
