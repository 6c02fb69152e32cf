/*
 * qlin: INT8 W8A8 linear layer for quantized training on AMD MI355X (gfx950).
 *
 * The layer stores each weight matrix as INT8 codes with one float magnitude
 * per output row and keeps no float master weight; it quantizes activations
 * per row on every call, optionally after a block-Hadamard rotation along the
 * contraction dimension; it runs the forward product and both backward
 * products as int8 x int8 -> int32 matrix products on the saved INT8 input;
 * and it updates the weight with an SGD step that stochastically requantizes
 * each row.  Sources: the mini_trainer "quantized-training" guide (feature
 * table; update paragraph; arithmetic paragraph on contractions above
 * 131,071) and OneTrainer PR #1681 "Int8 conv rot" (summary; commit notes 1
 * and 2).
 *
 * Conventions for every entry point:
 *  - All array pointers are device memory owned by the caller, row-major and
 *    contiguous, 16-byte aligned.  A pointer to an array with no element
 *    (for example any [M, *] array when M == 0) may be NULL.  The library
 *    allocates nothing and keeps no mutable global state, except the
 *    scratch array of qlin_product_noalloc (one per device, held until the
 *    process ends) and its looked-up address; calls on different streams are
 *    independent unless they share a qlin_product_ws workspace or are
 *    qlin_product_noalloc calls on the same device.
 *  - 'stream' is a hipStream_t (NULL means the null stream).  Every call only
 *    enqueues kernels on that stream and returns without synchronizing.
 *  - Arguments are validated before anything is launched: on any error the
 *    call returns a nonzero status and no output is touched.  Faults inside
 *    kernels surface at the caller's next synchronization.
 *  - Shapes: M (tokens) >= 0 is arbitrary; M == 0 is a no-op (except that
 *    qlin_bwd_dw then writes an all-zero dW).  N (out
 *    features) and K (in features) are multiples of 16.  The products take
 *    M, N and K up to 2^30 and outputs of fewer than 2^31 tiles of 256 x 256
 *    (QLIN_EUNSUPPORTED otherwise).  A contraction longer
 *    than QLIN_MAX_CONTRACTION is rejected with QLIN_EUNSUPPORTED, except by
 *    qlin_product_ws, which combines int32 chunks in int64.
 *  - Operand reach: the product kernels address each int8 operand with 32-bit
 *    byte offsets from a base that moves with the tile and the contraction,
 *    and must reach no further than 2,147,483,632 bytes from it.  The product
 *    calls (qlin_fwd, qlin_bwd_dx, qlin_bwd_dw, qlin_product_ws and
 *    qlin_gemm_s32) return QLIN_EUNSUPPORTED, before launching anything, for
 *    the shapes whose offsets could go past that, by these bounds:
 *      an operand strided along the contraction (dX: qw, whose rows hold K
 *      bytes; dW: qg2 and qx, rows of N and K bytes) needs
 *      (min(T, 128) - 1) * row_bytes + 256 <= 2,147,483,632, with T the
 *      contraction: row_bytes <= 16,909,312 once T >= 128;
 *      an operand contiguous along the contraction (forward: qx and qw, dX:
 *      qg1) needs (min(rows, 256) - 1) * T + t <= 2,147,483,632, with t = T
 *      within the int32 bound and t = 130,944 (one chunk) beyond it: only
 *      qlin_product_ws's long forward and dX contractions reach this, at
 *      T > 8,420,976 when the operand has 256 rows or more.
 *  - Arithmetic: IEEE binary32, round to nearest even, no fused multiply-add,
 *    IEEE division.  Results are deterministic and do not depend on the
 *    launch configuration, except col_sum of qlin_quantize_cols (fp32 sums
 *    combined in arbitrary order).
 */
#ifndef QLIN_H
#define QLIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define QLIN_OK 0
#define QLIN_EINVAL 1       /* null pointer, bad shape, misalignment, bad block/dtype */
#define QLIN_EUNSUPPORTED 2 /* contraction or row too long for this library */
#define QLIN_EDEVICE 3      /* the HIP runtime reported an error at launch */

/* Element types of floating inputs. */
#define QLIN_F32 0
#define QLIN_BF16 1

/* Products, for qlin_gemm_s32. */
#define QLIN_OP_FWD 0 /* acc[M,N] = qx[M,K]  . qw[N,K]^T */
#define QLIN_OP_DX 1  /* acc[M,K] = qg1[M,N] . qw[N,K]   */
#define QLIN_OP_DW 2  /* acc[N,K] = qg2[M,N]^T . qx[M,K] */

/* Longest contraction for which an int32 sum of int8 x int8 products cannot
 * overflow: 131071 * 128 * 128 < 2^31 (mini_trainer guide, arithmetic
 * paragraph).  The plain product calls reject longer ones; qlin_product_ws
 * takes them, adding exact int32 chunk sums in int64. */
#define QLIN_MAX_CONTRACTION 131071
/* Largest Hadamard block and longest row the row kernels accept. */
#define QLIN_MAX_HAD_BLOCK 512
#define QLIN_MAX_ROW 131072

/* Human-readable name of a status code (static storage). */
const char *qlin_status_string(int status);

/* Version of the C ABI declared here. */
int qlin_abi_version(void);

/*
 * Per-row dynamic INT8 quantization, optionally after a block-Hadamard
 * rotation (OneTrainer PR #1681: the activations are rotated along the
 * contraction dimension and quantized per row on every call; mini_trainer
 * guide: INT8 direction with a float magnitude per output row).
 *
 *   x         [rows, cols] fp32 or bf16 (dtype QLIN_F32 / QLIN_BF16), input.
 *   prescale  [cols] fp32 or NULL: multiplies each rotated element by the
 *             scale of its column (used to fold the weight row scales into
 *             dY before quantizing it for dX).
 *   had_block 0 (no rotation) or a power of two in [2, 512] dividing cols:
 *             each run of had_block elements is replaced by its normalized
 *             Walsh-Hadamard transform (Sylvester order, scaled by
 *             fl32(1/sqrt(had_block)), butterfly stages in ascending stride).
 *   q         [rows, cols] int8 output, s [rows] fp32 output:
 *             g = rotate(x) * prescale, a = max |g|, s = fl(a / 127) and
 *             q = rne(fl(g / s)) in [-127, 127]; a row with a == 0 gets
 *             s = 0 and q = 0.
 * rows >= 0; cols in [16, QLIN_MAX_ROW], a multiple of 16.
 */
int qlin_quantize_rows(const void *x, int dtype, int64_t rows, int64_t cols,
                       const float *prescale, int had_block, int8_t *q, float *s,
                       void *stream);

/*
 * Per-column dynamic INT8 quantization of x * prescale[:, None], the operand
 * of the weight-gradient product (mini_trainer guide, opening paragraph: the
 * backward matrix products are integer products on INT8 operands, the weight
 * gradient's on the saved INT8 input).  Scales sit on the output axis of that
 * product, never on its contraction (token) axis, so they factor out of the
 * token sum exactly.  q keeps the [rows, cols] layout of x.
 *
 *   x         [rows, cols] fp32 or bf16 input (dY, rows = tokens).
 *   prescale  [rows] fp32 or NULL (the activation row scales s_x).
 *   q         [rows, cols] int8 output; s [cols] fp32 output, defined as in
 *             qlin_quantize_rows but per column.
 *   col_sum   [cols] fp32 or NULL: sum over rows of the raw x (the bias
 *             gradient), accumulated in fp32 in an unspecified order.
 * rows >= 0; cols >= 16, a multiple of 16.  s (and col_sum) are also used as
 * accumulators during the call and must not alias x, prescale or q.
 */
int qlin_quantize_cols(const void *x, int dtype, int64_t rows, int64_t cols,
                       const float *prescale, int8_t *q, float *s, float *col_sum,
                       void *stream);

/*
 * Both quantizations of the output gradient dY in one call, reading dY twice
 * instead of three times: a first pass gathers the row maxima of the first,
 * the column maxima and sums of the second, a second pass writes both code
 * arrays (mini_trainer guide: the backward products are integer; the scales
 * of each operand sit on its product's output axis).
 * Results are those of
 *   qlin_quantize_rows(dy, prescale = sw, had_block = 0) -> (q1, s1)   and
 *   qlin_quantize_cols(dy, prescale = sx, col_sum)        -> (q2, s2, col_sum)
 * bit for bit, except col_sum (fp32 sums in an unspecified order; from 16
 * rows on it is fixed for a given shape, so repeated calls agree bit for bit).
 *
 *   dy       [rows, cols] fp32 or bf16 (rows = tokens, cols = out features).
 *   sw       [cols] fp32, the weight row scales (required).
 *   sx       [rows] fp32, the activation row scales (required when rows > 0).
 *   q1, s1   [rows, cols] int8 and [rows] fp32 outputs (operand of dX).
 *   q2, s2   [rows, cols] int8 and [cols] fp32 outputs (operand of dW).  q2
 *            also serves as scratch during the call, so it must not overlap
 *            any other argument.
 *   col_sum  [cols] fp32 or NULL (the bias gradient).
 * rows >= 0 (rows == 0 writes s2 = 0 and col_sum = 0); cols in
 * [16, QLIN_MAX_ROW], a multiple of 16; rows <= 1,048,560.
 */
int qlin_quantize_grad(const void *dy, int dtype, int64_t rows, int64_t cols, const float *sw,
                       const float *sx, int8_t *q1, float *s1, int8_t *q2, float *s2,
                       float *col_sum, void *stream);

/*
 * Block-Hadamard rotation of each row (the same transform as in
 * qlin_quantize_rows).  The transform is symmetric and orthogonal, so the
 * same call maps the rotated basis back (OneTrainer PR #1681: the weight
 * stays in the rotated basis, (xR)(WR)^T = xW^T).
 *   x [rows, cols] fp32 or bf16; y [rows, cols] fp32, may equal x when
 *   dtype is QLIN_F32 (in place), must not otherwise overlap it.
 *   block: power of two in [2, 512] dividing cols; cols a multiple of 16.
 */
int qlin_hadamard(const void *x, int dtype, int64_t rows, int64_t cols, int block,
                  float *y, void *stream);

/*
 * The represented weight in the original basis, for callers that need the
 * unquantized weight (OneTrainer PR #1681, commit note 2: LoRA, DoRA, offload
 * and export un-rotate the weight; the rotation is its own inverse):
 *   w[n, k] = fl(sw[n] * qw[n, k]), then, when had_block != 0, the rotation of
 *   each block of had_block elements (as in qlin_hadamard).
 *   qw [N, K] int8, sw [N] fp32 inputs; w [N, K] fp32 output, not overlapping
 *   them.  had_block: 0 or a power of two in [2, 512] dividing K; K a multiple
 *   of 16.
 */
int qlin_dequantize_weight(const int8_t *qw, const float *sw, int64_t N, int64_t K,
                           int had_block, float *w, void *stream);

/*
 * Forward product with fused dequant (mini_trainer guide: integer forward
 * product on INT8 weights; OneTrainer PR #1681: int8 x int8 -> int32
 * product of quantized activations and weights).
 *   qx [M,K] int8, sx [M]; qw [N,K] int8, sw [N]; bias [N] or NULL.
 *   y [M,N] fp32: y = fl(fl(fl32(acc) * sx[m]) * sw[n]) (+ bias[n]) with
 *   acc = sum_k qx[m,k] * qw[n,k] exact in int32.
 * K <= QLIN_MAX_CONTRACTION.  M <= 16 takes a weight-streaming path.
 */
int qlin_fwd(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
             const float *bias, int64_t M, int64_t N, int64_t K, float *y, void *stream);

/*
 * Input-gradient product (straight-through estimator across the activation
 * quantizer), optionally rotated back to the original basis.
 *   qg1 [M,N] int8, sg1 [M]: dY * sw[None, :] quantized per row
 *   (qlin_quantize_rows with prescale = sw); qw [N,K] int8 (rotated basis).
 *   dx [M,K] fp32: dx_r = fl(fl32(acc) * sg1[m]), acc = sum_n qg1[m,n] * qw[n,k];
 *   had_block = 0 stores dx_r; otherwise (a power of two in [2, 512]
 *   dividing K) each row of dx_r is rotated in blocks of had_block exactly
 *   as qlin_hadamard would (the rotation is its own inverse, OneTrainer PR
 *   #1681 commit note 2), fused into the product's epilogue for blocks up to
 *   128 and as a second kernel for larger blocks.
 * N <= QLIN_MAX_CONTRACTION.
 */
int qlin_bwd_dx(const int8_t *qg1, const float *sg1, const int8_t *qw, int64_t M,
                int64_t N, int64_t K, int had_block, float *dx, void *stream);

/*
 * Weight-gradient product on the saved INT8 input (mini_trainer guide:
 * saved Linear inputs are stored in INT8 for the backward pass).
 *   qg2 [M,N] int8, sg2 [N]: dY * sx[:, None] quantized per column
 *   (qlin_quantize_cols with prescale = sx); qx [M,K] int8 from the forward.
 *   dw [N,K] fp32: dw = fl(fl32(acc) * sg2[n]), acc = sum_m qg2[m,n] * qx[m,k].
 * M <= QLIN_MAX_CONTRACTION.
 */
int qlin_bwd_dw(const int8_t *qg2, const float *sg2, const int8_t *qx, int64_t M,
                int64_t N, int64_t K, float *dw, void *stream);

/*
 * Any of the three products with a caller workspace: the same results, bit
 * for bit, as qlin_fwd / qlin_bwd_dx / qlin_bwd_dw, for a contraction of any
 * length up to 2^31 - 1.
 *  - Beyond QLIN_MAX_CONTRACTION (mini_trainer guide, arithmetic paragraph,
 *    on contractions too long for an exact int32 sum) the contraction runs
 *    in chunks of at most 130,944 terms, each summed exactly in int32; the
 *    workspace adds the chunk sums in int64, and the int64 total, converted
 *    once to fp32, goes through the product's usual epilogue.
 *  - Within the bound the workspace balances the grid: the 256 x 256 output
 *    tiles left over after the last whole round of the chip's 256 compute
 *    units are each computed in two or three pieces along the contraction,
 *    whose int32 partial sums (exact) are added by the last piece to finish
 *    before the usual epilogue.  When a shape leaves nothing to balance,
 *    qlin_product_ws_bytes is 0 and the workspace is not touched.
 *
 *   op        QLIN_OP_FWD: a = qx [M,K], srow = sx, b = qw [N,K], scol = sw,
 *                          bias optional, out = y [M,N], had_block = 0;
 *             QLIN_OP_DX:  a = qg1 [M,N], srow = sg1, b = qw [N,K],
 *                          out = dx [M,K], had_block as in qlin_bwd_dx;
 *             QLIN_OP_DW:  a = qg2 [M,N], srow = sg2, b = qx [M,K],
 *                          out = dw [N,K], had_block = 0.
 *             scol and bias must be NULL except for the forward product.
 *   workspace device memory of at least qlin_product_ws_bytes(op, M, N, K)
 *             bytes, 16-byte aligned, overlapping no other argument (NULL
 *             when that size is 0).  Its first 4096 bytes hold arrival
 *             counters: they must be zero before the workspace's first use
 *             (allocate it zero-filled), and every completed call leaves them
 *             zero again.  The rest is scratch.  Calls that share a workspace
 *             must not run concurrently.
 */
int qlin_product_ws(int op, const int8_t *a, const float *srow, const int8_t *b,
                    const float *scol, const float *bias, int64_t M, int64_t N, int64_t K,
                    int had_block, float *out, void *workspace, size_t ws_bytes,
                    void *stream);

/*
 * qlin_product_ws for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same products, bit for bit, with the workspace taken from a scratch
 * array of QLIN_NOALLOC_SCRATCH_BYTES that the library holds in device
 * memory, one per device, for the life of the process.  Arguments are those
 * of qlin_product_ws without the workspace.  The call allocates nothing (no
 * hipMalloc, no allocating library routine) and uses the scratch of the
 * current device; 'stream' must belong to that device.
 *  - Within QLIN_MAX_CONTRACTION the scratch balances the last round of
 *    tiles when the shape's qlin_product_ws_bytes fits in it, after a small
 *    kernel zeroes the arrival counters it uses; when nothing is balanced or
 *    the pieces do not fit, the ordinary product runs (the same results).
 *  - Beyond QLIN_MAX_CONTRACTION the int64 sums (8 bytes per output, plus
 *    4096) must fit: larger shapes return QLIN_EUNSUPPORTED before anything
 *    is launched.
 * Every call on a device shares that device's scratch and leaves its last
 * contents there: calls that overlap in time on one device (on different
 * streams, or from different host threads) race and give wrong results.
 * The first call on each device looks up the scratch's address
 * (QLIN_EDEVICE if the runtime cannot).
 */
#define QLIN_NOALLOC_SCRATCH_BYTES (4096 + 160 * 262144)
int qlin_product_noalloc(int op, const int8_t *a, const float *srow, const int8_t *b,
                         const float *scol, const float *bias, int64_t M, int64_t N, int64_t K,
                         int had_block, float *out, void *stream);

/* Workspace bytes qlin_product_ws needs for this shape: beyond the int32
 * bound 4096 + 8 per output element; within it 4096 + 256 KiB per balancing
 * piece (at most 256 pieces), or 0 when nothing is balanced.  Returns 0 for
 * invalid arguments and for shapes the products do not support (M, N or K
 * above 2^30). */
size_t qlin_product_ws_bytes(int op, int64_t M, int64_t N, int64_t K);

/*
 * SGD step with stochastic requantization of each weight row, in place
 * (mini_trainer guide: updates stochastically requantize the represented
 * weight and no float master weight is retained; OneTrainer PR #1681: the
 * quantized weight is updated in its existing storage).
 *   qw [N,K] int8 and sw [N] fp32, read and overwritten.
 *   dw [N,K] fp32 weight gradient.
 *   Per row n: w = fl(fl(sw[n] * q) - fl(lr * dw)); s' = fl(max|w| / 127)
 *   (0 for an all-zero row); y = fl(w / s'); q' = floor(y) + (u < y -
 *   floor(y)) clamped to [-127, 127], where u = r * 2^-16 and r is the 16-bit
 *   half (i & 1) of word (i & 7) >> 1 of Philox4x32-10 (Salmon et al., SC'11)
 *   at counter (lo(i>>3), hi(i>>3), lo(step), hi(step)) and key (lo(seed),
 *   hi(seed)), i = n*K + k.  The result depends only on (inputs, lr, seed,
 *   step), so a run resumed at the same step reproduces it exactly.
 *   bias [N] and db [N] (both or neither): bias = fl(bias - fl(lr * db)).
 * K in [16, QLIN_MAX_ROW], a multiple of 16.
 */
int qlin_sgd_requant(int8_t *qw, float *sw, const float *dw, int64_t N, int64_t K,
                     float lr, uint64_t seed, uint64_t step, float *bias, const float *db,
                     void *stream);

/*
 * Row weight normalization (mini_trainer guide, feature table: an INT8
 * direction and a floating magnitude per output row; initial zero directions
 * are rejected).  A weight-normalized layer keeps per output row n the
 * direction codes q[n, :] with their scale s[n] (the direction v = s q, the
 * same storage as the absmax weight) and a magnitude g[n] trained as its own
 * parameter.  The represented weight is g q / ||q||, so the products take
 * qw = q with the column scale sw = fl(g / ||q||).  ||q|| = fl32(sqrt(sum
 * q^2)): the integer sum exact, the square root in double, rounded once.
 *
 * qlin_wn_init: g = fl(s ||q||) and sw = fl(g / ||q||), so the represented
 * weight starts as the absmax weight s q (within the rounding of sw).  An
 * all-zero row gives g = sw = 0: callers reject it (a zero direction).
 *   q [N, K] int8, s [N] fp32 inputs; g, sw [N] fp32 outputs.
 *   N >= 0; K in [16, QLIN_WN_MAX_ROW], a multiple of 16.
 */
#define QLIN_WN_MAX_ROW 32768
int qlin_wn_init(const int8_t *q, const float *s, int64_t N, int64_t K, float *g, float *sw,
                 void *stream);

/*
 * SGD step of a weight-normalized layer, in place, with dw the gradient of
 * the represented weight (the dW product's output).  Per row:
 *   dot = fl32(pairwise double sum of dw_k q_k)   (the products are exact;
 *         pairwise: the row zero-padded to a power of two, adjacent pairs
 *         added level by level)
 *   dg  = fl(dot / ||q||)                          (dL/dg)
 *   dv_k = fl(fl(g / fl(s ||q||)) * fl(dw_k - fl(fl(dg / ||q||) * q_k)))
 *                                                  (dL/dv, v = s q)
 *   w_k = fl(fl(s q_k) - fl(lr dv_k)), requantized exactly as by
 *         qlin_sgd_requant (new absmax scale s', Philox stochastic rounding
 *         keyed by seed, step and the element index)
 *   g'  = fl(g - fl(lr dg)),  sw' = fl(g' / ||q'||) (0 for all-zero codes).
 * A row whose codes are all zero has zero gradients.
 *   q [N, K] int8, s, g, sw [N] fp32: read and overwritten (sw is only
 *   written).  dw [N, K] fp32.  bias, db [N] (both or neither): bias =
 *   fl(bias - fl(lr db)).
 *   N >= 0; K in [16, QLIN_WN_MAX_ROW], a multiple of 16; lr finite.
 */
int qlin_wn_sgd_requant(int8_t *q, float *s, float *g, float *sw, const float *dw, int64_t N,
                        int64_t K, float lr, uint64_t seed, uint64_t step, float *bias,
                        const float *db, void *stream);

/*
 * AdamW step on the represented weight followed by the same stochastic
 * requantization of each row (mini_trainer guide, feature table: AdamW is
 * among the update paths covered on INT8 weights; update paragraph: updates
 * stochastically requantize the represented weight, no float master weight).
 * The guide gives no arithmetic; this is the published decoupled-weight-decay
 * algorithm with bias-corrected moments, in fp32:
 *   m' = fl(fl(b1*m) + fl(a1*g)),  v' = fl(fl(b2*v) + fl(fl(a2*g)*g)),
 *   d  = fl(fl(sqrt(v')*c2) + eps),
 *   w  = fl(fl(fl(s*q)*decay) - fl(c1*fl(m'/d)))
 * with constants computed in double from the fp32 arguments and rounded once:
 * a1 = 1-b1, a2 = 1-b2, c1 = lr/(1-b1^t), c2 = 1/sqrt(1-b2^t),
 * decay = 1-lr*weight_decay (t = step).  The row is then requantized exactly
 * as by qlin_sgd_requant with Philox step = step.
 *
 *   qw, sw   in/out as in qlin_sgd_requant; dw [N, K] fp32 gradient.
 *   m, v     [N, K] fp32 moments, in/out (zero before the first step); they
 *            must not overlap each other or dw.
 *   step     t >= 1, the AdamW step count and the Philox step.
 *   beta1, beta2 in [0, 1); eps > 0; weight_decay >= 0; all finite.
 *   bias, db, bias_m, bias_v: all four or none; the float bias [N] takes the
 *            same float update with its own moments [N].
 * N >= 0; K a multiple of 16, at most QLIN_MAX_ROW.
 */
int qlin_adamw_requant(int8_t *qw, float *sw, const float *dw, float *m, float *v, int64_t N,
                       int64_t K, float lr, float beta1, float beta2, float eps,
                       float weight_decay, uint64_t seed, uint64_t step, float *bias,
                       const float *db, float *bias_m, float *bias_v, void *stream);

/*
 * Raw int32 accumulators of one of the three products (same kernels as the
 * fused calls, no dequant), for exact verification of the integer forward
 * and backward products (mini_trainer guide, opening paragraph; OneTrainer
 * PR #1681, commit note 1: an int8 x int8 -> int32 product).  op is QLIN_OP_FWD,
 * QLIN_OP_DX or QLIN_OP_DW; a, b and the shape arguments mean what they mean
 * in qlin_fwd / qlin_bwd_dx / qlin_bwd_dw; c is [M,N], [M,K] or [N,K].
 */
int qlin_gemm_s32(int op, const int8_t *a, const int8_t *b, int64_t M, int64_t N,
                  int64_t K, int32_t *c, void *stream);

/*
 * Device-to-device copy of nbytes by a plain streaming kernel (16-byte loads
 * and stores, coalesced, every lane's loads issued before its stores).  It
 * computes nothing of the layer: it is the measured read+write bandwidth of
 * the device, the practical ceiling against which the memory-bound calls
 * (quantize, rotate, requant: HBM-bound steps of the path) are reported
 * beside the nameplate HBM bandwidth.
 *   src, dst  device buffers of nbytes, 16-byte aligned, not overlapping.
 *   nbytes    >= 0, a multiple of 16.
 */
int qlin_stream_copy(const void *src, void *dst, int64_t nbytes, void *stream);

/*
 * Matrix-core ceiling: the products' register tile and MFMA sequence with no
 * memory traffic.  Each of `workgroups` workgroups runs 8 waves; each wave
 * reads 24 fragments of 1 KiB (two 64-byte contraction steps of 8 row blocks
 * and 4 column blocks, lane l's 16 bytes at 16 l of a fragment, wave w
 * starting at fragment w) once from frags and then repeats, `iters` times,
 * the products' sequence of 64 v_mfma_i32_16x16x64_i8 (each block's two
 * steps back to back) into 8 x 4 blocks of 16 x 16 int32 sums.  It computes nothing of the layer: its rate
 * on random fragments, with one workgroup per compute unit, is the int8
 * matrix throughput the device sustains within its power limit, the practical
 * ceiling against which the products are reported beside the nameplate peak.
 *   frags       device buffer of QLIN_MFMA_CEILING_FRAG_BYTES int8 values,
 *               16-byte aligned.
 *   out         device buffer of workgroups * 512 * 4 int32, 16-byte aligned:
 *               lane t of workgroup g writes, at out[4 (512 g + t) + e], the
 *               sum over its 32 blocks of register e (int32, wrapping).
 *   workgroups  in [1, 65535]; iters in [1, 1048576].
 */
#define QLIN_MFMA_CEILING_FRAG_BYTES (24 * 1024)
int qlin_mfma_ceiling(const int8_t *frags, int32_t *out, int workgroups, int iters,
                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H */
