// Host-side launchers of the qlin kernels.  Arguments are validated by the
// C-ABI layer (api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlin {

void launch_quantize_rows(const void *x, bool bf16, int64_t rows, int64_t cols,
                          const float *prescale, int had, float cb, int8_t *q, float *s,
                          hipStream_t st);

void launch_quantize_cols(const void *x, bool bf16, int64_t rows, int64_t cols,
                          const float *prescale, int8_t *q, float *s, float *col_sum,
                          hipStream_t st);

// Both quantizations of the output gradient: rows of x * sw -> (q1, s1),
// columns of x * sx -> (q2, s2) and the column sums of x.  q2 serves as
// scratch for the row and column partials before its codes are written.
void launch_quantize_grad(const void *x, bool bf16, int64_t rows, int64_t cols, const float *sw,
                          const float *sx, int8_t *q1, float *s1, int8_t *q2, float *s2,
                          float *col_sum, hipStream_t st);

void launch_dequantize_weight(const int8_t *q, const float *sw, int64_t rows, int64_t cols,
                              int blk, float cb, float *w, hipStream_t st);

void launch_hadamard(const void *x, bool bf16, int64_t rows, int64_t cols, int blk, float cb,
                     float *y, hipStream_t st);

// Products.  op: 0 forward, 1 dX, 2 dW.  epi: 0 raw int32, 1 dequant.
struct ProductArgs {
    int op;
    const int8_t *a;
    const int8_t *b;
    int64_t M, N, K;
    const float *srow;  // sx, sg1 or sg2
    const float *scol;  // sw (forward only)
    const float *bias;  // forward only, may be null
    void *out;          // float* or int32_t*
    bool raw;           // int32 accumulators instead of dequantized floats
    int had = 0;        // dX only: rotate each output row in blocks of 'had' (<= 128)
    float had_scale = 1.0f;
    int64_t t_len = 0;        // contraction length of this launch (0: the full one)
    int64_t *ws = nullptr;    // int64 running sums of a split contraction
    int ws_mode = 0;          // 0 none, 1 store, 2 add, 3 finish from acc + ws
    // Workspace for balancing the last round of tiles (split_plan): arrival
    // counters in its first kSplitCountBytes (zero on entry, zero on exit),
    // then the pieces' int32 partial sums.  Null: no balancing.
    void *split_ws = nullptr;
};

void launch_product(const ProductArgs &p, hipStream_t st);

// Whether the product kernels can address every operand byte of this shape
// with their 32-bit buffer offsets (for contractions past the int32 bound,
// those of one chunk's launch).
bool product_addressable(int op, int64_t M, int64_t N, int64_t K);

// How a product balances its last round of 256 x 256 tiles over the chip:
// 'full' whole tiles, then each of the 'tail' remaining tiles in 'split'
// pieces along the contraction (split 1: no balancing).
struct SplitPlan {
    int full, tail, split;
};
constexpr size_t kSplitCountBytes = 4096;
SplitPlan split_plan(int op, int64_t M, int64_t N, int64_t K);
// Workspace bytes the plan needs (0 when it splits nothing).
size_t split_ws_bytes(const SplitPlan &sp);
// Zero n 32-bit words at p on the stream (a kernel, so graph capture holds
// no memset node).
void launch_zero_words(void *p, int n, hipStream_t st);

// A product whose contraction exceeds the int32 bound, in chunks combined in
// the int64 workspace ws [rows, cols] (8 bytes per output).
void launch_product_long(const ProductArgs &p, int64_t *ws, hipStream_t st);

// Streaming device copy of nbytes (a multiple of 16) between 16-byte aligned
// buffers: the reference for the memory-bound kernels' bandwidth.
void launch_stream_copy(const void *src, void *dst, int64_t nbytes, hipStream_t st);

// Matrix-core ceiling: `workgroups` workgroups of 8 waves repeat the
// products' MFMA sequence `iters` times on kMfmaCeilingFrags fragments of
// 1 KiB from frags; out gets each lane's sum of its 32 accumulator blocks
// (workgroups x 512 x 4 int32).
constexpr int kMfmaCeilingFrags = 24;
void launch_mfma_ceiling(const int8_t *frags, int32_t *out, int workgroups, int iters,
                         hipStream_t st);

void launch_sgd_requant(int8_t *qw, float *sw, const float *dw, int64_t N, int64_t K, float lr,
                        uint64_t seed, uint64_t step, float *bias, const float *db,
                        hipStream_t st);

// AdamW hyperparameters and the step constants derived from them on the host.
struct AdamConsts {
    float b1, b2, eps, a1, a2, c1, c2, decay;
};

// Row weight normalization: preparation and the SGD step (sgd.hip).
void launch_wn_init(const int8_t *q, const float *s, int64_t N, int64_t K, float *g, float *sw,
                    hipStream_t st);
void launch_wn_sgd_requant(int8_t *q, float *s, float *g, float *sw, const float *dw, int64_t N,
                           int64_t K, float lr, uint64_t seed, uint64_t step, float *bias,
                           const float *db, hipStream_t st);
void launch_adamw_requant(int8_t *qw, float *sw, const float *dw, float *m, float *v, int64_t N,
                          int64_t K, const AdamConsts &k, uint64_t seed, uint64_t step,
                          float *bias, const float *db, float *bm, float *bv, hipStream_t st);

} // namespace qlin
