// Row and column INT8 quantizers and the block-Hadamard rotation.
//
// Row quantization (OneTrainer PR #1681: activations rotated along the
// contraction dimension and quantized per row on every call): a workgroup
// holds one row at a time in registers (eight consecutive elements per lane)
// and walks rows grid-stride with the next row's loads in flight; rotation is
// done with in-lane and cross-lane (DPP) butterflies, the absmax reduced over
// the workgroup, then codes written as packed bytes.  One HBM read of x and
// one write of q.
//
// Column quantization (the weight-gradient operand; its scales sit on the
// product's output axis): pass 1 reduces |x * prescale[r]| over row slabs and
// merges slabs with an order-free integer atomicMax on the fp32 bits of the
// non-negative maxima; a tiny kernel turns maxima into scales; pass 2
// quantizes elementwise.  Both quantizations of dY in one call read it twice:
// once for the statistics of both (row and column maxima, column sums), once
// for both code arrays.
//
// Also here: the standalone rotation and the weight export (dequantize and
// rotate back).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace qlin {

// ------------------------------------------------------------ row quantizer

// Rotation of one 8-element chunk: HAD is the block size when it is known at
// compile time (16 .. 128; 0: no rotation), -1 for a block size given at run
// time.  With a fixed block the lane processes chunk had_chunk<HAD>(c) in
// place of c.  EXACT keeps the oracle's sign of exact zeros (needed where the
// rotated floats are the output; a quantizer does not need it).
template <int HAD, bool EXACT = false>
__device__ __forceinline__ void rotate8(float v[8], int had, float cb)
{
    if constexpr (HAD > 0)
        fwht8_fixed<HAD, EXACT>(v, cb);
    else if constexpr (HAD < 0)
        fwht8_lanes(v, had, cb);
}

template <int HAD>
__device__ __forceinline__ int64_t lane_chunk(int64_t c)
{
    if constexpr (HAD > 0)
        return had_chunk<HAD>(c);
    else
        return c;
}

// Grid-stride over rows.  Each pass issues the loads of the workgroup's next
// row before working on the current one, so HBM reads overlap the rotation,
// reduction and quantization.  Loads are unconditional (indexes past the row
// end are clamped to its last chunk and the values dropped) so that they all
// issue back to back.  The per-column prescale of the thread's chunks is
// loaded into registers once and reused for every row.
template <bool BF16, int THREADS, int J, int HAD>
__global__ __launch_bounds__(THREADS) void quant_rows_kernel(
    const void *__restrict__ x, int64_t rows, int64_t cols, const float *__restrict__ prescale,
    int had, float cb, int8_t *__restrict__ q, float *__restrict__ s)
{
    // 1024-thread workgroups have 128 registers per lane: no room for the
    // prescale or the next row's data, which they load when they need it.
    constexpr bool kKeepPrescale = THREADS <= 256;
    constexpr bool kPrefetch = THREADS <= 256;
    __shared__ float red[THREADS / kWave];
    const int t = threadIdx.x;
    const int64_t nch = cols / 8;
    // The chunk a lane processes in pass j; the permutation stays inside
    // groups of 16 chunks, all valid or all past the end (cols is a multiple
    // of 128 when HAD is 128, of 16 otherwise), and so does the clamp.
    auto chunk = [&](int j) {
        const int64_t c = lane_chunk<HAD>(t + (int64_t)j * THREADS);
        return c < nch ? c : nch - 1;
    };
    float p[kKeepPrescale ? J : 1][8];
    if (kKeepPrescale && prescale) {
#pragma unroll
        for (int j = 0; j < J; j++)
            load8<false>(prescale, chunk(j) * 8, p[kKeepPrescale ? j : 0]);
    }
    Raw8<BF16> cur[J];
    int64_t row = blockIdx.x;
#pragma unroll
    for (int j = 0; j < J; j++)
        cur[j] = load_raw8<BF16>(x, row * cols + chunk(j) * 8);
    for (; row < rows; row += gridDim.x) {
        const int64_t base = row * cols;
        const int64_t next = row + gridDim.x < rows ? row + gridDim.x : row;
        Raw8<BF16> nxt[kPrefetch ? J : 1];
        if constexpr (kPrefetch) {
#pragma unroll
            for (int j = 0; j < J; j++)
                nxt[j] = load_raw8<BF16>(x, next * cols + chunk(j) * 8);
        }
        float v[J][8];
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < J; j++) {
            const bool ok = t + (int64_t)j * THREADS < nch;
            unpack8<BF16>(cur[j], v[j]);
            // Chunk index c is the same function of the lane in every pass, so
            // lanes of one block stay together; a block is all valid or all
            // clamped because had divides cols.
            rotate8<HAD>(v[j], had, cb);
            if (prescale) {
                float pr[8];
                if constexpr (kKeepPrescale) {
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        pr[e] = p[j][e];
                } else {
                    load8<false>(prescale, chunk(j) * 8, pr);
                }
#pragma unroll
                for (int e = 0; e < 8; e++)
                    v[j][e] = v[j][e] * pr[e];
            }
            if (ok) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    amax = fmaxf(amax, __builtin_fabsf(v[j][e]));
            }
        }
        const float a = block_max<THREADS>(amax, red);
        const float sc = a / 127.0f;
        if (t == 0)
            s[row] = sc;
        const bool zero = (a == 0.0f);
        const bool subnormal = !zero && sc < 0x1p-126f;
        const float inv = recip_refined(sc);     // used only for a normal scale
#pragma unroll
        for (int j = 0; j < J; j++) {
            const int64_t c = lane_chunk<HAD>(t + (int64_t)j * THREADS);
            i32x2 out;
            if (zero) {
                out = i32x2{0, 0};
            } else if (subnormal) {
                float r[8];
#pragma unroll
                for (int e = 0; e < 8; e++)
                    r[e] = quant_code_exact(v[j][e], sc);
                out[0] = (int)pack4(r[0], r[1], r[2], r[3]);
                out[1] = (int)pack4(r[4], r[5], r[6], r[7]);
            } else {
                out = quant8(v[j], sc, inv);
            }
            if (c < nch)
                *reinterpret_cast<i32x2 *>(q + base + c * 8) = out;
        }
#pragma unroll
        for (int j = 0; j < J; j++)
            cur[j] = kPrefetch ? nxt[kPrefetch ? j : 0] : load_raw8<BF16>(x, next * cols + chunk(j) * 8);
    }
}

// Workgroups per launch: enough to fill the GPU several times over; each
// loops over rows.
constexpr int64_t kRowGrid = 4096;

template <bool BF16, int THREADS, int J, int HAD>
static void launch_rows_t(const void *x, int64_t rows, int64_t cols, const float *prescale,
                          int had, float cb, int8_t *q, float *s, hipStream_t st)
{
    const unsigned grid = (unsigned)(rows < kRowGrid ? rows : kRowGrid);
    hipLaunchKernelGGL((quant_rows_kernel<BF16, THREADS, J, HAD>), dim3(grid), dim3(THREADS), 0,
                       st, x, rows, cols, prescale, had, cb, q, s);
}

template <bool BF16, int HAD>
static void launch_rows_h(const void *x, int64_t rows, int64_t cols, const float *prescale,
                          int had, float cb, int8_t *q, float *s, hipStream_t st)
{
    // Registers per lane: 8 * J floats (and as many for the prescale).  256
    // threads cover 2048 elements per pass; rows longer than 16384 switch to
    // 1024 threads.
    const int64_t nch = cols / 8;
    const int64_t j256 = (nch + 255) / 256;
    switch (j256) {
    case 1: return launch_rows_t<BF16, 256, 1, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
    case 2: return launch_rows_t<BF16, 256, 2, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
    case 3: return launch_rows_t<BF16, 256, 3, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
    case 4: return launch_rows_t<BF16, 256, 4, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
    case 5: return launch_rows_t<BF16, 256, 5, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
    case 6: return launch_rows_t<BF16, 256, 6, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
    case 7: return launch_rows_t<BF16, 256, 7, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
    case 8: return launch_rows_t<BF16, 256, 8, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
    default: break;
    }
    const int64_t j1024 = (nch + 1023) / 1024;
    if (j1024 <= 4)
        return launch_rows_t<BF16, 1024, 4, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
    if (j1024 <= 8)
        return launch_rows_t<BF16, 1024, 8, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
    return launch_rows_t<BF16, 1024, 16, HAD>(x, rows, cols, prescale, had, cb, q, s, st);
}

template <bool BF16>
static void launch_rows_dt(const void *x, int64_t rows, int64_t cols, const float *prescale,
                           int had, float cb, int8_t *q, float *s, hipStream_t st)
{
    if (had == 0)
        launch_rows_h<BF16, 0>(x, rows, cols, prescale, had, cb, q, s, st);
    else if (had == 128)
        launch_rows_h<BF16, 128>(x, rows, cols, prescale, had, cb, q, s, st);
    else if (had == 64)
        launch_rows_h<BF16, 64>(x, rows, cols, prescale, had, cb, q, s, st);
    else
        launch_rows_h<BF16, -1>(x, rows, cols, prescale, had, cb, q, s, st);
}

void launch_quantize_rows(const void *x, bool bf16, int64_t rows, int64_t cols,
                          const float *prescale, int had, float cb, int8_t *q, float *s,
                          hipStream_t st)
{
    if (bf16)
        launch_rows_dt<true>(x, rows, cols, prescale, had, cb, q, s, st);
    else
        launch_rows_dt<false>(x, rows, cols, prescale, had, cb, q, s, st);
}

// --------------------------------------------------------- column quantizer

// Zero the per-column accumulators (a fill kernel rather than a memset so the
// sequence stays valid inside captured graphs).
__global__ void zero_cols_kernel(float *__restrict__ s, float *__restrict__ col_sum, int64_t cols)
{
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c < cols) {
        s[c] = 0.0f;
        if (col_sum)
            col_sum[c] = 0.0f;
    }
}

// Pass 1: each workgroup covers 512 columns (64 lanes x 8) and a slab of
// kColSlab rows split over 4 row lanes.  Maxima of |x * p[r]| are merged into
// s[] with atomicMax on the fp32 bit patterns (monotone for values >= 0);
// column sums of the raw x with fp32 atomicAdd.
constexpr int kColSlab = 256;

template <bool BF16>
__global__ __launch_bounds__(256) void colmax_kernel(const void *__restrict__ x, int64_t rows,
                                                     int64_t cols,
                                                     const float *__restrict__ prescale,
                                                     float *__restrict__ s,
                                                     float *__restrict__ col_sum)
{
    __shared__ float red_max[4][512];
    __shared__ float red_sum[4][512];
    const int lc = threadIdx.x % 64;
    const int lr = threadIdx.x / 64;
    const int64_t c0 = (int64_t)blockIdx.x * 512 + lc * 8;
    const int64_t r0 = (int64_t)blockIdx.y * kColSlab;
    const int64_t r1 = r0 + kColSlab < rows ? r0 + kColSlab : rows;
    float mx[8], sm[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        mx[e] = 0.0f;
        sm[e] = 0.0f;
    }
    if (c0 < cols) {
        for (int64_t r = r0 + lr; r < r1; r += 4) {
            float v[8];
            load8<BF16>(x, r * cols + c0, v);
            const float p = prescale ? prescale[r] : 1.0f;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                sm[e] = sm[e] + v[e];
                float g = prescale ? v[e] * p : v[e];
                mx[e] = fmaxf(mx[e], __builtin_fabsf(g));
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) {
        red_max[lr][lc * 8 + e] = mx[e];
        red_sum[lr][lc * 8 + e] = sm[e];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 512; i += 256) {
        const int64_t c = (int64_t)blockIdx.x * 512 + i;
        if (c >= cols)
            continue;
        float m = fmaxf(fmaxf(red_max[0][i], red_max[1][i]), fmaxf(red_max[2][i], red_max[3][i]));
        atomicMax(reinterpret_cast<unsigned int *>(s) + c, __float_as_uint(m));
        if (col_sum) {
            float t = ((red_sum[0][i] + red_sum[1][i]) + red_sum[2][i]) + red_sum[3][i];
            atomicAdd(col_sum + c, t);
        }
    }
}

// Column maxima -> scales, in place: s = fl(amax / 127).
__global__ void col_scale_kernel(float *__restrict__ s, int64_t cols)
{
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c < cols)
        s[c] = s[c] / 127.0f;
}

// Pass 2: codes.  Each thread owns 8 columns (so 8 reciprocals) and walks
// kColRows rows of them.
constexpr int kColRows = 16;

template <bool BF16>
__global__ __launch_bounds__(256) void colquant_kernel(const void *__restrict__ x, int64_t rows,
                                                       int64_t cols,
                                                       const float *__restrict__ prescale,
                                                       const float *__restrict__ s,
                                                       int8_t *__restrict__ q)
{
    const int64_t nch = cols / 8;
    const int64_t ch = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (ch >= nch)
        return;
    const int64_t c0 = ch * 8;
    float sc[8], inv[8];
    bool exact = false;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        sc[e] = s[c0 + e];
        inv[e] = 1.0f / sc[e];
        exact |= sc[e] < 0x1p-126f;   // zero or subnormal scale: exact path
    }
    const int64_t r0 = (int64_t)blockIdx.y * kColRows;
    const int64_t r1 = r0 + kColRows < rows ? r0 + kColRows : rows;
    for (int64_t r = r0; r < r1; r++) {
        float v[8], out[8];
        load8<BF16>(x, r * cols + c0, v);
        const float p = prescale ? prescale[r] : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            float g = prescale ? v[e] * p : v[e];
            if (!exact)
                out[e] = quant_code(g, sc[e], inv[e]);
            else
                out[e] = sc[e] == 0.0f ? 0.0f : quant_code_exact(g, sc[e]);
        }
        i32x2 w;
        w[0] = (int)pack4(out[0], out[1], out[2], out[3]);
        w[1] = (int)pack4(out[4], out[5], out[6], out[7]);
        *reinterpret_cast<i32x2 *>(q + r * cols + c0) = w;
    }
}

void launch_quantize_cols(const void *x, bool bf16, int64_t rows, int64_t cols,
                          const float *prescale, int8_t *q, float *s, float *col_sum,
                          hipStream_t st)
{
    const unsigned cblocks = (unsigned)((cols + 255) / 256);
    hipLaunchKernelGGL(zero_cols_kernel, dim3(cblocks), dim3(256), 0, st, s, col_sum, cols);
    if (rows > 0) {
        dim3 g1((unsigned)((cols + 511) / 512), (unsigned)((rows + kColSlab - 1) / kColSlab));
        if (bf16)
            hipLaunchKernelGGL(colmax_kernel<true>, g1, dim3(256), 0, st, x, rows, cols, prescale,
                               s, col_sum);
        else
            hipLaunchKernelGGL(colmax_kernel<false>, g1, dim3(256), 0, st, x, rows, cols,
                               prescale, s, col_sum);
    }
    hipLaunchKernelGGL(col_scale_kernel, dim3(cblocks), dim3(256), 0, st, s, cols);
    if (rows > 0) {
        dim3 g2((unsigned)((cols / 8 + 255) / 256), (unsigned)((rows + kColRows - 1) / kColRows));
        if (bf16)
            hipLaunchKernelGGL(colquant_kernel<true>, g2, dim3(256), 0, st, x, rows, cols,
                               prescale, s, q);
        else
            hipLaunchKernelGGL(colquant_kernel<false>, g2, dim3(256), 0, st, x, rows, cols,
                               prescale, s, q);
    }
}

// ------------------------------------------------ both dY quantizations
//
// Two reads of dY.  Pass 1 (grad_stats_kernel) reads it for the statistics
// of both quantizations: for each row, the maximum of |dY[r, c] * sw[c]| over
// each window of kStatCols columns, and for each column, the maximum of
// |dY[r, c] * sx[r]| and the sum of dY[r, c] over each group of rows.
// grad_scales_kernel reduces these partials into s1, s2 and the column sums
// (maxima are exact in any order; the sums run in a fixed order, so the
// result does not vary from run to run).  Pass 2 (grad_codes_kernel) reads dY
// again and writes both code arrays.  No kernel holds a whole row, so every
// width takes this path; the partials live in q2 until pass 2 overwrites it.
constexpr int kStatCols = 512;
constexpr int kStatBatch = 8;    // rows a lane loads before using any of them
// Waves of pass 1 (row groups x column windows).  At 7168 columns (14
// windows, workgroups of 4 windows) this gives 256 row groups and 1024
// workgroups, which at 4 waves per SIMD (120 registers per lane) are all
// resident at once (4096 waves gave 1168, and pass 1 ran 2-3% longer).
constexpr int kStatWaves = 3584;
constexpr int kCodeRows = 16;    // rows per thread in pass 2
// Offset of a dropped store: past any resource of pass 1 (rows * 4 bytes).
constexpr int kDropOffset = 0x7FFFFFF0;

// Maximum over the wave of each of kStatBatch values, left in lane 63: per
// step, one v_max_f32 whose first source is read through DPP.  The quad
// permutes and the half-row and row mirrors give every lane its 16-lane row's
// maximum, then row_bcast:15 (into rows 1 and 3) and row_bcast:31 (into rows
// 2 and 3) carry it up; the rows a step does not write keep their values.  As
// asm because the compiler does not fold a DPP move into the maximum.  The
// s_nop covers the two wait states a DPP read needs after a VALU write of its
// source; inside a step each instruction writes only its own register, which
// the next step reads eight instructions later.
#define QLIN_MAX_DPP_STEP(V, CTRL)                                                               \
    asm("s_nop 1\n\t"                                                                           \
        "v_max_f32_dpp %0, %0, %0 " CTRL " bank_mask:0xf\n\t"                                   \
        "v_max_f32_dpp %1, %1, %1 " CTRL " bank_mask:0xf\n\t"                                   \
        "v_max_f32_dpp %2, %2, %2 " CTRL " bank_mask:0xf\n\t"                                   \
        "v_max_f32_dpp %3, %3, %3 " CTRL " bank_mask:0xf\n\t"                                   \
        "v_max_f32_dpp %4, %4, %4 " CTRL " bank_mask:0xf\n\t"                                   \
        "v_max_f32_dpp %5, %5, %5 " CTRL " bank_mask:0xf\n\t"                                   \
        "v_max_f32_dpp %6, %6, %6 " CTRL " bank_mask:0xf\n\t"                                   \
        "v_max_f32_dpp %7, %7, %7 " CTRL " bank_mask:0xf"                                       \
        : "+v"(V[0]), "+v"(V[1]), "+v"(V[2]), "+v"(V[3]), "+v"(V[4]), "+v"(V[5]), "+v"(V[6]),    \
          "+v"(V[7]))

static_assert(kStatBatch == 8, "the DPP maximum steps take eight values");

__device__ __forceinline__ void wave_max8_to_last(float v[8])
{
    QLIN_MAX_DPP_STEP(v, "quad_perm:[1,0,3,2] row_mask:0xf");
    QLIN_MAX_DPP_STEP(v, "quad_perm:[2,3,0,1] row_mask:0xf");
    QLIN_MAX_DPP_STEP(v, "row_half_mirror row_mask:0xf");
    QLIN_MAX_DPP_STEP(v, "row_mirror row_mask:0xf");
    QLIN_MAX_DPP_STEP(v, "row_bcast:15 row_mask:0xa");
    QLIN_MAX_DPP_STEP(v, "row_bcast:31 row_mask:0xc");
}

#undef QLIN_MAX_DPP_STEP

// rowpart[win][rows]: row maxima over the 512-column window win;
// colpart[2 g][cols] and colpart[2 g + 1][cols]: column maxima and sums over
// the rows of row group g = blockIdx.y.  Each wave owns one window (the four
// waves of a workgroup sit side by side) and walks its group's batches of
// kStatBatch rows, which interleave with the other groups' (grid-stride).
// Slabs of consecutive rows per workgroup, or waves stacked in rows, ran at
// the same speed.
template <bool BF16>
__global__ __launch_bounds__(256) void grad_stats_kernel(const void *__restrict__ x, int64_t rows,
                                                         int64_t cols, const float *__restrict__ sw,
                                                         const float *__restrict__ sx,
                                                         float *__restrict__ rowpart,
                                                         float *__restrict__ colpart)
{
    const int lc = threadIdx.x % kWave;
    const int64_t win =
        (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    if (win * kStatCols >= cols)
        return;
    const int64_t c0 = win * kStatCols + lc * 8;
    const bool cok = c0 < cols;      // then all eight columns are (cols % 16 == 0)
    // Lanes past the last column read the last chunk (so that every load is
    // unconditional): their weight scales are zero and their column partials
    // are not written.  Rows past the end read the last row and are skipped.
    const int64_t cl = cok ? c0 : cols - 8;
    float w[8], mx[8], sm[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        w[e] = cok ? sw[c0 + e] : 0.0f;
        mx[e] = 0.0f;
        sm[e] = 0.0f;
    }
    // Row maxima go out through a buffer resource over this window's rows:
    // lane u < 8 stores row rb + u, and rows past the end (and lanes 8..63)
    // take an offset past the resource, whose stores the buffer unit drops.
    // So a batch issues the same memory operations on every path, and the
    // wait before a batch's arithmetic covers that batch's loads only.
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        rowpart + win * rows, (short)0, (int)(rows * 4), kRsrcWord3);
    const int64_t step = (int64_t)gridDim.y * kStatBatch;
    // Rows past the end read the last row.  A batch's eight row scales come
    // in one vector load (lane l holds row rb + l % 8's).
    Raw8<BF16> raw[2][kStatBatch];
    float pxv[2];
    auto fetch = [&](auto B, int64_t rb) {
        const int64_t rl = rb + (lc & 7);
        pxv[B()] = sx[rl < rows ? rl : rows - 1];
#pragma unroll
        for (int u = 0; u < kStatBatch; u++) {
            const int64_t r = rb + u < rows ? rb + u : rows - 1;
            raw[B()][u] = load_raw8<BF16>(x, r * cols + cl);
        }
    };
    auto reduce = [&](auto B, int64_t rb) {
        float rm[kStatBatch];
#pragma unroll
        for (int u = 0; u < kStatBatch; u++) {
            float v[8];
            unpack8<BF16>(raw[B()][u], v);
            const float px = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pxv[B()]), u));
            float m = 0.0f;
            if (rb + u < rows) {
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    sm[e] = sm[e] + v[e];
                    mx[e] = fmaxf(mx[e], __builtin_fabsf(v[e] * px));
                    m = fmaxf(m, __builtin_fabsf(v[e] * w[e]));
                }
            }
            rm[u] = m;
        }
        wave_max8_to_last(rm);
        float rv = 0.0f;
#pragma unroll
        for (int u = 0; u < kStatBatch; u++) {
            const float s = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rm[u]), kWave - 1));
            rv = lc == u ? s : rv;
        }
        const int64_t r = rb + lc;
        const int off = lc < kStatBatch && r < rows ? (int)(r * 4) : kDropOffset;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, rv), rp, off, 0, 0);
    };
    using Zero = std::integral_constant<int, 0>;
    using One = std::integral_constant<int, 1>;
    int64_t rb = (int64_t)blockIdx.y * kStatBatch;
    if constexpr (BF16) {
        // Two batches in registers: the next batch's loads are issued before
        // the current one is reduced, so the reads do not wait on the
        // arithmetic.  (fp32 rows would take 64 more registers per lane.)
        fetch(Zero{}, rb);
        for (; rb < rows; rb += 2 * step) {
            fetch(One{}, rb + step);
            reduce(Zero{}, rb);
            if (rb + step >= rows)
                break;
            fetch(Zero{}, rb + 2 * step);
            reduce(One{}, rb + step);
        }
    } else {
        for (; rb < rows; rb += step) {
            fetch(Zero{}, rb);
            reduce(Zero{}, rb);
        }
    }
    if (cok) {
        float *cm = colpart + 2 * (int64_t)blockIdx.y * cols;
        store8(cm, c0, mx);
        store8(cm + cols, c0, sm);
    }
}

// Partials -> s1 = fl(row max / 127), s2 = fl(column max / 127) and the column
// sums.  The first ceil(cols / 64) workgroups own 64 columns each: their 16
// waves take every 16th row group and are combined through LDS in a fixed
// order.  The workgroups after them own 1024 rows each.
__global__ __launch_bounds__(1024) void grad_scales_kernel(
    const float *__restrict__ rowpart, int wins, const float *__restrict__ colpart, int groups,
    int64_t rows, int64_t cols, float *__restrict__ s1, float *__restrict__ s2,
    float *__restrict__ col_sum)
{
    const int64_t cblocks = (cols + 63) / 64;
    if ((int64_t)blockIdx.x >= cblocks) {
        const int64_t r = ((int64_t)blockIdx.x - cblocks) * 1024 + threadIdx.x;
        if (r < rows) {
            float m = 0.0f;
            for (int k = 0; k < wins; k++)
                m = fmaxf(m, rowpart[k * rows + r]);
            s1[r] = m / 127.0f;
        }
        return;
    }
    __shared__ float red_max[16][64], red_sum[16][64];
    const int lc = threadIdx.x % 64, sl = threadIdx.x / 64;
    const int64_t c = (int64_t)blockIdx.x * 64 + lc;
    float m = 0.0f, sum = 0.0f;
    if (c < cols) {
#pragma unroll 4
        for (int g = sl; g < groups; g += 16) {
            m = fmaxf(m, colpart[(2 * (int64_t)g) * cols + c]);
            sum = sum + colpart[(2 * (int64_t)g + 1) * cols + c];
        }
    }
    red_max[sl][lc] = m;
    red_sum[sl][lc] = sum;
    __syncthreads();
    if (sl == 0 && c < cols) {
#pragma unroll
        for (int i = 1; i < 16; i++) {
            m = fmaxf(m, red_max[i][lc]);
            sum = sum + red_sum[i][lc];
        }
        s2[c] = m / 127.0f;
        if (col_sum)
            col_sum[c] = sum;
    }
}

// Eight codes rne(fl(g[e] / s[e])) with a scale per element, each s[e] > 0
// normal and inv[e] as quant8 takes it: the fast path and tie check of
// quant8, element by element.
__device__ __forceinline__ i32x2 quant8_each(const float g[8], const float s[8],
                                             const float inv[8])
{
    constexpr float kMagic = 0x1.8p23f;
    float f[8];
    float dmax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++)
        f[e] = code_fast(g[e], inv[e], dmax);
    if (!(dmax < 0.5f - 0x1p-14f)) {
#pragma unroll
        for (int e = 0; e < 8; e++)
            f[e] = __builtin_rintf(g[e] / s[e]) + kMagic;
    }
    auto pack = [&](int o) {
        const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(f[o + 1]), __float_as_uint(f[o]),
                                                  0x0C0C0400u);
        const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(f[o + 3]),
                                                  __float_as_uint(f[o + 2]), 0x04000C0Cu);
        return (int)(lo | hi);
    };
    return i32x2{pack(0), pack(4)};
}

// Pass 2: each thread owns 8 columns (their weight scales, column scales and
// reciprocals stay in registers) and walks kCodeRows rows, writing the row
// codes rne(fl(fl(dY * sw) / s1[r])) to q1 and the column codes
// rne(fl(fl(dY * sx[r]) / s2[c])) to q2.  A zero scale gives zero codes; a
// subnormal one (its reciprocal loses precision) the exact quotient.
template <bool BF16>
__global__ __launch_bounds__(256) void grad_codes_kernel(
    const void *__restrict__ x, int64_t rows, int64_t cols, const float *__restrict__ sw,
    const float *__restrict__ sx, const float *__restrict__ s1, const float *__restrict__ s2,
    int8_t *__restrict__ q1, int8_t *__restrict__ q2)
{
    const int64_t nch = cols / 8;
    const int64_t ch = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (ch >= nch)
        return;
    const int64_t c0 = ch * 8;
    float w[8], sc[8], inv[8];
    bool cexact = false;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        w[e] = sw[c0 + e];
        sc[e] = s2[c0 + e];
        inv[e] = recip_refined(sc[e]);     // unused for a zero or subnormal scale
        cexact |= sc[e] < 0x1p-126f;
    }
    const int64_t r0 = (int64_t)blockIdx.y * kCodeRows;
    const int64_t r1 = r0 + kCodeRows < rows ? r0 + kCodeRows : rows;
    for (int64_t r = r0; r < r1; r++) {
        float v[8], g[8];
        load8<BF16>(x, r * cols + c0, v);
        const float sr = s1[r];
#pragma unroll
        for (int e = 0; e < 8; e++)
            g[e] = v[e] * w[e];
        i32x2 o;
        if (sr == 0.0f) {
            o = i32x2{0, 0};
        } else if (sr < 0x1p-126f) {
            float c[8];
#pragma unroll
            for (int e = 0; e < 8; e++)
                c[e] = quant_code_exact(g[e], sr);
            o[0] = (int)pack4(c[0], c[1], c[2], c[3]);
            o[1] = (int)pack4(c[4], c[5], c[6], c[7]);
        } else {
            o = quant8(g, sr, recip_refined(sr));
        }
        *reinterpret_cast<i32x2 *>(q1 + r * cols + c0) = o;
        const float p = sx[r];
#pragma unroll
        for (int e = 0; e < 8; e++)
            g[e] = v[e] * p;
        if (!cexact) {
            o = quant8_each(g, sc, inv);
        } else {
            float c[8];
#pragma unroll
            for (int e = 0; e < 8; e++)
                c[e] = sc[e] == 0.0f ? 0.0f : quant_code_exact(g[e], sc[e]);
            o[0] = (int)pack4(c[0], c[1], c[2], c[3]);
            o[1] = (int)pack4(c[4], c[5], c[6], c[7]);
        }
        *reinterpret_cast<i32x2 *>(q2 + r * cols + c0) = o;
    }
}

void launch_quantize_grad(const void *x, bool bf16, int64_t rows, int64_t cols, const float *sw,
                          const float *sx, int8_t *q1, float *s1, int8_t *q2, float *s2,
                          float *col_sum, hipStream_t st)
{
    // Row groups: about kStatWaves waves in all, at most one per 16 rows, so
    // that the partials (4 bytes per row per column window, 8 per column per
    // group) fit in q2 from 16 rows on.  Fewer rows, or none, take the two
    // quantizers separately.
    const int64_t wins = (cols + kStatCols - 1) / kStatCols;
    int64_t groups = kStatWaves / wins;
    groups = groups < rows / 16 ? groups : rows / 16;
    if (rows == 0 || groups < 1 || 4 * (wins * rows + 2 * groups * cols) > rows * cols) {
        if (rows > 0)
            launch_quantize_rows(x, bf16, rows, cols, sw, 0, 1.0f, q1, s1, st);
        launch_quantize_cols(x, bf16, rows, cols, sx, q2, s2, col_sum, st);
        return;
    }
    float *rowpart = reinterpret_cast<float *>(q2);
    float *colpart = rowpart + wins * rows;
    const dim3 g1((unsigned)((wins + 3) / 4), (unsigned)groups);
    if (bf16)
        hipLaunchKernelGGL(grad_stats_kernel<true>, g1, dim3(256), 0, st, x, rows, cols, sw, sx,
                           rowpart, colpart);
    else
        hipLaunchKernelGGL(grad_stats_kernel<false>, g1, dim3(256), 0, st, x, rows, cols, sw, sx,
                           rowpart, colpart);
    const unsigned gs = (unsigned)((cols + 63) / 64 + (rows + 1023) / 1024);
    hipLaunchKernelGGL(grad_scales_kernel, dim3(gs), dim3(1024), 0, st, rowpart, (int)wins,
                       colpart, (int)groups, rows, cols, s1, s2, col_sum);
    const dim3 g2((unsigned)((cols / 8 + 255) / 256), (unsigned)((rows + kCodeRows - 1) / kCodeRows));
    if (bf16)
        hipLaunchKernelGGL(grad_codes_kernel<true>, g2, dim3(256), 0, st, x, rows, cols, sw, sx,
                           s1, s2, q1, q2);
    else
        hipLaunchKernelGGL(grad_codes_kernel<false>, g2, dim3(256), 0, st, x, rows, cols, sw, sx,
                           s1, s2, q1, q2);
}

// --------------------------------------------------------------- rotation

// Flat over 8-element chunks: a wave covers 64 consecutive chunks, so every
// block (at most 64 chunks, aligned) sits inside one wave.
template <bool BF16, int HAD>
__global__ __launch_bounds__(256) void hadamard_kernel(const void *__restrict__ x, int64_t nch,
                                                       int blk, float cb, float *__restrict__ y)
{
    // A fixed block size permutes chunks inside groups of 16, all valid or all
    // past the end (nch is then a multiple of 16).
    const int64_t c = lane_chunk<HAD>((int64_t)blockIdx.x * 256 + threadIdx.x);
    const bool ok = c < nch;
    float v[8];
    if (ok) {
        load8<BF16>(x, c * 8, v);
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
            v[e] = 0.0f;
    }
    rotate8<HAD, true>(v, blk, cb);
    if (ok)
        store8(y, c * 8, v);
}

// The represented weight in the original basis: w = fl(s[row] * q) for 8
// consecutive codes per lane, then (HAD != 0) the rotation of each block.
// Flat over 8-element chunks like the rotation kernel.
template <int HAD>
__global__ __launch_bounds__(256) void dequant_weight_kernel(const int8_t *__restrict__ q,
                                                             const float *__restrict__ sw,
                                                             int64_t nch, int64_t cols, int blk,
                                                             float cb, float *__restrict__ w)
{
    const int64_t c = lane_chunk<HAD>((int64_t)blockIdx.x * 256 + threadIdx.x);
    const bool ok = c < nch;
    float v[8];
    if (ok) {
        const i32x2 qv = *reinterpret_cast<const i32x2 *>(q + c * 8);
        const float s = sw[(c * 8) / cols];
#pragma unroll
        for (int e = 0; e < 8; e++)
            v[e] = s * (float)(int8_t)((uint32_t)qv[e / 4] >> (8 * (e % 4)));
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
            v[e] = 0.0f;
    }
    if (HAD != 0)
        rotate8<HAD, true>(v, blk, cb);
    if (ok)
        store8(w, c * 8, v);
}

void launch_dequantize_weight(const int8_t *q, const float *sw, int64_t rows, int64_t cols,
                              int blk, float cb, float *w, hipStream_t st)
{
    const int64_t nch = rows * cols / 8;
    const unsigned grid = (unsigned)((nch + 255) / 256);
    auto go = [&](auto h) {
        hipLaunchKernelGGL((dequant_weight_kernel<decltype(h)::value>), dim3(grid), dim3(256), 0,
                           st, q, sw, nch, cols, blk, cb, w);
    };
    switch (blk) {
    case 0: return go(std::integral_constant<int, 0>());
    case 16: return go(std::integral_constant<int, 16>());
    case 32: return go(std::integral_constant<int, 32>());
    case 64: return go(std::integral_constant<int, 64>());
    case 128: return go(std::integral_constant<int, 128>());
    default: return go(std::integral_constant<int, -1>());
    }
}

void launch_hadamard(const void *x, bool bf16, int64_t rows, int64_t cols, int blk, float cb,
                     float *y, hipStream_t st)
{
    const int64_t nch = rows * cols / 8;
    const unsigned grid = (unsigned)((nch + 255) / 256);
    auto go = [&](auto bf, auto h) {
        hipLaunchKernelGGL((hadamard_kernel<decltype(bf)::value, decltype(h)::value>), dim3(grid),
                           dim3(256), 0, st, x, nch, blk, cb, y);
    };
    auto with_block = [&](auto bf) {
        switch (blk) {
        case 16: return go(bf, std::integral_constant<int, 16>());
        case 32: return go(bf, std::integral_constant<int, 32>());
        case 64: return go(bf, std::integral_constant<int, 64>());
        case 128: return go(bf, std::integral_constant<int, 128>());
        default: return go(bf, std::integral_constant<int, -1>());
        }
    };
    if (bf16)
        with_block(std::true_type());
    else
        with_block(std::false_type());
}

} // namespace qlin
