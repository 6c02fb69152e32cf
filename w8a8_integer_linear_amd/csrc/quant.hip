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
// quantizes elementwise.  Both quantizations of dY in one call share the read
// of pass 1 with the row quantizer (column partials per workgroup, then a
// reduce).
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
//
// COLS (no rotation, 256 threads) also gathers, over the workgroup's rows, the
// column maxima of |x * colpre[row]| and the column sums of the raw x, and
// writes them to part[2 * blockIdx.x][cols] and part[2 * blockIdx.x + 1][cols]
// at the end: one read of dY serves both of its quantizations.
template <bool BF16, int THREADS, int J, int HAD, bool COLS>
__global__ __launch_bounds__(THREADS) void quant_rows_kernel(
    const void *__restrict__ x, int64_t rows, int64_t cols, const float *__restrict__ prescale,
    int had, float cb, int8_t *__restrict__ q, float *__restrict__ s,
    const float *__restrict__ colpre, float *__restrict__ part)
{
    static_assert(!COLS || (HAD == 0 && (THREADS == 512 || THREADS == 1024) && J <= 2),
                  "column partials: no rotation, 512 or 1024 threads, at most 16 columns per "
                  "lane");
    // 1024-thread workgroups have 128 registers per lane: no room for the
    // prescale or the next row's data, which they load when they need it.
    constexpr bool kKeepPrescale = THREADS <= 256 || COLS;
    constexpr bool kPrefetch = THREADS <= 256 || COLS;
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
    float cmax[COLS ? J : 1][8], csum[COLS ? J : 1][8];
    if constexpr (COLS) {
#pragma unroll
        for (int j = 0; j < J; j++)
#pragma unroll
            for (int e = 0; e < 8; e++) {
                cmax[j][e] = 0.0f;
                csum[j][e] = 0.0f;
            }
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
            if constexpr (COLS) {
                if (ok) {
                    const float cp = colpre ? colpre[row] : 1.0f;
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        csum[COLS ? j : 0][e] = csum[COLS ? j : 0][e] + v[j][e];
                        const float g = colpre ? v[j][e] * cp : v[j][e];
                        cmax[COLS ? j : 0][e] = fmaxf(cmax[COLS ? j : 0][e], __builtin_fabsf(g));
                    }
                }
            }
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
        const float inv = 1.0f / sc;
        const bool zero = (a == 0.0f);
        const bool subnormal = !zero && sc < 0x1p-126f;
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
    if constexpr (COLS) {
#pragma unroll
        for (int j = 0; j < J; j++) {
            const int64_t c = t + (int64_t)j * THREADS;
            if (c < nch) {
                store8(part + (2 * (int64_t)blockIdx.x) * cols, c * 8, cmax[j]);
                store8(part + (2 * (int64_t)blockIdx.x + 1) * cols, c * 8, csum[j]);
            }
        }
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
    hipLaunchKernelGGL((quant_rows_kernel<BF16, THREADS, J, HAD, false>), dim3(grid),
                       dim3(THREADS), 0, st, x, rows, cols, prescale, had, cb, q, s, nullptr,
                       nullptr);
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

// Partials from the fused row pass -> column scales s = fl(max / 127) and
// column sums.  A workgroup owns 64 columns; its 16 waves take every 16th
// workgroup partial and are combined through LDS (the maximum is exact in any
// order; the sums run in a fixed order, so the result is deterministic).
__global__ __launch_bounds__(1024) void grad_cols_reduce_kernel(const float *__restrict__ part,
                                                                int groups, int64_t cols,
                                                                float *__restrict__ s,
                                                                float *__restrict__ col_sum)
{
    __shared__ float red_max[16][64], red_sum[16][64];
    const int lc = threadIdx.x % 64, sl = threadIdx.x / 64;
    const int64_t c = (int64_t)blockIdx.x * 64 + lc;
    float m = 0.0f, sum = 0.0f;
    if (c < cols) {
#pragma unroll 4
        for (int g = sl; g < groups; g += 16) {
            m = fmaxf(m, part[(2 * (int64_t)g) * cols + c]);
            sum = sum + part[(2 * (int64_t)g + 1) * cols + c];
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
        s[c] = m / 127.0f;
        if (col_sum)
            col_sum[c] = sum;
    }
}

// The fused pass keeps the prescale and two partials per element it owns in
// registers, so it takes rows of up to 16384 columns: 2 chunks per lane at
// 512 threads up to 8192 columns, at 1024 threads (one workgroup per compute
// unit, half as many workgroups) above.
// Its workgroups write 8 bytes per column of partials into q2, which must
// therefore hold at least 8 * groups * cols bytes: groups <= rows / 8.
constexpr int64_t kGradMaxCols = 16384;
constexpr int64_t kGradMinRows = 512;
constexpr int kGradGroups = 512;

template <bool BF16, int THREADS, int J>
static void launch_grad_rows(const void *x, int64_t rows, int64_t cols, const float *sw,
                             const float *sx, int8_t *q1, float *s1, float *part, int groups,
                             hipStream_t st)
{
    hipLaunchKernelGGL((quant_rows_kernel<BF16, THREADS, J, 0, true>), dim3(groups),
                       dim3(THREADS), 0, st, x, rows, cols, sw, 0, 1.0f, q1, s1, sx, part);
}

void launch_quantize_grad(const void *x, bool bf16, int64_t rows, int64_t cols, const float *sw,
                          const float *sx, int8_t *q1, float *s1, int8_t *q2, float *s2,
                          float *col_sum, hipStream_t st)
{
    if (cols > kGradMaxCols || rows < kGradMinRows) {
        if (rows > 0)
            launch_quantize_rows(x, bf16, rows, cols, sw, 0, 1.0f, q1, s1, st);
        launch_quantize_cols(x, bf16, rows, cols, sx, q2, s2, col_sum, st);
        return;
    }
    const bool wide = cols > 8192;
    const int max_groups = wide ? kGradGroups / 2 : kGradGroups;
    const int groups = (int)(rows / 8 < max_groups ? rows / 8 : max_groups);
    float *part = reinterpret_cast<float *>(q2);
    const int64_t j = (cols / 8 + (wide ? 1023 : 511)) / (wide ? 1024 : 512);
    auto go = [&](auto bf) {
        constexpr bool B = decltype(bf)::value;
        if (wide)
            launch_grad_rows<B, 1024, 2>(x, rows, cols, sw, sx, q1, s1, part, groups, st);
        else if (j == 1)
            launch_grad_rows<B, 512, 1>(x, rows, cols, sw, sx, q1, s1, part, groups, st);
        else
            launch_grad_rows<B, 512, 2>(x, rows, cols, sw, sx, q1, s1, part, groups, st);
    };
    if (bf16)
        go(std::true_type());
    else
        go(std::false_type());
    hipLaunchKernelGGL(grad_cols_reduce_kernel, dim3((unsigned)((cols + 63) / 64)), dim3(1024), 0,
                       st, part, groups, cols, s2, col_sum);
    dim3 g2((unsigned)((cols / 8 + 255) / 256), (unsigned)((rows + kColRows - 1) / kColRows));
    if (bf16)
        hipLaunchKernelGGL(colquant_kernel<true>, g2, dim3(256), 0, st, x, rows, cols, sx, s2, q2);
    else
        hipLaunchKernelGGL(colquant_kernel<false>, g2, dim3(256), 0, st, x, rows, cols, sx, s2,
                           q2);
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
