// int8 x int8 -> int32 products of the layer on CDNA4 MFMA, with fused
// dequant epilogues (mini_trainer guide: integer forward and backward matrix
// products; OneTrainer PR #1681: int8 product of quantized activations and
// weights).
//
// One kernel template serves the three products.  C[i, j] = sum_t A(i, t) *
// B(j, t) where each operand is stored either with the contraction index
// contiguous ("row" operand: element (i, t) at base[i * ld + t]) or with the
// contraction index as the row ("km" operand: element (i, t) at base[t * ld +
// i]):
//   forward  A = qx  [M,K] row, B = qw [N,K] row          C = y  [M,N]
//   dX       A = qg1 [M,N] row, B = qw [N,K] km (t = n)   C = dx [M,K]
//   dW       A = qg2 [M,N] km,  B = qx [M,K] km (t = m)   C = dw [N,K]
// Both operands are staged in LDS with the contraction index contiguous, so
// the MFMA fragment reads are the same 16-byte reads for every layout; a km
// operand is loaded as 4 contraction rows x 8 bytes per lane and transposed in
// registers with byte permutes before it is written to LDS.
//
// Exactness: int32 accumulation of int8 products is exact for contractions up
// to 131,071 and does not depend on the order of k, so the placement of k
// inside an MFMA fragment only has to agree between A and B (it does: both
// are read with the same lane -> k map).
#include "common.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;            // contraction bytes per pipeline stage
constexpr int kLds = kBK + 16;     // LDS row stride in bytes (padding spreads banks)

struct GemmParams {
    const int8_t *a;
    const int8_t *b;
    int64_t lda, ldb, ldc;
    int R, S, T;                   // output rows, output cols, contraction
    const float *srow;
    const float *scol;
    const float *bias;
    void *out;
    int tiles_i, tiles_j;
};

// 4x4 byte transpose: x_r holds bytes (c0..c3) of row r, y_c gets bytes
// (r0..r3) of column c.  v_perm_b32 byte selectors: 0-3 pick bytes of the
// second source, 4-7 bytes of the first.
__device__ __forceinline__ void transpose4x4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                             uint32_t *y)
{
    const uint32_t t0 = __builtin_amdgcn_perm(x1, x0, 0x05010400u);
    const uint32_t t1 = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
    const uint32_t t2 = __builtin_amdgcn_perm(x1, x0, 0x07030602u);
    const uint32_t t3 = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
    y[0] = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
    y[1] = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
    y[2] = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
    y[3] = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
}

// Global -> register -> LDS staging of one operand tile of ROWS output rows
// by kBK contraction bytes.
template <int ROWS, bool KM>
struct Stage;

template <int ROWS>
struct Stage<ROWS, false> {
    static constexpr int N = ROWS * (kBK / 16) / kThreads;   // 16-byte chunks per lane
    i32x4 r[N];

    __device__ __forceinline__ void load(const int8_t *base, int64_t ld, int i0, int lim,
                                         int k0, int T)
    {
#pragma unroll
        for (int p = 0; p < N; p++) {
            const int c = threadIdx.x + p * kThreads;
            const int row = c / (kBK / 16);
            const int kc = c % (kBK / 16);
            const int gi = i0 + row;
            const int gk = k0 + kc * 16;
            if (gi < lim && gk < T)
                r[p] = *reinterpret_cast<const i32x4 *>(base + (int64_t)gi * ld + gk);
            else
                r[p] = i32x4{0, 0, 0, 0};
        }
    }

    __device__ __forceinline__ void store(int8_t *lds) const
    {
#pragma unroll
        for (int p = 0; p < N; p++) {
            const int c = threadIdx.x + p * kThreads;
            const int row = c / (kBK / 16);
            const int kc = c % (kBK / 16);
            *reinterpret_cast<i32x4 *>(lds + row * kLds + kc * 16) = r[p];
        }
    }
};

template <int ROWS>
struct Stage<ROWS, true> {
    // Units of 4 contraction rows x 8 output bytes; lanes of a wave take 16
    // consecutive contraction quads of 4 different column groups, which keeps
    // the transposed LDS writes spread over banks.
    static constexpr int N = (kBK / 4) * (ROWS / 8) / kThreads;
    i32x2 r[N][4];

    __device__ __forceinline__ void load(const int8_t *base, int64_t ld, int i0, int lim,
                                         int k0, int T)
    {
#pragma unroll
        for (int p = 0; p < N; p++) {
            const int u = threadIdx.x + p * kThreads;
            const int kq = u % (kBK / 4);
            const int ic = u / (kBK / 4);
            const int gi = i0 + ic * 8;
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                const int gk = k0 + kq * 4 + rr;
                if (gi < lim && gk < T)
                    r[p][rr] = *reinterpret_cast<const i32x2 *>(base + (int64_t)gk * ld + gi);
                else
                    r[p][rr] = i32x2{0, 0};
            }
        }
    }

    __device__ __forceinline__ void store(int8_t *lds) const
    {
#pragma unroll
        for (int p = 0; p < N; p++) {
            const int u = threadIdx.x + p * kThreads;
            const int kq = u % (kBK / 4);
            const int ic = u / (kBK / 4);
            uint32_t y[8];
            transpose4x4((uint32_t)r[p][0][0], (uint32_t)r[p][1][0], (uint32_t)r[p][2][0],
                         (uint32_t)r[p][3][0], y);
            transpose4x4((uint32_t)r[p][0][1], (uint32_t)r[p][1][1], (uint32_t)r[p][2][1],
                         (uint32_t)r[p][3][1], y + 4);
#pragma unroll
            for (int e = 0; e < 8; e++)
                *reinterpret_cast<uint32_t *>(lds + (ic * 8 + e) * kLds + kq * 4) = y[e];
        }
    }
};

enum { EPI_RAW = 0, EPI_ROWSCALE = 1, EPI_FWD = 2 };

// Tile order: workgroups are dispatched round-robin over the 8 XCDs, so
// consecutive ids are first regrouped per XCD (each XCD gets a contiguous
// range of tiles), then walked in groups of kGroup tile rows so that tiles
// running together share their A rows and B columns in that XCD's L2.
constexpr int kGroup = 8;

__device__ __forceinline__ void tile_of(int pid, int tiles_i, int tiles_j, int &ti, int &tj)
{
    const int n = tiles_i * tiles_j;
    const int q = n / 8, rem = n % 8;
    const int xcd = pid % 8, idx = pid / 8;
    const int lin = xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
    const int per_group = kGroup * tiles_j;
    const int g = lin / per_group;
    const int first = g * kGroup;
    const int gsize = tiles_i - first < kGroup ? tiles_i - first : kGroup;
    const int in = lin % per_group;
    ti = first + in % gsize;
    tj = in / gsize;
}

template <int BM, int BN, bool AKM, bool BKM, int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmParams p)
{
    constexpr int FM = BM / 64;    // 32x32 blocks per wave along rows (2 x 2 waves)
    constexpr int FN = BN / 64;
    __shared__ __attribute__((aligned(16))) int8_t smem[2][(BM + BN) * kLds];

    int ti, tj;
    tile_of(blockIdx.x, p.tiles_i, p.tiles_j, ti, tj);
    const int i0 = ti * BM, j0 = tj * BN;
    const int lane = __lane_id();
    const int w = threadIdx.x / kWave;
    const int wi = w / 2, wj = w % 2;

    Stage<BM, AKM> sa;
    Stage<BN, BKM> sb;
    i32x16 acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; a++)
#pragma unroll
        for (int b = 0; b < FN; b++)
            acc[a][b] = i32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    const int KT = (p.T + kBK - 1) / kBK;
    sa.load(p.a, p.lda, i0, p.R, 0, p.T);
    sb.load(p.b, p.ldb, j0, p.S, 0, p.T);
    sa.store(smem[0]);
    sb.store(smem[0] + BM * kLds);
    __syncthreads();

    for (int kt = 0; kt < KT; kt++) {
        const bool more = kt + 1 < KT;
        if (more) {
            sa.load(p.a, p.lda, i0, p.R, (kt + 1) * kBK, p.T);
            sb.load(p.b, p.ldb, j0, p.S, (kt + 1) * kBK, p.T);
        }
        const int8_t *la = smem[kt & 1];
        const int8_t *lb = la + BM * kLds;
#pragma unroll
        for (int kk = 0; kk < kBK / 32; kk++) {
            i32x4 af[FM], bf[FN];
            const int koff = kk * 32 + (lane / 32) * 16;
#pragma unroll
            for (int a = 0; a < FM; a++)
                af[a] = *reinterpret_cast<const i32x4 *>(
                    la + (wi * (BM / 2) + a * 32 + lane % 32) * kLds + koff);
#pragma unroll
            for (int b = 0; b < FN; b++)
                bf[b] = *reinterpret_cast<const i32x4 *>(
                    lb + (wj * (BN / 2) + b * 32 + lane % 32) * kLds + koff);
#pragma unroll
            for (int a = 0; a < FM; a++)
#pragma unroll
                for (int b = 0; b < FN; b++)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], acc[a][b], 0,
                                                                      0, 0);
        }
        if (more) {
            sa.store(smem[(kt + 1) & 1]);
            sb.store(smem[(kt + 1) & 1] + BM * kLds);
        }
        __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: lane l, register r holds column
    // l % 32 and row 8 * (r / 4) + 4 * (l / 32) + r % 4 of the block.
#pragma unroll
    for (int a = 0; a < FM; a++) {
#pragma unroll
        for (int b = 0; b < FN; b++) {
            const int j = j0 + wj * (BN / 2) + b * 32 + lane % 32;
            if (j >= p.S)
                continue;
            float cs = 0.0f, bj = 0.0f;
            if constexpr (EPI == EPI_FWD) {
                cs = p.scol[j];
                if (p.bias)
                    bj = p.bias[j];
            }
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int i = i0 + wi * (BM / 2) + a * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
                if (i >= p.R)
                    continue;
                const int64_t off = (int64_t)i * p.ldc + j;
                const int v = acc[a][b][r];
                if constexpr (EPI == EPI_RAW) {
                    static_cast<int32_t *>(p.out)[off] = v;
                } else {
                    float f = (float)v * p.srow[i];
                    if constexpr (EPI == EPI_FWD) {
                        f = f * cs;
                        if (p.bias)
                            f = f + bj;
                    }
                    static_cast<float *>(p.out)[off] = f;
                }
            }
        }
    }
}

template <int BM, int BN, bool AKM, bool BKM, int EPI>
void run_gemm(const GemmParams &p0, hipStream_t st)
{
    GemmParams p = p0;
    p.tiles_i = (p.R + BM - 1) / BM;
    p.tiles_j = (p.S + BN - 1) / BN;
    const unsigned grid = (unsigned)(p.tiles_i * p.tiles_j);
    hipLaunchKernelGGL((gemm_kernel<BM, BN, AKM, BKM, EPI>), dim3(grid), dim3(kThreads), 0, st,
                       p);
}

// Forward product for M <= 16 (decode-like shapes): the weight is streamed
// once; each workgroup owns 16 output columns and its 4 waves split the
// contraction in interleaved 64-byte steps, combining their int32 partials
// through LDS.  One 16x16x64 MFMA per step with A = the (zero-padded) 16
// rows of qx.  16x16 accumulator layout: lane l, register r holds column
// l % 16 and row 4 * (l / 16) + r.
template <bool RAW>
__global__ __launch_bounds__(256) void skinny_fwd_kernel(const int8_t *__restrict__ qx,
                                                         const float *__restrict__ sx,
                                                         const int8_t *__restrict__ qw,
                                                         const float *__restrict__ sw,
                                                         const float *__restrict__ bias, int M,
                                                         int N, int K, void *__restrict__ out)
{
    __shared__ i32x4 red[4][kWave];
    const int lane = __lane_id();
    const int w = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 16;
    const int col = lane % 16, g = lane / 16;
    const int8_t *xrow = qx + (int64_t)col * K;
    const int8_t *wrow = qw + (int64_t)(n0 + col) * K;
    const bool xok = col < M;
    i32x4 acc = {0, 0, 0, 0};
    const int steps = (K + 63) / 64;
    constexpr int U = 4;
    for (int s0 = w; s0 < steps; s0 += 4 * U) {
        i32x4 av[U], bv[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int k = (s0 + 4 * u) * 64 + g * 16;
            const bool ok = (s0 + 4 * u) < steps && k < K;
            bv[u] = ok ? *reinterpret_cast<const i32x4 *>(wrow + k) : i32x4{0, 0, 0, 0};
            av[u] = (ok && xok) ? *reinterpret_cast<const i32x4 *>(xrow + k) : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; u++)
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[u], bv[u], acc, 0, 0, 0);
    }
    red[w][lane] = acc;
    __syncthreads();
    if (w != 0)
        return;
    const i32x4 t = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    const int n = n0 + col;
    float cs = 0.0f, bn = 0.0f;
    if (!RAW) {
        cs = sw[n];
        if (bias)
            bn = bias[n];
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int m = 4 * g + r;
        if (m >= M)
            continue;
        if (RAW) {
            static_cast<int32_t *>(out)[(int64_t)m * N + n] = t[r];
        } else {
            float f = (float)t[r] * sx[m];
            f = f * cs;
            if (bias)
                f = f + bn;
            static_cast<float *>(out)[(int64_t)m * N + n] = f;
        }
    }
}

} // namespace

void launch_product(const ProductArgs &a, hipStream_t st)
{
    GemmParams p{};
    p.out = a.out;
    p.srow = a.srow;
    p.scol = a.scol;
    p.bias = a.bias;
    if (a.op == 0) {
        if (a.M <= 16) {
            const unsigned grid = (unsigned)(a.N / 16);
            if (a.raw)
                hipLaunchKernelGGL(skinny_fwd_kernel<true>, dim3(grid), dim3(256), 0, st, a.a,
                                   a.srow, a.b, a.scol, a.bias, (int)a.M, (int)a.N, (int)a.K,
                                   a.out);
            else
                hipLaunchKernelGGL(skinny_fwd_kernel<false>, dim3(grid), dim3(256), 0, st, a.a,
                                   a.srow, a.b, a.scol, a.bias, (int)a.M, (int)a.N, (int)a.K,
                                   a.out);
            return;
        }
        p.a = a.a; p.lda = a.K;
        p.b = a.b; p.ldb = a.K;
        p.R = (int)a.M; p.S = (int)a.N; p.T = (int)a.K; p.ldc = a.N;
        if (a.raw)
            run_gemm<128, 128, false, false, EPI_RAW>(p, st);
        else
            run_gemm<128, 128, false, false, EPI_FWD>(p, st);
    } else if (a.op == 1) {
        p.a = a.a; p.lda = a.N;
        p.b = a.b; p.ldb = a.K;
        p.R = (int)a.M; p.S = (int)a.K; p.T = (int)a.N; p.ldc = a.K;
        if (a.raw)
            run_gemm<128, 128, false, true, EPI_RAW>(p, st);
        else
            run_gemm<128, 128, false, true, EPI_ROWSCALE>(p, st);
    } else {
        p.a = a.a; p.lda = a.N;
        p.b = a.b; p.ldb = a.K;
        p.R = (int)a.N; p.S = (int)a.K; p.T = (int)a.M; p.ldc = a.K;
        if (a.raw)
            run_gemm<128, 128, true, true, EPI_RAW>(p, st);
        else
            run_gemm<128, 128, true, true, EPI_ROWSCALE>(p, st);
    }
}

} // namespace qlin
