// Matrix-core ceiling: the products' register tile and MFMA sequence with no
// memory traffic.  Every wave holds what a product wave holds in its main
// loop (8 x 4 blocks of 16 x 16 int32 sums, the fragments of two 64-byte
// contraction steps: 8 row blocks and 4 column blocks each) and repeats the
// products' sequence of 64 v_mfma_i32_16x16x64_i8 (row block, then column
// block, then the block's two steps back to back), 8 waves per workgroup,
// one workgroup per compute unit.  On random fragments its rate is the int8 matrix throughput the
// device sustains within its power limit, the practical ceiling the products
// are measured against beside the nameplate peak.
#include "common.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

// Fragment f of the buffer (24 of them, 1 KiB each: lane l's 16 bytes at
// 16 l) for wave w: wave w starts its 24 fragments at f = w, so the waves of a
// workgroup multiply different data.
__global__ __launch_bounds__(512, 1) void mfma_ceiling_kernel(const i32x4 *__restrict__ frags,
                                                              i32x4 *__restrict__ out, int iters)
{
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    i32x4 fa[2][8], fb[2][4];
#pragma unroll
    for (int s = 0; s < 2; s++) {
#pragma unroll
        for (int f = 0; f < 8; f++)
            fa[s][f] = frags[((w + 8 * s + f) % kMfmaCeilingFrags) * kWave + lane];
#pragma unroll
        for (int b = 0; b < 4; b++)
            fb[s][b] = frags[((w + 16 + 4 * s + b) % kMfmaCeilingFrags) * kWave + lane];
    }
    i32x4 acc[8][4];
#pragma unroll
    for (int f = 0; f < 8; f++)
#pragma unroll
        for (int b = 0; b < 4; b++)
            acc[f][b] = i32x4{0, 0, 0, 0};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int f = 0; f < 8; f++)
#pragma unroll
            for (int b = 0; b < 4; b++)
#pragma unroll
                for (int s = 0; s < 2; s++) {
                    // B first, as in the products: block (f, b) holds the
                    // 16 x 16 sums transposed.
                    acc[f][b] =
                        __builtin_amdgcn_mfma_i32_16x16x64_i8(fb[s][b], fa[s][f], acc[f][b], 0, 0, 0);
                    // (Keeps the products' order; left alone, the compiler
                    // regroups the MFMAs.)
                    __builtin_amdgcn_sched_barrier(0);
                }
    }
    i32x4 sum = {0, 0, 0, 0};
#pragma unroll
    for (int f = 0; f < 8; f++)
#pragma unroll
        for (int b = 0; b < 4; b++)
            sum += acc[f][b];
    out[(int64_t)blockIdx.x * 512 + threadIdx.x] = sum;
}

} // namespace

void launch_mfma_ceiling(const int8_t *frags, int32_t *out, int workgroups, int iters,
                         hipStream_t st)
{
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3((unsigned)workgroups), dim3(512), 0, st,
                       reinterpret_cast<const i32x4 *>(frags), reinterpret_cast<i32x4 *>(out),
                       iters);
}

} // namespace qlin
