// Streaming device copy: the practical HBM ceiling the memory-bound kernels
// of the layer (quantizers, rotation, requant) are measured against.  Each
// lane moves U 16-byte pieces per iteration, all loads issued before any
// store, with consecutive lanes on consecutive pieces; the grid walks the
// buffer in strides of its own size.  Measured on 512 MiB copies (MI355X):
// one piece per lane with one workgroup per 256 pieces (no second
// iteration) moved 6.16 TB/s; 2, 4 or 8 pieces per lane on grids of 256 to
// 32768 workgroups moved 4.8 to 5.8 TB/s.
#include "common.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4 *__restrict__ src,
                                                          u32x4 *__restrict__ dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n16;
         base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; k++) {
            const int64_t i = base + (int64_t)k * 256;
            v[k] = i < n16 ? src[i] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < U; k++) {
            const int64_t i = base + (int64_t)k * 256;
            if (i < n16)
                dst[i] = v[k];
        }
    }
}

} // namespace

void launch_stream_copy(const void *src, void *dst, int64_t nbytes, hipStream_t st)
{
    // One 16-byte piece per lane; the grid covers the buffer once, up to
    // 2^22 workgroups (2^30 lanes: within the dispatch's 32-bit lane count),
    // and walks longer buffers in strides of that size.
    const int64_t n16 = nbytes / 16;
    int64_t grid = (n16 + 255) / 256;
    grid = grid < ((int64_t)1 << 22) ? grid : ((int64_t)1 << 22);
    hipLaunchKernelGGL(stream_copy_kernel<1>, dim3((unsigned)grid), dim3(256), 0, st,
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n16);
}

} // namespace qlin
