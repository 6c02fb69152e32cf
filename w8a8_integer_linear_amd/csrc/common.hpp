// Device helpers shared by the qlin kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlin {

constexpr int kWave = 64;

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight consecutive elements starting at element index 'idx' (a multiple of 8)
// of an fp32 or bf16 array, widened to fp32 (bf16 -> fp32 is exact).
template <bool BF16>
__device__ __forceinline__ void load8(const void *base, int64_t idx, float v[8])
{
    if constexpr (BF16) {
        i32x4 w = *reinterpret_cast<const i32x4 *>(static_cast<const uint16_t *>(base) + idx);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            v[2 * e] = bf16_lo((uint32_t)w[e]);
            v[2 * e + 1] = bf16_hi((uint32_t)w[e]);
        }
    } else {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + idx);
        f32x4 a = p[0], b = p[1];
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
        v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    }
}

__device__ __forceinline__ void store8(float *base, int64_t idx, const float v[8])
{
    f32x4 *p = reinterpret_cast<f32x4 *>(base + idx);
    p[0] = f32x4{v[0], v[1], v[2], v[3]};
    p[1] = f32x4{v[4], v[5], v[6], v[7]};
}

// Normalised Walsh-Hadamard transform of blocks of 'blk' elements, with each
// lane holding eight consecutive elements of the row and the lanes of a block
// consecutive within the wave (blk / 8 lanes, aligned).  Stages run in
// ascending stride: strides 1, 2, 4 inside the lane, strides 8 .. blk/2
// across lanes (partner lane = lane ^ (stride / 8)).  The lower element of a
// pair becomes lo + hi and the upper one lo - hi; the block is then scaled by
// cb.  Every lane of the wave must call this (cross-lane exchange).
__device__ __forceinline__ void fwht8_lanes(float v[8], int blk, float cb)
{
    const int lane = __lane_id();
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
        if (h < blk) {
#pragma unroll
            for (int i = 0; i < 8; i++) {
                if ((i & h) == 0) {
                    float lo = v[i], hi = v[i + h];
                    v[i] = lo + hi;
                    v[i + h] = lo - hi;
                }
            }
        }
    }
    for (int m = 1; m < blk / 8; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float other = __shfl_xor(v[i], m);
            v[i] = upper ? other - v[i] : v[i] + other;
        }
    }
#pragma unroll
    for (int i = 0; i < 8; i++)
        v[i] = v[i] * cb;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = v + __shfl_xor(v, o);
    return v;
}

// Max over the workgroup; every thread gets the result.  'red' holds one
// float per wave.  Contains barriers: call from uniform control flow.
template <int THREADS>
__device__ __forceinline__ float block_max(float v, float *red)
{
    constexpr int NW = THREADS / kWave;
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    if (__lane_id() == 0)
        red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < NW; i++)
        r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

// INT8 code of g for scale s (> 0, normal): rne(fl(g / s)), |code| <= 127.
// Fast path: t = fl(g * inv) with inv = fl(1 / s) is within 2^-15 of fl(g / s)
// for |g| <= 127.01 s, so rne(t) equals rne(fl(g / s)) unless t lies within
// 2^-14 of a half-integer; those rare elements take the exact quotient.  The
// quotient is at most 127 (1 + 2^-22) < 127.5 in magnitude, so no clamp is
// needed.  Returned as a float holding the integer.
__device__ __forceinline__ float quant_code(float g, float s, float inv)
{
    float t = g * inv;
    float r = __builtin_rintf(t);
    float d = __builtin_fabsf(t - r);
    if (!(d < 0.5f - 0x1p-14f))
        r = __builtin_rintf(g / s);
    return r;
}

// Exact slow path for a scale s that is subnormal (loses relative precision):
// rne(fl(g / s)) clamped to [-127, 127].
__device__ __forceinline__ float quant_code_exact(float g, float s)
{
    float r = __builtin_rintf(g / s);
    return fminf(fmaxf(r, -127.0f), 127.0f);
}

// Pack the low bytes of four integer-valued floats into one dword.
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d)
{
    uint32_t ia = (uint32_t)(int)a & 0xFFu, ib = (uint32_t)(int)b & 0xFFu;
    uint32_t ic = (uint32_t)(int)c & 0xFFu, id = (uint32_t)(int)d & 0xFFu;
    return ia | (ib << 8) | (ic << 16) | (id << 24);
}

} // namespace qlin
