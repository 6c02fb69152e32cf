// Device helpers shared by the qlin kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlin {

constexpr int kWave = 64;

// Word 3 of a buffer resource for raw (unformatted) 32-bit accesses.
constexpr int kRsrcWord3 = 0x00020000;

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight consecutive elements of an fp32 or bf16 array as loaded from memory
// (16 or 32 bytes), before widening.
template <bool BF16> struct Raw8;
template <> struct Raw8<true> {
    i32x4 w;
};
template <> struct Raw8<false> {
    f32x4 a, b;
};

// Raw load of the eight elements starting at element index 'idx' (a multiple
// of 8).
template <bool BF16>
__device__ __forceinline__ Raw8<BF16> load_raw8(const void *base, int64_t idx)
{
    Raw8<BF16> r;
    if constexpr (BF16) {
        r.w = *reinterpret_cast<const i32x4 *>(static_cast<const uint16_t *>(base) + idx);
    } else {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + idx);
        r.a = p[0];
        r.b = p[1];
    }
    return r;
}

// Widen to fp32 (bf16 -> fp32 is exact).
template <bool BF16>
__device__ __forceinline__ void unpack8(const Raw8<BF16> &r, float v[8])
{
    if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            v[2 * e] = bf16_lo((uint32_t)r.w[e]);
            v[2 * e + 1] = bf16_hi((uint32_t)r.w[e]);
        }
    } else {
        v[0] = r.a[0]; v[1] = r.a[1]; v[2] = r.a[2]; v[3] = r.a[3];
        v[4] = r.b[0]; v[5] = r.b[1]; v[6] = r.b[2]; v[7] = r.b[3];
    }
}

// Eight consecutive elements starting at element index 'idx' (a multiple of 8)
// of an fp32 or bf16 array, widened to fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void *base, int64_t idx, float v[8])
{
    unpack8<BF16>(load_raw8<BF16>(base, idx), v);
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

// Fixed-size rotation of blocks of BLK in {16, 32, 64, 128} elements, each
// held by BLK / 8 consecutive lanes of a 16-lane row (eight consecutive
// elements per lane).
//
// The cross-lane stages run on DPP lane permutes, which inside a row of 16
// lanes reach partner lane ^ 1 and ^ 2 (quad permutes), ^ 7 (half-row mirror)
// and ^ 8 (row rotation by 8) in one instruction, but not ^ 4.  So for
// BLK >= 64 the lane with row position l holds chunk p = l ^ (3 * bit2(l)) of
// its block (an involution on 0..15): the chunk at distance 4 then sits in
// lane l ^ 7, the one at distance 8 in lane l ^ 8.  had_chunk() maps a chunk
// index to the one its lane processes.
//
// Each stage pairs the lower chunk (bit k of p clear) with the upper one; the
// oracle's lower result is lo + hi and the upper lo - hi.  A lane keeps its
// values multiplied by a sign sigma (+1 or -1, the same for its eight values)
// and computes w' = w + c * w_partner with c = +1 on the lower and -1 on the
// upper lane: partner and own sigma agree (they differ only in bit k, not yet
// processed), so the lower lane gets sigma (lo + hi) and the upper lane
// sigma (hi - lo) = -sigma (lo - hi), i.e. sigma flips on upper lanes.  Each
// value is one correctly rounded sum of +-lo and +-hi (the product by c is
// exact), so with the sign undone (exactly, in the final scaling by
// sigma * cb) the result is bit-identical to lo + hi and lo - hi, except
// for the sign of an exact zero (x - x is +0 whatever sign is carried).
// That is immaterial to a quantizer (a zero of either sign gives code 0 and
// leaves the absmax unchanged).  Kernels that output the rotated floats use
// the exact form (EXACT): v = fma(c, v, partner), i.e. lo + hi on the lower
// lane and lo - hi on the upper one, with the partner read by a separate DPP
// move: two instructions per value and stage, and no sign to undo.
template <int BLK>
__device__ __forceinline__ int64_t had_chunk(int64_t c)
{
    if constexpr (BLK >= 64)
        return c ^ (((c >> 2) & 1) * 3);
    else
        return c;
}

// One stage for all eight values: v += c * v[partner lane], as v_fmac_f32
// with its first source read through DPP.  Written as one asm block because
// the compiler does not fold a DPP move into a multiply-accumulate.  The
// s_nop covers the two wait states a DPP read needs after a VALU write of
// the same register; inside the block each instruction writes only its own
// register.
#define QLIN_FWHT_DPP_STAGE(CTRL)                                                                \
    asm("s_nop 1\n\t"                                                                           \
        "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
        "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
        "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
        "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
        "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
        "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
        "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
        "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                           \
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),    \
          "+v"(v[7])                                                                             \
        : "v"(c))

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int BLK, int K, bool EXACT>
__device__ __forceinline__ void fwht_lane_stage(float v[8], int p)
{
    static_assert(K < 4 && (8 << K) < BLK, "stage outside the block");
    const float c = ((p >> K) & 1) ? -1.0f : 1.0f;
    if constexpr (EXACT) {
        constexpr int kCtrl = K == 0 ? 0xB1 : K == 1 ? 0x4E : K == 2 ? 0x141 : 0x128;
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = __builtin_fmaf(c, v[i], dpp_mov<kCtrl>(v[i]));
    } else if constexpr (K == 0) {
        QLIN_FWHT_DPP_STAGE("quad_perm:[1,0,3,2]");
    } else if constexpr (K == 1) {
        QLIN_FWHT_DPP_STAGE("quad_perm:[2,3,0,1]");
    } else if constexpr (K == 2) {
        QLIN_FWHT_DPP_STAGE("row_half_mirror");
    } else {
        QLIN_FWHT_DPP_STAGE("row_ror:8");
    }
}

template <int BLK, bool EXACT>
__device__ __forceinline__ void fwht8_fixed(float v[8], float cb)
{
    static_assert(BLK >= 16 && BLK <= 128 && (BLK & (BLK - 1)) == 0, "block size");
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if ((i & h) == 0) {
                const float lo = v[i], hi = v[i + h];
                v[i] = lo + hi;
                v[i + h] = lo - hi;
            }
        }
    }
    const int p = (int)had_chunk<BLK>(__lane_id() & 15) & (BLK / 8 - 1);
    fwht_lane_stage<BLK, 0, EXACT>(v, p);
    if constexpr (BLK > 16)
        fwht_lane_stage<BLK, 1, EXACT>(v, p);
    if constexpr (BLK > 32)
        fwht_lane_stage<BLK, 2, EXACT>(v, p);
    if constexpr (BLK > 64)
        fwht_lane_stage<BLK, 3, EXACT>(v, p);
    const float scale = (!EXACT && (__builtin_popcount(p) & 1)) ? -cb : cb;
#pragma unroll
    for (int i = 0; i < 8; i++)
        v[i] = v[i] * scale;
}

// 1 / s for a normal s whose reciprocal is normal, within half an ulp plus a
// relative 2^-46: the hardware reciprocal (within 1 ulp) refined by one Newton
// step, three instructions against about twelve for a correctly rounded
// division.
__device__ __forceinline__ float recip_refined(float s)
{
    const float r = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(r, __builtin_fmaf(-s, r, 1.0f), r);
}

// Fast path of an INT8 code rne(fl(g / s)) for |g| <= 127.01 s, with inv =
// fl(1 / s) or recip_refined(s) (either is within 2^-24 (1 + 2^-22) of 1 / s,
// relatively).  The exact product g * inv is then within 2^-17 of g / s, and
// fl(g / s) within 2^-17 of g / s, so they are less than 2^-16 apart.
// f = fma(g, inv, 1.5 * 2^23) rounds the exact product to the nearest
// integer r (ties to even) in one rounding, and leaves r as the low byte of
// f's bits; d = fma(g, inv, -r) is the exact product's distance from r within
// 2^-25.  If |d| < 1/2 - 2^-14, fl(g / s) is less than 1/2 from r, so r is its
// rounded value; otherwise the caller takes the exact quotient.  Returns f;
// folds |d| into dmax.
__device__ __forceinline__ float code_fast(float g, float inv, float &dmax)
{
    constexpr float kMagic = 0x1.8p23f;
    const float f = __builtin_fmaf(g, inv, kMagic);
    const float d = __builtin_fmaf(g, inv, -(f - kMagic));
    dmax = fmaxf(dmax, __builtin_fabsf(d));
    return f;
}

// Eight INT8 codes rne(fl(g / s)) packed into two dwords, for a scale s > 0
// that is a normal number and inv as code_fast takes it.  If any of the eight
// fails code_fast's check, all eight take the exact quotient.  The quotient
// is at most 127 (1 + 2^-22) < 127.5 in magnitude, so no clamp is needed.
__device__ __forceinline__ i32x2 quant8(const float g[8], float s, float inv)
{
    constexpr float kMagic = 0x1.8p23f;
    float f[8];
    float dmax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++)
        f[e] = code_fast(g[e], inv, dmax);
    if (!(dmax < 0.5f - 0x1p-14f)) {
#pragma unroll
        for (int e = 0; e < 8; e++)
            f[e] = __builtin_rintf(g[e] / s) + kMagic;
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
//
// The barriers wait only for the workgroup's LDS operations: __syncthreads()
// would also wait for every outstanding global load of the wave, draining
// loads issued ahead of time for the next piece of work.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int THREADS>
__device__ __forceinline__ float block_max(float v, float *red)
{
    constexpr int NW = THREADS / kWave;
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    if (__lane_id() == 0)
        red[w] = v;
    lds_barrier();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < NW; i++)
        r = fmaxf(r, red[i]);
    lds_barrier();
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
