// Fused SGD and AdamW steps with stochastic requantization of each weight row
// (mini_trainer guide: updates stochastically requantize the represented
// weight; no floating master weight is retained; row kernels fuse the
// update; AdamW is among the covered update paths).  One workgroup per row;
// the updated row lives only in registers between the absmax reduction and
// the rounding.  AdamW reads and writes its fp32 moments in the same pass.
#include "common.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): per round, words 0 and
// 2 are multiplied by the round multipliers with full 64-bit products; the
// new counter is (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1,
// lo(M0*c0)); the key advances by the Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; r++) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        c[1] = (uint32_t)p1;
        c[3] = (uint32_t)p0;
        c[0] = n0;
        c[2] = n2;
    }
}

// AdamW state and step constants (computed on the host, each rounded once
// from double): a1 = 1 - b1, a2 = 1 - b2, c1 = lr / (1 - b1^t),
// c2 = 1 / sqrt(1 - b2^t), decay = 1 - lr * wd.
struct AdamParams {
    float *m, *v;          // [N, K] moments
    float *bm, *bv;        // [N] bias moments (with bias and db)
    float b1, b2, eps, a1, a2, c1, c2, decay;
};

// One AdamW element update: moments in place, returns the updated weight.
__device__ __forceinline__ float adamw_elem(const AdamParams &a, float w0, float g, float &m,
                                            float &v)
{
    m = a.b1 * m + a.a1 * g;
    v = a.b2 * v + (a.a2 * g) * g;
    const float d = __builtin_sqrtf(v) * a.c2 + a.eps;
    return w0 * a.decay - a.c1 * (m / d);
}

template <int THREADS, int J, bool ADAM>
__global__ __launch_bounds__(THREADS) void sgd_requant_kernel(
    int8_t *__restrict__ qw, float *__restrict__ sw, const float *__restrict__ dw, int64_t K,
    float lr, uint32_t seed_lo, uint32_t seed_hi, uint32_t step_lo, uint32_t step_hi,
    float *__restrict__ bias, const float *__restrict__ db, AdamParams ap)
{
    __shared__ float red[THREADS / kWave];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t nch = K / 8;
    const int64_t base = row * K;
    const float s = sw[row];
    float w[J][8];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t c = t + (int64_t)j * THREADS;
        if (c < nch) {
            const i32x2 qv = *reinterpret_cast<const i32x2 *>(qw + base + c * 8);
            float d[8], m[8], v[8];
            load8<false>(dw, base + c * 8, d);
            if constexpr (ADAM) {
                load8<false>(ap.m, base + c * 8, m);
                load8<false>(ap.v, base + c * 8, v);
            }
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int code = (int)(int8_t)((uint32_t)qv[e / 4] >> (8 * (e % 4)));
                const float cur = s * (float)code;
                if constexpr (ADAM) {
                    w[j][e] = adamw_elem(ap, cur, d[e], m[e], v[e]);
                } else {
                    const float upd = lr * d[e];
                    w[j][e] = cur - upd;
                }
                amax = fmaxf(amax, __builtin_fabsf(w[j][e]));
            }
            if constexpr (ADAM) {
                store8(ap.m, base + c * 8, m);
                store8(ap.v, base + c * 8, v);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++)
                w[j][e] = 0.0f;
        }
    }
    // block_max ends with a barrier, so every lane has read sw[row] before
    // lane 0 overwrites it below.
    const float a = block_max<THREADS>(amax, red);
    const float s2 = a / 127.0f;
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t c = t + (int64_t)j * THREADS;
        if (c >= nch)
            continue;
        float out[8];
        if (a == 0.0f) {
#pragma unroll
            for (int e = 0; e < 8; e++)
                out[e] = 0.0f;
        } else {
            // One Philox block per 8 consecutive elements: element index
            // i = base + 8c + e has i >> 3 = base / 8 + c and i & 7 = e
            // (K is a multiple of 16).
            const uint64_t blk = (uint64_t)(base / 8 + c);
            uint32_t x[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), step_lo, step_hi};
            philox4x32_10(x, seed_lo, seed_hi);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint32_t r16 = (x[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                const float y = w[j][e] / s2;
                const float f = floorf(y);
                const float frac = y - f;
                const float u = (float)r16 * 0x1p-16f;
                const float v = f + (u < frac ? 1.0f : 0.0f);
                out[e] = fminf(fmaxf(v, -127.0f), 127.0f);
            }
        }
        i32x2 o;
        o[0] = (int)pack4(out[0], out[1], out[2], out[3]);
        o[1] = (int)pack4(out[4], out[5], out[6], out[7]);
        *reinterpret_cast<i32x2 *>(qw + base + c * 8) = o;
    }
    if (t == 0) {
        sw[row] = s2;
        if constexpr (ADAM) {
            if (bias && db && ap.bm && ap.bv) {
                float m = ap.bm[row], v = ap.bv[row];
                bias[row] = adamw_elem(ap, bias[row], db[row], m, v);
                ap.bm[row] = m;
                ap.bv[row] = v;
            }
        } else if (bias && db) {
            bias[row] = bias[row] - lr * db[row];
        }
    }
}

template <int THREADS, int J, bool ADAM>
void launch_t(int8_t *qw, float *sw, const float *dw, int64_t N, int64_t K, float lr,
              uint64_t seed, uint64_t step, float *bias, const float *db, const AdamParams &ap,
              hipStream_t st)
{
    hipLaunchKernelGGL((sgd_requant_kernel<THREADS, J, ADAM>), dim3((unsigned)N), dim3(THREADS),
                       0, st, qw, sw, dw, K, lr, (uint32_t)seed, (uint32_t)(seed >> 32),
                       (uint32_t)step, (uint32_t)(step >> 32), bias, db, ap);
}

template <bool ADAM>
void launch_update(int8_t *qw, float *sw, const float *dw, int64_t N, int64_t K, float lr,
                   uint64_t seed, uint64_t step, float *bias, const float *db,
                   const AdamParams &ap, hipStream_t st)
{
    const int64_t nch = K / 8;
    const int64_t j256 = (nch + 255) / 256;
#define QLIN_LAUNCH(T, J) return launch_t<T, J, ADAM>(qw, sw, dw, N, K, lr, seed, step, bias, db, ap, st)
    switch (j256) {
    case 1: QLIN_LAUNCH(256, 1);
    case 2: QLIN_LAUNCH(256, 2);
    case 3: QLIN_LAUNCH(256, 3);
    case 4: QLIN_LAUNCH(256, 4);
    case 5: QLIN_LAUNCH(256, 5);
    case 6: QLIN_LAUNCH(256, 6);
    case 7: QLIN_LAUNCH(256, 7);
    case 8: QLIN_LAUNCH(256, 8);
    default: break;
    }
    const int64_t j1024 = (nch + 1023) / 1024;
    if (j1024 <= 4)
        QLIN_LAUNCH(1024, 4);
    if (j1024 <= 8)
        QLIN_LAUNCH(1024, 8);
    QLIN_LAUNCH(1024, 16);
#undef QLIN_LAUNCH
}

} // namespace

void launch_sgd_requant(int8_t *qw, float *sw, const float *dw, int64_t N, int64_t K, float lr,
                        uint64_t seed, uint64_t step, float *bias, const float *db,
                        hipStream_t st)
{
    launch_update<false>(qw, sw, dw, N, K, lr, seed, step, bias, db, AdamParams{}, st);
}

void launch_adamw_requant(int8_t *qw, float *sw, const float *dw, float *m, float *v, int64_t N,
                          int64_t K, const AdamConsts &k, uint64_t seed, uint64_t step,
                          float *bias, const float *db, float *bm, float *bv, hipStream_t st)
{
    AdamParams ap{m, v, bm, bv, k.b1, k.b2, k.eps, k.a1, k.a2, k.c1, k.c2, k.decay};
    launch_update<true>(qw, sw, dw, N, K, 0.0f, seed, step, bias, db, ap, st);
}

} // namespace qlin
