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
        // Three-input exclusive or in one instruction (truth table 0x96).
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[1], k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[3], k1, 0x96);
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

// A row's requant scale s2 > 0 with inv = fl(1 / s2); 'fast' when s2 lies in
// [2^-40, 2^40], the range in which row_quotient is exact.
struct RowScale {
    float s, inv;
    bool fast;
};

__device__ __forceinline__ RowScale row_scale(float s2)
{
    return RowScale{s2, 1.0f / s2, s2 >= 0x1p-40f && s2 <= 0x1p40f};
}

// fl(w / s) from the row's reciprocal inv = fl(1 / s), without a division:
// q = fl(w inv), then twice q = fl(q + r inv) with the remainder r = w - q s
// (exact by FMA).  The first correction leaves q within half an ulp plus
// about 2^-45 relative of w / s, i.e. faithful; from a faithful q and a
// correctly rounded reciprocal, one more correction yields the correctly
// rounded quotient (Markstein's theorem, IBM J. Res. Dev. 34(1), 1990),
// provided nothing underflows.  With s in [2^-40, 2^40] that holds whenever
// the result is 0 or at least 2^-40 in magnitude; smaller quotients must be
// recomputed by division.
__device__ __forceinline__ float row_quotient(float w, float s, float inv)
{
    float q = w * inv;
    float r = __builtin_fmaf(-q, s, w);
    q = __builtin_fmaf(r, inv, q);
    r = __builtin_fmaf(-q, s, w);
    return __builtin_fmaf(r, inv, q);
}

// Stochastic codes of one 8-element chunk w[8] for the row scale rs.s > 0:
// one Philox block per 8 consecutive elements of the row-major weight,
// counter (blk, step), key (seed); element e takes 16-bit half (e & 1) of
// word e >> 1 as u = r * 2^-16, and q = floor(y) + (u < y - floor(y)),
// y = fl(w / rs.s), clamped to [-127, 127].  Clamping y to [-127, 127] first
// gives the same codes (a y beyond 127 in magnitude has codes at the clamp
// either way) and keeps every code within reach of the packing below: the
// floor plus 1.5 * 2^23 is exact, its low byte is the floor's two's
// complement byte, and adding the stochastic carry to the bit pattern adds
// it to that byte.
__device__ __forceinline__ i32x2 sr_codes8(const float w[8], const RowScale &rs, uint64_t blk,
                                           uint32_t seed_lo, uint32_t seed_hi, uint32_t step_lo,
                                           uint32_t step_hi)
{
    constexpr float kMagic = 0x1.8p23f;
    uint32_t x[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), step_lo, step_hi};
    philox4x32_10(x, seed_lo, seed_hi);
    float y[8];
    bool slow = !rs.fast;
    if (rs.fast) {
#pragma unroll
        for (int e = 0; e < 8; e++) {
            y[e] = row_quotient(w[e], rs.s, rs.inv);
            slow |= w[e] != 0.0f && __builtin_fabsf(y[e]) < 0x1p-40f;
        }
    }
    if (slow) {
#pragma unroll
        for (int e = 0; e < 8; e++)
            y[e] = w[e] / rs.s;
    }
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const uint32_t r16 = (x[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const float yc = fminf(fmaxf(y[e], -127.0f), 127.0f);
        const float f = floorf(yc);
        const float frac = yc - f;
        const float u = (float)r16 * 0x1p-16f;
        b[e] = __float_as_uint(f + kMagic) + (u < frac ? 1u : 0u);
    }
    auto pack = [&](int o) {
        const uint32_t lo = __builtin_amdgcn_perm(b[o + 1], b[o], 0x0C0C0400u);
        const uint32_t hi = __builtin_amdgcn_perm(b[o + 3], b[o + 2], 0x04000C0Cu);
        return (int)(lo | hi);
    };
    return i32x2{pack(0), pack(4)};
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
    const RowScale rs = row_scale(a / 127.0f);
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t c = t + (int64_t)j * THREADS;
        if (c >= nch)
            continue;
        // One Philox block per 8 consecutive elements: element index i = base +
        // 8c + e has i >> 3 = base / 8 + c and i & 7 = e (K is a multiple of
        // 16).
        const i32x2 o = a == 0.0f ? i32x2{0, 0}
                                  : sr_codes8(w[j], rs, (uint64_t)(base / 8 + c), seed_lo,
                                              seed_hi, step_lo, step_hi);
        *reinterpret_cast<i32x2 *>(qw + base + c * 8) = o;
    }
    if (t == 0) {
        sw[row] = rs.s;
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

// ------------------------------------------------ row weight normalization

// Sum over the workgroup (exact: integers).  Ends with a barrier.
template <int THREADS>
__device__ __forceinline__ int64_t block_sum_i64(int64_t v, int64_t *red)
{
    constexpr int NW = THREADS / kWave;
#pragma unroll
    for (int m = 1; m < kWave; m *= 2)
        v += __shfl_xor(v, m);
    if (__lane_id() == 0)
        red[threadIdx.x / kWave] = v;
    __syncthreads();
    int64_t r = 0;
#pragma unroll
    for (int i = 0; i < NW; i++)
        r += red[i];
    __syncthreads();
    return r;
}

// Pairwise sum of x[0 .. P) (P a power of two): adjacent pairs, level by level.
template <int P>
__device__ __forceinline__ double pairwise_tree(double (&x)[P])
{
#pragma unroll
    for (int len = P; len > 1; len /= 2)
#pragma unroll
        for (int i = 0; i < len / 2; i++)
            x[i] = x[2 * i] + x[2 * i + 1];
    return x[0];
}

constexpr int pow2_at_least(int n)
{
    int p = 1;
    while (p < n)
        p *= 2;
    return p;
}

// ||q|| of a row from the exact integer sum of its squared codes: square root
// in double, rounded once to fp32.
__device__ __forceinline__ float code_norm(int64_t n2)
{
    return (float)__builtin_sqrt((double)n2);
}

// Packed codes of chunk c of the row at q (zeros past the row end), and code
// e of a packed chunk.
__device__ __forceinline__ i32x2 load_codes8(const int8_t *q, int64_t nch, int64_t c)
{
    return c < nch ? *reinterpret_cast<const i32x2 *>(q + c * 8) : i32x2{0, 0};
}

__device__ __forceinline__ int code_at(i32x2 v, int e)
{
    return (int)(int8_t)((uint32_t)v[e / 4] >> (8 * (e % 4)));
}

// One SGD step of a weight-normalized row (one workgroup per row): the
// represented weight is g q / ||q||, the direction s q.  dot = <dW, q> is a
// pairwise double sum in element order: a lane's 8 elements, adjacent lanes
// (the butterfly pairs lane l with l ^ m, so each pair adds the same two
// values), adjacent waves, then adjacent passes, the positions past the row
// end being zeros (the same sums as zero-padding the row to a power of two).
// Then dg = fl(dot / ||q||), dv_k = fl(fl(g / fl(s ||q||)) * fl(dW_k -
// fl(fl(dg / ||q||) * q_k))), w_k = fl(fl(s q_k) - fl(lr dv_k)), the SGD
// requant of w, g' = fl(g - fl(lr dg)) and sw' = fl(g' / ||q'||) (0 for an
// all-zero row).  A row whose codes are all zero has zero gradients.
template <int THREADS, int J>
__global__ __launch_bounds__(THREADS) void wn_sgd_kernel(
    int8_t *__restrict__ q, float *__restrict__ s, float *__restrict__ g, float *__restrict__ sw,
    const float *__restrict__ dw, int64_t K, float lr, uint32_t seed_lo, uint32_t seed_hi,
    uint32_t step_lo, uint32_t step_hi, float *__restrict__ bias, const float *__restrict__ db)
{
    constexpr int NW = THREADS / kWave;
    constexpr int JP = pow2_at_least(J);
    __shared__ double part[JP][NW];
    __shared__ int64_t isum[NW];
    __shared__ float red[NW];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const int wv = t / kWave;
    const int64_t nch = K / 8;
    const int64_t base = row * K;
    const float sr = s[row], gr = g[row];
    i32x2 qv[J];
    float d[J][8];
    int n2 = 0;
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t c = t + (int64_t)j * THREADS;
        qv[j] = load_codes8(q + base, nch, c);
        if (c < nch) {
            load8<false>(dw, base + c * 8, d[j]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++)
                d[j][e] = 0.0f;
        }
        double pr[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int qe = code_at(qv[j], e);
            n2 += qe * qe;
            pr[e] = (double)d[j][e] * (double)qe;     // exact
        }
        double ps = pairwise_tree(pr);
#pragma unroll
        for (int m = 1; m < kWave; m *= 2)
            ps = ps + __shfl_xor(ps, m);
        if (__lane_id() == 0)
            part[j][wv] = ps;
    }
    if (__lane_id() == 0) {
#pragma unroll
        for (int j = J; j < JP; j++)
            part[j][wv] = 0.0;
    }
    // The barriers inside also order the partial sums before their reads and
    // every lane's reads of s, g before lane 0 overwrites them.
    const float nrm = code_norm(block_sum_i64<THREADS>(n2, isum));
    double pj[JP];
#pragma unroll
    for (int j = 0; j < JP; j++) {
        double pw[NW];
#pragma unroll
        for (int i = 0; i < NW; i++)
            pw[i] = part[j][i];
        pj[j] = pairwise_tree(pw);
    }
    const float dot = (float)pairwise_tree(pj);
    float dg = 0.0f, a = 0.0f, b = 0.0f;
    if (nrm != 0.0f) {
        dg = dot / nrm;
        a = gr / (sr * nrm);
        b = dg / nrm;
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < J; j++) {
        const bool ok = t + (int64_t)j * THREADS < nch;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float qf = (float)code_at(qv[j], e);
            const float dv = nrm != 0.0f ? a * (d[j][e] - b * qf) : 0.0f;
            const float cur = sr * qf;
            const float upd = lr * dv;
            d[j][e] = ok ? cur - upd : 0.0f;          // the updated direction
            amax = fmaxf(amax, __builtin_fabsf(d[j][e]));
        }
    }
    const float am = block_max<THREADS>(amax, red);
    const RowScale rs = row_scale(am / 127.0f);
    int m2 = 0;
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t c = t + (int64_t)j * THREADS;
        if (c >= nch)
            continue;
        const i32x2 o = am == 0.0f ? i32x2{0, 0}
                                   : sr_codes8(d[j], rs, (uint64_t)(base / 8 + c), seed_lo,
                                               seed_hi, step_lo, step_hi);
        *reinterpret_cast<i32x2 *>(q + base + c * 8) = o;
#pragma unroll
        for (int e = 0; e < 8; e++)
            m2 += code_at(o, e) * code_at(o, e);
    }
    const float nrm2 = code_norm(block_sum_i64<THREADS>(m2, isum));
    if (t == 0) {
        const float g2 = gr - lr * dg;
        s[row] = rs.s;
        g[row] = g2;
        sw[row] = nrm2 == 0.0f ? 0.0f : g2 / nrm2;
        if (bias && db)
            bias[row] = bias[row] - lr * db[row];
    }
}

// Preparation of a weight-normalized row: g = fl(s ||q||), sw = fl(g /
// ||q||); an all-zero direction gives g = sw = 0 (callers reject it).
template <int THREADS>
__global__ __launch_bounds__(THREADS) void wn_init_kernel(const int8_t *__restrict__ q,
                                                          const float *__restrict__ s, int64_t K,
                                                          float *__restrict__ g,
                                                          float *__restrict__ sw)
{
    __shared__ int64_t isum[THREADS / kWave];
    const int64_t row = blockIdx.x;
    const int64_t nch = K / 8;
    int64_t n2 = 0;
    for (int64_t c = threadIdx.x; c < nch; c += THREADS) {
        const i32x2 v = load_codes8(q + row * K, nch, c);
#pragma unroll
        for (int e = 0; e < 8; e++)
            n2 += code_at(v, e) * code_at(v, e);
    }
    const float nrm = code_norm(block_sum_i64<THREADS>(n2, isum));
    if (threadIdx.x == 0) {
        const float gr = nrm == 0.0f ? 0.0f : s[row] * nrm;
        g[row] = gr;
        sw[row] = nrm == 0.0f ? 0.0f : gr / nrm;
    }
}

template <int THREADS, int J>
void launch_wn_t(int8_t *q, float *s, float *g, float *sw, const float *dw, int64_t N, int64_t K,
                 float lr, uint64_t seed, uint64_t step, float *bias, const float *db,
                 hipStream_t st)
{
    hipLaunchKernelGGL((wn_sgd_kernel<THREADS, J>), dim3((unsigned)N), dim3(THREADS), 0, st, q, s,
                       g, sw, dw, K, lr, (uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)step,
                       (uint32_t)(step >> 32), bias, db);
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

void launch_wn_init(const int8_t *q, const float *s, int64_t N, int64_t K, float *g, float *sw,
                    hipStream_t st)
{
    hipLaunchKernelGGL(wn_init_kernel<256>, dim3((unsigned)N), dim3(256), 0, st, q, s, K, g, sw);
}

// 256 threads for rows of up to 16384 elements (8 per lane per pass), 1024
// threads up to 32768 (QLIN_WN_MAX_ROW): the row's codes and gradient stay in
// registers between the dot product and the update.
void launch_wn_sgd_requant(int8_t *q, float *s, float *g, float *sw, const float *dw, int64_t N,
                           int64_t K, float lr, uint64_t seed, uint64_t step, float *bias,
                           const float *db, hipStream_t st)
{
    const int64_t nch = K / 8;
    const int64_t j256 = (nch + 255) / 256;
#define QLIN_WN(T, J) return launch_wn_t<T, J>(q, s, g, sw, dw, N, K, lr, seed, step, bias, db, st)
    switch (j256) {
    case 1: QLIN_WN(256, 1);
    case 2: QLIN_WN(256, 2);
    case 3: QLIN_WN(256, 3);
    case 4: QLIN_WN(256, 4);
    case 5: QLIN_WN(256, 5);
    case 6: QLIN_WN(256, 6);
    case 7: QLIN_WN(256, 7);
    case 8: QLIN_WN(256, 8);
    default: break;
    }
    QLIN_WN(1024, 4);
#undef QLIN_WN
}

} // namespace qlin
