// C-ABI entry points of libqlin: argument validation, then kernel launches on
// the caller's stream.  Every check runs before the first launch, so a
// rejected call leaves all outputs untouched; the validation itself makes no
// HIP call.
#include <math.h>

#include <mutex>

#include "qlin.h"
#include "launch.hpp"

namespace {

constexpr int kAbiVersion = 1;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool dtype_ok(int dt) { return dt == QLIN_F32 || dt == QLIN_BF16; }
bool dim16(int64_t v) { return v >= 16 && v % 16 == 0; }
bool hadamard_block_ok(int64_t cols, int b)
{
    return b >= 2 && b <= QLIN_MAX_HAD_BLOCK && pow2(b) && cols % b == 0;
}

// Optional pointers: 16-byte aligned when present.
bool opt_aligned(const void *p) { return p == nullptr || aligned16(p); }

// An array argument: non-null and 16-byte aligned unless it holds no element.
bool array_ok(const void *p, bool nonempty) { return nonempty ? (p && aligned16(p)) : opt_aligned(p); }

// a * b (and a * b * c) for non-negative sizes, saturated at INT64_MAX: a
// size check on the result then rejects the arguments as it would the exact
// product, and no argument can make the arithmetic overflow.
int64_t sat_mul(int64_t a, int64_t b)
{
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}
int64_t sat_mul(int64_t a, int64_t b, int64_t c) { return sat_mul(sat_mul(a, b), c); }

// Whether byte ranges [a, a + na) and [b, b + nb) intersect (empty ranges and
// null pointers never do).  Compared as integer addresses, ends saturated at
// the top of the address space.
bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    if (!a || !b || na <= 0 || nb <= 0)
        return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    const uintptr_t xe = (uint64_t)na > UINTPTR_MAX - x ? UINTPTR_MAX : x + (uintptr_t)na;
    const uintptr_t ye = (uint64_t)nb > UINTPTR_MAX - y ? UINTPTR_MAX : y + (uintptr_t)nb;
    return x < ye && y < xe;
}

// Longest contraction qlin_product_ws accepts (chunked into int32-exact pieces).
constexpr int64_t kMaxLongContraction = ((int64_t)1 << 31) - 1;

// Largest token count a call accepts (grid dimensions and int32 tile indices).
constexpr int64_t kMaxRows = (int64_t)1 << 30;

int finish()
{
    return hipGetLastError() == hipSuccess ? QLIN_OK : QLIN_EDEVICE;
}

// fl32(1 / sqrt(b)), the rotation's normalisation.
float hadamard_scale(int b) { return (float)(1.0 / sqrt((double)b)); }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

} // namespace

extern "C" {

const char *qlin_status_string(int status)
{
    switch (status) {
    case QLIN_OK: return "ok";
    case QLIN_EINVAL: return "invalid argument";
    case QLIN_EUNSUPPORTED: return "unsupported shape";
    case QLIN_EDEVICE: return "device error";
    default: return "unknown status";
    }
}

int qlin_abi_version(void) { return kAbiVersion; }

int qlin_quantize_rows(const void *x, int dtype, int64_t rows, int64_t cols,
                       const float *prescale, int had_block, int8_t *q, float *s, void *stream)
{
    if (!dtype_ok(dtype) || rows < 0 || !dim16(cols))
        return QLIN_EINVAL;
    if (!array_ok(x, rows > 0) || !array_ok(q, rows > 0) || (rows > 0 && !s) ||
        !opt_aligned(prescale))
        return QLIN_EINVAL;
    if (had_block != 0 && !hadamard_block_ok(cols, had_block))
        return QLIN_EINVAL;
    if (cols > QLIN_MAX_ROW || rows > kMaxRows)
        return QLIN_EUNSUPPORTED;
    if (rows == 0)
        return QLIN_OK;
    qlin::launch_quantize_rows(x, dtype == QLIN_BF16, rows, cols, prescale, had_block,
                               had_block ? hadamard_scale(had_block) : 1.0f, q, s,
                               as_stream(stream));
    return finish();
}

int qlin_quantize_cols(const void *x, int dtype, int64_t rows, int64_t cols,
                       const float *prescale, int8_t *q, float *s, float *col_sum, void *stream)
{
    if (!s || !dtype_ok(dtype) || rows < 0 || !dim16(cols))
        return QLIN_EINVAL;
    if (!array_ok(x, rows > 0) || !array_ok(q, rows > 0) || !opt_aligned(prescale))
        return QLIN_EINVAL;
    if (col_sum == s || (x && ((const void *)s == x || (const void *)col_sum == x)))
        return QLIN_EINVAL;
    if (rows > 65535LL * 16)          // grid.y of the quantize pass stays below 65536
        return QLIN_EUNSUPPORTED;
    qlin::launch_quantize_cols(x, dtype == QLIN_BF16, rows, cols, prescale, q, s, col_sum,
                               as_stream(stream));
    return finish();
}

int qlin_quantize_grad(const void *dy, int dtype, int64_t rows, int64_t cols, const float *sw,
                       const float *sx, int8_t *q1, float *s1, int8_t *q2, float *s2,
                       float *col_sum, void *stream)
{
    if (!dtype_ok(dtype) || rows < 0 || !dim16(cols))
        return QLIN_EINVAL;
    const bool any = rows > 0;
    if (!array_ok(dy, any) || !array_ok(q1, any) || !array_ok(q2, any) || !array_ok(s1, any) ||
        !array_ok(sx, any) || !array_ok(sw, true) || !array_ok(s2, true) || !opt_aligned(col_sum))
        return QLIN_EINVAL;
    // q2 is written (as scratch, then codes) while everything else is read or
    // written, so it overlaps nothing; s2 and col_sum are accumulators.
    const int64_t eb = dtype == QLIN_BF16 ? 2 : 4;
    const int64_t nq = sat_mul(rows, cols), ndy = sat_mul(rows, cols, eb);
    const int64_t nr = sat_mul(rows, 4), nc = sat_mul(cols, 4), ncs = col_sum ? nc : 0;
    if (any && (overlap(q2, nq, dy, ndy) || overlap(q2, nq, q1, nq) || overlap(q2, nq, s1, nr) ||
                overlap(q2, nq, sx, nr) || overlap(q2, nq, sw, nc) || overlap(q2, nq, s2, nc) ||
                overlap(q2, nq, col_sum, ncs) || overlap(q1, nq, dy, ndy)))
        return QLIN_EINVAL;
    if (overlap(s2, nc, col_sum, ncs) ||
        (any && (overlap(s2, nc, dy, ndy) || overlap(col_sum, ncs, dy, ndy))))
        return QLIN_EINVAL;
    if (cols > QLIN_MAX_ROW || rows > 65535LL * 16)
        return QLIN_EUNSUPPORTED;
    qlin::launch_quantize_grad(dy, dtype == QLIN_BF16, rows, cols, sw, sx, q1, s1, q2, s2,
                               col_sum, as_stream(stream));
    return finish();
}

int qlin_dequantize_weight(const int8_t *qw, const float *sw, int64_t N, int64_t K,
                           int had_block, float *w, void *stream)
{
    if (N < 0 || !dim16(K))
        return QLIN_EINVAL;
    if (!array_ok(qw, N > 0) || !array_ok(sw, N > 0) || !array_ok(w, N > 0))
        return QLIN_EINVAL;
    if (had_block != 0 && !hadamard_block_ok(K, had_block))
        return QLIN_EINVAL;
    if (N > 0 && (overlap(w, sat_mul(N, K, 4), qw, sat_mul(N, K)) ||
                  overlap(w, sat_mul(N, K, 4), sw, sat_mul(N, 4))))
        return QLIN_EINVAL;
    if (sat_mul(N, K) / 8 / 256 >= ((int64_t)1 << 31))
        return QLIN_EUNSUPPORTED;
    if (N == 0)
        return QLIN_OK;
    qlin::launch_dequantize_weight(qw, sw, N, K, had_block,
                                   had_block ? hadamard_scale(had_block) : 1.0f, w,
                                   as_stream(stream));
    return finish();
}

int qlin_hadamard(const void *x, int dtype, int64_t rows, int64_t cols, int block, float *y,
                  void *stream)
{
    if (!dtype_ok(dtype) || rows < 0 || !dim16(cols) || !hadamard_block_ok(cols, block))
        return QLIN_EINVAL;
    if (!array_ok(x, rows > 0) || !array_ok(y, rows > 0))
        return QLIN_EINVAL;
    // y may alias x only for an in-place fp32 call.
    if (dtype == QLIN_BF16 && rows > 0 &&
        overlap(x, sat_mul(rows, cols, 2), y, sat_mul(rows, cols, 4)))
        return QLIN_EINVAL;
    if (rows > (int64_t)1 << 40 || sat_mul(rows, cols) / 8 / 256 >= ((int64_t)1 << 31))
        return QLIN_EUNSUPPORTED;
    if (rows == 0)
        return QLIN_OK;
    qlin::launch_hadamard(x, dtype == QLIN_BF16, rows, cols, block, hadamard_scale(block), y,
                          as_stream(stream));
    return finish();
}

// Shared checks of the three products: shapes, pointers, then the contraction
// bound.  'a_rows' / 'b_rows' tell whether the operands hold any element and
// 'out_rows' whether the output does.
static int check_product(int op, const void *a, const void *b, void *out, int64_t M, int64_t N,
                         int64_t K, int64_t max_contraction = QLIN_MAX_CONTRACTION)
{
    if (M < 0 || !dim16(N) || !dim16(K))
        return QLIN_EINVAL;
    const bool has_m = M > 0;
    // forward and dX outputs have M rows; the dW output [N, K] exists for any M.
    const bool out_nonempty = op == QLIN_OP_DW ? true : has_m;
    const bool b_nonempty = op == QLIN_OP_DW ? has_m : true;
    if (!array_ok(a, has_m) || !array_ok(b, b_nonempty && has_m) || !array_ok(out, out_nonempty))
        return QLIN_EINVAL;
    const int64_t contraction = op == QLIN_OP_FWD ? K : (op == QLIN_OP_DX ? N : M);
    if (contraction > max_contraction || M > kMaxRows || N > kMaxRows || K > kMaxRows)
        return QLIN_EUNSUPPORTED;
    // The output's 256 x 256 tiles are counted (and indexed) as int.
    const int64_t rows = op == QLIN_OP_DW ? N : M, cols = op == QLIN_OP_FWD ? N : K;
    if (((rows + 255) / 256) * ((cols + 255) / 256) >= ((int64_t)1 << 31))
        return QLIN_EUNSUPPORTED;
    if (!qlin::product_addressable(op, M, N, K))
        return QLIN_EUNSUPPORTED;
    return QLIN_OK;
}

int qlin_fwd(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
             const float *bias, int64_t M, int64_t N, int64_t K, float *y, void *stream)
{
    int st = check_product(QLIN_OP_FWD, qx, qw, y, M, N, K);
    if (st != QLIN_OK)
        return st;
    if (M == 0)
        return QLIN_OK;
    if (!sx || !sw)
        return QLIN_EINVAL;
    qlin::ProductArgs p{QLIN_OP_FWD, qx, qw, M, N, K, sx, sw, bias, y, false};
    qlin::launch_product(p, as_stream(stream));
    return finish();
}

int qlin_bwd_dx(const int8_t *qg1, const float *sg1, const int8_t *qw, int64_t M, int64_t N,
                int64_t K, int had_block, float *dx, void *stream)
{
    int st = check_product(QLIN_OP_DX, qg1, qw, dx, M, N, K);
    if (st != QLIN_OK)
        return st;
    if (had_block != 0 && !hadamard_block_ok(K, had_block))
        return QLIN_EINVAL;
    if (M == 0)
        return QLIN_OK;
    if (!sg1)
        return QLIN_EINVAL;
    qlin::ProductArgs p{QLIN_OP_DX, qg1, qw, M, N, K, sg1, nullptr, nullptr, dx, false};
    const hipStream_t s = as_stream(stream);
    if (had_block >= 2 && had_block <= 128) {
        p.had = had_block;
        p.had_scale = hadamard_scale(had_block);
        qlin::launch_product(p, s);
    } else {
        qlin::launch_product(p, s);
        if (had_block)
            qlin::launch_hadamard(dx, false, M, K, had_block, hadamard_scale(had_block), dx, s);
    }
    return finish();
}

int qlin_bwd_dw(const int8_t *qg2, const float *sg2, const int8_t *qx, int64_t M, int64_t N,
                int64_t K, float *dw, void *stream)
{
    int st = check_product(QLIN_OP_DW, qg2, qx, dw, M, N, K);
    if (st != QLIN_OK)
        return st;
    if (!sg2)
        return QLIN_EINVAL;
    // An empty token range still defines dW (all zero).
    qlin::ProductArgs p{QLIN_OP_DW, qg2, qx, M, N, K, sg2, nullptr, nullptr, dw, false};
    qlin::launch_product(p, as_stream(stream));
    return finish();
}

size_t qlin_product_ws_bytes(int op, int64_t M, int64_t N, int64_t K)
{
    if (op < QLIN_OP_FWD || op > QLIN_OP_DW || M < 0 || N < 0 || K < 0)
        return 0;
    if (M > kMaxRows || N > kMaxRows || K > kMaxRows)
        return 0;       // a shape the products do not support
    const int64_t contraction = op == QLIN_OP_FWD ? K : (op == QLIN_OP_DX ? N : M);
    if (contraction <= QLIN_MAX_CONTRACTION)
        return qlin::split_ws_bytes(qlin::split_plan(op, M, N, K));
    const int64_t rows = op == QLIN_OP_DW ? N : M, cols = op == QLIN_OP_FWD ? N : K;
    return qlin::kSplitCountBytes + 8 * (size_t)rows * (size_t)cols;     // < 2^63 + 4096
}

// Validation shared by qlin_product_ws and qlin_product_noalloc once a
// workspace is needed: the shapes and pointers of the product (any
// contraction up to kMaxLongContraction), the rotation block and the
// scales.  Returns QLIN_OK, an error, or -1 for an empty forward or dX
// product (nothing to do).
static int check_ws_product(int op, const int8_t *a, const float *srow, const int8_t *b,
                            const float *scol, int64_t M, int64_t N, int64_t K, int had_block,
                            float *out)
{
    int st = check_product(op, a, b, out, M, N, K, kMaxLongContraction);
    if (st != QLIN_OK)
        return st;
    if (had_block != 0 && !hadamard_block_ok(K, had_block))
        return QLIN_EINVAL;
    if (M == 0)
        return -1;      // forward and dX outputs are empty (dW has M > 0 here)
    if (!srow || (op == QLIN_OP_FWD && !scol))
        return QLIN_EINVAL;
    return QLIN_OK;
}

// Launches a validated product that uses 'workspace' (the arrival counters
// in its first kSplitCountBytes, then partial or int64 sums).
static int launch_ws_product(int op, const int8_t *a, const float *srow, const int8_t *b,
                             const float *scol, const float *bias, int64_t M, int64_t N,
                             int64_t K, int had_block, float *out, void *workspace, bool is_long,
                             hipStream_t s)
{
    qlin::ProductArgs p{op, a, b, M, N, K, srow, scol, bias, out, false};
    if (op == QLIN_OP_DX && had_block >= 2 && had_block <= 128) {
        p.had = had_block;
        p.had_scale = hadamard_scale(had_block);
    }
    if (is_long) {
        int64_t *ws = reinterpret_cast<int64_t *>(static_cast<char *>(workspace) +
                                                  qlin::kSplitCountBytes);
        qlin::launch_product_long(p, ws, s);
    } else {
        p.split_ws = workspace;
        qlin::launch_product(p, s);
    }
    if (op == QLIN_OP_DX && had_block > 128)
        qlin::launch_hadamard(out, false, M, K, had_block, hadamard_scale(had_block), out, s);
    return finish();
}

// The ordinary product call of 'op' (no workspace).
static int plain_product(int op, const int8_t *a, const float *srow, const int8_t *b,
                         const float *scol, const float *bias, int64_t M, int64_t N, int64_t K,
                         int had_block, float *out, void *stream)
{
    if (op == QLIN_OP_FWD)
        return qlin_fwd(a, srow, b, scol, bias, M, N, K, out, stream);
    if (op == QLIN_OP_DX)
        return qlin_bwd_dx(a, srow, b, M, N, K, had_block, out, stream);
    return qlin_bwd_dw(a, srow, b, M, N, K, out, stream);
}

int qlin_product_ws(int op, const int8_t *a, const float *srow, const int8_t *b,
                    const float *scol, const float *bias, int64_t M, int64_t N, int64_t K,
                    int had_block, float *out, void *workspace, size_t ws_bytes, void *stream)
{
    if (op < QLIN_OP_FWD || op > QLIN_OP_DW)
        return QLIN_EINVAL;
    if (op != QLIN_OP_FWD && (scol || bias))
        return QLIN_EINVAL;
    if (op != QLIN_OP_DX && had_block != 0)
        return QLIN_EINVAL;
    const int64_t contraction = op == QLIN_OP_FWD ? K : (op == QLIN_OP_DX ? N : M);
    const bool is_long = contraction > QLIN_MAX_CONTRACTION;
    const size_t need = qlin_product_ws_bytes(op, M, N, K);
    if (!is_long && need == 0)     // nothing to balance: the ordinary product
        return plain_product(op, a, srow, b, scol, bias, M, N, K, had_block, out, stream);
    int st = check_ws_product(op, a, srow, b, scol, M, N, K, had_block, out);
    if (st != QLIN_OK)
        return st < 0 ? QLIN_OK : st;
    const int64_t rows = op == QLIN_OP_DW ? N : M, cols = op == QLIN_OP_FWD ? N : K;
    const int64_t la = op == QLIN_OP_FWD ? sat_mul(M, K) : sat_mul(M, N);
    const int64_t lb = op == QLIN_OP_DW ? sat_mul(M, K) : sat_mul(N, K);
    const int64_t nb = need > (size_t)INT64_MAX ? INT64_MAX : (int64_t)need;
    if (!workspace || !aligned16(workspace) || ws_bytes < need ||
        overlap(workspace, nb, out, sat_mul(rows, cols, 4)) || overlap(workspace, nb, a, la) ||
        overlap(workspace, nb, b, lb))
        return QLIN_EINVAL;
    return launch_ws_product(op, a, srow, b, scol, bias, M, N, K, had_block, out, workspace,
                             is_long, as_stream(stream));
}

// ------------------------------------------------------------ no allocation

// Scratch of qlin_product_noalloc: arrival counters, then partial or int64
// sums, exactly as in a qlin_product_ws workspace.  Each device that loads
// the library holds its own copy until the process ends; every call on a
// device shares that device's copy.  Host code never passes the array's name
// to a kernel or a copy (on the host it is only a stand-in for the symbol):
// it takes the device address hipGetSymbolAddress gives for the current
// device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[QLIN_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

// Device address of 'scratch' on the current device, looked up (with that
// device current) on the first call on it.
static int scratch_on_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QLIN_EDEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return QLIN_EDEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return QLIN_OK;
}

int qlin_product_noalloc(int op, const int8_t *a, const float *srow, const int8_t *b,
                         const float *scol, const float *bias, int64_t M, int64_t N, int64_t K,
                         int had_block, float *out, void *stream)
{
    if (op < QLIN_OP_FWD || op > QLIN_OP_DW)
        return QLIN_EINVAL;
    if (op != QLIN_OP_FWD && (scol || bias))
        return QLIN_EINVAL;
    if (op != QLIN_OP_DX && had_block != 0)
        return QLIN_EINVAL;
    const int64_t contraction = op == QLIN_OP_FWD ? K : (op == QLIN_OP_DX ? N : M);
    const bool is_long = contraction > QLIN_MAX_CONTRACTION;
    const size_t need = qlin_product_ws_bytes(op, M, N, K);
    // Within the int32 bound the scratch only balances the last round of
    // tiles: with nothing to balance, or more pieces than the scratch holds,
    // the ordinary product gives the same bits.
    if (!is_long && (need == 0 || need > (size_t)QLIN_NOALLOC_SCRATCH_BYTES))
        return plain_product(op, a, srow, b, scol, bias, M, N, K, had_block, out, stream);
    int st = check_ws_product(op, a, srow, b, scol, M, N, K, had_block, out);
    if (st != QLIN_OK)
        return st < 0 ? QLIN_OK : st;
    if (need > (size_t)QLIN_NOALLOC_SCRATCH_BYTES)
        return QLIN_EUNSUPPORTED;     // int64 sums of a long contraction do not fit
    void *ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != QLIN_OK)
        return st;
    const hipStream_t s = as_stream(stream);
    if (!is_long) {
        // The arrival counters of this call's split tiles start at zero
        // whatever an earlier call left.
        qlin::launch_zero_words(ws, qlin::split_plan(op, M, N, K).tail, s);
    }
    return launch_ws_product(op, a, srow, b, scol, bias, M, N, K, had_block, out, ws, is_long, s);
}

int qlin_gemm_s32(int op, const int8_t *a, const int8_t *b, int64_t M, int64_t N, int64_t K,
                  int32_t *c, void *stream)
{
    if (op != QLIN_OP_FWD && op != QLIN_OP_DX && op != QLIN_OP_DW)
        return QLIN_EINVAL;
    int st = check_product(op, a, b, c, M, N, K);
    if (st != QLIN_OK)
        return st;
    if (M == 0 && op != QLIN_OP_DW)
        return QLIN_OK;
    qlin::ProductArgs p{op, a, b, M, N, K, nullptr, nullptr, nullptr, c, true};
    qlin::launch_product(p, as_stream(stream));
    return finish();
}

int qlin_stream_copy(const void *src, void *dst, int64_t nbytes, void *stream)
{
    if (nbytes < 0 || nbytes % 16 != 0 || !array_ok(src, nbytes > 0) || !array_ok(dst, nbytes > 0))
        return QLIN_EINVAL;
    if (overlap(src, nbytes, dst, nbytes))
        return QLIN_EINVAL;
    if (nbytes == 0)
        return QLIN_OK;
    qlin::launch_stream_copy(src, dst, nbytes, as_stream(stream));
    return finish();
}

int qlin_mfma_ceiling(const int8_t *frags, int32_t *out, int workgroups, int iters,
                      void *stream)
{
    static_assert(QLIN_MFMA_CEILING_FRAG_BYTES == qlin::kMfmaCeilingFrags * 1024,
                  "fragment buffer size");
    if (workgroups < 1 || workgroups > 65535 || iters < 1 || iters > (1 << 20))
        return QLIN_EINVAL;
    if (!array_ok(frags, true) || !array_ok(out, true))
        return QLIN_EINVAL;
    if (overlap(frags, QLIN_MFMA_CEILING_FRAG_BYTES, out, (int64_t)workgroups * 512 * 16))
        return QLIN_EINVAL;
    qlin::launch_mfma_ceiling(frags, out, workgroups, iters, as_stream(stream));
    return finish();
}

int qlin_sgd_requant(int8_t *qw, float *sw, const float *dw, int64_t N, int64_t K, float lr,
                     uint64_t seed, uint64_t step, float *bias, const float *db, void *stream)
{
    if (N < 0 || !dim16(K))
        return QLIN_EINVAL;
    if (!array_ok(qw, N > 0) || !array_ok(dw, N > 0) || (N > 0 && !sw))
        return QLIN_EINVAL;
    if ((bias == nullptr) != (db == nullptr))
        return QLIN_EINVAL;
    if (!isfinite(lr))
        return QLIN_EINVAL;
    if (K > QLIN_MAX_ROW || N > kMaxRows)
        return QLIN_EUNSUPPORTED;
    if (N == 0)
        return QLIN_OK;
    qlin::launch_sgd_requant(qw, sw, dw, N, K, lr, seed, step, bias, db, as_stream(stream));
    return finish();
}

int qlin_wn_init(const int8_t *q, const float *s, int64_t N, int64_t K, float *g, float *sw,
                 void *stream)
{
    if (N < 0 || !dim16(K))
        return QLIN_EINVAL;
    const bool any = N > 0;
    if (!array_ok(q, any) || (any && (!s || !g || !sw)))
        return QLIN_EINVAL;
    const int64_t n4 = sat_mul(N, 4);
    if (any && (overlap(g, n4, sw, n4) || overlap(g, n4, s, n4) || overlap(sw, n4, s, n4)))
        return QLIN_EINVAL;
    if (K > QLIN_WN_MAX_ROW || N > kMaxRows)
        return QLIN_EUNSUPPORTED;
    if (N == 0)
        return QLIN_OK;
    qlin::launch_wn_init(q, s, N, K, g, sw, as_stream(stream));
    return finish();
}

int qlin_wn_sgd_requant(int8_t *q, float *s, float *g, float *sw, const float *dw, int64_t N,
                        int64_t K, float lr, uint64_t seed, uint64_t step, float *bias,
                        const float *db, void *stream)
{
    if (N < 0 || !dim16(K))
        return QLIN_EINVAL;
    const bool any = N > 0;
    if (!array_ok(q, any) || !array_ok(dw, any) || (any && (!s || !g || !sw)))
        return QLIN_EINVAL;
    if ((bias == nullptr) != (db == nullptr))
        return QLIN_EINVAL;
    if (!isfinite(lr))
        return QLIN_EINVAL;
    const int64_t n4 = sat_mul(N, 4);
    if (any && (overlap(g, n4, sw, n4) || overlap(g, n4, s, n4) || overlap(sw, n4, s, n4)))
        return QLIN_EINVAL;
    if (K > QLIN_WN_MAX_ROW || N > kMaxRows)
        return QLIN_EUNSUPPORTED;
    if (N == 0)
        return QLIN_OK;
    qlin::launch_wn_sgd_requant(q, s, g, sw, dw, N, K, lr, seed, step, bias, db,
                                as_stream(stream));
    return finish();
}

int qlin_adamw_requant(int8_t *qw, float *sw, const float *dw, float *m, float *v, int64_t N,
                       int64_t K, float lr, float beta1, float beta2, float eps,
                       float weight_decay, uint64_t seed, uint64_t step, float *bias,
                       const float *db, float *bias_m, float *bias_v, void *stream)
{
    if (N < 0 || !dim16(K) || step < 1)
        return QLIN_EINVAL;
    const bool any = N > 0;
    if (!array_ok(qw, any) || !array_ok(dw, any) || !array_ok(m, any) || !array_ok(v, any) ||
        (any && !sw))
        return QLIN_EINVAL;
    const int nb = (bias != nullptr) + (db != nullptr) + (bias_m != nullptr) + (bias_v != nullptr);
    if (nb != 0 && nb != 4)
        return QLIN_EINVAL;
    if (!isfinite(lr) || !isfinite(eps) || !(eps > 0.0f) || !isfinite(weight_decay) ||
        !(weight_decay >= 0.0f) || !(beta1 >= 0.0f && beta1 < 1.0f) ||
        !(beta2 >= 0.0f && beta2 < 1.0f))
        return QLIN_EINVAL;
    const int64_t nf = sat_mul(N, K, 4);
    if (any && (overlap(m, nf, v, nf) || overlap(m, nf, dw, nf) || overlap(v, nf, dw, nf)))
        return QLIN_EINVAL;
    if (K > QLIN_MAX_ROW || N > kMaxRows)
        return QLIN_EUNSUPPORTED;
    if (N == 0)
        return QLIN_OK;
    // Step constants, each computed in double and rounded once.
    const double b1 = beta1, b2 = beta2, t = (double)step;
    qlin::AdamConsts k;
    k.b1 = beta1;
    k.b2 = beta2;
    k.eps = eps;
    k.a1 = (float)(1.0 - b1);
    k.a2 = (float)(1.0 - b2);
    k.c1 = (float)((double)lr / (1.0 - pow(b1, t)));
    k.c2 = (float)(1.0 / sqrt(1.0 - pow(b2, t)));
    k.decay = (float)(1.0 - (double)lr * (double)weight_decay);
    qlin::launch_adamw_requant(qw, sw, dw, m, v, N, K, k, seed, step, bias, db, bias_m, bias_v,
                               as_stream(stream));
    return finish();
}

} // extern "C"
