"""GPU parity: every C-ABI call against the CPU oracle on identical seeded inputs.

Integer outputs (codes, int32 accumulators, stochastically rounded weights)
and the fp32 outputs are compared bit for bit: both sides follow the same
operation order (IEEE binary32, no FMA contraction, round to nearest even),
so the 1e-5 relative bound of the contract is met with zero difference.  The
one exception is the column sum (bias gradient), whose fp32 order is
unspecified: it is held to 1e-5 of the sum of magnitudes.
"""
import numpy as np
import pytest

import workloads
from tests.gpu_util import announce, assert_bitwise, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    return torch_cuda()


@pytest.fixture(scope="module")
def Q():
    import w8a8_integer_linear_amd as q
    return q


def _x(rng, rows, cols, bf16, scale=1.0):
    x = (rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(scale)).astype(np.float32)
    return workloads.f32_to_bf16_bits(x) if bf16 else x


# --------------------------------------------------------------- quantizers

ROW_CASES = [
    # rows, cols, had, bf16, prescale
    (64, 256, 0, False, False),        # tiny workload's activations
    (17, 5376, 128, True, False),      # forward activations, rotated
    (1, 16, 0, True, False),
    (15, 48, 16, False, True),
    (16, 7168, 0, True, True),         # dY * s_w for dX
    (65, 2048, 512, False, False),     # largest block, one 256-thread pass
    (3, 2064, 2, True, True),          # ragged second pass
    (5, 14336, 128, False, False),     # MLP fc2 input width
    (2, 20480, 256, True, False),      # 1024-thread path
    (2, 131072, 64, False, True),      # longest row
    (4500, 5376, 128, True, True),     # more rows than workgroups: rows grid-strided
    (4200, 20480, 0, False, True),     # grid-strided 1024-thread path
    (33, 1088, 64, True, True),        # fixed 64-block rotation, ragged pass
    (9, 384, 128, False, True),        # one partial 256-thread pass, 3 blocks
    (2, 5376, 128, True, False),       # two rows, fewer than the workgroups
    (33, 2560, 0, False, True),        # second pass 25% full
    (64, 768, 128, True, True),        # one pass 37.5% full, 6 blocks
]


@pytest.mark.parametrize("rows,cols,had,bf16,pre", ROW_CASES)
def test_quantize_rows(T, Q, orc, rows, cols, had, bf16, pre):
    rng = np.random.default_rng(rows * 131 + cols)
    x = _x(rng, rows, cols, bf16)
    p = rng.uniform(0.25, 4.0, cols).astype(np.float32) if pre else None
    announce("quantize_rows", rows, cols, had, bf16, pre)
    q, s = Q.qlin_quantize_rows(dev(x), prescale=None if p is None else dev(p), had_block=had)
    T.cuda.synchronize()
    qr, sr = orc.quantize_rows(x, prescale=p, had_block=had)
    assert_bitwise(host(s), sr, "scales")
    assert_bitwise(host(q), qr, "codes")


def _random_row_cases(n=12, seed=7101):
    """Seeded random quantizer shapes: 1..3000 rows, 16..40960 columns (a
    multiple of 16, of the block when rotating), any rotation block, fp32 or
    bf16 input, with or without a prescale."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        rows = int(rng.integers(1, 3000)) if i % 4 else int(rng.integers(1, 40))
        had = [0, 0, 2, 16, 32, 64, 128, 256, 512][int(rng.integers(0, 9))]
        unit = max(16, had)
        cols = unit * int(rng.integers(1, max(2, 40960 // unit // (8 if i % 4 else 1))))
        cases.append((i, rows, cols, had, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("i,rows,cols,had,bf16,pre", _random_row_cases())
def test_quantize_rows_random(T, Q, orc, i, rows, cols, had, bf16, pre):
    rng = np.random.default_rng(500 + i)
    x = _x(rng, rows, cols, bf16, 10.0 ** rng.uniform(-3, 3))
    p = rng.uniform(0.25, 4.0, cols).astype(np.float32) if pre else None
    announce("quantize_rows random", i, rows, cols, had, bf16, pre)
    q, s = Q.qlin_quantize_rows(dev(x), prescale=None if p is None else dev(p), had_block=had)
    T.cuda.synchronize()
    qr, sr = orc.quantize_rows(x, prescale=p, had_block=had)
    assert_bitwise(host(s), sr, "scales")
    assert_bitwise(host(q), qr, "codes")


def test_quantize_rows_edge_values(T, Q, orc):
    """Zero rows, subnormal scales, huge values, exact ties."""
    rows, cols = 6, 64
    x = np.zeros((rows, cols), np.float32)
    x[1, :] = np.float32(1e-40)                      # subnormal amax
    x[1, 3] = np.float32(-3e-40)
    x[2, :] = np.linspace(-3e38, 3e38, cols, dtype=np.float32)
    x[3, :8] = np.array([127, 0.5, 1.5, 2.5, -0.5, -2.5, 126.5, -126.5], np.float32) * 2.0 ** -6
    rng = np.random.default_rng(0)
    x[4] = rng.standard_normal(cols).astype(np.float32)
    x[5] = np.float32(7.0)
    announce("quantize_rows edge values")
    q, s = Q.qlin_quantize_rows(dev(x))
    T.cuda.synchronize()
    qr, sr = orc.quantize_rows(x)
    assert_bitwise(host(s), sr, "scales")
    assert_bitwise(host(q), qr, "codes")


COL_CASES = [(64, 128, False, True), (17, 48, True, True), (1, 16, False, False),
             (300, 7168, True, True), (12000, 272, True, True), (0, 32, True, True)]


@pytest.mark.parametrize("rows,cols,bf16,pre", COL_CASES)
def test_quantize_cols(T, Q, orc, rows, cols, bf16, pre):
    rng = np.random.default_rng(rows + 7 * cols)
    x = _x(rng, rows, cols, bf16, 0.01)
    p = rng.uniform(1e-3, 1e-1, rows).astype(np.float32) if pre else None
    announce("quantize_cols", rows, cols, bf16, pre)
    q, s, cs = Q.qlin_quantize_cols(dev(x), prescale=None if p is None else dev(p), want_sum=True)
    T.cuda.synchronize()
    qr, sr, csr = orc.quantize_cols(x, prescale=p, want_sum=True)
    assert_bitwise(host(s), sr, "scales")
    assert_bitwise(host(q), qr, "codes")
    xf = workloads.bf16_bits_to_f32(x) if bf16 else x
    bound = 1e-5 * np.abs(xf.astype(np.float64)).sum(axis=0) + 1e-30
    assert np.all(np.abs(host(cs).astype(np.float64) - csr) <= bound)


GRAD_CASES = [
    # rows, cols, bf16: the two-read path (rows >= 16) and the separate passes
    (600, 4096, True),
    (513, 7168, True),         # dY of the headline layer's width
    (1000, 8192, False),       # fp32 gradient
    (777, 4112, True),         # ragged last 512-column window and row batch
    (700, 8208, True),
    (600, 14336, False),       # the MLP's fc1 gradient width, fp32
    (520, 16400, True),        # more windows than the waves' budget fills
    (100, 256, False),         # one window, half of it past the last column
    (16, 1040, True),          # fewest rows of the two-read path: one row group
    (20, 131072, True),        # longest row: 256 windows
    (40, 131056, False),       # longest ragged row
    (15, 4096, True),          # too few rows: separate passes
    (1, 272, False),
]


@pytest.mark.parametrize("rows,cols,bf16", GRAD_CASES)
def test_quantize_grad(T, Q, orc, rows, cols, bf16):
    rng = np.random.default_rng(rows * 7 + cols)
    x = _x(rng, rows, cols, bf16, scale=0.01)
    xf = workloads.bf16_bits_to_f32(x) if bf16 else x
    if rows > 3:
        x[2] = 0                                  # an all-zero row
    x[:, 5] = 0                                   # and an all-zero column
    sw = rng.uniform(1e-3, 1e-2, cols).astype(np.float32)
    sx = rng.uniform(1e-3, 1e-1, rows).astype(np.float32)
    announce("quantize_grad", rows, cols, bf16)
    q1, s1, q2, s2, db = Q.qlin_quantize_grad(dev(x), dev(sw), dev(sx), want_sum=True)
    T.cuda.synchronize()
    q1r, s1r = orc.quantize_rows(x, prescale=sw)
    assert_bitwise(host(s1), s1r, "row scales")
    assert_bitwise(host(q1), q1r, "row codes")
    q2r, s2r, dbr = orc.quantize_cols(x, prescale=sx, want_sum=True)
    assert_bitwise(host(s2), s2r, "column scales")
    assert_bitwise(host(q2), q2r, "column codes")
    xf = workloads.bf16_bits_to_f32(x) if bf16 else x
    bound = 1e-5 * np.abs(xf.astype(np.float64)).sum(axis=0) + 1e-30
    assert np.all(np.abs(host(db).astype(np.float64) - dbr) <= bound)


def _random_grad_cases(n=8, seed=7303):
    """Seeded random dY shapes for both quantizations: mostly the two-read
    path (>= 16 rows), some of the separate passes."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        rows = int(rng.integers(16, 5000)) if i % 4 else int(rng.integers(1, 16))
        cols = 16 * int(rng.integers(1, 513 if i % 3 else 1024))
        cases.append((i, rows, cols, bool(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("i,rows,cols,bf16", _random_grad_cases())
def test_quantize_grad_random(T, Q, orc, i, rows, cols, bf16):
    rng = np.random.default_rng(1300 + i)
    x = _x(rng, rows, cols, bf16, scale=10.0 ** rng.uniform(-4, 1))
    sw = rng.uniform(1e-3, 1e-2, cols).astype(np.float32)
    sx = rng.uniform(1e-3, 1e-1, rows).astype(np.float32)
    announce("quantize_grad random", i, rows, cols, bf16)
    q1, s1, q2, s2, db = Q.qlin_quantize_grad(dev(x), dev(sw), dev(sx), want_sum=True)
    T.cuda.synchronize()
    q1r, s1r = orc.quantize_rows(x, prescale=sw)
    assert_bitwise(host(s1), s1r, "row scales")
    assert_bitwise(host(q1), q1r, "row codes")
    q2r, s2r, dbr = orc.quantize_cols(x, prescale=sx, want_sum=True)
    assert_bitwise(host(s2), s2r, "column scales")
    assert_bitwise(host(q2), q2r, "column codes")
    xf = workloads.bf16_bits_to_f32(x) if bf16 else x
    bound = 1e-5 * np.abs(xf.astype(np.float64)).sum(axis=0) + 1e-30
    assert np.all(np.abs(host(db).astype(np.float64) - dbr) <= bound)


def test_quantize_grad_random_sweep(T, Q, orc):
    """A wider seeded sweep of both dY quantizations in one test: 48 random
    shapes (16..4000 rows, up to 8192 columns, both dtypes, magnitudes over
    five decades), codes and scales bit for bit, db within its bound."""
    rng0 = np.random.default_rng(7404)
    for i in range(48):
        rows = int(rng0.integers(16, 4000))
        cols = 16 * int(rng0.integers(1, 513))
        bf16 = bool(i % 2)
        rng = np.random.default_rng(2300 + i)
        x = _x(rng, rows, cols, bf16, scale=10.0 ** rng.uniform(-4, 1))
        sw = rng.uniform(1e-3, 1e-2, cols).astype(np.float32)
        sx = rng.uniform(1e-3, 1e-1, rows).astype(np.float32)
        announce("quantize_grad sweep", i, rows, cols, bf16)
        q1, s1, q2, s2, db = Q.qlin_quantize_grad(dev(x), dev(sw), dev(sx), want_sum=True)
        T.cuda.synchronize()
        what = f"(case {i}: {rows} x {cols}, bf16 {bf16})"
        q1r, s1r = orc.quantize_rows(x, prescale=sw)
        assert_bitwise(host(s1), s1r, "row scales " + what)
        assert_bitwise(host(q1), q1r, "row codes " + what)
        q2r, s2r, dbr = orc.quantize_cols(x, prescale=sx, want_sum=True)
        assert_bitwise(host(s2), s2r, "column scales " + what)
        assert_bitwise(host(q2), q2r, "column codes " + what)
        xf = workloads.bf16_bits_to_f32(x) if bf16 else x
        bound = 1e-5 * np.abs(xf.astype(np.float64)).sum(axis=0) + 1e-30
        assert np.all(np.abs(host(db).astype(np.float64) - dbr) <= bound), "db " + what


def _fragment_matrix(frag):
    """A 1 KiB MFMA fragment (lane l's 16 bytes at 16 l) as the 16 x 64 block
    it carries: lane 16 g + r holds row r, contraction bytes 16 g .. 16 g + 15."""
    f = frag.reshape(4, 16, 16)                       # [g, r, j]
    return f.transpose(1, 0, 2).reshape(16, 64).astype(np.int64)


@pytest.mark.parametrize("iters", [1, 3])
def test_mfma_ceiling(T, Q, iters):
    """The matrix-core ceiling kernel does the products' MFMA work: every lane's
    sums against plain int64 matrix products of its wave's fragments."""
    rng = np.random.default_rng(31)
    frags = rng.integers(-128, 128, Q.MFMA_CEILING_FRAG_BYTES, dtype=np.int64).astype(np.int8)
    wg = 2
    announce("mfma ceiling", iters)
    out = T.zeros(wg * 512 * 4, dtype=T.int32, device="cuda")
    Q.qlin_mfma_ceiling(dev(frags), out, wg, iters)
    T.cuda.synchronize()
    got = host(out).reshape(wg, 8, 64, 4)
    fr = frags.reshape(24, 1024)
    lane = np.arange(64)
    for w in range(8):
        s = np.zeros((16, 16), np.int64)              # block sums [A row, B row]
        for st in range(2):
            for f in range(8):
                a = _fragment_matrix(fr[(w + 8 * st + f) % 24])
                for b in range(4):
                    bm = _fragment_matrix(fr[(w + 16 + 4 * st + b) % 24])
                    s += a @ bm.T
        # Lane l, register e holds row l % 16, column 4 (l // 16) + e.
        want = np.stack([s[lane % 16, 4 * (lane // 16) + e] for e in range(4)], axis=1) * iters
        want = want.astype(np.int64).astype(np.int32)
        for g in range(wg):
            assert np.array_equal(got[g, w], want), (g, w)


def test_quantize_grad_tiny_scales(T, Q, orc):
    """Zero, subnormal and normal row and column scales in one call: the code
    pass's exact quotients for subnormal scales, fast path elsewhere."""
    rows, cols = 64, 1024
    rng = np.random.default_rng(77)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    x[:32] *= np.float32(1e-36)                   # rows whose scales are subnormal
    x[:, :128] *= np.float32(1e-36)               # columns whose scales are subnormal
    x[40] = 0                                     # a zero row scale
    x[:, 200] = 0                                 # a zero column scale
    sw = rng.uniform(1e-3, 1e-2, cols).astype(np.float32)
    sx = rng.uniform(1e-3, 1e-1, rows).astype(np.float32)
    announce("quantize_grad tiny scales", rows, cols)
    q1, s1, q2, s2, db = Q.qlin_quantize_grad(dev(x), dev(sw), dev(sx), want_sum=True)
    T.cuda.synchronize()
    q1r, s1r = orc.quantize_rows(x, prescale=sw)
    q2r, s2r, _ = orc.quantize_cols(x, prescale=sx, want_sum=True)
    assert np.any((s1r > 0) & (s1r < np.float32(2.0 ** -126)))
    assert np.any((s2r > 0) & (s2r < np.float32(2.0 ** -126)))
    assert_bitwise(host(s1), s1r, "row scales")
    assert_bitwise(host(q1), q1r, "row codes")
    assert_bitwise(host(s2), s2r, "column scales")
    assert_bitwise(host(q2), q2r, "column codes")


def test_quantize_grad_no_tokens(T, Q, orc):
    cols = 64
    announce("quantize_grad rows=0")
    s2 = dev(np.full(cols, 7.0, np.float32))
    db = dev(np.full(cols, 7.0, np.float32))
    Q.qlin_quantize_grad(dev(np.zeros((0, cols), np.float32)), dev(np.ones(cols, np.float32)),
                         dev(np.ones(0, np.float32)), s2=s2, col_sum=db)
    T.cuda.synchronize()
    assert np.all(host(s2) == 0) and np.all(host(db) == 0)


@pytest.mark.parametrize("rows,cols,blk,bf16", [(3, 256, 128, False), (64, 5376, 128, False),
                                                (5, 1024, 512, True), (7, 64, 2, False),
                                                (9, 96, 32, True), (1, 16, 8, False),
                                                (4, 384, 64, True), (6, 160, 16, False),
                                                (2, 48, 16, True), (5, 4096, 128, True),
                                                (64, 1024, 128, False), (32, 512, 64, False),
                                                (16, 256, 16, False)])
def test_hadamard(T, Q, orc, rows, cols, blk, bf16):
    rng = np.random.default_rng(blk + rows)
    x = _x(rng, rows, cols, bf16)
    if cols in (1024, 512, 256) and not bf16:
        # small integers (and some -0.0): exact cancellations, signed zeros
        x = rng.integers(-3, 4, (rows, cols)).astype(np.float32)
        x[0, ::7] = np.float32(-0.0)
        x[1, :blk] = np.float32(-0.0)            # a block of -0.0: the oracle keeps some -0.0
    announce("hadamard", rows, cols, blk, bf16)
    xd = dev(x)
    if bf16:
        y = Q.qlin_hadamard(xd, blk)
    else:
        y = Q.qlin_hadamard(xd, blk, y=xd)          # in place
    T.cuda.synchronize()
    assert_bitwise(host(y), orc.hadamard(x, blk), "rotation")


@pytest.mark.parametrize("N,K,had", [(128, 256, 0), (64, 5376, 128), (7, 1024, 512),
                                     (9, 96, 32), (33, 1088, 64), (5, 48, 16), (3, 64, 2),
                                     (2, 4096, 256), (7168, 5376, 128)])
def test_dequantize_weight(T, Q, orc, N, K, had):
    rng = np.random.default_rng(N + K + had)
    q = _codes(rng, (N, K))
    s = rng.uniform(1e-4, 1e-1, N).astype(np.float32)
    announce("dequantize_weight", N, K, had)
    w = Q.qlin_dequantize_weight(dev(q), dev(s), had_block=had)
    T.cuda.synchronize()
    assert_bitwise(host(w), orc.dequantize_weight(q, s, had_block=had), "weight")


# ----------------------------------------------------------------- products

PRODUCT_SHAPES = [
    (64, 128, 256),      # tiny workload
    (1, 16, 16), (15, 48, 32), (16, 64, 80), (17, 48, 32),   # around the row floor
    (130, 272, 208),     # ragged tiles in every dimension
    (257, 144, 5376),    # long contraction
    (33, 4096, 64),      # many output columns
    (128, 384, 384),     # contractions of 1 and 3 full stages (the stage loop runs in pairs)
    (300, 400, 400),     # ragged last stages: 4 stages (fwd, dX) and 3 (dW)
]


def _codes(rng, shape):
    return rng.integers(-127, 128, size=shape).astype(np.int8)


@pytest.mark.parametrize("M,N,K", PRODUCT_SHAPES)
def test_gemm_s32(T, Q, orc, M, N, K):
    rng = np.random.default_rng(M + N + K)
    qx, qw, qg = _codes(rng, (M, K)), _codes(rng, (N, K)), _codes(rng, (M, N))
    for op, a, b in ((Q.QLIN_OP_FWD, qx, qw), (Q.QLIN_OP_DX, qg, qw), (Q.QLIN_OP_DW, qg, qx)):
        announce("gemm_s32", op, M, N, K)
        c = Q.qlin_gemm_s32(op, dev(a), dev(b), M, N, K)
        T.cuda.synchronize()
        assert_bitwise(host(c), orc.gemm_s32(op, a, b, M, N, K), f"acc op{op}")


def test_gemm_s32_extremes(T, Q, orc):
    """All +-127 codes at the longest contractions the test can afford."""
    M, N, K = 32, 32, 16384
    a = np.full((M, K), 127, np.int8)
    b = np.full((N, K), -127, np.int8)
    a[1] = -127
    announce("gemm_s32 extremes")
    c = Q.qlin_gemm_s32(Q.QLIN_OP_FWD, dev(a), dev(b), M, N, K)
    T.cuda.synchronize()
    assert_bitwise(host(c), orc.gemm_s32(0, a, b, M, N, K), "acc")


@pytest.mark.parametrize("op", [0, 1, 2])
def test_gemm_s32_longest_contraction(T, Q, orc, op):
    """All +-127 codes at the longest contraction the ABI accepts for each
    product (131,056 for the 16-aligned forward and dX contractions, 131,071
    tokens for dW), where |acc| reaches 131,071 * 127^2 = 2,114,044,159, just
    under 2^31."""
    L = 131071 if op == 2 else 131056
    if op == 0:
        M, N, K = 32, 48, L
        a, b = np.full((M, K), 127, np.int8), np.full((N, K), 127, np.int8)
    elif op == 1:
        M, N, K = 32, L, 48
        a, b = np.full((M, N), 127, np.int8), np.full((N, K), 127, np.int8)
    else:
        M, N, K = L, 32, 48
        a, b = np.full((M, N), 127, np.int8), np.full((M, K), 127, np.int8)
    if op == 2:
        a[:, 1] = -127      # output row 1 at the negative extreme
    else:
        a[1] = -127
    b[0, :8] = -1           # a few small codes so outputs differ
    announce("gemm_s32 longest contraction", op, M, N, K)
    c = Q.qlin_gemm_s32(op, dev(a), dev(b), M, N, K)
    T.cuda.synchronize()
    ref = orc.gemm_s32(op, a, b, M, N, K)
    assert np.abs(ref.astype(np.int64)).max() >= 2_000_000_000
    assert_bitwise(host(c), ref, "acc")


@pytest.mark.parametrize("M,N,K", PRODUCT_SHAPES)
@pytest.mark.parametrize("with_bias", [True, False])
def test_products_dequant(T, Q, orc, M, N, K, with_bias):
    rng = np.random.default_rng(3 * M + N)
    qx, qw, qg = _codes(rng, (M, K)), _codes(rng, (N, K)), _codes(rng, (M, N))
    sx = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    sg1 = rng.uniform(1e-6, 1e-4, M).astype(np.float32)
    sg2 = rng.uniform(1e-6, 1e-4, N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32) * np.float32(0.01) if with_bias else None
    announce("fwd", M, N, K, with_bias)
    y = Q.qlin_fwd(dev(qx), dev(sx), dev(qw), dev(sw), None if b is None else dev(b))
    T.cuda.synchronize()
    assert_bitwise(host(y), orc.fwd(qx, sx, qw, sw, b), "y")
    if with_bias:
        return
    announce("bwd_dx", M, N, K)
    dx = Q.qlin_bwd_dx(dev(qg), dev(sg1), dev(qw))
    T.cuda.synchronize()
    assert_bitwise(host(dx), orc.bwd_dx(qg, sg1, qw), "dx")
    announce("bwd_dw", M, N, K)
    dw = Q.qlin_bwd_dw(dev(qg), dev(sg2), dev(qx))
    T.cuda.synchronize()
    assert_bitwise(host(dw), orc.bwd_dw(qg, sg2, qx), "dw")


def _random_skinny_cases(n=8, seed=7202):
    """Seeded random shapes for the weight-streaming forward: 1..16 tokens,
    up to 8192 output features (grids past one workgroup per compute unit take
    the 1024-byte chunks), contractions of 16..12288."""
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 17)), 16 * int(rng.integers(1, 513)),
             16 * int(rng.integers(1, 769)), bool(rng.integers(0, 2))) for i in range(n)]


@pytest.mark.parametrize("i,M,N,K,with_bias", _random_skinny_cases())
def test_skinny_forward_random(T, Q, orc, i, M, N, K, with_bias):
    rng = np.random.default_rng(900 + i)
    qx, qw = _codes(rng, (M, K)), _codes(rng, (N, K))
    sx = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    announce("skinny random", i, M, N, K, with_bias)
    c = Q.qlin_gemm_s32(Q.QLIN_OP_FWD, dev(qx), dev(qw), M, N, K)
    y = Q.qlin_fwd(dev(qx), dev(sx), dev(qw), dev(sw), None if bias is None else dev(bias))
    T.cuda.synchronize()
    assert_bitwise(host(c), orc.gemm_s32(0, qx, qw, M, N, K), "acc")
    assert_bitwise(host(y), orc.fwd(qx, sx, qw, sw, bias), "y")


@pytest.mark.parametrize("M,N,K", [(2, 48, 4112), (16, 32, 8192), (1, 16, 12352), (7, 64, 16)])
def test_skinny_forward_chunks(T, Q, orc, M, N, K):
    """The weight-streaming kernel walks the contraction in chunks of 4096
    bytes: several chunks, a ragged last one, a one-step contraction."""
    rng = np.random.default_rng(M * 7 + K)
    qx, qw = _codes(rng, (M, K)), _codes(rng, (N, K))
    sx = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    announce("skinny chunks", M, N, K)
    c = Q.qlin_gemm_s32(Q.QLIN_OP_FWD, dev(qx), dev(qw), M, N, K)
    y = Q.qlin_fwd(dev(qx), dev(sx), dev(qw), dev(sw), dev(bias))
    T.cuda.synchronize()
    assert_bitwise(host(c), orc.gemm_s32(0, qx, qw, M, N, K), "acc")
    assert_bitwise(host(y), orc.fwd(qx, sx, qw, sw, bias), "y")


@pytest.mark.parametrize("M", [1, 4, 15, 16])
def test_skinny_forward(T, Q, orc, M):
    """M <= 16 takes the weight-streaming kernel (skinny workload: 4096 -> 4096)."""
    d = workloads.skinny(M, K=4096, N=4096)
    qw, sw = orc.prepare_weight(d["w"])
    qx, sx = orc.quantize_rows(d["x"])
    announce("skinny fwd", M)
    y = Q.qlin_fwd(dev(qx), dev(sx), dev(qw), dev(sw))
    c = Q.qlin_gemm_s32(Q.QLIN_OP_FWD, dev(qx), dev(qw), M, 4096, 4096)
    T.cuda.synchronize()
    assert_bitwise(host(c), orc.gemm_s32(0, qx, qw, M, 4096, 4096), "acc")
    assert_bitwise(host(y), orc.fwd(qx, sx, qw, sw), "y")
    bias = np.linspace(-1, 1, 4096, dtype=np.float32)
    y2 = Q.qlin_fwd(dev(qx), dev(sx), dev(qw), dev(sw), dev(bias))
    T.cuda.synchronize()
    assert_bitwise(host(y2), orc.fwd(qx, sx, qw, sw, bias), "y+bias")


def _random_product_cases(n=10, seed=20261203):
    """Seeded random shapes: any token count, feature counts multiples of 16,
    contractions long enough (>= 8 stages of 128) for some tiles to be split
    along the contraction, and a rotation block that divides K."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(rng.integers(1, 1500))
        N = 16 * int(rng.integers(1, 100))
        K = 16 * int(rng.integers(1, 100))
        if i % 3 == 1:
            K = 128 * (K // 128 + 1)            # the widest fused rotation
            had = 128
        elif i % 3 == 2:
            hads = [h for h in (64, 32, 16, 8, 4, 2) if K % h == 0]
            had = hads[int(rng.integers(0, len(hads)))]
        else:
            had = 0
        cases.append((i, M, N, K, had, bool(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("i,M,N,K,had,with_bias", _random_product_cases())
def test_products_random_shapes(T, Q, orc, i, M, N, K, had, with_bias):
    """The three products through qlin_product_ws (tiles split along the
    contraction where the shape allows) and the plain entry points, bit for
    bit against the oracle, on seeded random shapes."""
    rng = np.random.default_rng(1000 + i)
    qx, qw, qg = _codes(rng, (M, K)), _codes(rng, (N, K)), _codes(rng, (M, N))
    sx = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    sg1 = rng.uniform(1e-6, 1e-4, M).astype(np.float32)
    sg2 = rng.uniform(1e-6, 1e-4, N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32) if with_bias else None
    y_ref = orc.fwd(qx, sx, qw, sw, b)
    dx_ref = orc.bwd_dx(qg, sg1, qw)
    if had:
        dx_ref = orc.hadamard(dx_ref, had)
    dw_ref = orc.bwd_dw(qg, sg2, qx)
    announce("random products", i, M, N, K, had, with_bias)
    y = Q.qlin_product_ws(Q.QLIN_OP_FWD, dev(qx), dev(sx), dev(qw), M, N, K, scol=dev(sw),
                          bias=None if b is None else dev(b))
    dx = Q.qlin_product_ws(Q.QLIN_OP_DX, dev(qg), dev(sg1), dev(qw), M, N, K, had_block=had)
    dw = Q.qlin_product_ws(Q.QLIN_OP_DW, dev(qg), dev(sg2), dev(qx), M, N, K)
    y2 = Q.qlin_fwd(dev(qx), dev(sx), dev(qw), dev(sw), None if b is None else dev(b))
    dx2 = Q.qlin_bwd_dx(dev(qg), dev(sg1), dev(qw), had_block=had)
    dw2 = Q.qlin_bwd_dw(dev(qg), dev(sg2), dev(qx))
    T.cuda.synchronize()
    for got, ref, what in ((y, y_ref, "y"), (dx, dx_ref, "dx"), (dw, dw_ref, "dw"),
                           (y2, y_ref, "y plain"), (dx2, dx_ref, "dx plain"),
                           (dw2, dw_ref, "dw plain")):
        assert_bitwise(host(got), ref, what)


def test_products_random_sweep(T, Q, orc):
    """A wider seeded sweep in one test: 120 random shapes up to 3000 tokens
    and 2032 features, the three products through qlin_product_ws and the
    plain entry points, bit for bit against the oracle."""
    rng0 = np.random.default_rng(777001)
    for i in range(120):
        M = int(rng0.integers(1, 3000))
        N, K = 16 * int(rng0.integers(1, 128)), 16 * int(rng0.integers(1, 128))
        had = [0, 128, 64, 16][i % 4]
        if had and K % had:
            K = had * (K // had + 1)
        rng = np.random.default_rng(5000 + i)
        qx, qw, qg = _codes(rng, (M, K)), _codes(rng, (N, K)), _codes(rng, (M, N))
        sx = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
        sg1 = rng.uniform(1e-6, 1e-4, M).astype(np.float32)
        sg2 = rng.uniform(1e-6, 1e-4, N).astype(np.float32)
        b = rng.standard_normal(N).astype(np.float32) if i % 2 else None
        announce("random sweep", i, M, N, K, had)
        y_ref = orc.fwd(qx, sx, qw, sw, b)
        dx_ref = orc.bwd_dx(qg, sg1, qw)
        if had:
            dx_ref = orc.hadamard(dx_ref, had)
        dw_ref = orc.bwd_dw(qg, sg2, qx)
        bias = None if b is None else dev(b)
        got = [
            (Q.qlin_product_ws(Q.QLIN_OP_FWD, dev(qx), dev(sx), dev(qw), M, N, K, scol=dev(sw),
                               bias=bias), y_ref, "y"),
            (Q.qlin_product_ws(Q.QLIN_OP_DX, dev(qg), dev(sg1), dev(qw), M, N, K, had_block=had),
             dx_ref, "dx"),
            (Q.qlin_product_ws(Q.QLIN_OP_DW, dev(qg), dev(sg2), dev(qx), M, N, K), dw_ref, "dw"),
            (Q.qlin_fwd(dev(qx), dev(sx), dev(qw), dev(sw), bias), y_ref, "y plain"),
            (Q.qlin_bwd_dx(dev(qg), dev(sg1), dev(qw), had_block=had), dx_ref, "dx plain"),
            (Q.qlin_bwd_dw(dev(qg), dev(sg2), dev(qx)), dw_ref, "dw plain"),
        ]
        T.cuda.synchronize()
        for out, ref, what in got:
            assert_bitwise(host(out), ref, f"{what} (case {i}: {M} x {N} x {K}, block {had})")


@pytest.mark.parametrize("M,N,K,had", [(64, 128, 256, 128), (130, 272, 384, 128), (17, 48, 512, 64),
                                       (33, 64, 256, 2), (40, 32, 64, 16), (5, 16, 1024, 256),
                                       (3, 16, 512, 512), (257, 144, 5376, 128)])
def test_bwd_dx_rotated_back(T, Q, orc, M, N, K, had):
    """dX rotated back in the product's epilogue (blocks <= 128) or by a second
    kernel (larger blocks) equals the oracle's dX followed by its rotation."""
    rng = np.random.default_rng(M * 3 + had)
    qg, qw = _codes(rng, (M, N)), _codes(rng, (N, K))
    sg1 = rng.uniform(1e-6, 1e-4, M).astype(np.float32)
    announce("bwd_dx rotated", M, N, K, had)
    dx = Q.qlin_bwd_dx(dev(qg), dev(sg1), dev(qw), had_block=had)
    T.cuda.synchronize()
    assert_bitwise(host(dx), orc.hadamard(orc.bwd_dx(qg, sg1, qw), had), "dx")


def test_dw_empty_tokens(T, Q, orc):
    N, K = 32, 48
    announce("bwd_dw M=0")
    dw = Q.qlin_bwd_dw(dev(np.zeros((0, N), np.int8)), dev(np.ones(N, np.float32)),
                       dev(np.zeros((0, K), np.int8)))
    T.cuda.synchronize()
    assert np.all(host(dw) == 0)


LONG_CASES = [
    # op, M, N, K, had: contractions above 131,071 (3 chunks, 2 chunks)
    (2, 300_000, 32, 48, 0),
    (1, 32, 200_000, 256, 128),
    (1, 20, 140_000, 512, 256),      # rotation block too wide to fuse: separate pass
    (0, 20, 48, 262_144, 0),         # forward with bias; 20 rows use the tiled kernel
    (0, 3, 32, 140_032, 0),          # a skinny M takes the tiled kernel too
]


@pytest.mark.parametrize("op,M,N,K,had", LONG_CASES)
def test_long_contraction(T, Q, orc, op, M, N, K, had):
    rng = np.random.default_rng(op * 7 + M)
    sa = (M, K) if op == 0 else (M, N)
    sb = (N, K) if op in (0, 1) else (M, K)
    a = _codes(rng, sa)
    b = _codes(rng, sb)
    # output row 0 has columns whose sums pass 2^31
    if op == 0:
        a[0] = 127
        b[:4] = 127
    elif op == 1:
        a[0] = 127
        b[:, :4] = 127
    else:
        a[:, 0] = 127
        b[:, :4] = 127
    R, C = {0: (M, N), 1: (M, K), 2: (N, K)}[op]
    srow = rng.uniform(1e-4, 1e-2, R).astype(np.float32)
    scol = rng.uniform(1e-2, 1e-1, N).astype(np.float32) if op == 0 else None
    bias = rng.standard_normal(N).astype(np.float32) if op == 0 else None
    announce("long contraction", op, M, N, K, had)
    out = Q.qlin_product_ws(op, dev(a), dev(srow), dev(b), M, N, K,
                            scol=None if scol is None else dev(scol),
                            bias=None if bias is None else dev(bias), had_block=had)
    T.cuda.synchronize()
    ii, jj = np.repeat(np.arange(R), C), np.tile(np.arange(C), R)
    acc = orc.gemm_s64_at(op, a, b, M, N, K, ii[:C], jj[:C])
    assert np.abs(acc).max() > 2 ** 31          # row 0 overflows int32
    ref = orc.op_at_long(op, a, srow, b, scol, bias, M, N, K, ii, jj).reshape(R, C)
    if had:
        ref = orc.hadamard(ref, had)
    assert_bitwise(host(out), ref, "long product")


def test_product_ws_within_bound_is_the_plain_call(T, Q, orc):
    rng = np.random.default_rng(1)
    M, N, K = 130, 272, 208
    qg = _codes(rng, (M, N))
    qx = _codes(rng, (M, K))
    s = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    announce("product_ws within the bound")
    a = Q.qlin_product_ws(2, dev(qg), dev(s), dev(qx), M, N, K)
    b = Q.qlin_bwd_dw(dev(qg), dev(s), dev(qx))
    T.cuda.synchronize()
    assert_bitwise(host(a), host(b), "dW")


SPLIT_CASES = [
    # op, M, N, K, had, bias.  A grid of more tiles than one round of the chip
    # (256) leaves a partial last round; with a workspace those tiles are split
    # along the contraction (here 272 tiles: 256 whole, 16 in 3 pieces each).
    (0, 4352, 4096, 4096, 0, True),
    (1, 4352, 4096, 4096, 128, False),   # rotation in the epilogue of the last piece
    (2, 4096, 4352, 4096, 0, False),
    # Fewer tiles than one round: every tile split; ragged rows, columns and
    # contraction (the last piece of a dW split gets the partial stage).
    (0, 700, 1040, 1008, 0, True),
    (2, 3000, 1040, 528, 0, False),
    (1, 600, 2048, 512, 64, False),
    (1, 300, 1024, 1024, 256, False),    # rotation too wide to fuse: separate pass
]


@pytest.mark.parametrize("op,M,N,K,had,with_bias", SPLIT_CASES)
def test_product_split_tail(T, Q, orc, op, M, N, K, had, with_bias):
    """Products through the workspace entry point with their last round of
    tiles split along the contraction: bitwise equal to the ordinary call over
    the whole output (twice on one workspace, whose arrival counters the
    first call must leave at zero), and to the oracle on whole sampled output
    rows, taken from the split tiles and from whole ones."""
    rng = np.random.default_rng(op * 1009 + M + K)
    need = Q.qlin_product_ws_bytes(op, M, N, K)
    assert need > 0, "the case must split"
    sa = (M, K) if op == 0 else (M, N)
    sb = (N, K) if op in (0, 1) else (M, K)
    a, b = _codes(rng, sa), _codes(rng, sb)
    R, C = {0: (M, N), 1: (M, K), 2: (N, K)}[op]
    srow = rng.uniform(1e-4, 1e-2, R).astype(np.float32)
    scol = rng.uniform(1e-2, 1e-1, N).astype(np.float32) if op == 0 else None
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    da, db_, ds = dev(a), dev(b), dev(srow)
    dsc = None if scol is None else dev(scol)
    dbias = None if bias is None else dev(bias)
    announce("split tail", op, M, N, K, had, need)
    ws = T.zeros(need, dtype=T.uint8, device="cuda")
    outs = [host(Q.qlin_product_ws(op, da, ds, db_, M, N, K, scol=dsc, bias=dbias,
                                   had_block=had, workspace=ws)) for _ in range(2)]
    if op == 0:
        plain = Q.qlin_fwd(da, ds, db_, dsc, dbias)
    elif op == 1:
        plain = Q.qlin_bwd_dx(da, ds, db_, had_block=had)
    else:
        plain = Q.qlin_bwd_dw(da, ds, db_)
    T.cuda.synchronize()
    assert np.all(host(ws[:4096]) == 0), "arrival counters left non-zero"
    plain = host(plain)
    assert_bitwise(outs[0], plain, "split vs plain")
    assert_bitwise(outs[1], plain, "second call on the workspace")
    # whole output rows: the last two (in the last, split, tile row) and two others
    rows = np.unique(np.r_[R - 1, R - 2, rng.integers(0, R, 2)])
    ii, jj = np.repeat(rows, C), np.tile(np.arange(C), len(rows))
    ref = orc.op_at(op, a, srow, b, scol, bias, M, N, K, ii, jj).reshape(len(rows), C)
    if had:
        ref = orc.hadamard(ref, had)
    assert_bitwise(outs[0][rows], ref, "sampled rows")


# ------------------------------------------------------------------ update

SGD_CASES = [(128, 256, True), (64, 5376, False), (7, 16, True), (3, 20480, False),
             (5, 14336, True)]


@pytest.mark.parametrize("N,K,with_bias", SGD_CASES)
def test_sgd_requant(T, Q, orc, N, K, with_bias):
    rng = np.random.default_rng(N * K)
    qw = _codes(rng, (N, K))
    qw[:, 0] = 127
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    dw = rng.standard_normal((N, K)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    db = rng.standard_normal(N).astype(np.float32) if with_bias else None
    for seed, step, lr in ((0, 0, 1e-3), (123456789012, 2 ** 33 + 5, 0.5), (1, 7, 0.0)):
        announce("sgd_requant", N, K, seed, step, lr)
        qd, sd, dd = dev(qw), dev(sw), dev(dw)
        bd = None if bias is None else dev(bias)
        Q.qlin_sgd_requant(qd, sd, dd, lr, seed, step, bias=bd,
                           db=None if db is None else dev(db))
        T.cuda.synchronize()
        qr, sr, br = orc.sgd_requant(qw, sw, dw, lr, seed, step, bias=bias, db=db)
        assert_bitwise(host(sd), sr, "scales")
        assert_bitwise(host(qd), qr, "codes")
        if bias is not None:
            assert_bitwise(host(bd), br, "bias")


WN_CASES = [(4, 16, False), (33, 272, True), (16, 2064, False), (64, 5376, True),
            (8, 14336, False), (4, 20480, True), (2, 32768, False)]


@pytest.mark.parametrize("N,K,with_bias", WN_CASES)
def test_weight_norm_steps(T, Q, orc, N, K, with_bias):
    """Weight-normalized layer: preparation, then three chained SGD steps
    (each step's oracle inputs are the oracle's own previous outputs); one row
    has all-zero codes (no direction: zero gradients).  Bit for bit."""
    rng = np.random.default_rng(N * K + 5)
    q = _codes(rng, (N, K))
    q[:, 0] = 127
    s = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    announce("wn_init", N, K)
    gd, swd = Q.qlin_wn_init(dev(q), dev(s))
    T.cuda.synchronize()
    g, sw = orc.wn_init(q, s)
    assert_bitwise(host(gd), g, "g")
    assert_bitwise(host(swd), sw, "sw")
    q[N // 2] = 0                       # a row without a direction from here on
    s[N // 2] = 0.0
    g[N // 2] = np.float32(1.5)
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    d = {k: (None if a is None else dev(a)) for k, a in
         dict(q=q, s=s, g=g, sw=sw, bias=bias).items()}
    for step, lr in ((1, 1e-2), (2, 0.3), (3, 0.0)):
        dw = (rng.standard_normal((N, K)) * 10.0 ** rng.uniform(-4, -1)).astype(np.float32)
        db = rng.standard_normal(N).astype(np.float32) if with_bias else None
        announce("wn_sgd_requant", N, K, step, lr)
        Q.qlin_wn_sgd_requant(d["q"], d["s"], d["g"], d["sw"], dev(dw), lr, seed=77, step=step,
                              bias=d["bias"], db=None if db is None else dev(db))
        T.cuda.synchronize()
        q, s, g, sw, bias = orc.wn_sgd_requant(q, s, g, dw, lr, 77, step, bias=bias, db=db)
        for key, ref in (("q", q), ("s", s), ("g", g), ("sw", sw), ("bias", bias)):
            if ref is not None:
                assert_bitwise(host(d[key]), ref, f"{key} after step {step}")


def _random_update_cases(n=8, seed=7404):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 600)), 16 * int(rng.integers(1, 2048 if i % 2 else 256)),
             bool(rng.integers(0, 2))) for i in range(n)]


@pytest.mark.parametrize("i,N,K,with_bias", _random_update_cases())
def test_updates_random(T, Q, orc, i, N, K, with_bias):
    """SGD, AdamW and weight-normalized SGD on seeded random shapes, one step
    each from the same state, bit for bit."""
    rng = np.random.default_rng(1400 + i)
    qw = _codes(rng, (N, K))
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    dw = (rng.standard_normal((N, K)) * 10.0 ** rng.uniform(-4, 0)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    db = rng.standard_normal(N).astype(np.float32) if with_bias else None
    lr, seed, step = 0.05, 99 + i, 1 + i
    announce("updates random", i, N, K, with_bias)
    q, s, b = dev(qw), dev(sw), None if bias is None else dev(bias)
    Q.qlin_sgd_requant(q, s, dev(dw), lr, seed, step, bias=b, db=None if db is None else dev(db))
    T.cuda.synchronize()
    qr, sr, br = orc.sgd_requant(qw, sw, dw, lr, seed, step, bias=bias, db=db)
    assert_bitwise(host(q), qr, "sgd codes")
    assert_bitwise(host(s), sr, "sgd scales")
    if bias is not None:
        assert_bitwise(host(b), br, "sgd bias")
    q, s = dev(qw), dev(sw)
    m, v = dev(np.zeros((N, K), np.float32)), dev(np.zeros((N, K), np.float32))
    Q.qlin_adamw_requant(q, s, dev(dw), m, v, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                         weight_decay=0.01, seed=seed, step=step)
    T.cuda.synchronize()
    qa, sa, ma, va = orc.adamw_requant(qw, sw, dw, np.zeros((N, K), np.float32),
                                       np.zeros((N, K), np.float32), 1e-3, 0.9, 0.999, 1e-8,
                                       0.01, seed, step)[:4]
    for got, ref, what in ((q, qa, "adamw codes"), (s, sa, "adamw scales"), (m, ma, "m"),
                           (v, va, "v")):
        assert_bitwise(host(got), ref, what)
    qw[:, 0] = 127
    g0, sw0 = orc.wn_init(qw, sw)
    q, s, g, swd = dev(qw), dev(sw), dev(g0), dev(sw0)
    Q.qlin_wn_sgd_requant(q, s, g, swd, dev(dw), lr, seed, step)
    T.cuda.synchronize()
    qn, sn, gn, swn, _ = orc.wn_sgd_requant(qw, sw, g0, dw, lr, seed, step)
    for got, ref, what in ((q, qn, "wn codes"), (s, sn, "wn scales"), (g, gn, "wn g"),
                           (swd, swn, "wn sw")):
        assert_bitwise(host(got), ref, what)


ADAMW_CASES = [(128, 256, True), (64, 5376, False), (7, 16, True), (3, 20480, False),
               (5, 14336, True)]


@pytest.mark.parametrize("N,K,with_bias", ADAMW_CASES)
def test_adamw_requant(T, Q, orc, N, K, with_bias):
    """Three chained AdamW steps; each step's inputs on the oracle side are the
    oracle's own previous outputs."""
    rng = np.random.default_rng(N * K + 3)
    qw = _codes(rng, (N, K))
    qw[:, 0] = 127
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    m = np.zeros((N, K), np.float32)
    v = np.zeros((N, K), np.float32)
    bias = rng.standard_normal(N).astype(np.float32) if with_bias else None
    bm = np.zeros(N, np.float32) if with_bias else None
    bv = np.zeros(N, np.float32) if with_bias else None
    d = {k: (None if a is None else dev(a)) for k, a in
         dict(qw=qw, sw=sw, m=m, v=v, bias=bias, bm=bm, bv=bv).items()}
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    for t in (1, 2, 3):
        g = (rng.standard_normal((N, K)) * 10.0 ** rng.uniform(-3, 1)).astype(np.float32)
        db = rng.standard_normal(N).astype(np.float32) if with_bias else None
        announce("adamw_requant", N, K, with_bias, t)
        Q.qlin_adamw_requant(d["qw"], d["sw"], dev(g), d["m"], d["v"], seed=13, step=t,
                             bias=d["bias"], db=None if db is None else dev(db),
                             bias_m=d["bm"], bias_v=d["bv"], **hp)
        T.cuda.synchronize()
        qw, sw, m, v, bias, bm, bv = orc.adamw_requant(
            qw, sw, g, m, v, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"],
            13, t, bias=bias, db=db, bm=bm, bv=bv)
        assert_bitwise(host(d["m"]), m, f"m step {t}")
        assert_bitwise(host(d["v"]), v, f"v step {t}")
        assert_bitwise(host(d["sw"]), sw, f"scales step {t}")
        assert_bitwise(host(d["qw"]), qw, f"codes step {t}")
        if with_bias:
            assert_bitwise(host(d["bias"]), bias, f"bias step {t}")
            assert_bitwise(host(d["bm"]), bm, f"bias m step {t}")
            assert_bitwise(host(d["bv"]), bv, f"bias v step {t}")


def test_sgd_extreme_scales(T, Q, orc):
    """Rows whose requant scale lies outside [2^-40, 2^40] and elements whose
    quotient w / s' is below 2^-40 in magnitude (normal and subnormal w) take
    the kernel's division path; the rest of each row its reciprocal path.
    Both must give the oracle's codes."""
    rng = np.random.default_rng(404)
    N, K = 12, 1024
    qw = _codes(rng, (N, K))
    qw[:, 0] = 127
    sw = np.full(N, 1e-3, np.float32)
    sw[0], sw[1] = 1e-20, 2e-14           # scales below 2^-40
    sw[2], sw[3] = 3e13, 1e18             # scales above 2^40
    sw[4] = np.float32(2.0 ** -40)        # the bounds themselves
    sw[5] = np.float32(2.0 ** 40)
    dw = rng.standard_normal((N, K)).astype(np.float32)
    dw[:6] *= sw[:6, None]
    # rows 6-11: zero codes with tiny or zero gradients beside full-size ones
    for r, mag in ((6, 1e-30), (7, 1e-36), (8, 1e-41), (9, 0.0)):
        qw[r, 1::2] = 0
        dw[r, 1::2] = mag * rng.choice([-1.0, 1.0], K // 2).astype(np.float32)
    qw[10, 8:] = 0                         # whole chunks of tiny quotients
    dw[10, 8:] = 1e-33
    qw[11] = 0                             # one normal element, the rest subnormal w
    qw[11, 0] = 127
    dw[11, 1:] = rng.choice([-1.0, 1.0], K - 1).astype(np.float32) * np.float32(1e-36)
    lr = 1e-3
    for seed, step in ((0, 0), (5, 2 ** 31 + 3)):
        announce("sgd_requant extreme scales", seed, step)
        qd, sd = dev(qw), dev(sw)
        Q.qlin_sgd_requant(qd, sd, dev(dw), lr, seed, step)
        T.cuda.synchronize()
        qr, sr, _ = orc.sgd_requant(qw, sw, dw, lr, seed, step)
        assert_bitwise(host(sd), sr, "scales")
        assert_bitwise(host(qd), qr, "codes")


def test_sgd_zero_rows(T, Q, orc):
    N, K = 4, 64
    qw = np.zeros((N, K), np.int8)
    qw[1] = 5
    sw = np.array([0.0, 0.5, 0.0, 1e-3], np.float32)
    dw = np.zeros((N, K), np.float32)
    dw[2, 3] = 1.0
    announce("sgd_requant zero rows")
    qd, sd = dev(qw), dev(sw)
    Q.qlin_sgd_requant(qd, sd, dev(dw), 0.25, 0, 0)
    T.cuda.synchronize()
    qr, sr, _ = orc.sgd_requant(qw, sw, dw, 0.25, 0, 0)
    assert_bitwise(host(sd), sr, "scales")
    assert_bitwise(host(qd), qr, "codes")


# --------------------------------------------------------- error behaviour

def test_rejected_calls_leave_outputs_untouched(T, Q):
    x = T.randn(4, 48, device="cuda")
    q = T.full((4, 48), 5, dtype=T.int8, device="cuda")
    s = T.full((4,), 3.0, device="cuda")
    with pytest.raises(Q.QlinError):
        Q.qlin_quantize_rows(x, had_block=32, q=q, s=s)     # 32 does not divide 48
    qw = T.zeros((16, 131072), dtype=T.int8, device="cuda")
    y = T.full((2, 16), 7.0, device="cuda")
    with pytest.raises(Q.QlinError):
        Q.qlin_fwd(T.zeros((2, 131072), dtype=T.int8, device="cuda"),
                   T.ones(2, device="cuda"), qw, T.ones(16, device="cuda"), y=y)
    T.cuda.synchronize()
    assert bool((q == 5).all()) and bool((s == 3.0).all()) and bool((y == 7.0).all())


# ------------------------------------------------------------ streaming copy

@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 16 * 777])
def test_stream_copy(T, Q, nbytes):
    """The bandwidth reference copies every byte (ragged last iteration and
    a grid that walks the buffer more than once included)."""
    announce("stream copy", nbytes)
    g = T.Generator(device="cuda")
    g.manual_seed(nbytes)
    src = T.randint(0, 256, (nbytes,), dtype=T.uint8, device="cuda", generator=g)
    dst = T.zeros(nbytes + 64, dtype=T.uint8, device="cuda")
    Q._native.qlin_stream_copy(src, dst[:nbytes])
    T.cuda.synchronize()
    assert T.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].count_nonzero()) == 0


# ------------------------------------------------------------- repetition

def test_products_repeated(T, Q, orc):
    """Small products launched many times in a row, every output compared bit
    for bit with the oracle.  A race between the waves of a workgroup (such as
    the end of the main loop against the epilogue's staging in LDS) shows as
    a few wrong outputs in some launches only; two-stage contractions with
    ragged edges, and split last rounds on one reused workspace."""
    reps = 100
    for M, N, K in [(130, 272, 208), (64, 528, 320)]:
        rng = np.random.default_rng(7 * M + N)
        qx, qw, qg = _codes(rng, (M, K)), _codes(rng, (N, K)), _codes(rng, (M, N))
        for op, a, b in ((Q.QLIN_OP_FWD, qx, qw), (Q.QLIN_OP_DX, qg, qw), (Q.QLIN_OP_DW, qg, qx)):
            announce("repeated gemm_s32", op, M, N, K, reps)
            ref = orc.gemm_s32(op, a, b, M, N, K)
            da, db = dev(a), dev(b)
            outs = [Q.qlin_gemm_s32(op, da, db, M, N, K) for _ in range(reps)]
            T.cuda.synchronize()
            for r, c in enumerate(outs):
                assert_bitwise(host(c), ref, f"op{op} {M}x{N}x{K} launch {r}")
    reps = 40
    for op, M, N, K in [(0, 700, 1040, 1008), (2, 3000, 1040, 528)]:
        rng = np.random.default_rng(op * 31 + M)
        sa = (M, K) if op == 0 else (M, N)
        sb = (N, K) if op == 0 else (M, K)
        a, b = _codes(rng, sa), _codes(rng, sb)
        R = M if op == 0 else N
        srow = rng.uniform(1e-4, 1e-2, R).astype(np.float32)
        scol = rng.uniform(1e-2, 1e-1, N).astype(np.float32) if op == 0 else None
        need = Q.qlin_product_ws_bytes(op, M, N, K)
        assert need > 0, "the case must split"
        announce("repeated split", op, M, N, K, reps)
        ref = orc.fwd(a, srow, b, scol) if op == 0 else orc.bwd_dw(a, srow, b)
        ws = T.zeros(need, dtype=T.uint8, device="cuda")
        da, db, ds = dev(a), dev(b), dev(srow)
        dsc = None if scol is None else dev(scol)
        outs = [Q.qlin_product_ws(op, da, ds, db, M, N, K, scol=dsc, workspace=ws)
                for _ in range(reps)]
        T.cuda.synchronize()
        for r, c in enumerate(outs):
            assert_bitwise(host(c), ref, f"split op{op} launch {r}")
        assert np.all(host(ws[:4096]) == 0), "arrival counters left non-zero"
