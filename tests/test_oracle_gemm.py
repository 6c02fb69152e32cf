"""Pins of the oracle's integer products and dequant epilogues (mini_trainer
guide: integer forward and backward matrix products on INT8 weights and saved
INT8 inputs; contractions up to 131,071 stay exact in int32)."""
import numpy as np
import pytest

SHAPES = [(1, 16, 16), (17, 48, 32), (64, 128, 256), (37, 80, 112)]


def _codes(rng, shape):
    return rng.integers(-127, 128, size=shape).astype(np.int8)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_s32_vs_brute_force(orc, M, N, K):
    rng = np.random.default_rng(M * 7 + N)
    qx, qw = _codes(rng, (M, K)), _codes(rng, (N, K))
    qg = _codes(rng, (M, N))
    i64 = lambda a: a.astype(np.int64)
    assert np.array_equal(orc.gemm_s32(orc.OP_FWD, qx, qw, M, N, K), i64(qx) @ i64(qw).T)
    assert np.array_equal(orc.gemm_s32(orc.OP_DX, qg, qw, M, N, K), i64(qg) @ i64(qw))
    assert np.array_equal(orc.gemm_s32(orc.OP_DW, qg, qx, M, N, K), i64(qg).T @ i64(qx))


def test_gemm_s32_at_matches_full(orc):
    rng = np.random.default_rng(1)
    M, N, K = 33, 48, 64
    qx, qw, qg = _codes(rng, (M, K)), _codes(rng, (N, K)), _codes(rng, (M, N))
    for op, a, b, (R, C) in ((orc.OP_FWD, qx, qw, (M, N)), (orc.OP_DX, qg, qw, (M, K)),
                             (orc.OP_DW, qg, qx, (N, K))):
        full = orc.gemm_s32(op, a, b, M, N, K)
        ii, jj = rng.integers(0, R, 200), rng.integers(0, C, 200)
        assert np.array_equal(orc.gemm_s32_at(op, a, b, M, N, K, ii, jj), full[ii, jj])


def test_contraction_bound(orc):
    """131,071 * 128 * 128 < 2^31 = 131,072 * 128 * 128: the longest contraction that
    is exact in int32 for any int8 codes; one more is rejected."""
    K = 131071
    assert K * 128 * 128 < 2 ** 31 == (K + 1) * 128 * 128
    a = np.full((1, K), 127, np.int8)
    b = np.full((1, K), -127, np.int8)
    assert orc.gemm_s32(orc.OP_FWD, a, b, 1, 1, K)[0, 0] == -K * 127 * 127
    with pytest.raises(orc.OracleError):
        orc.gemm_s32(orc.OP_FWD, np.zeros((1, K + 1), np.int8), np.zeros((1, K + 1), np.int8),
                     1, 1, K + 1)


def test_fwd_epilogue_vs_float64(orc):
    rng = np.random.default_rng(2)
    M, N, K = 40, 48, 96
    qx, qw = _codes(rng, (M, K)), _codes(rng, (N, K))
    sx = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    y = orc.fwd(qx, sx, qw, sw, b)
    acc = qx.astype(np.float64) @ qw.astype(np.float64).T
    ref = acc * sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64) + b
    mag = np.abs(acc * sx[:, None] * sw[None, :]) + np.abs(b)
    assert np.all(np.abs(y - ref) <= 4 * 2.0 ** -24 * mag + 1e-30)
    y0 = orc.fwd(qx, sx, qw, sw, None)
    assert np.all(np.abs(y0 - (ref - b)) <= 3 * 2.0 ** -24 * np.abs(ref - b) + 1e-30)


def _exact_operand(rng, rows, cols, lo=-20, hi=0):
    """Rows exactly representable by (int8 codes, power-of-two scale)."""
    q = rng.integers(-127, 128, size=(rows, cols)).astype(np.int32)
    q[np.arange(rows), rng.integers(0, cols, rows)] = 127
    e = rng.integers(lo, hi, rows)
    s = np.ldexp(np.float32(1.0), e).astype(np.float32)
    return (q * s[:, None].astype(np.float64)).astype(np.float32)


def test_fwd_exact_brute_force(orc):
    """Exactly quantizable X and W: the layer equals fl32(X W^T + b) in float64."""
    rng = np.random.default_rng(3)
    M, N, K = 24, 32, 64
    x = _exact_operand(rng, M, K)
    w = _exact_operand(rng, N, K)
    b = (rng.integers(-1000, 1000, N) * 2.0 ** -12).astype(np.float32)
    qx, sx = orc.quantize_rows(x)
    qw, sw = orc.quantize_rows(w)
    y = orc.fwd(qx, sx, qw, sw, b)
    ref = (x.astype(np.float64) @ w.astype(np.float64).T + b).astype(np.float32)
    assert np.array_equal(y, ref)


def test_bwd_exact_brute_force(orc):
    """dX = dY W and dW = dY^T X exactly, with power-of-two scales throughout."""
    rng = np.random.default_rng(4)
    M, N, K = 24, 32, 64
    x = _exact_operand(rng, M, K)
    w = _exact_operand(rng, N, K)
    qx, sx = orc.quantize_rows(x)
    qw, sw = orc.quantize_rows(w)
    # dY whose rows (after the s_w prescale) and columns (after the s_x
    # prescale) are exactly quantizable: one shared power-of-two magnitude.
    dyq = rng.integers(-127, 128, size=(M, N)).astype(np.int32)
    dyq[:, 0] = 127
    dyq[0, :] = 127
    sw_e = np.log2(sw).astype(int)
    sx_e = np.log2(sx).astype(int)
    dy = (dyq * np.ldexp(1.0, -sw_e)[None, :] * np.ldexp(1.0, -sx_e)[:, None] * 2.0 ** -30)
    dy = dy.astype(np.float32)
    qg1, sg1 = orc.quantize_rows(dy, prescale=sw)
    dx = orc.bwd_dx(qg1, sg1, qw)
    w_eff = qw.astype(np.float64) * sw[:, None]
    assert np.array_equal(dx, (dy.astype(np.float64) @ w_eff).astype(np.float32))
    qg2, sg2 = orc.quantize_cols(dy, prescale=sx)
    dw = orc.bwd_dw(qg2, sg2, qx)
    x_eff = qx.astype(np.float64) * sx[:, None]
    assert np.array_equal(dw, (dy.astype(np.float64).T @ x_eff).astype(np.float32))


def test_op_at_matches_full(orc):
    rng = np.random.default_rng(5)
    M, N, K = 19, 32, 48
    qx, qw, qg = _codes(rng, (M, K)), _codes(rng, (N, K)), _codes(rng, (M, N))
    sx, sw = rng.random(M).astype(np.float32), rng.random(N).astype(np.float32)
    sg = rng.random(M).astype(np.float32)
    sgc = rng.random(N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    cases = [(orc.OP_FWD, qx, sx, qw, sw, b, orc.fwd(qx, sx, qw, sw, b)),
             (orc.OP_DX, qg, sg, qw, None, None, orc.bwd_dx(qg, sg, qw)),
             (orc.OP_DW, qg, sgc, qx, None, None, orc.bwd_dw(qg, sgc, qx))]
    for op, a, sr, bb, sc, bias, full in cases:
        R, C = full.shape
        ii, jj = rng.integers(0, R, 100), rng.integers(0, C, 100)
        got = orc.op_at(op, a, sr, bb, sc, bias, M, N, K, ii, jj)
        assert np.array_equal(got, full[ii, jj])


def test_rejects_long_contractions(orc):
    with pytest.raises(orc.OracleError):
        orc.bwd_dw(np.zeros((131072, 16), np.int8), np.zeros(16, np.float32),
                   np.zeros((131072, 16), np.int8))


def test_dw_rows_and_brute_force(orc):
    rng = np.random.default_rng(6)
    M, N, K = 45, 32, 48
    qg, qx = _codes(rng, (M, N)), _codes(rng, (M, K))
    sg = rng.random(N).astype(np.float32)
    full = orc.bwd_dw(qg, sg, qx)
    acc = qg.astype(np.int64).T @ qx.astype(np.int64)
    assert np.array_equal(full, (acc.astype(np.float32) * sg[:, None]).astype(np.float32))
    rows = np.array([31, 0, 7, 7])
    assert np.array_equal(orc.bwd_dw_rows(qg, sg, qx, rows), full[rows])
