"""Pins of the oracle's long contractions (mini_trainer guide, arithmetic
paragraph: contractions above 131,071 combine bounded int32 partial dot
products in int64 before scaling)."""
import numpy as np
import pytest


def _mats(op, L, rng, fill=None):
    if op == 0:
        M, N, K = 3, 4, L
        sa, sb = (M, K), (N, K)
    elif op == 1:
        M, N, K = 3, L, 4
        sa, sb = (M, N), (N, K)
    else:
        M, N, K = L, 3, 4
        sa, sb = (M, N), (M, K)
    if fill is None:
        a = rng.integers(-127, 128, sa).astype(np.int8)
        b = rng.integers(-127, 128, sb).astype(np.int8)
    else:
        a = np.full(sa, fill, np.int8)
        b = np.full(sb, fill, np.int8)
    return M, N, K, a, b


def _ref(op, a, b):
    a64, b64 = a.astype(np.int64), b.astype(np.int64)
    return a64 @ b64.T if op == 0 else (a64 @ b64 if op == 1 else a64.T @ b64)


@pytest.mark.parametrize("op", [0, 1, 2])
def test_exact_beyond_int32(orc, op):
    """All 127 codes over 300,000 terms: 4.8e9, beyond int32, exact in int64."""
    rng = np.random.default_rng(op)
    M, N, K, a, b = _mats(op, 300_000, rng, fill=127)
    R, C = _ref(op, a, b).shape
    ii, jj = np.repeat(np.arange(R), C), np.tile(np.arange(C), R)
    got = orc.gemm_s64_at(op, a, b, M, N, K, ii, jj)
    assert np.all(got == 300_000 * 127 * 127) and got[0] > 2 ** 31


@pytest.mark.parametrize("op", [0, 1, 2])
def test_random_long_matches_numpy(orc, op):
    rng = np.random.default_rng(10 + op)
    M, N, K, a, b = _mats(op, 200_003, rng)
    ref = _ref(op, a, b)
    R, C = ref.shape
    ii, jj = np.repeat(np.arange(R), C), np.tile(np.arange(C), R)
    assert np.array_equal(orc.gemm_s64_at(op, a, b, M, N, K, ii, jj), ref.reshape(-1))


def test_dequant_converts_once(orc):
    """fl32 of the exact int64 sum, then the usual epilogue (dW here): an int64
    sum that is not representable in fp32 rounds to nearest even once."""
    L = 300_001
    M, N, K = L, 2, 2
    a = np.full((M, N), 127, np.int8)
    b = np.full((M, K), 127, np.int8)
    b[0, 0] = 1                         # sum = 127 * (127 * (L - 1) + 1), odd, > 2^24
    s = np.array([0.5, 2.0 ** -20], np.float32)
    out = orc.op_at_long(2, a, s, b, None, None, M, N, K, np.array([0, 1]), np.array([0, 0]))
    acc = 127 * (127 * (L - 1) + 1)
    assert acc > 2 ** 31
    assert np.array_equal(out, (np.float32(acc) * s).astype(np.float32))


def test_agrees_with_the_bounded_path(orc):
    """Below the bound the long path is the ordinary dequantized product."""
    rng = np.random.default_rng(7)
    M, N, K = 5, 6, 4096
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sx = rng.uniform(0.1, 1, M).astype(np.float32)
    sw = rng.uniform(0.1, 1, N).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    ii, jj = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    assert np.array_equal(orc.op_at_long(0, a, sx, b, sw, bias, M, N, K, ii, jj),
                          orc.op_at(0, a, sx, b, sw, bias, M, N, K, ii, jj))
