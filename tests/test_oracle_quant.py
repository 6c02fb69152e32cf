"""Pins of the oracle's absmax INT8 quantizers (OneTrainer PR #1681: per-row
activation quantization on every call; mini_trainer guide: INT8 direction with a
floating magnitude per output row; tiny workload: per-row absmax/127 with
round-half-even)."""
import numpy as np
import pytest

import workloads


def _exact_rows(rng, rows, cols, exps):
    """Integer rows in [-127, 127], each holding one +-127, times 2^e."""
    q = rng.integers(-127, 128, size=(rows, cols)).astype(np.int32)
    pos = rng.integers(0, cols, size=rows)
    q[np.arange(rows), pos] = np.where(rng.random(rows) < 0.5, 127, -127)
    scale = np.ldexp(np.float32(1.0), np.asarray(exps)).astype(np.float32)
    return q.astype(np.int8), scale, (q.astype(np.float32) * scale[:, None]).astype(np.float32)


def test_exactly_quantizable_rows(orc):
    rng = np.random.default_rng(0)
    q_ref, s_ref, x = _exact_rows(rng, 20, 96, rng.integers(-20, 5, size=20))
    q, s = orc.quantize_rows(x)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s, s_ref)


def test_round_half_to_even(orc):
    # g/s lands exactly on halves: 0.5, 1.5, 2.5, -0.5, -2.5, 126.5 -> 0, 2, 2, 0, -2, 126.
    row = np.array([127, 0.5, 1.5, 2.5, -0.5, -2.5, 126.5, -126.5], np.float32) * np.float32(2.0 ** -6)
    q, s = orc.quantize_rows(row[None, :])
    assert s[0] == np.float32(2.0 ** -6)
    assert q[0].tolist() == [127, 0, 2, 2, 0, -2, 126, -126]


def test_invariants_random_rows(orc):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((2000, 64)) * rng.uniform(1e-3, 1e3, (2000, 1))).astype(np.float32)
    q, s = orc.quantize_rows(x)
    assert np.all(np.abs(q).max(axis=1) == 127)          # the absmax element maps to +-127
    assert np.all(s == (np.abs(x).max(axis=1) / np.float32(127)).astype(np.float32))
    err = np.abs(x.astype(np.float64) - s[:, None].astype(np.float64) * q)
    assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -20))
    assert q.min() >= -127


def test_power_of_two_scaling_invariance(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    q0, s0 = orc.quantize_rows(x)
    for e in (-7, 3, 11):
        q1, s1 = orc.quantize_rows((x * np.float32(2.0 ** e)).astype(np.float32))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** e)).astype(np.float32))


def test_zero_row(orc):
    x = np.zeros((3, 32), np.float32)
    x[1, 5] = 3.0
    q, s = orc.quantize_rows(x)
    assert s[0] == 0 and s[2] == 0 and np.all(q[[0, 2]] == 0)
    assert q[1, 5] == 127 and s[1] == np.float32(3.0) / np.float32(127)


def test_sign_symmetry(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((10, 48)).astype(np.float32)
    q, s = orc.quantize_rows(x)
    qn, sn = orc.quantize_rows(-x)
    assert np.array_equal(qn, -q) and np.array_equal(s, sn)


def test_prescale_power_of_two(orc):
    """A per-column prescale by powers of two equals quantizing the scaled input."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    p = np.ldexp(np.float32(1.0), rng.integers(-4, 4, 64)).astype(np.float32)
    p[::3] *= -1
    q1, s1 = orc.quantize_rows(x, prescale=p)
    q2, s2 = orc.quantize_rows((x * p).astype(np.float32))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_rotation_then_prescale_order(orc):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    p = np.ldexp(np.float32(1.0), rng.integers(-3, 3, 256)).astype(np.float32)
    q1, s1 = orc.quantize_rows(x, prescale=p, had_block=128)
    q2, s2 = orc.quantize_rows((orc.hadamard(x, 128) * p).astype(np.float32))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_rotation_of_one_hot_rows(orc):
    """A one-hot row rotates to a +-c_b row with the Hadamard row's signs."""
    import scipy.linalg
    b = 128
    x = np.zeros((b, 2 * b), np.float32)
    x[np.arange(b), np.arange(b)] = 5.0
    q, s = orc.quantize_rows(x, had_block=b)
    H = scipy.linalg.hadamard(b)
    assert np.array_equal(q[:, :b], (127 * H).astype(np.int8))
    assert np.all(q[:, b:] == 0)


def test_bf16_matches_decoded(orc):
    rng = np.random.default_rng(6)
    xb = workloads.f32_to_bf16_bits(rng.standard_normal((7, 256)).astype(np.float32))
    a = orc.quantize_rows(xb, had_block=64)
    b = orc.quantize_rows(workloads.bf16_bits_to_f32(xb), had_block=64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_cols_equals_rows_of_transpose(orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((37, 48)).astype(np.float32)
    p = rng.uniform(0.5, 2.0, 37).astype(np.float32)
    qc, sc = orc.quantize_cols(x, prescale=p)
    qr, sr = orc.quantize_rows(np.ascontiguousarray(x.T), prescale=p)
    assert np.array_equal(qc, qr.T) and np.array_equal(sc, sr)


def test_cols_exact_and_sum(orc):
    rng = np.random.default_rng(8)
    q_ref, s_ref, xt = _exact_rows(rng, 16, 40, rng.integers(-10, 3, 16))
    x = np.ascontiguousarray(xt.T)             # columns are exactly quantizable
    q, s, cs = orc.quantize_cols(x, want_sum=True)
    assert np.array_equal(q, q_ref.T) and np.array_equal(s, s_ref)
    assert np.allclose(cs, x.astype(np.float64).sum(axis=0), rtol=0,
                       atol=1e-6 * np.abs(x).sum(axis=0).max())


def test_cols_prescale_and_zero_columns(orc):
    x = np.zeros((5, 16), np.float32)
    x[:, 3] = [10, -20, 60, -254, 999]
    p = np.array([1, 1, 0.5, 0.5, 0], np.float32)
    q, s = orc.quantize_cols(x, prescale=p)
    assert s[3] == np.float32(1.0)
    assert q[:, 3].tolist() == [10, -20, 30, -127, 0]
    assert np.all(s[np.arange(16) != 3] == 0)


def test_degenerate_shapes(orc):
    q, s = orc.quantize_rows(np.zeros((0, 16), np.float32))
    assert q.shape == (0, 16) and s.shape == (0,)
    q, s = orc.quantize_cols(np.zeros((0, 16), np.float32))
    assert np.all(s == 0)
    with pytest.raises(orc.OracleError):
        orc.quantize_rows(np.zeros((2, 96), np.float32), had_block=64)


def test_prepare_weight_rejects_zero_rows(orc):
    w = np.ones((3, 16), np.float32)
    w[1] = 0
    with pytest.raises(ValueError):
        orc.prepare_weight(w)
