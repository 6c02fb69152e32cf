"""Pins of the oracle's Philox generator and the SGD stochastic requantization
(mini_trainer guide: updates stochastically requantize represented weights; no
floating master weight is retained).

Philox4x64-10 is checked against numpy's independent implementation; the
4x32 instance shares its round structure and uses the 32-bit constants of
Salmon et al. (SC'11)."""
import numpy as np
import pytest


def _numpy_philox_block(ctr, key):
    """numpy increments the 256-bit counter, then generates one block."""
    bg = np.random.Philox(key=np.array(key, np.uint64), counter=np.array(ctr, np.uint64))
    return bg.random_raw(4)


def _inc256(ctr):
    c = [int(v) for v in ctr]
    for i in range(4):
        c[i] = (c[i] + 1) % (1 << 64)
        if c[i] != 0:
            break
    return np.array(c, np.uint64)


def test_philox4x64_matches_numpy(orc):
    rng = np.random.default_rng(0)
    cases = [([0, 0, 0, 0], [0, 0]), ([2 ** 64 - 1, 5, 0, 0], [1, 2])]
    cases += [(rng.integers(0, 2 ** 63, 4, dtype=np.uint64).tolist(),
               rng.integers(0, 2 ** 63, 2, dtype=np.uint64).tolist()) for _ in range(50)]
    for ctr, key in cases:
        assert np.array_equal(orc.philox4x64_10(_inc256(ctr), key), _numpy_philox_block(ctr, key))


def test_philox4x32_statistics(orc):
    """Uniform 16-bit halves; distinct counters and keys give distinct blocks."""
    outs = np.array([orc.philox4x32_10([i, 0, 3, 0], [11, 0]) for i in range(4096)], np.uint32)
    halves = np.concatenate([outs & 0xFFFF, outs >> 16]).ravel()
    counts = np.bincount(halves >> 8, minlength=256)     # top byte of each half
    expected = halves.size / 256
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)              # ~6 sigma
    assert len({tuple(o) for o in outs}) == 4096
    other_key = orc.philox4x32_10([0, 0, 3, 0], [12, 0])
    other_step = orc.philox4x32_10([0, 0, 4, 0], [11, 0])
    assert not np.array_equal(other_key, outs[0]) and not np.array_equal(other_step, outs[0])


def test_philox4x32_avalanche(orc):
    rng = np.random.default_rng(1)
    flips = []
    for _ in range(200):
        c = rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32)
        k = rng.integers(0, 2 ** 32, 2, dtype=np.uint64).astype(np.uint32)
        bit = rng.integers(0, 128)
        c2 = c.copy()
        c2[bit // 32] ^= np.uint32(1 << (bit % 32))
        d = orc.philox4x32_10(c, k) ^ orc.philox4x32_10(c2, k)
        flips.append(sum(bin(int(v)).count("1") for v in d))
    assert 60 < np.mean(flips) < 68                       # ~64 of 128 bits flip


def test_sr_bits_counter_layout(orc):
    """Element i uses block i >> 3 at counter (i>>3, step), half (i & 1) of word (i & 7) >> 1."""
    seed, step = 0x1234_5678_9ABC, 77
    for i in (0, 1, 7, 8, 12345, 2 ** 35 + 3):
        blk = i >> 3
        x = orc.philox4x32_10([blk & 0xFFFFFFFF, blk >> 32, step, 0],
                              [seed & 0xFFFFFFFF, seed >> 32])
        assert orc.sr_bits16(seed, step, i) == (int(x[(i & 7) >> 1]) >> (16 * (i & 1))) & 0xFFFF


def _pow2_codes(rng, N, K, lo=-10, hi=-2):
    q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    q[:, 0] = 127
    s = np.ldexp(np.float32(1.0), rng.integers(lo, hi, N)).astype(np.float32)
    return q, s


def test_zero_lr_fixed_point_pow2(orc):
    rng = np.random.default_rng(2)
    q, s = _pow2_codes(rng, 16, 64)
    q2, s2, _ = orc.sgd_requant(q, s, np.ones((16, 64), np.float32), 0.0, seed=3, step=0)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_exact_update(orc):
    """w = s q - lr dW exactly representable on the old grid: deterministic codes."""
    s = np.array([2.0 ** -3], np.float32)
    q = np.array([[127, 100, -50, 0, 3, -127, 64, 1]], np.int8)
    lr = 0.5
    steps = np.array([[0, 6, -4, 2, 0, 0, -1, 1]], np.float32)    # code units
    dw = (steps * s[0] / lr).astype(np.float32)                     # lr*dW = steps*s
    q2, s2, _ = orc.sgd_requant(q, s, dw, lr, seed=0, step=0)
    assert s2[0] == s[0]
    assert q2[0].tolist() == [127, 94, -46, -2, 3, -127, 65, 0]


def test_membership_and_unbiased(orc):
    rng = np.random.default_rng(4)
    N, K = 4, 64
    q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    s = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    dw = rng.standard_normal((N, K)).astype(np.float32)
    lr = 1e-3
    w32 = (s[:, None] * q.astype(np.float32) - np.float32(lr) * dw).astype(np.float32)
    w = w32.astype(np.float64)
    T = 400
    acc = np.zeros((N, K))
    for step in range(T):
        q2, s2, _ = orc.sgd_requant(q, s, dw, lr, seed=9, step=step)
        y = w32 / s2[:, None]                            # IEEE fp32 division
        f = np.floor(y)
        assert np.all((q2 == f) | (q2 == f + 1) | (np.abs(q2) == 127))
        acc += s2[:, None].astype(np.float64) * q2
    mean = acc / T
    step_size = s2[:, None].astype(np.float64)
    # E[s q'] = w up to 2^-16 of a step; the sample mean has std <= step/(2 sqrt(T)).
    z = (mean - w) / (step_size / (2 * np.sqrt(T)))
    assert np.abs(z).max() < 5.5
    assert abs(z.mean()) < 0.3                          # no systematic bias


def test_zero_lr_changes_are_rare_and_small(orc):
    rng = np.random.default_rng(5)
    q = rng.integers(-127, 128, size=(64, 256)).astype(np.int8)
    q[:, 0] = -127                        # a quantized row always holds its +-127
    s = rng.uniform(1e-4, 1e-1, 64).astype(np.float32)
    q2, s2, _ = orc.sgd_requant(q, s, np.zeros((64, 256), np.float32), 0.0, seed=1, step=0)
    d = q2.astype(np.int32) - q
    assert np.abs(d).max() <= 1 and (d != 0).mean() < 0.05


def test_zero_row_and_bias(orc):
    q = np.zeros((2, 16), np.int8)
    q[1, :] = 10
    s = np.array([0.5, 0.25], np.float32)
    dw = np.zeros((2, 16), np.float32)
    bias = np.array([1.0, -2.0], np.float32)
    db = np.array([4.0, -8.0], np.float32)
    q2, s2, b2 = orc.sgd_requant(q, s, dw, 0.25, seed=0, step=0, bias=bias, db=db)
    assert s2[0] == 0 and np.all(q2[0] == 0)
    assert np.all(q2[1] == 127) and s2[1] == np.float32(2.5) / np.float32(127)
    assert b2.tolist() == [0.0, 0.0]


def test_seed_and_step_select_the_stream(orc):
    rng = np.random.default_rng(6)
    q = rng.integers(-127, 128, size=(8, 128)).astype(np.int8)
    s = rng.uniform(1e-3, 1e-2, 8).astype(np.float32)
    dw = rng.standard_normal((8, 128)).astype(np.float32)
    a = orc.sgd_requant(q, s, dw, 1e-3, seed=1, step=5)[0]
    b = orc.sgd_requant(q, s, dw, 1e-3, seed=1, step=5)[0]
    c = orc.sgd_requant(q, s, dw, 1e-3, seed=1, step=6)[0]
    d = orc.sgd_requant(q, s, dw, 1e-3, seed=2, step=5)[0]
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_row_ids_key_the_stream(orc):
    """Updating selected rows with their global ids equals updating the full matrix."""
    rng = np.random.default_rng(7)
    q = rng.integers(-127, 128, size=(9, 64)).astype(np.int8)
    s = rng.uniform(1e-3, 1e-2, 9).astype(np.float32)
    dw = rng.standard_normal((9, 64)).astype(np.float32)
    qf, sf, _ = orc.sgd_requant(q, s, dw, 1e-2, seed=4, step=2)
    rows = np.array([8, 3, 5])
    qs, ss, _ = orc.sgd_requant(q[rows], s[rows], dw[rows], 1e-2, seed=4, step=2, row_ids=rows)
    assert np.array_equal(qs, qf[rows]) and np.array_equal(ss, sf[rows])
