"""Bit-exact second implementations of the oracle's fp32 readings.

The oracle's floating-point steps are fixed operation by operation (the
readings of the pages it states in its header).  Each test here recomputes
one of them with numpy float32 arrays, whose elementwise operations are single
IEEE binary32 roundings (division included, and ``np.rint`` rounds half to
even), and compares every bit.  Each test also checks that a plausible
misreading of the same step changes the result on its data, so a mistake of
that kind in the oracle would fail here.

Passages: OneTrainer PR #1681, summary and verification paragraph (a
block-Hadamard rotation along the contraction dimension, an orthogonal
rotation buffer; per-row activation quantization, absmax / 127 with
round-half-even in the tiny workload); mini_trainer "quantized-training" guide,
opening paragraph and update paragraph (integer products with float scales;
stochastic requantization of the represented weight on update).  Philox4x32-10
follows Salmon et al., "Parallel random numbers: as easy as 1, 2, 3" (SC'11);
it is compared here with Triton's implementation run by Triton's CPU
interpreter.
"""
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import workloads

F = np.float32
BLOCKS = [2, 4, 8, 16, 32, 64, 128, 256, 512]
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32 if a.dtype == np.float32 else np.uint8)


# ------------------------------------------------------------------ rotation

def rotate_replica(x, b, ascending=True):
    """Block butterfly in float32: stride h pairs i and i + h (bit h of i
    clear) into (lo + hi, lo - hi); strides ascending; then one multiply by
    fl32(1 / sqrt(b))."""
    y = np.array(x, F, copy=True)
    rows, cols = y.shape
    strides = []
    h = 1
    while h < b:
        strides.append(h)
        h *= 2
    for h in (strides if ascending else strides[::-1]):
        v = y.reshape(rows, cols // b, b // (2 * h), 2, h)
        lo = v[..., 0, :].copy()
        hi = v[..., 1, :].copy()
        v[..., 0, :] = lo + hi
        v[..., 1, :] = lo - hi
    return y * F(1.0 / np.sqrt(np.float64(b)))


@pytest.mark.parametrize("b", BLOCKS)
def test_rotation_replica(orc, b):
    rng = np.random.default_rng(100 + b)
    x = (rng.standard_normal((6, 2 * b)) * rng.uniform(1e-3, 1e3, (6, 1))).astype(F)
    ref = rotate_replica(x, b)
    assert np.array_equal(bits(orc.hadamard(x, b)), bits(ref))
    xb = workloads.f32_to_bf16_bits(x)
    assert np.array_equal(bits(orc.hadamard(xb, b)),
                          bits(rotate_replica(workloads.bf16_bits_to_f32(xb), b)))
    if b >= 4:
        # The stage order fixes the rounding: descending strides differ.
        assert not np.array_equal(bits(ref), bits(rotate_replica(x, b, ascending=False)))


# ---------------------------------------------------------------- quantizers

def quant_replica(g):
    """Rows of g (float32): s = fl(amax / 127), q = clamp(rne(fl(g / s))),
    all-zero rows give s = 0, q = 0."""
    s = (np.abs(g).max(axis=1) / F(127)).astype(F)
    safe = np.where(s == 0, F(1), s).astype(F)
    q = np.clip(np.rint(g / safe[:, None]), -127, 127)
    q[s == 0] = 0
    return q.astype(np.int8), s


def quant_reciprocal(g):
    """The same with g * fl(1 / s) in place of the division."""
    s = (np.abs(g).max(axis=1) / F(127)).astype(F)
    r = (F(1) / np.where(s == 0, F(1), s)).astype(F)
    return np.clip(np.rint(g * r[:, None]), -127, 127).astype(np.int8)


def near_ties(rng, rows, cols):
    """Rows whose values sit within a few ulps of (k + 1/2) s, with s the
    row's own scale: where the quotient's last bit decides the code."""
    amax = rng.uniform(0.5, 2.0, rows).astype(F) * np.ldexp(F(1), rng.integers(-20, 20, rows))
    s = (amax / F(127)).astype(F)
    k = rng.integers(-127, 127, (rows, cols)).astype(np.float64)
    g = ((k + 0.5) * s.astype(np.float64)[:, None]).astype(F)
    for _ in range(3):
        step = rng.integers(-1, 2, (rows, cols))
        g = np.where(step > 0, np.nextafter(g, F(np.inf)),
                     np.where(step < 0, np.nextafter(g, F(-np.inf)), g)).astype(F)
    g = np.clip(g, -amax[:, None], amax[:, None]).astype(F)
    g[:, 0] = amax
    return g


def test_quantizer_replica_random_rows(orc):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((300, 192)) * rng.uniform(1e-4, 1e4, (300, 1))).astype(F)
    x[7] = 0
    q, s = orc.quantize_rows(x)
    qr, sr = quant_replica(x)
    assert np.array_equal(q, qr) and np.array_equal(bits(s), bits(sr))


def test_quantizer_replica_near_ties(orc):
    rng = np.random.default_rng(12)
    g = near_ties(rng, 200, 256)
    q, s = orc.quantize_rows(g)
    qr, sr = quant_replica(g)
    assert np.array_equal(q, qr) and np.array_equal(bits(s), bits(sr))
    # A reciprocal multiply instead of the division moves some codes here.
    assert np.count_nonzero(quant_reciprocal(g) != qr) > 0


@pytest.mark.parametrize("b", [0, 16, 128])
def test_quantizer_replica_rotation_and_prescale(orc, b):
    """Rows are rotated first, then prescaled per column, then quantized."""
    rng = np.random.default_rng(13 + b)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((40, 512)).astype(F))
    p = rng.uniform(0.01, 3.0, 512).astype(F)
    q, s = orc.quantize_rows(x, prescale=p, had_block=b)
    xf = workloads.bf16_bits_to_f32(x)
    g = (rotate_replica(xf, b) if b else xf) * p
    qr, sr = quant_replica(g)
    assert np.array_equal(q, qr) and np.array_equal(bits(s), bits(sr))
    if b:
        # Prescaling before the rotation is another operator, other codes.
        g2 = rotate_replica(xf * p, b)
        assert not np.array_equal(quant_replica(g2)[0], qr)


def test_column_quantizer_replica(orc):
    """Columns of x * prescale[row], and the column sums of the raw x added in
    increasing row order."""
    rng = np.random.default_rng(14)
    x = workloads.f32_to_bf16_bits((rng.standard_normal((300, 96)) * 0.01).astype(F))
    p = rng.uniform(0.001, 0.1, 300).astype(F)
    q, s, cs = orc.quantize_cols(x, prescale=p, want_sum=True)
    xf = workloads.bf16_bits_to_f32(x)
    qr, sr = quant_replica(np.ascontiguousarray((xf * p[:, None]).T))
    assert np.array_equal(q, qr.T) and np.array_equal(bits(s), bits(sr))
    assert np.array_equal(bits(cs), bits(np.cumsum(xf, axis=0, dtype=F)[-1]))


# ----------------------------------------------------------------- epilogues

def _codes(rng, shape):
    return rng.integers(-127, 128, size=shape).astype(np.int8)


def test_forward_epilogue_replica(orc):
    """y = fl(fl(fl(fl32(acc) * sx[m]) * sw[n]) + b[n])."""
    rng = np.random.default_rng(15)
    M, N, K = 48, 80, 320
    qx, qw = _codes(rng, (M, K)), _codes(rng, (N, K))
    sx = rng.uniform(1e-3, 1e-1, M).astype(F)
    sw = rng.uniform(1e-4, 1e-2, N).astype(F)
    b = (rng.standard_normal(N) * 0.05).astype(F)
    acc = (qx.astype(np.int64) @ qw.astype(np.int64).T).astype(F)
    base = (acc * sx[:, None]) * sw[None, :]
    assert np.array_equal(bits(orc.fwd(qx, sx, qw, sw)), bits(base))
    assert np.array_equal(bits(orc.fwd(qx, sx, qw, sw, b)), bits(base + b[None, :]))
    # Multiplying by the product of the two scales rounds differently.
    other = acc * (sx[:, None] * sw[None, :])
    assert not np.array_equal(bits(base), bits(other))


def test_backward_epilogue_replicas(orc):
    """dX = fl(fl32(acc) * sg1[m]) (rotated basis), dW = fl(fl32(acc) * sg2[n])."""
    rng = np.random.default_rng(16)
    M, N, K = 64, 48, 96
    qg, qw, qx = _codes(rng, (M, N)), _codes(rng, (N, K)), _codes(rng, (M, K))
    sg1 = rng.uniform(1e-6, 1e-3, M).astype(F)
    sg2 = rng.uniform(1e-6, 1e-3, N).astype(F)
    i64 = lambda a: a.astype(np.int64)
    dx = (i64(qg) @ i64(qw)).astype(F) * sg1[:, None]
    dw = (i64(qg).T @ i64(qx)).astype(F) * sg2[:, None]
    assert np.array_equal(bits(orc.bwd_dx(qg, sg1, qw)), bits(dx))
    assert np.array_equal(bits(orc.bwd_dw(qg, sg2, qx)), bits(dw))


# -------------------------------------------------------------------- Philox

def _triton_blocks(ctr, key):
    pytest.importorskip("triton")
    lines = "\n".join(" ".join(str(int(v)) for v in (*c, *k)) for c, k in zip(ctr, key))
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "philox_triton_ref.py")],
                       input=lines, capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        pytest.skip(f"Triton's interpreter did not run: {r.stderr[-400:]}")
    return np.array([list(map(int, l.split())) for l in r.stdout.split("\n") if l.strip()],
                    np.uint64).astype(np.uint32)


def test_philox4x32_matches_triton(orc):
    rng = np.random.default_rng(17)
    m = 2 ** 32 - 1
    ctr = [[0, 0, 0, 0], [m, m, m, m], [1, 0, 0, 0], [0, 0, 1, 0]]
    key = [[0, 0], [m, m], [0, 0], [0, 0]]
    ctr += rng.integers(0, 2 ** 32, (60, 4), dtype=np.uint64).tolist()
    key += rng.integers(0, 2 ** 32, (60, 2), dtype=np.uint64).tolist()
    ref = _triton_blocks(ctr, key)
    got = np.array([orc.philox4x32_10(c, k) for c, k in zip(ctr, key)], np.uint32)
    assert np.array_equal(got, ref)


def test_philox_weyl_constants_share_the_golden_and_sqrt3_bits():
    """The 32-bit key increments are the top halves of the 64-bit ones (the
    fractional bits of the golden ratio and of sqrt(3) - 1), whose 4x64
    instance equals numpy's Philox."""
    src = open(os.path.join(ROOT, "oracle", "qlin_oracle.c")).read()
    inst = {}
    for m in re.finditer(r"DEFINE_PHILOX4\((\w+),[^)]*?(0x[0-9A-Fa-f]+)u?l*,\s*(0x[0-9A-Fa-f]+)u?l*,"
                         r"\s*(0x[0-9A-Fa-f]+)u?l*,\s*(0x[0-9A-Fa-f]+)u?l*\)", src):
        inst[m.group(1)] = [int(v, 16) for v in m.groups()[1:]]
    w32, w64 = inst["orc_philox4x32_10"][2:], inst["orc_philox4x64_10"][2:]
    assert w32 == [w >> 32 for w in w64]
    from fractions import Fraction
    import decimal
    decimal.getcontext().prec = 60
    phi = (decimal.Decimal(5).sqrt() - 1) / 2
    s3 = decimal.Decimal(3).sqrt() - 1
    assert w64[0] == int(phi * 2 ** 64) and w64[1] == int(s3 * 2 ** 64)


# ---------------------------------------------------------------- SGD update

def r16_replica(orc, seed, step, idx):
    """16-bit uniforms of element indices idx: half (i & 1) of word
    (i & 7) >> 1 of the Philox4x32-10 block at counter (i >> 3, step), key
    seed."""
    out = np.empty(idx.size, np.uint32)
    key = [seed & 0xFFFFFFFF, seed >> 32]
    cache = {}
    for t, i in enumerate(idx.tolist()):
        blk = i >> 3
        if blk not in cache:
            cache[blk] = orc.philox4x32_10([blk & 0xFFFFFFFF, blk >> 32, step & 0xFFFFFFFF,
                                            step >> 32], key)
        out[t] = (int(cache[blk][(i & 7) >> 1]) >> (16 * (i & 1))) & 0xFFFF
    return out


def sgd_replica(orc, qw, sw, dw, lr, seed, step, row0=0, assoc="plain"):
    N, K = qw.shape
    cur = sw[:, None] * qw.astype(F)
    if assoc == "plain":
        w = cur - F(lr) * dw                       # fl(fl(s q) - fl(lr dW))
    else:                                          # fl(s fl(q - fl(fl(lr dW) / s)))
        w = sw[:, None] * (qw.astype(F) - (F(lr) * dw) / sw[:, None])
    s1 = (np.abs(w).max(axis=1) / F(127)).astype(F)
    y = w / np.where(s1 == 0, F(1), s1)[:, None]
    f = np.floor(y)
    idx = (np.arange(N, dtype=np.int64)[:, None] + row0) * K + np.arange(K, dtype=np.int64)
    u = r16_replica(orc, seed, step, idx.ravel()).reshape(N, K).astype(F) * F(2.0 ** -16)
    q = np.clip(f + (u < (y - f)), -127, 127)
    q[s1 == 0] = 0
    return q.astype(np.int8), s1


def test_sgd_requant_replica(orc):
    rng = np.random.default_rng(18)
    N, K = 24, 600
    qw = _codes(rng, (N, K))
    sw = rng.uniform(1e-4, 1e-2, N).astype(F)
    dw = (rng.standard_normal((N, K)) * 2.0).astype(F)
    b = rng.standard_normal(N).astype(F)
    db = rng.standard_normal(N).astype(F)
    lr, seed, step = 1e-3, 0xDEADBEEF12, 5
    q, s, b1 = orc.sgd_requant(qw, sw, dw, lr, seed, step, bias=b, db=db)
    qr, sr = sgd_replica(orc, qw, sw, dw, lr, seed, step)
    assert np.array_equal(q, qr) and np.array_equal(bits(s), bits(sr))
    assert np.array_equal(bits(b1), bits(b - F(lr) * db))
    # Rows keyed by their global index (a slice of a larger weight).
    q2, s2, _ = orc.sgd_requant(qw[5:9], sw[5:9], dw[5:9], lr, seed, step,
                                row_ids=np.arange(5, 9))
    assert np.array_equal(q2, qr[5:9]) and np.array_equal(bits(s2), bits(sr[5:9]))
    # Another association of the update gives other codes or scales here.
    qa, sa = sgd_replica(orc, qw, sw, dw, lr, seed, step, assoc="scaled")
    assert not (np.array_equal(qa, qr) and np.array_equal(bits(sa), bits(sr)))


def test_sgd_requant_exact_ties(orc):
    """Every quotient's fraction equals its own uniform exactly: the rounding
    goes up only when u < frac, so each code stays at floor(y)."""
    rng = np.random.default_rng(19)
    N, K, seed, step, e = 8, 256, 77, 3, -9
    idx = (np.arange(N, dtype=np.int64)[:, None] * K + np.arange(K)).ravel()
    u = r16_replica(orc, seed, step, idx).reshape(N, K).astype(np.float64) / 65536.0
    f = rng.integers(-127, 126, (N, K)).astype(np.float64)
    y = f + u
    y[:, 0] = 127.0
    w = np.ldexp(y, e).astype(F)
    assert np.array_equal(w.astype(np.float64), np.ldexp(y, e))    # exact
    qw = np.zeros((N, K), np.int8)
    sw = np.full(N, 0.5, F)
    q, s, _ = orc.sgd_requant(qw, sw, -w, 1.0, seed, step)    # w = 0 - 1 * (-w)
    assert np.all(s == F(2.0 ** e))
    expect = f.astype(np.int64)
    expect[:, 0] = 127
    assert np.array_equal(q.astype(np.int64), expect)
    qr, _ = sgd_replica(orc, qw, sw, -w, 1.0, seed, step)
    assert np.array_equal(q, qr)
    # Most fractions are nonzero, so rounding up on u <= frac would move them.
    assert np.count_nonzero(u[:, 1:] > 0) > 0.9 * N * (K - 1)
