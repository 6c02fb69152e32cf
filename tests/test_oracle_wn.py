"""Pins of the oracle's row weight normalization (mini_trainer guide, feature
table: an INT8 direction and a floating magnitude per output row; zero
directions rejected).  The represented weight is W = g v / ||v|| with v = s q.

The gradients are checked against central finite differences of that map in
float64 (an independent route to the same derivatives), the direction
gradient against its orthogonality to v, the pairwise dot product against an
exactly rounded sum, the preparation against the absmax weight it starts
from, and the update against its closed forms and the unbiasedness of the
stochastic rounding."""
import math

import numpy as np
import pytest


def _row_state(rng, N, K):
    q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    q[:, 0] = 127                      # full-range rows (absmax code 127)
    s = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    g = rng.uniform(0.5, 2.0, N).astype(np.float32)
    dw = (rng.standard_normal((N, K)) * 1e-2).astype(np.float32)
    return q, s, g, dw


def _loss(g, v, G):
    """Linear loss <W, G> of the represented weight W = g v / ||v||, float64."""
    return float(np.dot(g * v / np.linalg.norm(v), G))


@pytest.mark.parametrize("K", [16, 48, 160])
def test_gradients_match_finite_differences(orc, K):
    rng = np.random.default_rng(K)
    q, s, g, dw = _row_state(rng, 3, K)
    dg, dv = orc.wn_grads(q, s, g, dw)
    for n in range(3):
        v = s[n].astype(np.float64) * q[n].astype(np.float64)
        G = dw[n].astype(np.float64)
        gn = float(g[n])
        h = 1e-6 * gn
        fd_g = (_loss(gn + h, v, G) - _loss(gn - h, v, G)) / (2 * h)
        assert abs(dg[n] - fd_g) <= 1e-5 * abs(fd_g) + 1e-9
        fd_v = np.empty(K)
        for k in range(K):
            e = np.zeros(K)
            hv = 1e-6 * max(abs(v[k]), float(s[n]))
            e[k] = hv
            fd_v[k] = (_loss(gn, v + e, G) - _loss(gn, v - e, G)) / (2 * hv)
        scale = np.abs(fd_v).max()
        assert np.abs(dv[n] - fd_v).max() <= 1e-4 * scale


def test_direction_gradient_is_orthogonal_to_the_direction(orc):
    rng = np.random.default_rng(7)
    q, s, g, dw = _row_state(rng, 16, 5376)
    _, dv = orc.wn_grads(q, s, g, dw)
    qf = q.astype(np.float64)
    dvf = dv.astype(np.float64)
    inner = np.abs((dvf * qf).sum(1))
    bound = 1e-5 * np.linalg.norm(dvf, axis=1) * np.linalg.norm(qf, axis=1)
    assert np.all(inner <= bound)


@pytest.mark.parametrize("K", [16, 2064, 5376])
def test_magnitude_gradient_is_the_exact_dot_product(orc, K):
    """dg = fl(dot / ||q||) with dot within one fp32 rounding of the exactly
    rounded sum of dW_k q_k (the pairwise double sum is far more precise)."""
    rng = np.random.default_rng(K + 1)
    q, s, g, dw = _row_state(rng, 8, K)
    dg, _ = orc.wn_grads(q, s, g, dw)
    for n in range(8):
        exact = math.fsum(float(a) * float(b) for a, b in zip(dw[n], q[n]))
        nrm = np.float32(math.sqrt(int((q[n].astype(np.int64) ** 2).sum())))
        ref = np.float32(np.float32(exact) / nrm)
        assert abs(int(dg[n].view(np.int32)) - int(ref.view(np.int32))) <= 2


def test_norm_of_codes_is_exact(orc):
    """||q|| for rows whose sum of squares is a perfect square: g / sw."""
    q = np.zeros((2, 32), np.int8)
    q[0, :4] = [3, 4, 0, 0]            # norm 5
    q[1, :2] = [127, 127]              # norm 127 sqrt(2)
    s = np.ones(2, np.float32)
    g, sw = orc.wn_init(q, s)
    assert g[0] == np.float32(5.0)
    assert g[1] == np.float32(127 * math.sqrt(2))


def test_init_represents_the_absmax_weight(orc):
    rng = np.random.default_rng(3)
    q, s, _, _ = _row_state(rng, 64, 256)
    g, sw = orc.wn_init(q, s)
    norms = np.linalg.norm(q.astype(np.float64), axis=1)
    assert np.allclose(g, s.astype(np.float64) * norms, rtol=2e-7, atol=0)
    ulps = np.abs(sw.view(np.int32).astype(np.int64) - s.view(np.int32).astype(np.int64))
    assert ulps.max() <= 2


def test_init_rejects_zero_directions(orc):
    q = np.ones((3, 16), np.int8)
    q[1] = 0
    with pytest.raises(orc.OracleError):
        orc.wn_init(q, np.ones(3, np.float32))


def test_zero_lr_step_keeps_the_state(orc):
    rng = np.random.default_rng(5)
    q, s, g, dw = _row_state(rng, 32, 128)
    q2, s2, g2, sw2, _ = orc.wn_sgd_requant(q, s, g, dw, 0.0, seed=9, step=1)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2, s)
    assert np.array_equal(g2, g)
    nrm = np.sqrt((q.astype(np.int64) ** 2).sum(1).astype(np.float64)).astype(np.float32)
    assert np.array_equal(sw2, g / nrm)


def test_step_closed_forms(orc):
    """g' = fl(g - fl(lr dg)); s' is the absmax scale of w = fl(fl(s q) -
    fl(lr dv)); codes are floor or ceil of w / s'; sw' = fl(g' / ||q'||)."""
    rng = np.random.default_rng(11)
    q, s, g, dw = _row_state(rng, 16, 256)
    lr = np.float32(0.05)
    dg, dv = orc.wn_grads(q, s, g, dw)
    q2, s2, g2, sw2, _ = orc.wn_sgd_requant(q, s, g, dw, lr, seed=1, step=3)
    assert np.array_equal(g2, g - lr * dg)
    w = s[:, None] * q.astype(np.float32) - lr * dv
    assert np.array_equal(s2, np.abs(w).max(1) / np.float32(127))
    y = w / s2[:, None]
    assert np.all((q2 == np.floor(y)) | (q2 == np.ceil(y)))
    nrm = np.sqrt((q2.astype(np.int64) ** 2).sum(1).astype(np.float64)).astype(np.float32)
    assert np.array_equal(sw2, g2 / nrm)


def test_requant_of_the_direction_is_unbiased(orc):
    """Over many seeds the mean represented direction s' q' is the float
    update w (stochastic rounding is unbiased), to within its sampling error."""
    rng = np.random.default_rng(13)
    q, s, g, dw = _row_state(rng, 1, 64)
    lr = np.float32(0.2)
    _, dv = orc.wn_grads(q, s, g, dw)
    w = (s[:, None] * q.astype(np.float32) - lr * dv)[0].astype(np.float64)
    acc = np.zeros(64)
    T = 400
    for seed in range(T):
        q2, s2, _, _, _ = orc.wn_sgd_requant(q, s, g, dw, lr, seed=seed, step=1)
        acc += s2[0] * q2[0].astype(np.float64)
    mean = acc / T
    step = np.abs(w).max() / 127
    assert np.abs(mean - w).max() <= 4 * step * 0.5 / math.sqrt(T)


def test_bias_step(orc):
    rng = np.random.default_rng(17)
    q, s, g, dw = _row_state(rng, 8, 32)
    b = rng.standard_normal(8).astype(np.float32)
    db = rng.standard_normal(8).astype(np.float32)
    lr = np.float32(0.01)
    _, _, _, _, b2 = orc.wn_sgd_requant(q, s, g, dw, lr, seed=1, step=1, bias=b, db=db)
    assert np.array_equal(b2, b - lr * db)
