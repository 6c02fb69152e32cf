"""Pins of the oracle's AdamW stochastic requant (mini_trainer guide, feature
table: AdamW is among the update paths with coverage on INT8 weights; the
guide gives no arithmetic, so the oracle follows the published decoupled-
weight-decay algorithm with bias-corrected moments).

The float update is checked against torch's own AdamW run in float64 from the
same represented weight, over several steps; the requant tail against the SGD
requant, which has its own pins."""
import numpy as np
import pytest
import torch

import workloads  # noqa: F401  (keeps the import layout of the other oracle tests)

LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


def f32(x):
    """The fp32 value the oracle receives, as a Python float (torch then runs
    on exactly the same hyperparameters)."""
    return float(np.float32(x))


def _state(rng, N, K):
    qw = rng.integers(-127, 128, (N, K)).astype(np.int8)
    qw[:, 0] = 127
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    return qw, sw


def _torch_step(w0, g, m0, v0, t, wd):
    """One step of torch.optim.AdamW in float64 from the given point: parameter
    w0, moments (m0, v0) after t - 1 steps.  Returns (param, exp_avg,
    exp_avg_sq)."""
    p = torch.nn.Parameter(torch.tensor(w0.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=f32(LR), betas=(f32(B1), f32(B2)), eps=f32(EPS),
                            weight_decay=f32(wd))
    opt.state[p] = {"step": torch.tensor(float(t - 1), dtype=torch.float64),
                    "exp_avg": torch.tensor(m0.astype(np.float64)),
                    "exp_avg_sq": torch.tensor(v0.astype(np.float64))}
    p.grad = torch.tensor(g.astype(np.float64))
    opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_float_update_matches_torch_adamw(orc, wd):
    rng = np.random.default_rng(3)
    N, K = 8, 96
    qw, sw = _state(rng, N, K)
    w0 = sw[:, None] * qw.astype(np.float32)
    grads = [rng.standard_normal((N, K)).astype(np.float32) * np.float32(s)
             for s in (1.0, 0.1, 3.0, 1e-3)]
    m = np.zeros((N, K), np.float32)
    v = np.zeros((N, K), np.float32)
    for t, g in enumerate(grads, start=1):
        pt, mt, vt = _torch_step(w0, g, m, v, t, wd)
        m0, v0 = m, v
        w, m, v = orc.adamw_update(qw, sw, g, m, v, LR, B1, B2, EPS, wd, t)
        # One step from the same fp32 state: a few roundings per value, i.e. a
        # few ulps of the terms it sums.
        gm = np.abs(g.astype(np.float64))
        assert np.all(np.abs(m - mt) <= 1e-6 * (B1 * np.abs(m0) + (1 - B1) * gm) + 1e-30)
        assert np.all(np.abs(v - vt) <= 1e-6 * (B2 * v0 + (1 - B2) * gm * gm) + 1e-30)
        step = np.abs(w0 * (1 - f32(LR) * f32(wd)) - pt)
        assert np.all(np.abs(w - pt) <= 1e-6 * (np.abs(w0) + step) + 1e-12)
        assert np.max(step) > 1e-4        # the update is far above that tolerance


def test_first_step_is_a_sign_step(orc):
    """t = 1 from zero moments, no decay: the step is lr * g / (|g| + eps)."""
    rng = np.random.default_rng(4)
    qw, sw = _state(rng, 4, 64)
    g = rng.standard_normal((4, 64)).astype(np.float32)
    z = np.zeros((4, 64), np.float32)
    w, m, v = orc.adamw_update(qw, sw, g, z, z, LR, B1, B2, EPS, 0.0, 1)
    w0 = (sw[:, None] * qw.astype(np.float32)).astype(np.float64)
    step = f32(LR) * g.astype(np.float64) / (np.abs(g.astype(np.float64)) + f32(EPS))
    assert np.all(np.abs((w0 - w) - step) <= 1e-6 * (np.abs(w0) + LR))
    a1, a2 = orc.adamw_constants(LR, B1, B2, 0.0, 1)[:2]
    assert np.all(m == a1 * g)
    assert np.all(v == (a2 * g) * g)


def test_constants_are_rounded_once(orc):
    a1, a2, c1, c2, decay = orc.adamw_constants(LR, B1, B2, 0.01, 5)
    b1, b2, lr = float(np.float32(B1)), float(np.float32(B2)), float(np.float32(LR))
    assert a1 == np.float32(1 - b1) and a2 == np.float32(1 - b2)
    assert c1 == np.float32(lr / (1 - b1 ** 5))
    assert c2 == np.float32(1 / np.sqrt(1 - b2 ** 5))
    assert decay == np.float32(1 - lr * float(np.float32(0.01)))


def test_zero_lr_requant_equals_sgd_requant(orc):
    """lr = 0 and no decay leave the represented weight as it is; the requant
    (scales, Philox-keyed codes) must then be exactly the SGD one at lr = 0."""
    rng = np.random.default_rng(5)
    qw, sw = _state(rng, 16, 256)
    g = rng.standard_normal((16, 256)).astype(np.float32)
    z = np.zeros_like(g)
    q_a, s_a, m, v, *_ = orc.adamw_requant(qw, sw, g, z, z, 0.0, B1, B2, EPS, 0.0, 11, 3)
    q_s, s_s, _ = orc.sgd_requant(qw, sw, z, 0.0, 11, 3)
    assert np.array_equal(q_a, q_s) and np.array_equal(s_a, s_s)
    # the moments still advance
    assert np.all(m == orc.adamw_constants(0.0, B1, B2, 0.0, 3)[0] * g)


def test_requant_uses_the_float_update(orc):
    """Codes and scales are the requant of exactly the float update."""
    rng = np.random.default_rng(6)
    qw, sw = _state(rng, 8, 128)
    g = rng.standard_normal((8, 128)).astype(np.float32)
    m = rng.standard_normal((8, 128)).astype(np.float32) * np.float32(0.1)
    v = rng.uniform(0, 1, (8, 128)).astype(np.float32)
    w, m1, v1 = orc.adamw_update(qw, sw, g, m, v, LR, B1, B2, EPS, 0.01, 4)
    q2, s2, m2, v2, *_ = orc.adamw_requant(qw, sw, g, m, v, LR, B1, B2, EPS, 0.01, 9, 4)
    assert np.array_equal(m1, m2) and np.array_equal(v1, v2)
    assert np.array_equal(s2, (np.abs(w).max(axis=1) / np.float32(127)).astype(np.float32))
    # Exact codes: floor(y) + (u < frac(y)), u from the Philox stream at step t.
    y = (w / s2[:, None]).astype(np.float32)
    f = np.floor(y)
    bits = np.array([orc.sr_bits16(9, 4, i) for i in range(w.size)], np.float32)
    u = bits.reshape(w.shape) * np.float32(2.0 ** -16)
    ref = np.clip(f + (u < (y - f)), -127, 127).astype(np.int8)
    assert np.array_equal(q2, ref)
    assert np.mean(q2 != f) > 0.2           # the random draws decide many codes


def test_bias_matches_torch_adamw(orc):
    rng = np.random.default_rng(7)
    N, K = 32, 16
    qw, sw = _state(rng, N, K)
    b = rng.standard_normal(N).astype(np.float32)
    grads = [rng.standard_normal(N).astype(np.float32) for _ in range(3)]
    p = torch.nn.Parameter(torch.tensor(b.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=f32(LR), betas=(f32(B1), f32(B2)), eps=f32(EPS),
                            weight_decay=f32(0.01))
    bm = np.zeros(N, np.float32)
    bv = np.zeros(N, np.float32)
    cur = b
    z = np.zeros((N, K), np.float32)
    for t, db in enumerate(grads, start=1):
        p.grad = torch.tensor(db.astype(np.float64))
        opt.step()
        _, _, _, _, cur, bm, bv = orc.adamw_requant(qw, sw, z, z, z, LR, B1, B2, EPS, 0.01, 0, t,
                                                    bias=cur, db=db, bm=bm, bv=bv)
        ref = p.detach().numpy()
        assert np.all(np.abs(cur - ref) <= 1e-5 * (np.abs(ref) + LR))
        with torch.no_grad():
            p.copy_(torch.tensor(cur.astype(np.float64)))
