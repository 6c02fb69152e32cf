"""End-to-end checks of the oracle's training step against float64 brute force.

The quantized layer approximates the float layer (mini_trainer guide: integer
forward/backward products with per-row scales; OneTrainer PR #1681: the int8
route's error against the dequantized weight).  These are tolerance bands, the
exact pins live in the per-function tests."""
import hashlib
import os

import numpy as np
import pytest

import workloads
from tests.golden import read_kv, HERE as GOLDEN


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_tiny_train_step_bands(orc):
    d = workloads.tiny()
    x, w, b, dy, lr = d["x"], d["w"], d["b"], d["dy"], d["lr"]
    qw, sw = orc.prepare_weight(w)
    qx, sx = orc.quantize_rows(x)
    y = orc.fwd(qx, sx, qw, sw, b)
    w_eff = qw.astype(np.float64) * sw[:, None]
    ref_y = x.astype(np.float64) @ w_eff.T + b
    assert _rel(y, ref_y) < 2e-2                      # activation quantization only
    qg1, sg1 = orc.quantize_rows(dy, prescale=sw)
    dx = orc.bwd_dx(qg1, sg1, qw)
    assert _rel(dx, dy.astype(np.float64) @ w_eff) < 2e-2
    qg2, sg2, db = orc.quantize_cols(dy, prescale=sx, want_sum=True)
    dw = orc.bwd_dw(qg2, sg2, qx)
    x_eff = qx.astype(np.float64) * sx[:, None]
    assert _rel(dw, dy.astype(np.float64).T @ x_eff) < 2e-2
    assert np.allclose(db, dy.astype(np.float64).sum(0), atol=1e-5)
    qw2, sw2, b2 = orc.sgd_requant(qw, sw, dw, lr, seed=0, step=0, bias=b, db=db)
    w_new = qw2.astype(np.float64) * sw2[:, None]
    target = w_eff - lr * dw
    # stochastic rounding moves each weight by less than one new step
    assert np.all(np.abs(w_new - target) <= sw2[:, None] * (1 + 1e-5))
    assert np.allclose(b2, b - np.float32(lr) * db, atol=1e-7)


@pytest.mark.parametrize("rotate,lo,hi", [(True, 5e-3, 1.5e-2), (False, 2e-2, 6e-2)])
def test_accuracy_band_against_page(orc, rotate, lo, hi):
    """Activation-quantization error against the dequantized weight.

    The page reports 9.43e-03 for its int8 route with rotation; with the 1% x8
    outlier channels and no rotation the error is several times larger, which
    is what the rotation is for."""
    page = float(read_kv("accuracy_band.txt")["int8_relative_error"])
    d = workloads.linear(256, 5376, 512, seed=0)
    x = workloads.bf16_bits_to_f32(d["x"])
    blk = 128 if rotate else 0
    qw, sw = orc.prepare_weight(d["w"], had_block=blk)
    qx, sx = orc.quantize_rows(d["x"], had_block=blk)
    y = orc.fwd(qx, sx, qw, sw)
    xr = orc.hadamard(x, 128).astype(np.float64) if rotate else x.astype(np.float64)
    ref = xr @ (qw.astype(np.float64) * sw[:, None]).T
    err = _rel(y, ref)
    assert lo < err < hi
    if rotate:
        assert abs(err - page) / page < 0.25


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:32]


def tiny_step_digests(orc):
    """Digests of every output of the tiny training step (regression guard)."""
    d = workloads.tiny()
    qw, sw = orc.prepare_weight(d["w"])
    qx, sx = orc.quantize_rows(d["x"])
    y = orc.fwd(qx, sx, qw, sw, d["b"])
    qg1, sg1 = orc.quantize_rows(d["dy"], prescale=sw)
    dx = orc.bwd_dx(qg1, sg1, qw)
    qg2, sg2, db = orc.quantize_cols(d["dy"], prescale=sx, want_sum=True)
    dw = orc.bwd_dw(qg2, sg2, qx)
    qw2, sw2, b2 = orc.sgd_requant(qw, sw, dw, d["lr"], seed=0, step=0, bias=d["b"], db=db)
    return {"weight": _digest(qw, sw), "x": _digest(qx, sx), "y": _digest(y),
            "g1": _digest(qg1, sg1), "dx": _digest(dx), "g2": _digest(qg2, sg2, db),
            "dw": _digest(dw), "update": _digest(qw2, sw2, b2)}


def test_tiny_step_digests(orc):
    """The stored digests were written by tests/golden/make_golden.py from the oracle."""
    stored = read_kv("tiny_step_digests.txt")
    assert tiny_step_digests(orc) == stored
