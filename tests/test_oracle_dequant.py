"""Pins of the oracle's weight export: the represented weight fl(s * q),
rotated back to the original basis (OneTrainer PR #1681, commit note 2:
callers that need the unquantized weight un-rotate it; the rotation is
orthogonal and its own inverse)."""
import numpy as np
import pytest
from scipy.linalg import hadamard

import workloads


def test_no_rotation_is_the_scaled_codes(orc):
    rng = np.random.default_rng(0)
    q = rng.integers(-127, 128, (16, 64)).astype(np.int8)
    s = rng.uniform(1e-4, 1e-1, 16).astype(np.float32)
    assert np.array_equal(orc.dequantize_weight(q, s), s[:, None] * q.astype(np.float32))


@pytest.mark.parametrize("b", [2, 16, 128, 512])
def test_rotation_matches_the_hadamard_matrix(orc, b):
    rng = np.random.default_rng(b)
    N, K = 8, 1024
    q = rng.integers(-127, 128, (N, K)).astype(np.int8)
    s = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    w = orc.dequantize_weight(q, s, had_block=b)
    H = hadamard(b).astype(np.float64) / np.sqrt(b)
    base = (s[:, None] * q.astype(np.float32)).astype(np.float64)
    ref = (base.reshape(N, K // b, b) @ H).reshape(N, K)
    mag = (np.abs(base).reshape(N, K // b, b).sum(axis=2, keepdims=True) / np.sqrt(b))
    tol = (np.log2(b) + 2) * 2.0 ** -24 * np.broadcast_to(mag, (N, K // b, b)).reshape(N, K)
    assert np.all(np.abs(w - ref) <= tol)


@pytest.mark.parametrize("b", [0, 128])
def test_round_trip_error_bound(orc, b):
    """prepare (rotate, quantize) then export: within the quantization error,
    which the orthogonal rotation carries over unchanged in norm."""
    d = workloads.linear(4, 256, 64, with_dy=False, had_block=b, seed=3)
    w = d["w"]
    q, s = orc.prepare_weight(w, had_block=b)
    back = orc.dequantize_weight(q, s, had_block=b)
    blk = b if b else 1
    err = (back - w).astype(np.float64).reshape(64, -1, blk)
    norm = np.sqrt((err ** 2).sum(axis=2))
    bound = (s.astype(np.float64)[:, None] / 2) * np.sqrt(blk) * (1 + 1e-5) + 1e-7
    assert np.all(norm <= bound)
    assert np.abs(back - w).max() > 0       # the export is lossy, as expected
