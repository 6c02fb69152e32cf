"""Pins of the oracle's block-Hadamard rotation (OneTrainer PR #1681: rotation
along the contraction dimension; orthogonal rotation buffer; the identity
(xR)(WR)^T = xW^T that lets the weight stay in the rotated basis)."""
import numpy as np
import pytest
import scipy.linalg

from tests.golden import read_kv
import workloads

BLOCKS = [2, 4, 8, 16, 32, 64, 128, 256, 512]


def _ref_rotate(x, b):
    """float64 block rotation with scipy's Sylvester Hadamard matrix."""
    H = scipy.linalg.hadamard(b).astype(np.float64) / np.sqrt(b)
    rows, cols = x.shape
    xb = x.astype(np.float64).reshape(rows, cols // b, b)
    return (xb @ H).reshape(rows, cols)


@pytest.mark.parametrize("b", BLOCKS)
def test_matches_scipy_hadamard(orc, b):
    rng = np.random.default_rng(b)
    x = rng.standard_normal((5, 3 * b)).astype(np.float32)
    y = orc.hadamard(x, b)
    ref = _ref_rotate(x, b)
    # fp32 butterfly: log2(b) rounded stages plus one scaling; errors scale
    # with the block's 2-norm.  A wrong sign or index gives O(1) errors.
    nrm = np.linalg.norm(x.astype(np.float64).reshape(5, 3, b), axis=2)
    bound = (np.log2(b) + 2) * 2.0 ** -23 * np.repeat(nrm, b, axis=1)
    assert np.all(np.abs(y - ref) <= bound)


def test_orthogonality_page_value(orc):
    g = read_kv("hadamard_orthogonality.txt")
    b = int(g["block"])
    R = orc.hadamard(np.eye(b, dtype=np.float32), b)
    dev = float(np.abs(R @ R.T - np.eye(b, dtype=np.float32)).max())
    assert dev <= 1e-6
    assert f"{dev:.2e}" == g["max_abs_deviation"]
    # Every entry is +-c_b exactly: the butterfly of a one-hot row is exact.
    assert np.all(np.abs(R) == np.float32(orc.hadamard_scale(b)))


def test_scale_constant(orc):
    for b in BLOCKS:
        c = orc.hadamard_scale(b)
        assert c == float(np.float32(1.0 / np.sqrt(np.float64(b))))
    assert np.float32(orc.hadamard_scale(128)).view(np.uint32) == 0x3DB504F3


@pytest.mark.parametrize("b", [2, 16, 128])
def test_involution(orc, b):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 2 * b)).astype(np.float32)
    back = orc.hadamard(orc.hadamard(x, b), b)
    assert np.max(np.abs(back - x)) <= 4 * np.log2(b) * 2.0 ** -23 * np.abs(x).max() * np.sqrt(b)


def test_rotation_identity_xw(orc):
    """(xR)(WR)^T == x W^T (OneTrainer PR #1681, commit note 2)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    w = rng.standard_normal((5, 256)).astype(np.float32)
    lhs = orc.hadamard(x, 128).astype(np.float64) @ orc.hadamard(w, 128).astype(np.float64).T
    rhs = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.max(np.abs(lhs - rhs)) < 1e-4


def test_block_independence(orc):
    """Each block is rotated on its own: changing block 1 leaves block 0 alone."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 256)).astype(np.float32)
    y0 = orc.hadamard(x, 128)
    x2 = x.copy()
    x2[:, 128:] += 1.0
    y1 = orc.hadamard(x2, 128)
    assert np.array_equal(y0[:, :128], y1[:, :128])
    assert not np.array_equal(y0[:, 128:], y1[:, 128:])


def test_bf16_input_is_exact_decode(orc):
    rng = np.random.default_rng(5)
    xb = workloads.f32_to_bf16_bits(rng.standard_normal((3, 256)).astype(np.float32))
    assert np.array_equal(orc.hadamard(xb, 64), orc.hadamard(workloads.bf16_bits_to_f32(xb), 64))


@pytest.mark.parametrize("b,cols", [(3, 12), (1, 8), (1024, 1024), (128, 192), (0, 16)])
def test_rejects_bad_blocks(orc, b, cols):
    with pytest.raises(orc.OracleError):
        orc.hadamard(np.zeros((1, cols), np.float32), b)


def test_bf16_cast_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(4096) * 10).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.f32_to_bf16_bits(x), ref)
