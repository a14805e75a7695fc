"""Pins of the oracle's channel rotation against things other than itself: a worked
example written by hand, the library Hadamard matrix, orthogonality, the involution,
dot-product preservation, the spread of one outlier channel, and the purpose of the
pre-pass (lower quantization error on data with an outlier channel)."""
import os
import numpy as np
import pytest
import scipy.linalg

from oracle import rotate as RO
from oracle import quant as Q

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_examples():
    n = 0
    for line in open(os.path.join(GOLD, "hadamard_d4.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("|")
        x = np.array([float(t) for t in lhs.split()])
        y = np.array([float(t) for t in rhs.split()])
        assert np.allclose(RO.rotate_rows(x), y, rtol=0, atol=1e-15), (x, y)
        n += 1
    assert n == 3


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 64, 128, 256])
def test_matrix_is_the_library_hadamard_and_orthogonal(d):
    h = RO.hadamard(d)
    assert np.array_equal(h, scipy.linalg.hadamard(d))
    assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_involution_and_dot_products(d):
    rng = np.random.default_rng(d)
    x, y = rng.standard_normal((5, d)), rng.standard_normal((5, d))
    rx, ry = RO.rotate_rows(x), RO.rotate_rows(y)
    assert np.allclose(RO.rotate_rows(rx), x, rtol=0, atol=1e-12)
    assert np.allclose((rx * ry).sum(-1), (x * y).sum(-1), rtol=1e-12, atol=1e-12)
    assert np.allclose(np.linalg.norm(rx, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
def test_one_outlier_channel_is_spread(d):
    for c in (0, 5, d - 1):
        e = np.zeros(d)
        e[c] = 10.0
        r = RO.rotate_rows(e)
        assert np.allclose(np.abs(r), 10.0 / np.sqrt(d), rtol=0, atol=1e-12)


def test_rotation_lowers_quantization_error_on_outlier_channels():
    """The pre-pass's purpose: 2-bit per-token V groups of 64 channels over rows with one
    channel scaled by 10 lose less (relative L2 error of the dequantized rows) when the
    rows are rotated first and rotated back after dequantization."""
    rng = np.random.default_rng(7)
    N, d, G = 256, 128, 64
    v = rng.standard_normal((N, d)).astype(np.float32)
    v[:, 17] *= 10.0
    v = Q.bf16_round(v)

    def err(x):
        codes, s, z = Q.quantize_v(x, 2, G, "f32")
        return Q.dequantize_v(codes, s, z, G)

    plain = err(v)
    rv = Q.bf16_round(RO.rotate_rows(v).astype(np.float32))
    rot = RO.rotate_rows(err(rv))
    rel = lambda a: np.linalg.norm(a - v) / np.linalg.norm(v)
    assert rel(rot) < 0.8 * rel(plain), (rel(rot), rel(plain))
