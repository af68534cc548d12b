"""Pins of the oracle's block Walsh-Hadamard transform. CPU only."""

import numpy as np
import pytest
import scipy.linalg

from oracle.hadamard import fwht, fwht_f64
from tests.conftest import read_golden


def test_fwht_golden_examples():
    for row in read_golden("fwht_examples.txt"):
        txt = " ".join(row)
        b, xin, xout = [p.strip() for p in txt.split("|")]
        B = int(b)
        x = np.array([float(t) for t in xin.split()], np.float32)
        y = np.array([float(t) for t in xout.split()], np.float32)
        assert (fwht(x, B) == y).all(), (B, fwht(x, B), y)


@pytest.mark.parametrize("B", [2, 4, 8, 16, 32, 64, 128])
def test_fwht_equals_dense_sylvester_matrix(B):
    """Small-integer inputs keep every float32 sum exact, so the butterflies must
    equal scipy's dense Sylvester matrix product exactly."""
    rng = np.random.default_rng(B)
    x = rng.integers(-1000, 1000, size=(37, B)).astype(np.float32)
    H = scipy.linalg.hadamard(B).astype(np.float64)
    assert (fwht(x, B).astype(np.float64) == x.astype(np.float64) @ H.T).all()


@pytest.mark.parametrize("B", [16, 128])
def test_fwht_orthogonality_and_involution(B):
    I = np.eye(B, dtype=np.float32)
    H = fwht(I, B).astype(np.float64)        # rows are H e_i = columns of H
    assert (H @ H.T == B * np.eye(B)).all()   # H H^T = B I
    rng = np.random.default_rng(1)
    x = rng.integers(-50, 50, size=(9, B)).astype(np.float32)
    assert (fwht(fwht(x, B), B) == B * x).all()


def test_fwht_blocks_are_independent():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    y = fwht(x, 128)
    for b in range(4):
        assert (y[:, 128 * b:128 * (b + 1)] == fwht(x[:, 128 * b:128 * (b + 1)], 128)).all()


def test_fwht_float32_rounding_is_small_and_parseval_holds():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((1000, 128)) * 0.02).astype(np.float32)
    y32 = fwht(x, 128).astype(np.float64)
    y64 = fwht_f64(x.astype(np.float64), 128)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    assert np.allclose(y64, x.astype(np.float64) @ H.T, rtol=1e-12, atol=1e-15)
    # seven roundings of sums whose magnitude is at most ||x||_1
    bound = 7 * 2.0 ** -24 * np.sum(np.abs(x), axis=1, dtype=np.float64)[:, None]
    assert np.all(np.abs(y32 - y64) <= bound)
    ratio = np.sum(y32 ** 2, axis=1) / (128 * np.sum(x.astype(np.float64) ** 2, axis=1))
    assert np.allclose(ratio, 1.0, rtol=1e-5)
