"""Block Walsh-Hadamard transform: the Hadamard part of TACO's ASH transform.

Test infrastructure only (see the package docstring).

[TACO] Fig. 7 applies an "ASH transform" after adaptive rescaling and before
dual-scale quantization; Fig. 8 shows the distribution before and after a
Hadamard-based transform; Fig. 13 compares against a "standard Hadamard".
The pages give neither normalisation, block size nor evaluation order.
Readings: the unnormalised Sylvester matrix (entries +-1, natural order) on
each contiguous block of B elements along the hidden dimension; the 1/B of
the inverse is an exact power of two and the forward 1/sqrt(B) is left to the
tensor scale. Evaluation order (it fixes the float32 rounding): butterflies
with half-width h = 1, 2, 4, ..., B/2, each pair (i, i + h) with i & h == 0
becoming (y[i] + y[i+h], y[i] - y[i+h]).
"""

import numpy as np


def _butterflies(y, B):
    h = 1
    while h < B:
        # index i = j*2h + t*h + r, t = the bit of weight h
        v = y.reshape(-1, B // (2 * h), 2, h)
        a = v[:, :, 0, :]
        b = v[:, :, 1, :]
        y = np.stack([a + b, a - b], axis=2).reshape(-1, B)
        h *= 2
    return y


def fwht(x, B):
    """Unnormalised FWHT of every contiguous B-block of ``x``, in float32.

    ``x`` is any float32 array whose last-axis length is a multiple of B.
    Returns an array of the same shape. B must be a power of two.
    """
    x = np.asarray(x, dtype=np.float32)
    assert B >= 1 and (B & (B - 1)) == 0 and x.shape[-1] % B == 0
    shape = x.shape
    y = _butterflies(x.reshape(-1, B).astype(np.float32), B)
    return y.astype(np.float32).reshape(shape)


def fwht_f64(x, B):
    """The same transform in float64 (used by tests as a higher-precision check)."""
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape
    return _butterflies(x.reshape(-1, B), B).reshape(shape)
