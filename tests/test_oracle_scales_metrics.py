"""Pins of the oracle's error metrics and of its FP8 tensor-scale rules.

* mse, rel_mse, rel_l2 against hand-worked fractions (tests/golden/
  metrics_examples.txt).
* The data-driven tensor scale ([TACO] Fig. 7, "adaptive rescaling"; reading:
  g = RN(A / M), A the abs-max of the transformed tensor, M = 448 for E4M3 and
  57344 for E5M2): on inputs whose transformed abs-max A is known in closed
  form, g must be the float32 nearest to A / M in exact rational arithmetic;
  on random inputs the element holding A must dequantize to exactly RN(M * g)
  (its scaled value rounds to the format's largest code whichever block
  exponent the rounding of g gives it).
* The clamps of g and of the gather-stage g' = g_0 + ... + g_{N-1} to
  [2^-60, 2^60], and the in-order float32 sum of g'.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import codecs as cd
from oracle.formats import bf16_bits_to_f32, f32_to_bf16_bits
import workloads as W
from tests.conftest import read_golden

F32 = np.float32


def _vec(s):
    return np.array([float(Fraction(v)) for v in s.split(",")], dtype=np.float64)


def test_metrics_golden():
    rows = read_golden("metrics_examples.txt")
    assert len(rows) >= 4
    for name, a, b, mse, rmse, rl2 in rows:
        a, b = _vec(a), _vec(b)
        assert oracle.mse(a, b) == pytest.approx(float(Fraction(mse)), rel=1e-15, abs=0), name
        assert oracle.rel_mse(a, b) == pytest.approx(float(Fraction(rmse)), rel=1e-15, abs=0), name
        assert oracle.rel_l2(a, b) == pytest.approx(float(Fraction(rl2)), rel=1e-15, abs=0), name


def test_metrics_accept_float32_and_shapes():
    # the metrics widen to float64 before squaring: float32 inputs whose
    # squares overflow float32 still give the exact ratio
    a = np.full((2, 3), 3e30, np.float32)
    b = np.full((2, 3), 1e30, np.float32)
    assert oracle.rel_mse(a, b) == pytest.approx(4.0, rel=1e-6)
    assert oracle.mse(np.zeros(0), np.zeros(0)) == 0.0


def _nearest_f32(q: Fraction):
    """The float32 nearest to the rational q > 0, ties to the even mantissa,
    found by exact comparison of neighbouring candidates."""
    c = F32(float(q))
    cands = [np.nextafter(c, F32(0)), c, np.nextafter(c, F32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - q), int(np.asarray(v).view(np.uint32)) & 1))
    return F32(best)


def _two_spike_tensor(a, b, c):
    """Three rows of 256 (two 128-blocks each), zero except: row 0 block 0 holds
    a at index 0 and b at index 1; row 2 block 1 holds c at index 0. The
    Sylvester transform of the first block is a + b or a - b at every index
    (column 1 of H_128 alternates in sign), of the second c at every index:
    the transformed abs-max is max(|a| + |b|, |c|) when a and b have opposite
    signs."""
    x = np.zeros((3, 256), np.float32)
    x[0, 0], x[0, 1], x[2, 128] = a, b, c
    bits = f32_to_bf16_bits(x)
    assert (bf16_bits_to_f32(bits) == x).all(), "the spikes must be exact in bf16"
    return bits


@pytest.mark.parametrize("fmt,M", [(cd.FP8_DUAL, 448), (cd.FP8E5_DUAL, 57344)])
def test_auto_tensor_scale_is_the_nearest_float_to_transformed_absmax_over_M(fmt, M):
    # a = -3 * 2^-5, b = 2.75 * 2^-5: the transformed abs-max is 5.75 * 2^-5.
    # The untransformed abs-max (c = 2^-3) and the signed maximum of the
    # transformed values (also c) are both smaller, so taking either gives a
    # different g.
    a, b, c = -3 * 2.0 ** -5, 2.75 * 2.0 ** -5, 2.0 ** -3
    A = Fraction(5.75) * Fraction(1, 32)
    codec = cd.Codec(fmt, 128, True)
    comp = oracle.compress(codec, _two_spike_tensor(a, b, c))
    want = _nearest_f32(A / M)
    assert comp.tensor_scale.view(np.uint32) == want.view(np.uint32), (comp.tensor_scale, want)
    # without the transform the abs-max is max(|a|, |b|, |c|) = c
    comp0 = oracle.compress(cd.Codec(fmt, 128, False), _two_spike_tensor(a, b, c))
    assert comp0.tensor_scale.view(np.uint32) == _nearest_f32(Fraction(c) / M).view(np.uint32)


# seeds 800-802: the abs-max block gets k = 0 (its scaled maximum rounds to
# at most M and encodes to the largest code); seeds 812, 828, 840: the
# rounding of g and 1/g leaves the scaled maximum just above M, the block
# exponent is -1 and the value encodes to M / 2, which 2^-k brings back to M
@pytest.mark.parametrize("fmt,M", [(cd.FP8_DUAL, 448.0), (cd.FP8E5_DUAL, 57344.0)])
@pytest.mark.parametrize("seed,k", [(800, 0), (801, 0), (802, 0), (812, -1), (828, -1), (840, -1)])
def test_absmax_element_dequantizes_to_M_times_g(fmt, M, seed, k):
    codec = cd.Codec(fmt, 128, True)
    x = W.random_bits((32, 512), seed=seed, sigma=0.02, body="t3")
    comp = oracle.compress(codec, x)
    y = cd.transform(codec, x).reshape(-1)
    i = int(np.argmax(np.abs(y)))
    assert comp.scale[i // 128] == k
    dq = oracle.dequantize(comp)
    g = comp.tensor_scale
    assert abs(dq[i]) == F32(F32(M) * g), (dq[i], M, g)
    assert np.sign(dq[i]) == np.sign(y[i])
    # and no dequantized value exceeds it
    assert np.max(np.abs(dq)) == F32(F32(M) * g)


@pytest.mark.parametrize("fmt", [cd.FP8_DUAL, cd.FP8E5_DUAL])
def test_tensor_scale_clamps(fmt):
    codec = cd.Codec(fmt, 128, True)
    # transformed abs-max 2^-100: A / M is far below 2^-60
    tiny = _two_spike_tensor(2.0 ** -100, 0.0, 0.0)
    assert oracle.compress(codec, tiny).tensor_scale == F32(2.0 ** -60)
    # transformed abs-max 2^100: A / M is far above 2^60
    huge = _two_spike_tensor(2.0 ** 100, 0.0, 0.0)
    c = oracle.compress(codec, huge)
    assert c.tensor_scale == F32(2.0 ** 60)
    # the clamped scale still brings every block into range: the spike
    # dequantizes to itself (a power of two, exact through every step)
    assert np.max(np.abs(oracle.dequantize(c))) == F32(2.0 ** 100)
    # an all-zero tensor takes g = 1
    assert oracle.compress(codec, np.zeros((2, 128), np.uint16)).tensor_scale == F32(1.0)


def test_gather_scale_sum_order_and_clamps():
    # sequential float32 sum: 1 + 2^-24 rounds back to 1 (a tie, to even)
    # twice, whereas summing the two small terms first would give 1 + 2^-23
    assert cd.sum_tensor_scales([1.0, 2.0 ** -24, 2.0 ** -24]) == F32(1.0)
    assert cd.sum_tensor_scales([2.0 ** -24, 2.0 ** -24, 1.0]) == F32(1.0 + 2.0 ** -23)
    assert cd.sum_tensor_scales([0.5, 0.25, 0.125]) == F32(0.875)
    assert cd.sum_tensor_scales([2.0 ** 60, 2.0 ** 60]) == F32(2.0 ** 60)
    assert cd.sum_tensor_scales([2.0 ** -61]) == F32(2.0 ** -60)
