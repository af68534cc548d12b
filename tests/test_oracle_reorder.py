"""Pins of the oracle's data-driven reshaping (chunk_order, reorder_columns,
restore_columns, compress_reordered, decode_reordered): a hand-worked order,
brute force on small inputs, ties, the exact inverse, and what the order does
to the blocks of the reordered tensor."""

import numpy as np
import pytest

import oracle
from oracle import codecs as cd
from oracle.formats import bf16_bits_to_f32, f32_to_bf16_bits
import workloads as W


def test_hand_worked_order():
    # four groups of 8 channels; their largest magnitudes over both rows are
    # 1.5 (group 0), 4 (group 1, from row 1, negative), 0.25 (group 2) and 4
    # (group 3): order 1, 3 (equal statistics by group index), 0, 2
    x = np.zeros((2, 32), np.float32)
    x[0, 3], x[1, 1] = 1.5, -1.0
    x[1, 12] = -4.0
    x[0, 17] = 0.25
    x[0, 31], x[1, 24] = 4.0, 2.0
    assert oracle.chunk_order(f32_to_bf16_bits(x)).tolist() == [1, 3, 0, 2]


@pytest.mark.parametrize("seed", range(4))
def test_order_matches_a_brute_force_sort(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((5, 64)) * rng.choice([0.01, 1.0, 30.0], size=64)).astype(np.float32)
    x[:, 8:16] = x[:, 40:48]                        # two groups with the same statistic
    bits = f32_to_bf16_bits(x)
    v = bf16_bits_to_f32(bits)
    stat = [max(abs(float(v[r, c])) for r in range(5) for c in range(8 * j, 8 * j + 8)) for j in range(8)]
    want = sorted(range(8), key=lambda j: (-stat[j], j))
    assert oracle.chunk_order(bits).tolist() == want


def test_reorder_and_restore_are_inverse_permutations():
    rng = np.random.default_rng(3)
    x = rng.integers(0, 1 << 16, size=(3, 128), dtype=np.uint16)
    order = rng.permutation(16)
    y = oracle.reorder_columns(x, order)
    assert (y[:, 8 * 5 + 2] == x[:, 8 * order[5] + 2]).all()
    assert (oracle.restore_columns(y, order) == x).all()
    assert (oracle.reorder_columns(x, np.arange(16)) == x).all()
    with pytest.raises(AssertionError):
        oracle.reorder_columns(x, np.r_[order[:-1], order[0]])        # not a permutation


def test_reordered_blocks_have_non_increasing_maxima():
    w = W.WORKLOADS["qwen-tp"]
    x = W.make_shard(w, 0, chunks=[0])
    order = oracle.chunk_order(x)
    y = bf16_bits_to_f32(oracle.reorder_columns(x, order))
    bmax = np.abs(y).max(axis=0).reshape(-1, 128).max(axis=1)
    assert (np.diff(bmax) <= 0).all()
    # the 51 outlier channels of this workload sit in the first blocks
    first = set((8 * order[:64, None] + np.arange(8)).reshape(-1).tolist())
    assert set(W.outlier_channels(w).tolist()) <= first


def _exact_input(codec, rng, rows=4, cols=512):
    """Values the codec reproduces exactly in any order of the 8-channel
    groups. FP8 with the transform and g = 1: one +-2^-3 per group, so any
    128-block's transform is even multiples of 2^-3 up to 16 times that (at
    most four significant bits: E4M3 values after the block exponent), undone
    exactly. INT8: multiples of 1/4 with +-127/4 in every group (s = 1/4).
    INT4 asymmetric: multiples of 1/4 in [-7/4, 2] with both ends in every
    group (s = 1/4, z = 7)."""
    x = np.zeros((rows, cols), np.float32)
    if codec.format == cd.FP8_DUAL:
        for r in range(rows):
            for j in range(cols // 8):
                x[r, 8 * j + rng.integers(0, 8)] = rng.choice([-0.125, 0.125])
    elif codec.format == cd.INT8_SYM:
        x = rng.integers(-127, 128, size=(rows, cols)).astype(np.float32)
        x[:, ::8] = 127.0
        x = x * np.float32(0.25)
    else:
        x = rng.integers(-7, 9, size=(rows, cols)).astype(np.float32)
        x[:, ::8], x[:, 1::8] = -7.0, 8.0
        x = x * np.float32(0.25)
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("codec", [cd.Codec.fp8(128, True), cd.Codec.int8_sym(), cd.Codec.int4_asym()],
                         ids=["fp8-h", "i8s", "i4a"])
def test_decode_reordered_inverts_the_reordering(codec):
    rng = np.random.default_rng(5)
    bits = _exact_input(codec, rng)
    order = rng.permutation(64)
    g = 1.0 if codec.format == cd.FP8_DUAL else None
    c = oracle.compress_reordered(codec, bits, order, tensor_scale=g)
    assert (oracle.decode_reordered(c, order) == bf16_bits_to_f32(bits)).all()
    # without the inverse the decode is the reordered tensor
    assert (oracle.decode(c) == bf16_bits_to_f32(oracle.reorder_columns(bits, order))).all()
    # and the compressed buffer is that of the reordered tensor
    ref = oracle.compress(codec, oracle.reorder_columns(bits, order), tensor_scale=g)
    assert (c.codes == ref.codes).all()
