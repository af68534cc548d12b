"""The seeded input generators: deterministic, chunk-addressable, and shaped as
stated for each workload. CPU only."""

import numpy as np

import workloads as W
from oracle.formats import bf16_bits_to_f32


def test_shapes_and_determinism():
    w = W.WORKLOADS["taco-tiny"]
    a = W.make_shard(w, 0)
    b = W.make_shard(w, 0)
    c = W.make_shard(w, 1)
    assert a.shape == (w.rows, w.cols) and a.dtype == np.uint16
    assert (a == b).all() and not (a == c).all()


def test_chunk_subset_equals_full_rows():
    w = W.WORKLOADS["gpt-tp"]
    full = W.make_shard(w, 2)
    ch = W.sample_chunks(w, 3, seed=1)
    part = W.make_shard(w, 2, chunks=ch)
    assert (part == full[W.chunk_rows(ch, w.rows)]).all()


def test_distributions():
    w = W.WORKLOADS["gpt-tp"]
    x = bf16_bits_to_f32(W.make_shard(w, 0, chunks=[0, 1]))
    chans = W.outlier_channels(w)
    assert len(chans) == 4
    body = np.delete(x, chans, axis=1)
    assert abs(body.std() / 0.02 - 1) < 0.02
    assert abs(x[:, chans].std() / (0.02 * 20) - 1) < 0.05
    t = W.WORKLOADS["flashcomm"]
    y = bf16_bits_to_f32(W.make_shard(t, 0, chunks=[0]))
    # Student-t(3): median |t| = 0.7649 -> median |x| = 0.05 * 0.7649
    assert abs(np.median(np.abs(y)) / (0.05 * 0.7649) - 1) < 0.03
    tiny = W.WORKLOADS["taco-tiny"]
    z = bf16_bits_to_f32(W.make_shard(tiny, 0))
    big = np.abs(z) >= 10 * 0.02 * 0.99
    assert abs(big.sum() - round(0.001 * tiny.n)) <= 5
