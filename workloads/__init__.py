"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only makes input tensors (bf16 bit patterns). It contains none of
the codec arithmetic, so the oracle and the HIP path can both take their
inputs from here without sharing anything else.

The pages quantize real activations of GPT, Qwen, LLaMA and Gemma models; no
model, weight or dataset is available, so each workload below is a seeded
random tensor with the shape and value distribution stated for it:

* taco-tiny      2048 x 1024, N(0, 0.02), 0.1 % point outliers at +-U[10, 50] sigma
                 per shard; FP8 dual-scale with 128-point Hadamard; 2 shards
                 summed to FP32.
* gpt-tp         4096 x 4096, N(0, 0.02), 4 hidden channels scaled x20 (the same
                 channels in every shard); FP8 dual-scale; 4 shards, sum
                 re-quantized to FP8.
* equarx         8192 x 5120, N(0, 1); symmetric INT8, block 64; 8 shards, sum
                 re-quantized to INT8.
* flashcomm      8192 x 8192, 0.05 * Student-t(3) (down-projection-like heavy
                 tails); asymmetric INT4 group 128; 8 shards, sum re-quantized to
                 asymmetric INT8 group 128.
* qwen-tp        32768 x 5120, 0.02 * Student-t(3), 1 % of hidden channels x100;
                 FP8 dual-scale; 8 shards, sum re-quantized to FP8.

Generation is split into blocks of ROW_CHUNK rows, each with its own seed
derived from (workload seed, shard, chunk), so any subset of rows can be
regenerated alone and the result does not depend on the thread count.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os
from typing import Optional, Sequence

import numpy as np

ROW_CHUNK = 256

FP8_DUAL, INT8_SYM, INT4_ASYM, INT8_ASYM = 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    cols: int
    shards: int
    seed: int
    body: str                 # "normal" or "t3"
    sigma: float
    in_format: int
    in_block: int
    hadamard: bool
    out_format: Optional[int]  # None: the FP32 sum is the output
    out_block: Optional[int]
    point_outlier_frac: float = 0.0
    point_outlier_range: tuple = (10.0, 50.0)
    channel_count: int = 0
    channel_gain: float = 1.0
    gemm: bool = False         # a bf16 [rows, cols] x [cols, cols] product overlaps the codec

    @property
    def n(self):
        return self.rows * self.cols


WORKLOADS = {
    "taco-tiny": Workload("taco-tiny", 2048, 1024, 2, 1000, "normal", 0.02,
                          FP8_DUAL, 128, True, None, None,
                          point_outlier_frac=0.001),
    "gpt-tp": Workload("gpt-tp", 4096, 4096, 4, 2000, "normal", 0.02,
                       FP8_DUAL, 128, True, FP8_DUAL, 128,
                       channel_count=4, channel_gain=20.0),
    "equarx": Workload("equarx", 8192, 5120, 8, 3000, "normal", 1.0,
                       INT8_SYM, 64, False, INT8_SYM, 64),
    "flashcomm": Workload("flashcomm", 8192, 8192, 8, 4000, "t3", 0.05,
                          INT4_ASYM, 128, False, INT8_ASYM, 128),
    "qwen-tp": Workload("qwen-tp", 32768, 5120, 8, 5000, "t3", 0.02,
                        FP8_DUAL, 128, True, FP8_DUAL, 128,
                        channel_count=51, channel_gain=100.0, gemm=True),
}

ORDER = ["taco-tiny", "gpt-tp", "equarx", "flashcomm", "qwen-tp"]


def f32_to_bf16_rne(x):
    """float32 -> bf16 bit patterns, nearest-even (input preparation only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def outlier_channels(w: Workload):
    if w.channel_count == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([w.seed, 7777])
    return np.sort(rng.choice(w.cols, size=w.channel_count, replace=False))


def _chunk(w: Workload, shard: int, chunk: int, chans):
    r0 = chunk * ROW_CHUNK
    nr = min(ROW_CHUNK, w.rows - r0)
    rng = np.random.default_rng([w.seed, shard, chunk])
    if w.body == "normal":
        x = rng.standard_normal((nr, w.cols), dtype=np.float32) * np.float32(w.sigma)
    else:
        x = (rng.standard_t(3, size=(nr, w.cols)) * w.sigma).astype(np.float32)
    if len(chans):
        x[:, chans] *= np.float32(w.channel_gain)
    return f32_to_bf16_rne(x)


def _point_outliers(w: Workload, shard: int, bits):
    """Replace round(frac * n) uniformly chosen entries by +-U[lo, hi] * sigma."""
    n = w.n
    k = int(round(w.point_outlier_frac * n))
    if k == 0:
        return bits
    rng = np.random.default_rng([w.seed, shard, 999_983])
    pos = rng.choice(n, size=k, replace=False)
    lo, hi = w.point_outlier_range
    mag = rng.uniform(lo, hi, size=k) * w.sigma
    sgn = np.where(rng.integers(0, 2, size=k) == 1, 1.0, -1.0)
    flat = bits.reshape(-1)
    flat[pos] = f32_to_bf16_rne((sgn * mag).astype(np.float32))
    return bits


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def make_shard(w: Workload, shard: int, chunks: Optional[Sequence[int]] = None):
    """bf16 bit patterns (uint16) of one shard.

    chunks=None: the whole [rows, cols] tensor. Otherwise only the listed row
    chunks (each ROW_CHUNK rows), stacked in the given order; point outliers
    need the whole tensor and are only placed when chunks is None.
    """
    chans = outlier_channels(w)
    nchunks = (w.rows + ROW_CHUNK - 1) // ROW_CHUNK
    sel = list(range(nchunks)) if chunks is None else list(chunks)
    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(lambda c: _chunk(w, shard, c, chans), sel))
    bits = np.concatenate(parts, axis=0) if parts else np.zeros((0, w.cols), np.uint16)
    if chunks is None and w.point_outlier_frac > 0:
        bits = _point_outliers(w, shard, bits)
    return bits


def chunk_rows(chunks: Sequence[int], rows: int):
    """Row indices covered by the listed chunks, in order."""
    out = []
    for c in chunks:
        out.extend(range(c * ROW_CHUNK, min(rows, (c + 1) * ROW_CHUNK)))
    return np.asarray(out, dtype=np.int64)


def sample_chunks(w: Workload, count: int, seed: int = 0):
    """A seeded choice of row chunks for sampled full-size checks (always
    includes the first and the last chunk)."""
    nchunks = (w.rows + ROW_CHUNK - 1) // ROW_CHUNK
    rng = np.random.default_rng([w.seed, 4242, seed])
    mid = rng.choice(np.arange(1, max(2, nchunks - 1)), size=min(count, max(1, nchunks - 2)), replace=False)
    return sorted(set([0, nchunks - 1] + [int(c) for c in mid]))


def random_bits(shape, seed, sigma=1.0, body="normal"):
    """Small seeded bf16 tensors for edge-case and brute-force tests."""
    rng = np.random.default_rng(seed)
    if body == "normal":
        x = rng.standard_normal(shape).astype(np.float32) * np.float32(sigma)
    elif body == "t3":
        x = (rng.standard_t(3, size=shape) * sigma).astype(np.float32)
    elif body == "uniform":
        x = rng.uniform(-sigma, sigma, size=shape).astype(np.float32)
    else:
        raise ValueError(body)
    return f32_to_bf16_rne(x)
