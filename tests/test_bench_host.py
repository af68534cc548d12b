"""Host-side checks of the bench (no GPU): the one-GPU contract and the
algorithmic bytes its roofline divides by."""

import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


# Bytes per element each kernel must move, from the formats: bf16 input 2 B;
# FP8 code 1 B + one int8 exponent per 128; INT8 symmetric 1 B + one float32
# scale per 64; asymmetric codes (INT4: 1/2 B, INT8: 1 B) + a float32 scale and
# a uint8 zero point per 128. A reduce reads N shards and writes one
# re-quantized output (or a float32 sum).
PER_ELEMENT = {
    "taco-tiny": (2 + 1 + 1 / 128, 2 * (1 + 1 / 128) + 4),
    "gpt-tp": (2 + 1 + 1 / 128, 4 * (1 + 1 / 128) + (1 + 1 / 128)),
    "equarx": (2 + 1 + 4 / 64, 8 * (1 + 4 / 64) + (1 + 4 / 64)),
    "flashcomm": (2 + 0.5 + 5 / 128, 8 * (0.5 + 5 / 128) + (1 + 5 / 128)),
    "qwen-tp": (2 + 1 + 1 / 128, 8 * (1 + 1 / 128) + (1 + 1 / 128)),
}


@pytest.mark.parametrize("name", sorted(PER_ELEMENT))
def test_algorithmic_bytes_per_element(name):
    w = W.WORKLOADS[name]
    comp, red = bench.algorithmic_bytes(w)
    want_c, want_r = PER_ELEMENT[name]
    # FP8 buffers also carry a 16-byte tensor-scale header: at most 16 B per
    # shard, far below one part in 10^5 of these sizes
    assert comp == pytest.approx(want_c * w.n, rel=1e-5, abs=16)
    assert red == pytest.approx(want_r * w.n, rel=1e-5, abs=16 * (w.shards + 1))
