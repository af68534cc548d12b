"""CPU oracle for compressing and decompressing tensor-parallel activations.

TEST INFRASTRUCTURE ONLY. Nothing in the product library imports, links or
runs this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code, table or
constant generator with the HIP path under ``quantized_compression_tensor_amd``.

Sources, cited by page title and the section / figure / equation on it:

* [TACO]  "TACO: Efficient Communication Compression of Intermediate Tensors
  for Scalable Tensor-Parallel LLM Training" (Pith review page): abstract,
  Fig. 3 (E4M3 vs E5M2), Fig. 6 with Eq. (3) (FP8 error bound), Fig. 7
  (adaptive rescaling -> ASH transform -> dual-scale quantization), Fig. 8
  (Hadamard-based reshaping of the distribution), Fig. 13 (standard
  Hadamard baseline).
* [EQuARX] "EQuARX: Efficient Quantized AllReduce in XLA for Distributed
  Machine Learning Acceleration" (Pith review page): "What carries the
  argument" (block-wise symmetric int8 with an abs-max scale, one FP32 scale
  per 64 entries, dequantize to FP32 before adding), Fig. 7 (MSE).
* [FlashComm] "Flash Communication: Reducing Tensor Parallelization
  Bottleneck for Fast Large Language Model Inference" (Pith review page):
  "What carries the argument" (asymmetric group-128 quantization, two-step
  All-Reduce: sum locally, re-quantize to INT8), Algorithm 1 (dequantization
  takes codes, zero point and scale), free parameters (group size 128; INT4
  reduce stage, INT8 gather stage).
* [FP8] "FP8 Formats for Deep Learning" (cited in TACO's reference list) for
  the E4M3 bit layout (bias 7, no infinities, S.1111.111 is NaN, max 448) and
  the E5M2 one (bias 15, IEEE infinities and NaNs, max 57344).

Precision. Every floating-point step is IEEE-754 binary32 with one
round-to-nearest-even per operation and no fused multiply-add, in the stated
order. binary32 is what the pages fix for the sums (EQuARX: dequantize to
FP32 before adding; FlashComm: sum locally before re-quantizing), and every
quantization code is decided in the precision of the kernels that must
reproduce it bit for bit. Metrics accumulate in float64.

Where the pages leave a step open the oracle takes one plain reading; each is
listed, with its reason, in the repository's design notes and repeated in the
docstring of the function that implements it.

Parity status. Formats, transform, reduction, the ring hop and the rings
built from it, the INT8 / asymmetric codecs, the error metrics and the FP8
tensor-scale rules (data-driven g, its clamps, the gather-stage sum) are
pinned by closed forms, hand-worked values, brute force and library
cross-checks in ``tests/``. TACO's reshaping, ASH transform and dual-scale quantization are
never defined on the pages (the referee on the TACO page says the reshaping
and adaptive scales are "not quantified"), so ``compress_fp8_dual`` and its
inverse (with E4M3 or E5M2 codes) are pinned only to the readings they
implement: parity unpinned against the paper itself. The E5M2 format itself
is pinned like E4M3.
"""

from .formats import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    decode_e4m3,
    encode_e4m3,
    decode_e5m2,
    encode_e5m2,
    pack_int4,
    unpack_int4,
)
from .hadamard import fwht, fwht_f64  # noqa: F401
from .codecs import (  # noqa: F401
    FP8_DUAL,
    FP8E5_DUAL,
    FP8_FORMATS,
    INT8_SYM,
    INT4_ASYM,
    INT8_ASYM,
    Codec,
    Compressed,
    block_exponent,
    compress,
    dequantize,
    decompress_reduce,
    ring_hop,
    full_loop_ring,
    semi_loop_ring,
    requantize,
    decode,
    chunk_order,
    reorder_columns,
    restore_columns,
    compress_reordered,
    decode_reordered,
    auto_tensor_scale,
    sum_tensor_scales,
    decode_gemm,
)
from .metrics import rel_mse, rel_l2, mse  # noqa: F401
