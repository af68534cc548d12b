"""Pins of the oracle's consumer product decode(A) @ W^T ([FlashComm] "What
carries the argument" and Fig. 8: the gathered activation is dequantized and
handed to the next layer).

The expected values are built without the oracle: each code is decoded from
the format's definition with exact rational arithmetic (torch's own FP8 and
bf16 conversions supply the E4M3 / E5M2 code values and the nearest-even
bf16 rounding), and the products are summed as fractions."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs as cd
import oracle


def _bf16(v: float) -> Fraction:
    """Nearest-even bf16 of a float32 value, by torch's conversion."""
    return Fraction(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).float().item())


def _f32(fr: Fraction) -> float:
    """Nearest float32 of an exact value held exactly in a double."""
    d = float(fr)
    assert Fraction(d) == fr, "the exact decoded value must fit a double"
    return float(np.float32(d))


def _fp8_value(code: int, e5: bool) -> Fraction:
    dt = torch.float8_e5m2 if e5 else torch.float8_e4m3fn
    return Fraction(torch.tensor([code], dtype=torch.uint8).view(dt).float().item())


def _decoded_rows(c: cd.Compressed):
    """bf16 values of the decoded activation, as fractions, from the definitions:
    INT8 symmetric q * s, asymmetric (q - z) * s, FP8 dec(q) * 2^-k * g; each
    rounded once to float32 and then to bf16."""
    M, K, B = c.rows, c.cols, c.codec.block
    f = c.codec.format
    if f == cd.INT4_ASYM:
        q = np.empty(M * K, np.int64)
        q[0::2] = c.codes & 0xF
        q[1::2] = c.codes >> 4
    elif f == cd.INT8_SYM:
        q = c.codes.view(np.int8).astype(np.int64)
    else:
        q = c.codes.astype(np.int64)
    out = []
    for i in range(M * K):
        b = i // B
        if f in cd.FP8_FORMATS:
            g = Fraction(float(c.tensor_scale))
            v = _fp8_value(int(q[i]), f == cd.FP8E5_DUAL) * Fraction(2) ** (-int(c.scale[b])) * g
        elif f == cd.INT8_SYM:
            v = int(q[i]) * Fraction(float(c.scale[b]))
        else:
            v = (int(q[i]) - int(c.zero[b])) * Fraction(float(c.scale[b]))
        out.append(_bf16(_f32(v)))
    return [out[r * K:(r + 1) * K] for r in range(M)]


def _handmade(fmt, M, K, seed):
    rng = np.random.default_rng(seed)
    codec = {cd.INT8_SYM: cd.Codec.int8_sym(), cd.INT8_ASYM: cd.Codec.int8_asym(),
             cd.INT4_ASYM: cd.Codec.int4_asym(), cd.FP8_DUAL: cd.Codec.fp8(64, False),
             cd.FP8E5_DUAL: cd.Codec.fp8e5(128, False)}[fmt]
    nb = M * K // codec.block
    if fmt in cd.FP8_FORMATS:
        # finite codes only (E4M3: not S.1111.111; E5M2: exponent field below 31)
        codes = rng.integers(0, 256, M * K).astype(np.uint8)
        if fmt == cd.FP8_DUAL:
            codes[(codes & 0x7F) == 0x7F] = 0x3C
        else:
            codes[(codes & 0x7C) == 0x7C] = 0x3C
        return cd.Compressed(codec, M, K, codes, rng.integers(-5, 6, nb).astype(np.int8),
                             tensor_scale=np.float32(0.37182818))   # many mantissa bits: the bf16 rounding matters
    scale = (rng.random(nb) * 0.05 + 0.001).astype(np.float32)
    if fmt == cd.INT8_SYM:
        codes = rng.integers(-127, 128, M * K).astype(np.int8).view(np.uint8)
        return cd.Compressed(codec, M, K, codes, scale)
    top = 15 if fmt == cd.INT4_ASYM else 255
    q = rng.integers(0, top + 1, M * K).astype(np.uint8)
    codes = oracle.pack_int4(q) if fmt == cd.INT4_ASYM else q
    zero = rng.integers(0, top + 1, nb).astype(np.uint8)
    return cd.Compressed(codec, M, K, codes, scale, zero)


FMTS = [cd.INT8_SYM, cd.INT8_ASYM, cd.INT4_ASYM, cd.FP8_DUAL, cd.FP8E5_DUAL]


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_gemm_equals_exact_sum(fmt):
    M, K, N = 2, 128, 3
    c = _handmade(fmt, M, K, seed=fmt)
    rng = np.random.default_rng(100 + fmt)
    w_bits = rng.integers(0, 1 << 16, (N, K)).astype(np.uint16)
    w_bits[(w_bits & 0x7F80) == 0x7F80] = 0x3F80    # finite weights only
    w = [[Fraction(float(v)) for v in oracle.bf16_bits_to_f32(row)] for row in w_bits]
    a = _decoded_rows(c)
    out, mag = oracle.decode_gemm(c, w_bits)
    assert out.shape == (M, N) and mag.shape == (M, N)
    for m in range(M):
        for n in range(N):
            exact = sum(a[m][k] * w[n][k] for k in range(K))
            absum = sum(abs(a[m][k] * w[n][k]) for k in range(K))
            tol = float(absum) * 2.0 ** -50
            assert abs(out[m, n] - float(exact)) <= tol, (m, n)
            assert abs(mag[m, n] - float(absum)) <= tol, (m, n)


def test_identity_weight_returns_the_decoded_activation():
    c = _handmade(cd.INT8_ASYM, 3, 256, seed=9)
    eye = np.where(np.eye(256, dtype=bool), np.uint16(0x3F80), np.uint16(0))   # bf16 1.0 on the diagonal
    out, _ = oracle.decode_gemm(c, eye)
    want = oracle.bf16_bits_to_f32(cd.decode(c, "bf16")).astype(np.float64)
    assert np.array_equal(out, want)


def test_weight_rows_are_output_features():
    """W is [N, K]: output column n uses row n of W (a transposed W would be
    caught by a non-square shape error and by this column selection)."""
    c = _handmade(cd.INT8_SYM, 2, 128, seed=4)
    w = np.zeros((5, 128), np.uint16)
    cols = [7, 0, 127, 64, 3]
    for n, k in enumerate(cols):
        w[n, k] = 0x4000   # 2.0
    out, _ = oracle.decode_gemm(c, w)
    a = oracle.bf16_bits_to_f32(cd.decode(c, "bf16")).astype(np.float64)
    assert np.array_equal(out, 2.0 * a[:, cols])
    with pytest.raises(ValueError):
        oracle.decode_gemm(c, np.zeros((128, 5), np.uint16))
