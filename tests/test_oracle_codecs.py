"""Pins of the oracle's codecs, reduce and decode against brute force, closed
forms, the TACO page's Eq. (3) bound and hand-worked examples. CPU only."""

import math

import numpy as np
import pytest

import oracle
from oracle import codecs as cd
from oracle import formats as fm
from oracle.hadamard import fwht
import workloads as W
from tests.conftest import read_golden
from tests.test_oracle_formats import nearest_code_bruteforce, nearest_e5m2_bruteforce

F32 = np.float32


def bits_of(x):
    return W.f32_to_bf16_rne(np.asarray(x, np.float32))


# ------------------------------------------------------- block exponent --

def k_bruteforce(m):
    """Largest k in [-64, 63] with m * 2^k <= 448 (exact in float64); -64 if none."""
    m = float(m)
    if m == 0.0:
        return 0
    best = -64
    for k in range(-64, 64):
        if m * 2.0 ** k <= 448.0:
            best = k
    return best


def k_probe_values():
    base = []
    for j in range(-140, 130, 3):
        for c in (448.0, 224.0, 256.0, 0.875 * 512, 1.0, 300.0):
            v = F32(min(c * 2.0 ** j, 3.0e38))
            if np.isfinite(v) and v > 0:
                base += [v, np.nextafter(v, F32(np.inf)), np.nextafter(v, F32(0))]
    base += [F32(0), F32(1e-45), F32(3.4e38), F32(2.0 ** -126), F32(2.0 ** -149)]
    return np.array(base, np.float32)


def test_block_exponent_bruteforce():
    m = k_probe_values()
    got = cd.block_exponent(m)
    want = np.array([k_bruteforce(v) for v in m])
    assert (got == want).all(), m[got != want]


def test_block_exponent_postcondition():
    m = k_probe_values()
    k = cd.block_exponent(m)
    v = m.astype(np.float64) * np.exp2(k.astype(np.float64))
    live = (m > 0) & (k > -64) & (k < 63)
    assert np.all(v[live] <= 448.0) and np.all(v[live] > 224.0)


def test_block_exponent_infinity():
    assert cd.block_exponent(np.array([np.inf], np.float32))[0] == -64


# ------------------------------------------------------------- FP8 dual --

@pytest.mark.parametrize("B", [16, 32, 128])
@pytest.mark.parametrize("gexp", [0, -3, 5])
def test_fp8_dual_bruteforce_small_integers(B, gexp):
    """Small-integer inputs make the FWHT exact; a power-of-two g makes the scaled
    values exact; then every code must be the brute-force nearest E4M3 code of
    y * 2^(k - gexp), with k from the brute-force exponent search."""
    rng = np.random.default_rng(B + 7 * (gexp + 10))
    x = rng.integers(-9, 10, size=(3, 2 * B)).astype(np.float32)
    x[0, :B] = 0.0                                 # an all-zero block
    x[1, :B] = 0.0
    x[1, 3] = 5.0                                  # a single spike
    codec = cd.Codec.fp8(B, True)
    c = oracle.compress(codec, bits_of(x), tensor_scale=F32(2.0 ** gexp))
    y = fwht(x.reshape(-1), B).astype(np.float64).reshape(-1, B)
    w = y * 2.0 ** -gexp
    kk = np.array([k_bruteforce(F32(np.max(np.abs(b)))) for b in w])
    v = (w * np.exp2(kk)[:, None]).reshape(-1)
    v = np.where(y.reshape(-1) == 0, 0.0, v)
    assert (c.scale.astype(int) == kk).all()
    assert (c.codes == nearest_code_bruteforce(v.astype(np.float32))).all()
    assert c.tensor_scale == F32(2.0 ** gexp)


def test_fp8_dual_auto_scale_and_block_range():
    x = W.random_bits((64, 256), seed=3, sigma=0.02)
    codec = cd.Codec.fp8()
    c = oracle.compress(codec, x)
    y = cd.transform(codec, x)
    A = np.max(np.abs(y))
    assert c.tensor_scale == F32(A) / F32(448.0)
    v = c.prequant.reshape(-1, 128)
    vmax = np.max(np.abs(v), axis=1)
    assert np.all(vmax <= 448.0) and np.all(vmax > 224.0)
    # the block holding the tensor maximum keeps k such that 448 * 2^-k * g ~ A
    dq = oracle.dequantize(c)
    assert abs(np.max(np.abs(dq)) - A) <= A * 2.0 ** -4


def test_fp8_dual_error_within_eq3_bound():
    """TACO Eq. (3), applied where the rounding happens (the scaled value v),
    then carried back through the exact power-of-two and g scalings."""
    x = W.random_bits((128, 512), seed=9, sigma=0.02)
    codec = cd.Codec.fp8()
    c = oracle.compress(codec, x)
    y = cd.transform(codec, x).astype(np.float64)
    dq = oracle.dequantize(c).astype(np.float64)
    v = c.prequant.astype(np.float64)
    av = np.abs(v)
    ulp = np.where(av >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(av, 1e-300))) - 3), 2.0 ** -9)
    k = np.repeat(c.scale.astype(np.float64), 128)
    g = float(c.tensor_scale)
    # rounding error of v, plus the two float32 roundings (y / g and * g)
    bound = (ulp / 2) * 2.0 ** -k * g + 2 * 2.0 ** -24 * np.abs(y) + 2.0 ** -24 * np.abs(dq)
    assert np.all(np.abs(dq - y) <= bound * (1 + 1e-9))


def test_fp8_dual_rel_mse_statistics():
    """rel-MSE of a 3-mantissa-bit float on values spread over a binade is about
    2^-6 / 12 * E[(2^e / x)^2] ~ 7e-4; the block scale keeps values out of the
    subnormal range, so the round trip should land near that."""
    x = W.random_bits((256, 1024), seed=21, sigma=0.02)
    codec = cd.Codec.fp8()
    c = oracle.compress(codec, x)
    xr = oracle.decode(c)
    r = oracle.rel_mse(xr, fm.bf16_bits_to_f32(x))
    assert 4e-4 < r < 1.1e-3, r


def test_hadamard_helps_on_outlier_channels():
    """TACO Fig. 8 / Fig. 13: the Hadamard transform spreads outlier channels over
    the block, which lowers the error of per-block FP8 scaling."""
    w = W.WORKLOADS["gpt-tp"]
    x = W.make_shard(w, 0, chunks=[0])
    u = fm.bf16_bits_to_f32(x)
    on = oracle.rel_mse(oracle.decode(oracle.compress(cd.Codec.fp8(128, True), x)), u)
    off = oracle.rel_mse(oracle.decode(oracle.compress(cd.Codec.fp8(128, False), x)), u)
    assert on < off


def test_fp8_decode_bf16_is_rounded_f32_decode():
    x = W.random_bits((8, 256), seed=5, sigma=0.5)
    c = oracle.compress(cd.Codec.fp8(), x)
    assert (oracle.decode(c, "bf16") == fm.f32_to_bf16_bits(oracle.decode(c))).all()


def test_fp8_zero_is_positive_code():
    x = np.zeros((2, 128), np.float32)
    x[1, 0] = -0.0
    c = oracle.compress(cd.Codec.fp8(), bits_of(x))
    assert (c.codes == 0).all() and (c.scale == 0).all() and c.tensor_scale == 1.0


def test_fp8_saturates_when_block_exponent_clamps():
    """A stale, far too small g forces k to its lower clamp: codes saturate at 448."""
    x = np.full((1, 128), 1.0e4, np.float32)
    c = oracle.compress(cd.Codec.fp8(128, False), bits_of(x), tensor_scale=F32(2.0 ** -60))
    assert c.scale[0] == -64
    assert (c.codes == 0x7E).all()


# ------------------------------------------------------- FP8 dual, E5M2 --

def k_bruteforce_e5(m):
    """Largest k in [-64, 63] with m * 2^k <= 57344 (exact in float64); -64 if none."""
    m = float(m)
    if m == 0.0:
        return 0
    best = -64
    for k in range(-64, 64):
        if m * 2.0 ** k <= 57344.0:
            best = k
    return best


def test_block_exponent_e5m2_bruteforce_and_range():
    m = np.concatenate([k_probe_values(), np.array([57344.0, 28672.0, 57345.0, 28671.0], np.float32)])
    got = cd.block_exponent(m, cd.FP8E5_DUAL)
    want = np.array([k_bruteforce_e5(v) for v in m])
    assert (got == want).all(), m[got != want]
    v = m.astype(np.float64) * np.exp2(got.astype(np.float64))
    live = (m > 0) & (got > -64) & (got < 63)
    assert np.all(v[live] <= 57344.0) and np.all(v[live] > 28672.0)


@pytest.mark.parametrize("B", [16, 128])
@pytest.mark.parametrize("gexp", [0, 4])
def test_fp8e5_dual_bruteforce_small_integers(B, gexp):
    """As for E4M3: exact FWHT and power-of-two scalings, so every code must be
    the brute-force nearest E5M2 code of y * 2^(k - gexp)."""
    rng = np.random.default_rng(B + 11 * (gexp + 3))
    x = rng.integers(-9, 10, size=(3, 2 * B)).astype(np.float32)
    x[0, :B] = 0.0
    x[1, :B] = 0.0
    x[1, 3] = 5.0
    codec = cd.Codec.fp8e5(B, True)
    c = oracle.compress(codec, bits_of(x), tensor_scale=F32(2.0 ** gexp))
    y = fwht(x.reshape(-1), B).astype(np.float64).reshape(-1, B)
    w = y * 2.0 ** -gexp
    kk = np.array([k_bruteforce_e5(F32(np.max(np.abs(b)))) for b in w])
    v = (w * np.exp2(kk)[:, None]).reshape(-1)
    v = np.where(y.reshape(-1) == 0, 0.0, v)
    assert (c.scale.astype(int) == kk).all()
    assert (c.codes == nearest_e5m2_bruteforce(v.astype(np.float32))).all()


def test_fp8e5_dual_auto_scale_and_error_bound():
    """g = RN(A / 57344); TACO Eq. (3) with m = 2 at the scaled value, carried
    back through the exact power-of-two and g scalings."""
    x = W.random_bits((128, 512), seed=19, sigma=0.02)
    codec = cd.Codec.fp8e5()
    c = oracle.compress(codec, x)
    y = cd.transform(codec, x).astype(np.float64)
    assert c.tensor_scale == F32(F32(np.max(np.abs(y))) / F32(57344.0))
    dq = oracle.dequantize(c).astype(np.float64)
    av = np.abs(c.prequant.astype(np.float64))
    ulp = np.where(av >= 2.0 ** -14, np.exp2(np.floor(np.log2(np.maximum(av, 1e-300))) - 2), 2.0 ** -16)
    k = np.repeat(c.scale.astype(np.float64), 128)
    g = float(c.tensor_scale)
    bound = (ulp / 2) * 2.0 ** -k * g + 2 * 2.0 ** -24 * np.abs(y) + 2.0 ** -24 * np.abs(dq)
    assert np.all(np.abs(dq - y) <= bound * (1 + 1e-9))
    vmax = np.max(av.reshape(-1, 128), axis=1)
    assert np.all(vmax <= 57344.0) and np.all(vmax > 28672.0)


def test_fp8e5_dual_rel_mse_statistics():
    """Two mantissa bits: about 2^-4 / 12 * E[(2^e / x)^2] ~ 2.8e-3, four times
    the E4M3 figure."""
    x = W.random_bits((256, 1024), seed=21, sigma=0.02)
    r5 = oracle.rel_mse(oracle.decode(oracle.compress(cd.Codec.fp8e5(), x)), fm.bf16_bits_to_f32(x))
    r4 = oracle.rel_mse(oracle.decode(oracle.compress(cd.Codec.fp8(), x)), fm.bf16_bits_to_f32(x))
    assert 1.6e-3 < r5 < 4.4e-3, r5
    assert 3.0 < r5 / r4 < 5.0, (r5, r4)


def test_fp8e5_saturates_when_block_exponent_clamps():
    x = np.full((1, 128), 1.0e12, np.float32)
    c = oracle.compress(cd.Codec.fp8e5(128, False), bits_of(x), tensor_scale=F32(2.0 ** -60))
    assert c.scale[0] == -64
    assert (c.codes == 0x7B).all()


def test_fp8e5_reduce_requant_pair_and_sum_scale():
    xs = [W.random_bits((16, 256), seed=40 + r, sigma=0.02) for r in range(3)]
    codec = cd.Codec.fp8e5()
    shards = [oracle.compress(codec, x) for x in xs]
    acc, rq = oracle.decompress_reduce(shards, codec)
    assert rq.tensor_scale == cd.sum_tensor_scales([s.tensor_scale for s in shards])
    with pytest.raises(AssertionError):
        oracle.decompress_reduce(shards, cd.Codec.fp8())        # E5M2 -> E4M3 is not a pair


# ---------------------------------------------------------- INT formats --

def _golden_int_rows():
    out = []
    for row in read_golden("int_codecs_examples.txt"):
        kind, vin, qout, z = [p.strip() for p in " ".join(row).split("|")]
        out.append((kind, [float(t) for t in vin.split()], [int(t) for t in qout.split()], z[2:]))
    return out


def test_int_codecs_golden():
    for kind, vin, qout, z in _golden_int_rows():
        if kind == "sym8":
            codec, B = cd.Codec.int8_sym(), 64
        elif kind == "asym4":
            codec, B = cd.Codec.int4_asym(), 128
        else:
            codec, B = cd.Codec.int8_asym(), 128
        x = np.zeros((1, B), np.float32)
        x[0, :len(vin)] = vin
        c = oracle.compress(codec, bits_of(x))
        if kind == "asym4":
            q = fm.unpack_int4(c.codes).astype(int)
        elif kind == "sym8":
            q = c.codes.view(np.int8).astype(int)
        else:
            q = c.codes.astype(int)
        assert list(q[:len(qout)]) == qout, (kind, vin, q[:len(qout)])
        if z != "-":
            assert int(c.zero[0]) == int(z)
            assert (q[len(qout):] == int(z)).all()        # zeros encode to z
        else:
            assert (q[len(qout):] == 0).all()


def test_int8_sym_extremes_and_error_bound():
    x = W.random_bits((64, 512), seed=13, sigma=1.0)
    u = fm.bf16_bits_to_f32(x).reshape(-1, 64)
    c = oracle.compress(cd.Codec.int8_sym(), x)
    q = c.codes.view(np.int8).reshape(-1, 64).astype(int)
    # the abs-max element of each block lands exactly on +-127
    i = np.argmax(np.abs(u), axis=1)
    assert (np.abs(q[np.arange(len(i)), i]) == 127).all()
    dq = oracle.dequantize(c).reshape(-1, 64).astype(np.float64)
    s = c.scale.astype(np.float64)[:, None]
    assert np.all(np.abs(dq - u) <= s / 2 * (1 + 2.0 ** -20) + 2.0 ** -24 * np.abs(u))


def test_int8_sym_mse_is_s2_over_12():
    x = W.random_bits((512, 1024), seed=17, sigma=1.0)
    c = oracle.compress(cd.Codec.int8_sym(), x)
    err = oracle.dequantize(c).astype(np.float64) - fm.bf16_bits_to_f32(x).reshape(-1)
    pred = np.mean(np.repeat(c.scale.astype(np.float64) ** 2 / 12.0, 64))
    assert abs(np.mean(err ** 2) / pred - 1.0) < 0.05


@pytest.mark.parametrize("codec", [cd.Codec.int4_asym(), cd.Codec.int8_asym()])
def test_asym_zero_exact_and_bounds(codec):
    x = W.random_bits((32, 1024), seed=19, sigma=0.05, body="t3")
    xf = fm.bf16_bits_to_f32(x)
    xf[:, ::7] = 0.0                          # zeros everywhere
    x = bits_of(xf)
    c = oracle.compress(codec, x)
    dq = oracle.dequantize(c).reshape(-1)
    u = xf.reshape(-1).astype(np.float64)
    assert (dq[u == 0] == 0).all()            # zero round-trips exactly
    qmax = (1 << codec.bits) - 1
    assert (c.zero <= qmax).all()
    s = np.repeat(c.scale.astype(np.float64), 128)
    assert np.all(np.abs(dq - u) <= s / 2 * (1 + 2.0 ** -18) + 2.0 ** -23 * np.abs(u) + 1e-30)


def test_tiny_blocks_quantize_to_zero():
    x = np.zeros((1, 256), np.float32)
    x[0, 5] = 1e-35                           # below 2^-100: a zero block
    x[0, 128 + 5] = 1.0
    for codec in (cd.Codec.int8_sym(), cd.Codec.int4_asym()):
        c = oracle.compress(codec, bits_of(x))
        assert c.scale[0] == 0
        dq = oracle.dequantize(c)
        assert dq[5] == 0 and dq[128 + 5] == np.float32(1.0)


# ---------------------------------------------------- reduce and decode --

def _shards(codec, n=3, shape=(16, 256), sigma=0.02, body="normal"):
    return [oracle.compress(codec, W.random_bits(shape, seed=100 + r, sigma=sigma, body=body))
            for r in range(n)]


ALL_CODECS = [cd.Codec.fp8(), cd.Codec.fp8(64, False), cd.Codec.int8_sym(),
              cd.Codec.int4_asym(), cd.Codec.int8_asym()]


@pytest.mark.parametrize("codec", ALL_CODECS)
def test_reduce_single_shard_is_dequantize(codec):
    s = _shards(codec, 1)
    acc, _ = oracle.decompress_reduce(s)
    assert (acc.reshape(-1) == oracle.dequantize(s[0])).all()


@pytest.mark.parametrize("codec", ALL_CODECS)
def test_reduce_ignores_all_zero_shards(codec):
    s = _shards(codec, 2)
    z = oracle.compress(codec, np.zeros((16, 256), np.uint16))
    a, _ = oracle.decompress_reduce(s)
    b, _ = oracle.decompress_reduce([s[0], z, s[1], z])
    assert (a == b).all()


def test_reduce_is_sequential_float32_sum():
    s = _shards(cd.Codec.int8_sym(), 5, sigma=1.0)
    acc, _ = oracle.decompress_reduce(s)
    exact = sum(oracle.dequantize(t).astype(np.float64) for t in s)
    mags = sum(np.abs(oracle.dequantize(t)).astype(np.float64) for t in s)
    # five float32 additions: each rounding is at most half an ulp of a partial sum
    assert np.all(np.abs(acc.reshape(-1) - exact) <= 5 * 2.0 ** -24 * mags)
    # and the order is fixed: the same shards in reverse order may round differently,
    # the oracle's own sum must be reproducible bit for bit
    acc2, _ = oracle.decompress_reduce(s)
    assert (acc2 == acc).all()


def test_taco_reduce_is_linear_through_the_transform():
    codec = cd.Codec.fp8()
    s = _shards(codec, 4, shape=(8, 512))
    acc, rq = oracle.decompress_reduce(s, codec)
    lhs = fwht(acc.reshape(-1), 128) / 128.0
    rhs = sum(oracle.decode(t).reshape(-1).astype(np.float64) for t in s)
    assert oracle.rel_l2(lhs, rhs) < 1e-6
    # the requantized sum carries g' = sum of g_r and decodes near the exact sum
    gsum = sum(float(t.tensor_scale) for t in s)
    assert abs(float(rq.tensor_scale) - gsum) <= 4 * 2.0 ** -24 * gsum
    assert oracle.rel_mse(oracle.decode(rq).reshape(-1), rhs) < 2e-3


def test_taco_requant_never_saturates_with_summed_scale():
    codec = cd.Codec.fp8()
    s = _shards(codec, 8, shape=(16, 512), sigma=3.0)
    _, rq = oracle.decompress_reduce(s, codec)
    assert (rq.scale > -64).all()
    assert np.max(np.abs(rq.prequant)) <= 448.0


def test_requantize_standalone_matches_reduce_requant():
    codec = cd.Codec.int8_asym()
    s = _shards(cd.Codec.int4_asym(), 3, sigma=0.05, body="t3")
    acc, rq = oracle.decompress_reduce(s, codec)
    rq2 = oracle.requantize(codec, acc)
    assert (rq.codes == rq2.codes).all() and (rq.scale == rq2.scale).all() and (rq.zero == rq2.zero).all()


def test_equarx_one_shot_mse_below_ring_figure():
    """Context check (EQuARX page, Fig. 7 / "If this is right": MSE 0.0014 with both
    ring stages quantized on N(0,1)): a one-shot 8-shard sum with one gather-stage
    requantization must do no worse than that ring figure."""
    w = W.WORKLOADS["equarx"]
    shards = [oracle.compress(cd.Codec.int8_sym(), W.make_shard(w, r, chunks=[0])) for r in range(8)]
    exact = sum(fm.bf16_bits_to_f32(W.make_shard(w, r, chunks=[0])).astype(np.float64) for r in range(8))
    _, rq = oracle.decompress_reduce(shards, cd.Codec.int8_sym())
    m = oracle.mse(oracle.decode(rq), exact)
    assert m < 0.0014, m


def test_empty_tensor():
    for codec in ALL_CODECS:
        c = oracle.compress(codec, np.zeros((0, 256), np.uint16))
        assert c.codes.size == 0 and c.scale.size == 0
        acc, rq = oracle.decompress_reduce([c, c])
        assert acc.shape == (0, 256)


def test_bad_shapes_rejected():
    with pytest.raises(AssertionError):
        oracle.compress(cd.Codec.fp8(), np.zeros((2, 100), np.uint16))
    with pytest.raises(AssertionError):
        oracle.compress(cd.Codec(cd.INT8_SYM, 128), np.zeros((2, 256), np.uint16))
    with pytest.raises(AssertionError):
        cd.check_pair(cd.Codec.int8_sym(), cd.Codec.int8_asym())
