"""The three codecs, the decompress-reduce(-requantize) step and the decode.

Test infrastructure only (see the package docstring). All arithmetic is
float32 with one rounding per operation, in the order written; integer steps
are exact.

Layout of the input: a row-major [rows, cols] tensor of bf16 bit patterns.
Quantization blocks are B contiguous elements along ``cols`` (B divides
cols), so the tensor is simply a sequence of n / B blocks.
"""

from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .formats import (
    E4M3_MAX,
    E5M2_MAX,
    bf16_bits_to_f32,
    decode_e4m3,
    decode_e5m2,
    encode_e4m3,
    encode_e5m2,
    f32_to_bf16_bits,
    pack_int4,
    unpack_int4,
)
from .hadamard import fwht

F32 = np.float32

FP8_DUAL = 1    # TACO: Hadamard blocks + tensor scale g + per-block power-of-two exponent
INT8_SYM = 2    # EQuARX: symmetric abs-max int8, one float32 scale per 64 entries
INT4_ASYM = 3   # FlashComm: asymmetric min/max, group 128, 4-bit codes packed two per byte
INT8_ASYM = 4   # FlashComm: the same scheme at 8 bits, used for the gather stage
FP8E5_DUAL = 5  # TACO's dual-scale scheme with E5M2 codes (the other FP8 format of Fig. 3)

FP8_FORMATS = (FP8_DUAL, FP8E5_DUAL)
# largest finite code value of each FP8 format, written 0.875 * 2^P
FP8_MAX = {FP8_DUAL: E4M3_MAX, FP8E5_DUAL: E5M2_MAX}
_FP8_P = {FP8_DUAL: 9, FP8E5_DUAL: 16}
_FP8_ENC = {FP8_DUAL: encode_e4m3, FP8E5_DUAL: encode_e5m2}
_FP8_DEC = {FP8_DUAL: decode_e4m3, FP8E5_DUAL: decode_e5m2}

# Reading: the tensor scale g is kept within [2^-60, 2^60] so that g * 2^-k and
# (1/g) * 2^k stay normal float32 numbers for every block exponent k.
G_MIN = F32(2.0 ** -60)
G_MAX = F32(2.0 ** 60)
K_MIN, K_MAX = -64, 63          # block exponent stored as int8
# Reading: a block whose abs-max (symmetric) or range (asymmetric) is below
# 2^-100 is stored as all-zero codes with a zero scale, so 127/A and
# qmax/r never overflow float32.
TINY = F32(2.0 ** -100)


@dataclass(frozen=True)
class Codec:
    format: int
    block: int
    hadamard: bool = False

    @property
    def bits(self):
        return 4 if self.format == INT4_ASYM else 8

    @staticmethod
    def fp8(block=128, hadamard=True):
        return Codec(FP8_DUAL, block, bool(hadamard))

    @staticmethod
    def fp8e5(block=128, hadamard=True):
        return Codec(FP8E5_DUAL, block, bool(hadamard))

    @staticmethod
    def int8_sym(block=64):
        return Codec(INT8_SYM, block, False)

    @staticmethod
    def int4_asym(block=128):
        return Codec(INT4_ASYM, block, False)

    @staticmethod
    def int8_asym(block=128):
        return Codec(INT8_ASYM, block, False)


@dataclass
class Compressed:
    """One compressed shard, as separate arrays.

    codes: uint8 [n] (INT4: packed, [n / 2]); for INT8_SYM the bytes are int8.
    scale: FP8_DUAL -> int8 block exponents k [n / B]; otherwise float32 s [n / B].
    zero:  asymmetric formats -> uint8 zero points z [n / B]; else None.
    tensor_scale: FP8_DUAL -> float32 g; else None.
    """
    codec: Codec
    rows: int
    cols: int
    codes: np.ndarray
    scale: np.ndarray
    zero: Optional[np.ndarray] = None
    tensor_scale: Optional[np.float32] = None
    prequant: Optional[np.ndarray] = None   # the float32 fed to the rounding step


# ---------------------------------------------------------------- TACO FP8 --

def block_exponent(m, fmt=FP8_DUAL):
    """Per-block power-of-two exponent k of the dual-scale reading.

    Reading of [TACO]'s Dual-Scale Quantization (named in the abstract and
    Fig. 7, never defined): the second scale of a block is 2^k with k the
    largest integer such that m * 2^k <= 448, where m is the block's largest
    magnitude after the tensor scale; k is clamped to the int8 range
    [-64, 63]; k = 0 for an all-zero block; an infinite m has no such k and
    gets the lower clamp. With m = f * 2^E (f in [0.5, 1)) the largest k is
    9 - E if f <= 0.875 (448 = 0.875 * 2^9) and 8 - E otherwise, which puts
    the block maximum in (224, 448]. For E5M2 the same rule holds with
    57344 = 0.875 * 2^16: k = 16 - E or 15 - E, the maximum in (28672, 57344].
    """
    P = _FP8_P[fmt]
    m = np.asarray(m, dtype=np.float32).astype(np.float64)
    fin = np.isfinite(m) & (m > 0)
    f, E = np.frexp(np.where(fin, m, 1.0))
    k = np.where(f <= 0.875, P, P - 1) - E.astype(np.int64)
    k = np.clip(k, K_MIN, K_MAX)
    k = np.where(m == 0, 0, k)
    k = np.where(np.isinf(m), K_MIN, k)
    return k.astype(np.int64)


def auto_tensor_scale(y, fmt=FP8_DUAL):
    """Tensor scale g from the data (reading of [TACO] Fig. 7 "adaptive rescaling").

    g = RN(A / M) with A = max |y| over the whole tensor in the transformed
    domain and M the format's largest value (448 for E4M3, 57344 for E5M2), so
    the tensor maximum maps onto the largest code; g = 1 for an all-zero
    tensor; g is clamped to [2^-60, 2^60].
    """
    y = np.asarray(y, dtype=np.float32)
    A = np.max(np.abs(y)) if y.size else F32(0)
    if A == 0:
        return F32(1.0)
    g = F32(A) / F32(FP8_MAX[fmt])
    return F32(min(max(g, G_MIN), G_MAX))


def sum_tensor_scales(gs):
    """Tensor scale of a sum of shards: g' = g_0 + g_1 + ... in order, clamped.

    Reading: the pages do not say how the gather-stage FP8 tensor is scaled.
    Since every |dequantized value| <= M * 2^-k * g_r (M = 448 or 57344), the
    sum of the g_r bounds the sum without a second pass over it.
    """
    acc = F32(0)
    for g in gs:
        acc = F32(acc + F32(g))
    return F32(min(max(acc, G_MIN), G_MAX))


def _quantize_fp8_dual(y, g, B, fmt=FP8_DUAL):
    """Dual-scale FP8 quantization of transformed values y (float32, flat).

    w = RN(y * RN(1/g)); a w that is exactly zero is +0 (reading: the sign of
    an exact zero carries nothing); m = max |w| per block; k from
    ``block_exponent``; v = w * 2^k; q = E4M3 (or E5M2) code of v.
    """
    g = F32(g)
    inv_g = F32(F32(1.0) / g)
    yb = y.reshape(-1, B)
    w = yb * inv_g
    w = np.where(yb == 0, F32(0.0), w).astype(np.float32)
    m = np.max(np.abs(w), axis=1) if w.size else np.zeros(0, np.float32)
    k = block_exponent(m, fmt)
    v = np.ldexp(w, k[:, None]).astype(np.float32)
    q = _FP8_ENC[fmt](v)
    return q.reshape(-1), k.astype(np.int8), v.reshape(-1)


def _dequantize_fp8_dual(codes, k, g, B, fmt=FP8_DUAL):
    """x' = RN(dec(q) * 2^-k * g): dec(q) * 2^-k is exact, one rounding for g."""
    d = _FP8_DEC[fmt](codes).reshape(-1, B)
    t = np.ldexp(d, -k.astype(np.int64)[:, None]).astype(np.float32)
    return (t * F32(g)).astype(np.float32).reshape(-1)


# ------------------------------------------------------------- EQuARX INT8 --

def _quantize_int8_sym(u, B):
    """Block-wise symmetric int8 ([EQuARX], "What carries the argument").

    Per block: A = max |u| (abs-max reduction); s = RN(A / 127) is the FP32
    scale that travels with the block; q = clamp(round(RN(u * RN(127 / A))),
    -127, 127), rounding to nearest even. Readings: the code range is the
    symmetric [-127, 127]; the codes come from multiplying by the rounded
    reciprocal; a block with A < 2^-100 stores s = 0 and zero codes.
    """
    ub = u.reshape(-1, B)
    A = np.max(np.abs(ub), axis=1) if ub.size else np.zeros(0, np.float32)
    live = A >= TINY
    Asafe = np.where(live, A, F32(1.0)).astype(np.float32)
    s = np.where(live, Asafe / F32(127.0), F32(0.0)).astype(np.float32)
    inv = (F32(127.0) / Asafe).astype(np.float32)
    t = (ub * inv[:, None]).astype(np.float32)
    q = np.clip(np.rint(t), -127, 127)
    q = np.where(live[:, None], q, 0).astype(np.int8)
    t = np.where(live[:, None], t, F32(0.0)).astype(np.float32)
    return q.reshape(-1), s, t.reshape(-1)


def _dequantize_int8_sym(q, s, B):
    """Dequantize to FP32 before any addition ([EQuARX]): RN(q * s)."""
    qf = q.astype(np.int8).astype(np.float32).reshape(-1, B)
    return (qf * s[:, None]).astype(np.float32).reshape(-1)


# --------------------------------------------------------- FlashComm asym --

def _quantize_asym(u, B, bits):
    """Asymmetric min/max quantization per group ([FlashComm], "What carries
    the argument"; Algorithm 1 dequantizes from codes, zero point and scale).

    The formulas (the page's Eq. (1)-(4)) are not printed; reading, with
    qmax = 2^bits - 1: lo = min(min u, 0), hi = max(max u, 0) (the range always
    holds zero, so zero is exact); r = RN(hi - lo); s = RN(r / qmax);
    inv = RN(qmax / r); zero point z = clamp(round(RN(-lo * inv)), 0, qmax);
    q = clamp(round(RN(u * inv)) + z, 0, qmax); rounding to nearest even.
    A group with r < 2^-100 stores s = 0, z = 0 and zero codes.
    """
    qmax = F32((1 << bits) - 1)
    ub = u.reshape(-1, B)
    if ub.size:
        lo = np.minimum(np.min(ub, axis=1), F32(0.0)).astype(np.float32)
        hi = np.maximum(np.max(ub, axis=1), F32(0.0)).astype(np.float32)
    else:
        lo = hi = np.zeros(0, np.float32)
    r = (hi - lo).astype(np.float32)
    live = r >= TINY
    rsafe = np.where(live, r, F32(1.0)).astype(np.float32)
    s = np.where(live, rsafe / qmax, F32(0.0)).astype(np.float32)
    inv = (qmax / rsafe).astype(np.float32)
    z = np.clip(np.rint((-lo * inv).astype(np.float32)), 0, qmax)
    t = (ub * inv[:, None]).astype(np.float32)
    q = np.clip(np.rint(t) + z[:, None], 0, qmax)
    q = np.where(live[:, None], q, 0).astype(np.uint8)
    z = np.where(live, z, 0).astype(np.uint8)
    t = np.where(live[:, None], t, F32(0.0)).astype(np.float32)
    return q.reshape(-1), s, z, t.reshape(-1)


def _dequantize_asym(q, s, z, B):
    """RN(float(q - z) * s); q - z is an exact small integer."""
    d = (q.reshape(-1, B).astype(np.int64) - z.astype(np.int64)[:, None]).astype(np.float32)
    return (d * s[:, None]).astype(np.float32).reshape(-1)


# ------------------------------------------------------------ public API ---

def _check(codec, cols):
    B = codec.block
    if codec.format in FP8_FORMATS:
        assert B in (16, 32, 64, 128), "FP8 block must be 16, 32, 64 or 128"
    elif codec.format == INT8_SYM:
        assert B == 64, "INT8_SYM block is 64"
    elif codec.format in (INT4_ASYM, INT8_ASYM):
        assert B == 128, "asymmetric group is 128"
    else:
        raise ValueError("unknown format")
    assert cols % B == 0, "cols must be a multiple of the block"


def _pack(codec, rows, cols, q, s, z=None, g=None, pre=None):
    codes = pack_int4(q) if codec.format == INT4_ASYM else q.view(np.uint8).copy()
    return Compressed(codec, rows, cols, codes, s, z, g, pre)


def quantize_values(codec, y, rows, cols, tensor_scale=None):
    """Quantize float32 values that are already in the codec's domain.

    For FP8_DUAL, ``y`` is taken to be in the transformed (Hadamard) domain and
    no transform is applied; ``tensor_scale`` None means the data-driven g.
    """
    _check(codec, cols)
    y = np.ascontiguousarray(y, dtype=np.float32).reshape(-1)
    B = codec.block
    if codec.format in FP8_FORMATS:
        g = auto_tensor_scale(y, codec.format) if tensor_scale is None else F32(tensor_scale)
        q, k, v = _quantize_fp8_dual(y, g, B, codec.format)
        return _pack(codec, rows, cols, q, k, None, g, v)
    if codec.format == INT8_SYM:
        q, s, t = _quantize_int8_sym(y, B)
        return _pack(codec, rows, cols, q, s, None, None, t)
    q, s, z, t = _quantize_asym(y, B, codec.bits)
    return _pack(codec, rows, cols, q, s, z, None, t)


def transform(codec, x_bits):
    """Widen bf16 to float32 and, for FP8_DUAL with hadamard, apply the block FWHT.

    Reading of [TACO]'s "data-driven reshaping": the [rows, cols] tensor is
    viewed as [n / B, B] blocks along the hidden dimension (no data movement).
    """
    u = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16)).reshape(-1)
    if codec.format in FP8_FORMATS and codec.hadamard:
        return fwht(u, codec.block)
    return u


def compress(codec, x_bits, tensor_scale=None):
    """Compress one bf16 shard of shape [rows, cols] (uint16 bit patterns).

    FP8_DUAL ([TACO] Fig. 7): widen, block FWHT (if enabled), tensor scale g
    (given, or from this tensor when None), per-block exponent, E4M3 codes.
    INT8_SYM ([EQuARX]) and INT4_ASYM / INT8_ASYM ([FlashComm]) quantize the
    widened values directly.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    y = transform(codec, x_bits)
    return quantize_values(codec, y, rows, cols, tensor_scale)


def dequantize(c: Compressed):
    """Dequantize one shard to float32 (FP8_DUAL: still in the transformed domain)."""
    B = c.codec.block
    if c.codec.format in FP8_FORMATS:
        return _dequantize_fp8_dual(c.codes, c.scale, c.tensor_scale, B, c.codec.format)
    if c.codec.format == INT8_SYM:
        return _dequantize_int8_sym(c.codes.view(np.int8), c.scale, B)
    q = unpack_int4(c.codes) if c.codec.format == INT4_ASYM else c.codes
    return _dequantize_asym(q, c.scale, c.zero, B)


ALLOWED_PAIRS = {
    (FP8_DUAL, FP8_DUAL),
    (FP8E5_DUAL, FP8E5_DUAL),
    (INT8_SYM, INT8_SYM),
    (INT4_ASYM, INT8_ASYM),
    (INT8_ASYM, INT8_ASYM),
}


def check_pair(cin: Codec, cout: Codec):
    assert (cin.format, cout.format) in ALLOWED_PAIRS, "unsupported format pair"
    if cin.format in FP8_FORMATS:
        assert cin.block == cout.block and cin.hadamard == cout.hadamard
    else:
        assert cin.block == cout.block


def decompress_reduce(shards: List[Compressed], out_codec: Optional[Codec] = None):
    """Sum N compressed shards in FP32 and optionally re-quantize the sum.

    Each shard is dequantized to FP32 before it is added ([EQuARX]); the sum
    is acc = ((0 + x_0) + x_1) + ... + x_{N-1}, one float32 rounding per add
    (reading: a fixed shard order stands in for the ring order). The partial
    sum is then re-quantized for the gather stage ([FlashComm] re-quantizes to
    INT8 for the All-Gather; [EQuARX] quantizes both stages): FP8_DUAL with
    g' = sum of the shard tensor scales and no second transform (the FWHT is
    linear and shared, so the sum of transformed shards is the transform of
    the sum), INT8_SYM, or INT8_ASYM.

    Returns (acc float32 [rows, cols], Compressed or None).
    """
    assert len(shards) >= 1
    c0 = shards[0]
    for s in shards:
        assert s.codec == c0.codec and (s.rows, s.cols) == (c0.rows, c0.cols)
    acc = np.zeros(c0.rows * c0.cols, dtype=np.float32)
    for s in shards:
        acc = (acc + dequantize(s)).astype(np.float32)
    rq = None
    if out_codec is not None:
        check_pair(c0.codec, out_codec)
        g = None
        if out_codec.format in FP8_FORMATS:
            g = sum_tensor_scales([s.tensor_scale for s in shards])
        rq = quantize_values(out_codec, acc, c0.rows, c0.cols, g)
    return acc.reshape(c0.rows, c0.cols), rq


def ring_hop(incoming: Optional[Compressed], local_bits, out_codec: Codec, in_codec: Optional[Codec] = None):
    """One hop of a quantized ring reduce-scatter.

    [EQuARX] "What carries the argument": on each hop the received shard is
    dequantized to FP32 before the receiver adds its own contribution, and the
    partial sum is quantized again before it is sent on; the full-loop ring
    takes N - 1 such hops ("Extended reading notes"). Reading: the sum is
    acc = (0 + dequant(incoming)) + f32(local), one float32 rounding per add
    (the order of the decompress-reduce with the local bf16 shard as the last
    addend); incoming None is the first hop (acc = 0 + f32(local)). The
    partial sum is quantized with out_codec (INT8_SYM -> INT8_SYM,
    INT4_ASYM / INT8_ASYM -> INT8_ASYM). Transform-free formats only: the FP8
    codec's shards live in the Hadamard domain and its gather scale needs the
    local tensor's abs-max, so it is not a ring codec here.

    Returns (acc float32 [rows, cols], Compressed in out_codec).
    """
    x = bf16_bits_to_f32(np.asarray(local_bits, dtype=np.uint16))
    rows, cols = x.shape
    assert out_codec.format in (INT8_SYM, INT8_ASYM), "ring hops use INT8 codecs"
    acc = np.zeros(rows * cols, dtype=np.float32)
    if incoming is not None:
        assert (incoming.rows, incoming.cols) == (rows, cols)
        check_pair(incoming.codec, out_codec)
        acc = (acc + dequantize(incoming)).astype(np.float32)
    elif in_codec is not None:
        check_pair(in_codec, out_codec)
    acc = (acc + x.reshape(-1)).astype(np.float32)
    return acc.reshape(rows, cols), quantize_values(out_codec, acc, rows, cols, None)


def full_loop_ring(locals_bits, codec: Codec):
    """The full-loop ring for one chunk ([EQuARX] "What carries the argument":
    bandwidth-optimal, N - 1 hops): rank 0 quantizes its shard, every later
    rank r = 1 .. N-1 dequantizes what it received, adds its own shard and
    quantizes again (``ring_hop``); the last rank's output is what the
    all-gather sends. Returns the Compressed result in ``codec`` (INT8_SYM or
    INT8_ASYM)."""
    q = None
    for x in locals_bits:
        _, q = ring_hop(q, x, codec, in_codec=codec)
    return q


def semi_loop_ring(locals_bits, codec: Codec):
    """The semi-loop ring for one chunk ([EQuARX] "What carries the argument":
    it uses both ring directions to halve the number of quantization hops; its
    adder chain is a figure the page does not reproduce). Reading: with N >= 2
    ranks and h = N // 2, ranks 0 .. h-1 form a chain in one direction and
    ranks N-1 .. h a chain in the other, each link a ``ring_hop`` as in the
    full loop (every rank quantizes what it sends on); the two chains' outputs
    meet, are dequantized to FP32 and added in the order (first chain, second
    chain), and the sum is quantized once for the all-gather
    (``decompress_reduce`` of the two). The longest chain has N - h
    quantizations instead of the full loop's N.

    Returns the Compressed result in ``codec``."""
    n = len(locals_bits)
    assert n >= 2, "the semi-loop needs two ranks or more"
    h = n // 2
    first = full_loop_ring(locals_bits[:h], codec)
    second = full_loop_ring(locals_bits[h:][::-1], codec)
    _, rq = decompress_reduce([first, second], codec)
    return rq


# ------------------------------------------------ data-driven reshaping -----

CHUNK = 8   # channels per reordered group (the kernels move 16-byte bf16 vectors)


def chunk_order(stats_bits):
    """Data-driven reshaping of the hidden dimension ([TACO] abstract and
    "What carries the argument": the tensor is reshaped adaptively, from the
    data, before the Adaptive Scale-Hadamard Transform; the page does not say
    how). Reading: the hidden channels are taken in groups of CHUNK = 8
    consecutive channels; each group's statistic is its largest magnitude over
    every row of a statistics tensor (e.g. an earlier step's activation, the
    same on every rank); the groups are ordered by that statistic, largest
    first, equal statistics by group index, so that the blocks of the reordered
    tensor hold channels of similar magnitude.

    Returns order (int64 [cols / 8]): reordered group j is original group
    order[j]."""
    x = bf16_bits_to_f32(np.asarray(stats_bits, dtype=np.uint16))
    rows, cols = x.shape
    assert cols % CHUNK == 0
    m = np.max(np.abs(x), axis=0) if rows else np.zeros(cols, np.float32)
    g = np.max(m.reshape(-1, CHUNK), axis=1)
    g = np.where(np.isnan(g), np.float32(np.inf), g)   # reading: a NaN group sorts as the largest
    return np.lexsort((np.arange(g.size), -g.astype(np.float64))).astype(np.int64)


def _column_map(order, cols):
    order = np.asarray(order, dtype=np.int64)
    assert order.size * CHUNK == cols and np.array_equal(np.sort(order), np.arange(order.size)), \
        "order must be a permutation of the channel groups"
    return (order[:, None] * CHUNK + np.arange(CHUNK)[None, :]).reshape(-1)


def reorder_columns(x, order):
    """Columns of a [rows, cols] array in reordered form: reordered column
    8 j + i is original column 8 order[j] + i."""
    x = np.asarray(x)
    return x[:, _column_map(order, x.shape[1])]


def restore_columns(y, order):
    """Inverse of reorder_columns."""
    y = np.asarray(y)
    out = np.empty_like(y)
    out[:, _column_map(order, y.shape[1])] = y
    return out


def compress_reordered(codec, x_bits, order, tensor_scale=None):
    """compress() of the reordered tensor: the codec sees the channel groups in
    the data-driven order (the compressed buffer, the reduce and the
    requantization all work in that order)."""
    return compress(codec, reorder_columns(np.asarray(x_bits, dtype=np.uint16), order), tensor_scale)


def decode_reordered(c, order, out_dtype="f32"):
    """decode() followed by the inverse reordering of the channels."""
    return restore_columns(decode(c, out_dtype), order)


def requantize(codec, x_f32, tensor_scale=None):
    """Quantize a caller-supplied float32 tensor (FP8: taken as transformed values)."""
    x = np.asarray(x_f32, dtype=np.float32)
    rows, cols = x.shape
    return quantize_values(codec, x, rows, cols, tensor_scale)


def decode(c: Compressed, out_dtype="f32"):
    """Consumer-side decode: dequantize and undo the transform.

    FP8_DUAL with hadamard: x = FWHT(y') * 2^-log2(B) (the Sylvester matrix is
    its own inverse up to 1/B); an exactly-zero result is +0.
    Returns float32 [rows, cols], or bf16 bit patterns if out_dtype == "bf16".
    """
    y = dequantize(c)
    if c.codec.format in FP8_FORMATS and c.codec.hadamard:
        B = c.codec.block
        t = fwht(y, B)
        x = np.ldexp(t, -int(np.log2(B))).astype(np.float32)
        x = np.where(t == 0, F32(0.0), x).astype(np.float32)
    else:
        x = y
    x = x.reshape(c.rows, c.cols)
    if out_dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def decode_gemm(c: Compressed, w_bits):
    """The consumer of a gathered activation: decode(A) @ W^T.

    [FlashComm] "What carries the argument" and Fig. 8: the quantized volume is
    dequantized on the receiving side and handed to the next computation, here
    a linear layer with weight W (bf16 bit patterns [N, K], the rows of W are
    the output features). The activation is the bf16 tensor decode() writes;
    the products are summed in float64, so the result is the exact value of
    the product up to float64 rounding.

    Returns (out, mag), both float64 [M, N]: out = A W^T and mag = |A| |W|^T,
    the sum of the magnitudes of the products, which bounds any summation
    order's rounding error when scaled by the unit roundoff of the
    accumulator.
    """
    a = bf16_bits_to_f32(decode(c, "bf16")).astype(np.float64)
    w = bf16_bits_to_f32(np.asarray(w_bits, dtype=np.uint16)).astype(np.float64)
    if w.ndim != 2 or w.shape[1] != c.cols:
        raise ValueError("W must be [N, K] with K the activation's cols")
    return a @ w.T, np.abs(a) @ np.abs(w).T
