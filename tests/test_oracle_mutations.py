"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one. A pin set that lets a dropped term, a wrong sign, a wrong index
or a wrong constant through would not be worth trusting."""

import numpy as np
import pytest

from oracle import codecs as cd
from oracle import formats as fm
from oracle import hadamard as hd
import tests.test_oracle_codecs as TC
import tests.test_oracle_formats as TF
import tests.test_oracle_hadamard as TH


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_encoder_ties_away_from_zero_is_caught(monkeypatch):
    real = fm.encode_e4m3

    def bad(v):
        v = np.asarray(v, np.float32)
        # nudge exact ties upward: rounds half away from zero
        return real(np.where(np.isfinite(v), v * np.float32(1 + 2 ** -22), v))
    monkeypatch.setattr(fm, "encode_e4m3", bad)
    assert _fails(TF.test_e4m3_rounding_golden)


def test_encoder_without_saturation_is_caught(monkeypatch):
    real = fm.encode_e4m3

    def bad(v):
        c = real(v)
        big = np.abs(np.asarray(v, np.float32)) > 464
        return np.where(big, np.uint8(0x7F) | (c & 0x80), c).astype(np.uint8)
    monkeypatch.setattr(fm, "encode_e4m3", bad)
    assert _fails(TF.test_e4m3_rounding_golden)


def test_swapped_butterfly_is_caught(monkeypatch):
    def bad(y, B):
        h = 1
        while h < B:
            v = y.reshape(-1, B // (2 * h), 2, h)
            a, b = v[:, :, 0, :], v[:, :, 1, :]
            y = np.stack([a - b, a + b], axis=2).reshape(-1, B)
            h *= 2
        return y
    monkeypatch.setattr(hd, "_butterflies", bad)
    assert _fails(TH.test_fwht_golden_examples)
    assert _fails(TH.test_fwht_equals_dense_sylvester_matrix, 8)


def test_skipped_butterfly_stage_is_caught(monkeypatch):
    def bad(y, B):
        h = 2
        while h < B:
            v = y.reshape(-1, B // (2 * h), 2, h)
            a, b = v[:, :, 0, :], v[:, :, 1, :]
            y = np.stack([a + b, a - b], axis=2).reshape(-1, B)
            h *= 2
        return y
    monkeypatch.setattr(hd, "_butterflies", bad)
    assert _fails(TH.test_fwht_equals_dense_sylvester_matrix, 16)


def test_exponent_threshold_and_offset_errors_are_caught(monkeypatch):
    real = cd.block_exponent
    monkeypatch.setattr(cd, "block_exponent", lambda m, *f: real(m, *f) + 1)
    assert _fails(TC.test_block_exponent_bruteforce)
    monkeypatch.setattr(cd, "block_exponent",
                        lambda m, *f: np.where(np.asarray(m) > 0, real(np.asarray(m) * np.float32(0.99), *f), 0))
    assert _fails(TC.test_block_exponent_bruteforce)


def test_int8_scale_over_128_is_caught(monkeypatch):
    real = cd._quantize_int8_sym

    def bad(u, B):
        q, s, t = real(u, B)
        return q, (s * np.float32(127.0 / 128.0)).astype(np.float32), t
    monkeypatch.setattr(cd, "_quantize_int8_sym", bad)
    assert _fails(TC.test_int8_sym_extremes_and_error_bound)


def test_asym_zero_point_sign_error_is_caught(monkeypatch):
    real = cd._quantize_asym

    def bad(u, B, bits):
        q, s, z, t = real(u, B, bits)
        qmax = (1 << bits) - 1
        return q, s, (qmax - z).astype(np.uint8), t
    monkeypatch.setattr(cd, "_quantize_asym", bad)
    assert _fails(TC.test_int_codecs_golden)


def test_dequant_dropping_tensor_scale_is_caught(monkeypatch):
    def bad(codes, k, g, B, fmt=cd.FP8_DUAL):
        d = fm.decode_e4m3(codes).reshape(-1, B)
        return np.ldexp(d, -k.astype(np.int64)[:, None]).astype(np.float32).reshape(-1)
    monkeypatch.setattr(cd, "_dequantize_fp8_dual", bad)
    assert _fails(TC.test_fp8_dual_error_within_eq3_bound)


def test_requant_with_max_scale_instead_of_sum_is_caught(monkeypatch):
    monkeypatch.setattr(cd, "sum_tensor_scales", lambda gs: np.float32(max(gs)))
    assert _fails(TC.test_taco_reduce_is_linear_through_the_transform) or \
        _fails(TC.test_taco_requant_never_saturates_with_summed_scale)


def test_int4_nibble_order_swap_is_caught(monkeypatch):
    def bad(q):
        q = np.asarray(q, np.uint8)
        return ((q[..., 1::2] & 0xF) | ((q[..., 0::2] & 0xF) << 4)).astype(np.uint8)
    monkeypatch.setattr(fm, "pack_int4", bad)
    assert _fails(TF.test_int4_pack_roundtrip_exhaustive)


def _bad_ring_hop(sign, keep_incoming):
    """A ring hop with the local term's sign flipped, or the incoming dropped."""
    import oracle

    def bad(incoming, local_bits, out_codec, in_codec=None):
        x = fm.bf16_bits_to_f32(np.asarray(local_bits, dtype=np.uint16))
        rows, cols = x.shape
        acc = np.zeros(rows * cols, dtype=np.float32)
        if incoming is not None and keep_incoming:
            acc = (acc + cd.dequantize(incoming)).astype(np.float32)
        acc = (acc + np.float32(sign) * x.reshape(-1)).astype(np.float32)
        return acc.reshape(rows, cols), cd.quantize_values(out_codec, acc, rows, cols, None)
    return bad


@pytest.mark.parametrize("sign,keep", [(-1.0, True), (1.0, False)], ids=["sign", "dropped"])
def test_ring_hop_mistakes_are_caught(monkeypatch, sign, keep):
    import oracle
    import tests.test_oracle_ring as TR
    monkeypatch.setattr(oracle, "ring_hop", _bad_ring_hop(sign, keep))
    assert _fails(TR.test_hop_sum_is_exact_when_every_term_is_representable)
    assert _fails(TR.test_ring_mse_matches_the_reported_values)


def test_e5m2_encoder_mistakes_are_caught(monkeypatch):
    real = fm.encode_e5m2

    def ties_away(v):
        v = np.asarray(v, np.float32)
        return real(np.where(np.isfinite(v), v * np.float32(1 + 2 ** -22), v))
    monkeypatch.setattr(fm, "encode_e5m2", ties_away)
    assert _fails(TF.test_e5m2_rounding_golden)

    def no_saturation(v):
        c = real(v)
        big = np.abs(np.asarray(v, np.float32)) > 57344
        return np.where(big, np.uint8(0x7C) | (c & 0x80), c).astype(np.uint8)
    monkeypatch.setattr(fm, "encode_e5m2", no_saturation)
    assert _fails(TF.test_e5m2_special_values)


def test_e5m2_decoder_bias_error_is_caught(monkeypatch):
    real = fm.decode_e5m2
    monkeypatch.setattr(fm, "decode_e5m2", lambda c: (real(c) * np.float32(2.0)).astype(np.float32))
    assert _fails(TF.test_e5m2_landmarks_golden)


def test_e5m2_exponent_with_the_e4m3_limit_is_caught(monkeypatch):
    real = cd.block_exponent
    monkeypatch.setattr(cd, "block_exponent", lambda m, *f: real(m))
    assert _fails(TC.test_block_exponent_e5m2_bruteforce_and_range)


# ---------------------------------------------- metrics and tensor scales --
import oracle  # noqa: E402
import tests.test_oracle_ring as TR  # noqa: E402
import tests.test_oracle_scales_metrics as TS  # noqa: E402


@pytest.mark.parametrize("name,bad", [
    ("mse", lambda a, b: float(np.sum((np.asarray(a, np.float64) - np.asarray(b, np.float64)) ** 2))),
    ("rel_mse", lambda a, b: float(np.mean((np.asarray(a, np.float64) - np.asarray(b, np.float64)) ** 2))
     / float(np.sum(np.asarray(b, np.float64) ** 2))),
    ("rel_l2", lambda a, b: float(np.sum((np.asarray(a, np.float64) - np.asarray(b, np.float64)) ** 2))
     / float(np.sum(np.asarray(b, np.float64) ** 2))),                        # no square roots
    ("rel_l2", lambda a, b: float(np.linalg.norm(np.asarray(a, np.float64) - np.asarray(b, np.float64)))
     / float(np.linalg.norm(np.asarray(a, np.float64)))),                     # the other reference
], ids=["mse-sum", "rel_mse-mean", "rel_l2-no-sqrt", "rel_l2-swapped"])
def test_metric_mistakes_are_caught(monkeypatch, name, bad):
    monkeypatch.setattr(oracle, name, bad)
    assert _fails(TS.test_metrics_golden)


def _auto_scale_variant(absfn=np.abs, M=None, clamp=True):
    def f(y, fmt=cd.FP8_DUAL):
        y = np.asarray(y, np.float32)
        A = np.max(absfn(y)) if y.size else np.float32(0)
        if A == 0:
            return np.float32(1.0)
        g = np.float32(A) / np.float32(M if M is not None else cd.FP8_MAX[fmt])
        return np.float32(min(max(g, cd.G_MIN), cd.G_MAX)) if clamp else np.float32(g)
    return f


@pytest.mark.parametrize("bad", [
    _auto_scale_variant(absfn=lambda y: y),          # signed maximum instead of the abs-max
    _auto_scale_variant(M=447.0),                    # wrong constant
    _auto_scale_variant(M=448.0),                    # the E4M3 constant for both formats
], ids=["signed-max", "M-447", "M-448-for-e5m2"])
def test_auto_tensor_scale_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(cd, "auto_tensor_scale", bad)
    caught = _fails(TS.test_auto_tensor_scale_is_the_nearest_float_to_transformed_absmax_over_M, cd.FP8_DUAL, 448) \
        or _fails(TS.test_auto_tensor_scale_is_the_nearest_float_to_transformed_absmax_over_M, cd.FP8E5_DUAL, 57344)
    assert caught


def test_auto_scale_from_untransformed_values_is_caught(monkeypatch):
    real = cd.quantize_values

    def bad(codec, y, rows, cols, tensor_scale=None):
        if codec.format in cd.FP8_FORMATS and tensor_scale is None:
            # the abs-max of the inverse-transformed values (the input domain)
            x = hd.fwht(np.asarray(y, np.float32).reshape(-1), codec.block) / np.float32(codec.block)
            tensor_scale = cd.auto_tensor_scale(x, codec.format)
        return real(codec, y, rows, cols, tensor_scale)
    monkeypatch.setattr(cd, "quantize_values", bad)
    assert _fails(TS.test_auto_tensor_scale_is_the_nearest_float_to_transformed_absmax_over_M, cd.FP8_DUAL, 448)


def test_missing_tensor_scale_clamp_is_caught(monkeypatch):
    monkeypatch.setattr(cd, "auto_tensor_scale", _auto_scale_variant(clamp=False))
    assert _fails(TS.test_tensor_scale_clamps, cd.FP8_DUAL)


@pytest.mark.parametrize("bad", [
    lambda gs: np.float32(min(max(np.float32(sum(float(g) for g in gs)), cd.G_MIN), cd.G_MAX)),   # float64 sum
    lambda gs: np.float32(sum(np.float32(g) for g in gs)),                                          # no clamp
], ids=["f64-sum", "no-clamp"])
def test_gather_scale_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(cd, "sum_tensor_scales", bad)
    assert _fails(TS.test_gather_scale_sum_order_and_clamps)


@pytest.mark.parametrize("bad", [
    lambda xs, codec: cd.full_loop_ring(xs, codec),                                                # no second direction
    lambda xs, codec: cd.decompress_reduce([cd.full_loop_ring(xs[:len(xs) // 2], codec),
                                            cd.full_loop_ring(xs[len(xs) // 2 + 1:][::-1], codec)],
                                           codec)[1],                                              # a rank dropped
], ids=["full-loop", "dropped-rank"])
def test_semi_loop_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(oracle, "semi_loop_ring", bad)
    assert _fails(TR.test_semi_loop_ring_error_statistics)


# ---------------------------------------------------- data-driven reshaping --
import tests.test_oracle_reorder as TO  # noqa: E402


def _order_variant(desc=True, ties_by_index=True, chunk=8):
    def f(stats_bits):
        x = fm.bf16_bits_to_f32(np.asarray(stats_bits, dtype=np.uint16))
        g = np.max(np.abs(x), axis=0).reshape(-1, chunk).max(axis=1).astype(np.float64)
        idx = np.arange(g.size) if ties_by_index else -np.arange(g.size)
        return np.lexsort((idx, -g if desc else g)).astype(np.int64)
    return f


@pytest.mark.parametrize("bad", [_order_variant(desc=False), _order_variant(ties_by_index=False),
                                 _order_variant(chunk=16)], ids=["ascending", "ties-reversed", "groups-of-16"])
def test_order_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(oracle, "chunk_order", bad)
    assert _fails(TO.test_hand_worked_order) or any(_fails(TO.test_order_matches_a_brute_force_sort, s)
                                                    for s in range(4))


def test_restore_with_the_order_itself_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "restore_columns", lambda y, order: oracle.reorder_columns(y, order))
    assert _fails(TO.test_reorder_and_restore_are_inverse_permutations)


def _gemm_variant(kind):
    def bad(c, w_bits):
        if kind == "f32_activation":
            a = cd.decode(c, "f32").astype(np.float64)
        else:
            a = fm.bf16_bits_to_f32(cd.decode(c, "bf16")).astype(np.float64)
        w = fm.bf16_bits_to_f32(np.asarray(w_bits, np.uint16)).astype(np.float64)
        if kind == "magnitude_weight":
            w = np.abs(w)
        if kind == "reversed_k":
            w = w[:, ::-1]
        return a @ w.T, np.abs(a) @ np.abs(w).T
    return bad


@pytest.mark.parametrize("kind", ["f32_activation", "magnitude_weight", "reversed_k"])
def test_decode_gemm_mistakes_are_caught(monkeypatch, kind):
    import oracle
    import tests.test_oracle_gemm as TG
    monkeypatch.setattr(oracle, "decode_gemm", _gemm_variant(kind))
    assert _fails(TG.test_decode_gemm_equals_exact_sum, cd.INT8_ASYM)
    assert _fails(TG.test_decode_gemm_equals_exact_sum, cd.FP8_DUAL)
