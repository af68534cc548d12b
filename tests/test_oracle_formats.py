"""Pins of the oracle's number formats against closed forms, brute force and a
library (torch's float8_e4m3fn / bfloat16 casts). CPU only."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as fm
from tests.conftest import read_golden


def all_finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


# ---------------------------------------------------------------- decode --

def test_e4m3_landmarks_golden():
    for code, val in read_golden("e4m3_landmarks.txt"):
        got = fm.decode_e4m3(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == np.float32(float(val)), (code, got, val)
            assert np.signbit(got) == val.startswith("-"), code


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = fm.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert (np.signbit(ours) == np.signbit(ref))[~np.isnan(ours)].all()


def test_e4m3_decode_grid_structure():
    """Positive finite codes are strictly increasing; subnormals are evenly spaced
    by 2^-9; each normal binade holds 8 values spaced 2^(e-3)."""
    pos = fm.decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64)
    assert np.all(np.diff(pos) > 0)
    assert np.allclose(np.diff(pos[:9]), 2.0 ** -9, rtol=0, atol=0)
    for e in range(1, 16):
        b = pos[8 * e: 8 * e + 8]
        if len(b) < 2:
            continue
        step = 2.0 ** (e - 7 - 3)
        assert np.all(np.diff(b) == step)
        assert b[0] == 2.0 ** (e - 7)
    assert pos[-1] == 448.0


# ---------------------------------------------------------------- encode --

def nearest_code_bruteforce(v):
    """Nearest finite E4M3 code by exhaustive search; ties to the even code
    (even mantissa); saturate beyond 448; sign kept for zero results."""
    codes = np.array([c for c in range(0, 0x7F)], dtype=np.uint8)   # non-negative finite
    vals = fm.decode_e4m3(codes).astype(np.float64)
    out = np.empty(len(v), dtype=np.uint8)
    for i, x in enumerate(np.asarray(v, np.float64)):
        a = min(abs(x), 448.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        if len(best) == 2:
            best = [b for b in best if (codes[b] & 1) == 0]
        c = int(codes[best[0]])
        out[i] = c | (0x80 if math.copysign(1.0, x) < 0 else 0)
    return out


def test_e4m3_rounding_golden():
    rows = read_golden("e4m3_rounding.txt")
    v = np.array([float(r[0]) for r in rows], np.float32)
    want = np.array([int(r[1], 16) for r in rows], np.uint8)
    got = fm.encode_e4m3(v)
    assert (got == want).all(), list(zip(v, got, want))


def test_e4m3_roundtrip_every_finite_code():
    c = all_finite_codes()
    assert (fm.encode_e4m3(fm.decode_e4m3(c)) == c).all()


def bf16_all_finite():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = fm.bf16_bits_to_f32(bits)
    return x[np.isfinite(x)]


@pytest.mark.parametrize("scale_exp", [0, -8, 6])
def test_e4m3_encode_bruteforce_all_bf16(scale_exp):
    """Every finite bf16 value (times 2^s, landing in and around the E4M3 range),
    against the exhaustive nearest-code search."""
    with np.errstate(over="ignore"):
        x = (bf16_all_finite() * np.float32(2.0 ** scale_exp)).astype(np.float32)
    # keep the interesting span: around and inside [2^-12, 2^10]
    a = np.abs(x)
    x = x[((a > 2.0 ** -12) & (a < 2.0 ** 10)) | (a == 0)]
    assert (fm.encode_e4m3(x) == nearest_code_bruteforce(x)).all()


def test_e4m3_midpoints_and_neighbours():
    vals = fm.decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    v = np.concatenate([mids, up, dn, -mids, -up, -dn, [448, 464, 480, 1e30, -1e30]]).astype(np.float32)
    assert (fm.encode_e4m3(v) == nearest_code_bruteforce(v)).all()


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 0.01,
        rng.standard_normal(20000) * 30,
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (fm.encode_e4m3(v) == ref).all()


def test_e4m3_special_values():
    v = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 448.0, 464.0], np.float32)
    got = fm.encode_e4m3(v)
    assert list(got) == [0x7F, 0x7E, 0xFE, 0x00, 0x80, 0x7E, 0x7E]


# -------------------------------------------------------- Eq. (3) bound --

def test_eq3_ulp_bound_golden():
    for x, bound in read_golden("eq3_bound.txt"):
        x, bound = np.float32(float(x)), float(bound)
        err = abs(float(fm.decode_e4m3(fm.encode_e4m3(np.array([x])))[0]) - float(x))
        assert err <= bound, (x, err, bound)
        # round-to-nearest achieves half the bound
        assert err <= bound / 2


def test_eq3_ulp_bound_random():
    rng = np.random.default_rng(11)
    x = np.exp2(rng.uniform(-6, math.log2(448), 200000)).astype(np.float32)
    x = np.where(rng.integers(0, 2, x.size) == 1, -x, x).astype(np.float32)
    err = np.abs(fm.decode_e4m3(fm.encode_e4m3(x)).astype(np.float64) - x)
    ulp = np.exp2(np.floor(np.log2(np.abs(x).astype(np.float64))) - 3)
    assert np.all(err <= ulp / 2)
    # subnormal inputs: absolute error at most half of 2^-9
    xs = rng.uniform(-2.0 ** -6, 2.0 ** -6, 100000).astype(np.float32)
    errs = np.abs(fm.decode_e4m3(fm.encode_e4m3(xs)).astype(np.float64) - xs)
    assert np.all(errs <= 2.0 ** -10)


# ------------------------------------------------------ bf16 and INT4 --

def test_bf16_widen_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = fm.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        [0.0, -0.0, 1e-40, -1e-40, 3.3e38]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (fm.f32_to_bf16_bits(x) == ref).all()


def test_int4_pack_roundtrip_exhaustive():
    b = np.arange(256, dtype=np.uint8)
    q = fm.unpack_int4(b)
    assert (fm.pack_int4(q) == b).all()
    assert q[2 * 0x3A] == 0xA and q[2 * 0x3A + 1] == 0x3   # low nibble first


def test_rint_is_nearest_even():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 0.49999997, 2.5000002, -63.5, 126.5], np.float32)
    want = [0, 2, 2, -0, -2, -2, 0, 3, -64, 126]
    assert list(np.rint(x).astype(int)) == want


# ------------------------------------------------------------------ E5M2 --

def all_finite_e5m2_codes():
    return np.array([c for c in range(256) if (c & 0x7C) != 0x7C], dtype=np.uint8)


def nearest_e5m2_bruteforce(v):
    """Nearest finite E5M2 code by exhaustive search; ties to the even code
    (even mantissa); saturate beyond 57344; sign kept for zero results."""
    codes = np.array([c for c in range(0, 0x7C)], dtype=np.uint8)   # non-negative finite
    vals = fm.decode_e5m2(codes).astype(np.float64)
    out = np.empty(len(v), dtype=np.uint8)
    for i, x in enumerate(np.asarray(v, np.float64)):
        a = min(abs(x), 57344.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        if len(best) == 2:
            best = [b for b in best if (codes[b] & 1) == 0]
        c = int(codes[best[0]])
        out[i] = c | (0x80 if math.copysign(1.0, x) < 0 else 0)
    return out


def test_e5m2_landmarks_golden():
    for code, val in read_golden("e5m2_landmarks.txt"):
        got = fm.decode_e5m2(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == np.float32(float(val)), (code, got, val)
            assert np.signbit(got) == val.startswith("-"), code


def test_e5m2_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = fm.decode_e5m2(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float32).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert (np.signbit(ours) == np.signbit(ref))[~np.isnan(ours)].all()


def test_e5m2_decode_grid_structure():
    """Positive finite codes are strictly increasing; subnormals are evenly spaced
    by 2^-16; each normal binade holds 4 values spaced 2^(e-15-2)."""
    pos = fm.decode_e5m2(np.arange(0, 0x7C, dtype=np.uint8)).astype(np.float64)
    assert np.all(np.diff(pos) > 0)
    assert np.all(np.diff(pos[:5]) == 2.0 ** -16)
    for e in range(1, 31):
        b = pos[4 * e: 4 * e + 4]
        assert b[0] == 2.0 ** (e - 15)
        assert np.all(np.diff(b) == 2.0 ** (e - 15 - 2))
    assert pos[-1] == 57344.0


def test_e5m2_rounding_golden():
    rows = read_golden("e5m2_rounding.txt")
    v = np.array([float(r[0]) for r in rows], np.float32)
    want = np.array([int(r[1], 16) for r in rows], np.uint8)
    got = fm.encode_e5m2(v)
    assert (got == want).all(), list(zip(v, got, want))


def test_e5m2_roundtrip_every_finite_code():
    c = all_finite_e5m2_codes()
    assert (fm.encode_e5m2(fm.decode_e5m2(c)) == c).all()


@pytest.mark.parametrize("scale_exp", [0, -14, 12])
def test_e5m2_encode_bruteforce_all_bf16(scale_exp):
    """Every finite bf16 value (times 2^s, landing in and around the E5M2 range),
    against the exhaustive nearest-code search."""
    with np.errstate(over="ignore"):
        x = (bf16_all_finite() * np.float32(2.0 ** scale_exp)).astype(np.float32)
    a = np.abs(x)
    x = x[((a > 2.0 ** -19) & (a < 2.0 ** 17)) | (a == 0)]
    assert (fm.encode_e5m2(x) == nearest_e5m2_bruteforce(x)).all()


def test_e5m2_midpoints_and_neighbours():
    vals = fm.decode_e5m2(np.arange(0, 0x7C, dtype=np.uint8)).astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    v = np.concatenate([mids, up, dn, -mids, -up, -dn, [57344, 61440, 65536, 1e30, -1e30]]).astype(np.float32)
    assert (fm.encode_e5m2(v) == nearest_e5m2_bruteforce(v)).all()


def test_e5m2_encode_matches_torch_in_range():
    """torch's cast rounds to nearest even and does not saturate; inside
    [-57344, 57344] the two must agree."""
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.uniform(-57344, 57344, 20000),
        rng.standard_normal(20000) * 1e-4,
        rng.standard_normal(20000) * 300,
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert (fm.encode_e5m2(v) == ref).all()


def test_e5m2_special_values():
    v = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 57344.0, 61440.0], np.float32)
    got = fm.encode_e5m2(v)
    assert list(got) == [0x7F, 0x7B, 0xFB, 0x00, 0x80, 0x7B, 0x7B]


def test_e5m2_eq3_ulp_bound_random():
    """[TACO] Eq. (3) with m = 2: |e| <= 2^(floor(log2|x|) - 2) in the normal
    range; nearest rounding gives half of it. Subnormals: absolute error at
    most half of 2^-16."""
    rng = np.random.default_rng(13)
    x = np.exp2(rng.uniform(-14, math.log2(57344), 200000)).astype(np.float32)
    x = np.where(rng.integers(0, 2, x.size) == 1, -x, x).astype(np.float32)
    err = np.abs(fm.decode_e5m2(fm.encode_e5m2(x)).astype(np.float64) - x)
    ulp = np.exp2(np.floor(np.log2(np.abs(x).astype(np.float64))) - 2)
    assert np.all(err <= ulp / 2)
    xs = rng.uniform(-2.0 ** -14, 2.0 ** -14, 100000).astype(np.float32)
    errs = np.abs(fm.decode_e5m2(fm.encode_e5m2(xs)).astype(np.float64) - xs)
    assert np.all(errs <= 2.0 ** -17)
