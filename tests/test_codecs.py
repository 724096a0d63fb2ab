"""Pins for the oracle's number formats (CPU only).

Every bfloat16 pattern and every e4m3 code is checked; the encoders are
cross-checked against torch's CPU conversions (library routines) and against
values fixed by the formats' definitions (tests/golden/*.txt).
"""
import os

import numpy as np
import pytest
import torch

from oracle.codecs import (bf16_decode, bf16_encode, e4m3_decode, e4m3_encode, E4M3_MAX,
                           e5m2_decode, e5m2_encode, E5M2_MAX)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _parse_float(s):
    return float.fromhex(s) if "0x" in s else float(s)


def test_bf16_golden_values():
    for val, bits in _read_table("bf16_known.txt"):
        v = _parse_float(val)
        got = int(bf16_encode(np.array([v]))[0])
        assert got == int(bits, 16), (val, hex(got), bits)


def test_bf16_all_patterns_roundtrip():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_decode(bits)
    finite = np.isfinite(vals)
    assert np.array_equal(bf16_encode(vals[finite]), bits[finite])
    # infinities round-trip too
    inf = np.isinf(vals)
    assert np.array_equal(bf16_encode(vals[inf]), bits[inf])
    # decode matches torch's view of the same bits
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), np.isnan(vals))
    assert np.array_equal(t[finite], vals[finite])


def test_bf16_midpoints_round_to_even():
    bits = np.arange(0x0000, 0x7F7F, dtype=np.uint16)   # positive finite, next one finite
    lo = bf16_decode(bits)
    hi = bf16_decode(bits + 1)
    mid = (lo + hi) / 2                                 # exact in float64
    got = bf16_encode(mid)
    even = np.where(bits % 2 == 0, bits, bits + 1).astype(np.uint16)
    assert np.array_equal(got, even)
    # just above / below the midpoint go to the nearer neighbour
    above = np.nextafter(mid, np.inf)
    below = np.nextafter(mid, -np.inf)
    assert np.array_equal(bf16_encode(above), (bits + 1).astype(np.uint16))
    assert np.array_equal(bf16_encode(below), bits)
    # the negative side is symmetric
    assert np.array_equal(bf16_encode(-mid), even | np.uint16(0x8000))


def test_bf16_overflow_and_nan():
    big = bf16_decode(np.array([0x7F7F], np.uint16))[0]
    ulp = 2.0 ** (127 - 7)
    assert bf16_encode(np.array([big + ulp / 2]))[0] == 0x7F80     # tie -> even -> inf
    assert bf16_encode(np.array([big + ulp / 2 - 2.0 ** 80]))[0] == 0x7F7F
    assert bf16_encode(np.array([np.nan]))[0] & 0x7F80 == 0x7F80


def test_bf16_matches_torch_on_random_f32():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-60, 60, 1_000_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_encode(x.astype(np.float64)), ref)


def test_bf16_single_rounding_from_float64():
    # A float64 just above a bf16 midpoint whose float32 rounding lands on the
    # midpoint: a single rounding goes up; f64->f32->bf16 would go to even.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert bf16_encode(np.array([v]))[0] == 0x3F81


def test_e4m3_golden_values():
    for val, code in _read_table("e4m3_known.txt"):
        got = int(e4m3_encode(np.array([float(val)]))[0])
        assert got == int(code, 16), (val, hex(got), code)
        dec = e4m3_decode(np.array([int(code, 16)], np.uint8))[0]
        assert dec == float(val)


def test_e4m3_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_decode(codes)
    nan = np.isnan(vals)
    assert set(codes[nan].tolist()) == {0x7F, 0xFF}
    assert np.nanmax(vals) == E4M3_MAX and np.nanmin(vals) == -E4M3_MAX
    assert np.array_equal(e4m3_encode(vals[~nan]), codes[~nan])
    # matches torch's decoding of the same codes
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], vals[~nan])
    # the positive finite values are strictly increasing with the code
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_e4m3_midpoints_and_saturation():
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mid = (pos[:-1] + pos[1:]) / 2
    got = e4m3_encode(mid)
    lo_codes = np.arange(0x7E, dtype=np.uint8)
    even = np.where(lo_codes % 2 == 0, lo_codes, lo_codes + 1).astype(np.uint8)
    assert np.array_equal(got, even)
    assert e4m3_encode(np.array([449.0, 464.0, 1e9, -1e9])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00          # tie below min subnormal -> 0
    assert e4m3_encode(np.array([2.0 ** -10 * 1.0001]))[0] == 0x01


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(11)
    x = (rng.uniform(-448, 448, 500_000) * np.exp(rng.uniform(-12, 0, 500_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x.astype(np.float64)), ref)


def test_e5m2_all_codes():
    """Every code decodes to its format-definition value (torch's float8_e5m2 as a
    second reading), and every finite value encodes back to its code."""
    codes = np.arange(256, dtype=np.uint8)
    vals = e5m2_decode(codes)
    fin = np.isfinite(vals)
    assert fin.sum() == 248 and np.isinf(vals).sum() == 2 and np.isnan(vals).sum() == 6
    assert np.array_equal(e5m2_encode(vals[fin]), codes[fin])
    t = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(vals[fin], t[fin])
    assert vals[0x7B] == E5M2_MAX == 1.75 * 2.0 ** 15
    assert vals[0x01] == 2.0 ** -16 and vals[0x04] == 2.0 ** -14      # min subnormal, min normal
    assert vals[0x3C] == 1.0 and vals[0x3D] == 1.25 and vals[0xBE] == -1.5


def test_e5m2_midpoints_and_saturation():
    pos = e5m2_decode(np.arange(0x7C, dtype=np.uint8))
    mid = (pos[:-1] + pos[1:]) / 2
    got = e5m2_encode(mid)
    # ties go to the even code (the code with an even mantissa field)
    want = np.where(np.arange(0x7B) % 2 == 0, np.arange(0x7B), np.arange(1, 0x7C)).astype(np.uint8)
    assert np.array_equal(got, want)
    assert e5m2_encode(np.array([57345.0, 61440.0, 1e9, -1e9])).tolist() == [0x7B, 0x7B, 0x7B, 0xFB]
    assert e5m2_encode(np.array([2.0 ** -17]))[0] == 0x00          # tie below min subnormal -> 0
    assert e5m2_encode(np.array([2.0 ** -17 * 1.0001]))[0] == 0x01


def test_e5m2_matches_torch_in_range():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-12, 10, 200000))).astype(np.float32)
    x = np.clip(x, -E5M2_MAX, E5M2_MAX)
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(e5m2_encode(x.astype(np.float64)), ref)
