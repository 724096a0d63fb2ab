"""Number formats used by the oracle, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 stored fraction bits; the
upper half of an IEEE binary32.  Rounding is round-to-nearest-even (RNE),
overflow goes to infinity.

e4m3 (OCP 8-bit floating point, "E4M3FN"): 1 sign bit, 4 exponent bits
(bias 7), 3 fraction bits, subnormals m·2^-9, largest finite 448 = 1.75·2^8,
no infinities, NaN = S.1111.111.  The pages use E4M3 for forward
activation×weight GEMMs ("Megatron-LM deep architecture", FP8 hybrid
precision section).  Rounding is RNE; values beyond ±448 saturate to ±448.

e5m2 (OCP 8-bit floating point, "E5M2"): 1 sign bit, 5 exponent bits
(bias 15), 2 fraction bits, subnormals m·2^-16, largest finite 57344 =
1.75·2^15, infinities S.11111.00 and NaNs S.11111.xx.  The pages use E5M2
for the gradients of the backward pass ("Megatron-LM deep architecture", FP8
hybrid precision section).  Rounding is RNE; values beyond ±57344 saturate to
±57344 (the GPU path clamps before converting).

The encoders round a float64 value once, directly to the target grid.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
_BF16_OVERFLOW = 2.0 ** 128


def _round_to_grid(x: np.ndarray, frac_bits: int, emin: int) -> np.ndarray:
    """Round float64 `x` to the nearest value with `frac_bits` fraction bits.

    The grid spacing in the binade [2^e, 2^(e+1)) is 2^(e - frac_bits), and
    below the smallest normal binade (e < emin) it stays 2^(emin - frac_bits)
    (subnormals).  Ties go to the even neighbour (numpy.rint).  No overflow
    handling: the caller applies its format's range.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(np.abs(x))          # |x| = m·2^e, m in [0.5, 1)
    e = np.maximum(e - 1, emin)         # leading-bit exponent, clamped to emin
    q = e - frac_bits                   # exponent of the grid spacing
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def bf16_encode(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (uint16), RNE, overflow to ±inf."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_grid(x, 7, -126)
    r = np.where(np.abs(r) >= _BF16_OVERFLOW, np.copysign(np.inf, x), r)
    r = np.where(np.isnan(x), np.nan, r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    codes = np.arange(256)
    sign = np.where(codes >= 128, -1.0, 1.0)
    E = (codes >> 3) & 0xF
    m = codes & 7
    mag = np.where(E == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, E - 7))
    val = sign * mag
    val[(E == 15) & (m == 7)] = np.nan
    return val


_E4M3_VALUES = _e4m3_table()
# non-negative finite codes 0x00..0x7E in increasing order of value
_E4M3_POS = _E4M3_VALUES[:0x7F].copy()


def e4m3_decode(codes) -> np.ndarray:
    """e4m3 codes (uint8) -> float64 (exact); NaN for 0x7F / 0xFF."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """float64 -> e4m3 codes (uint8), RNE, saturating to ±448; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_grid(x, 3, -6)
    mag = np.minimum(np.abs(r), E4M3_MAX)
    idx = np.searchsorted(_E4M3_POS, mag)
    if not np.all(_E4M3_POS[np.minimum(idx, 0x7E)][~np.isnan(mag)] == mag[~np.isnan(mag)]):
        raise AssertionError("e4m3 rounding produced an off-grid value")
    code = idx.astype(np.uint8) | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def _e5m2_table() -> np.ndarray:
    codes = np.arange(256)
    sign = np.where(codes >= 128, -1.0, 1.0)
    E = (codes >> 2) & 0x1F
    m = codes & 3
    mag = np.where(E == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.ldexp(1.0, E - 15))
    val = sign * mag
    val[(E == 31) & (m == 0)] = sign[(E == 31) & (m == 0)] * np.inf
    val[(E == 31) & (m != 0)] = np.nan
    return val


_E5M2_VALUES = _e5m2_table()
# non-negative finite codes 0x00..0x7B in increasing order of value
_E5M2_POS = _E5M2_VALUES[:0x7C].copy()


def e5m2_decode(codes) -> np.ndarray:
    """e5m2 codes (uint8) -> float64 (exact); ±inf for 0x7C / 0xFC, NaN for the rest of E = 31."""
    return _E5M2_VALUES[np.asarray(codes, dtype=np.uint8)]


def e5m2_encode(x) -> np.ndarray:
    """float64 -> e5m2 codes (uint8), RNE, saturating to ±57344; NaN -> 0x7E."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_grid(x, 2, -14)
    mag = np.minimum(np.abs(r), E5M2_MAX)
    idx = np.searchsorted(_E5M2_POS, mag)
    if not np.all(_E5M2_POS[np.minimum(idx, 0x7B)][~np.isnan(mag)] == mag[~np.isnan(mag)]):
        raise AssertionError("e5m2 rounding produced an off-grid value")
    code = idx.astype(np.uint8) | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(x), np.uint8(0x7E), code).astype(np.uint8)
