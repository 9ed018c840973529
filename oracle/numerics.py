"""Number formats, decoded exactly into float64.  Test infrastructure only.

bf16: the upper 16 bits of an IEEE-754 binary32.

OCP FP8 e4m3fn (the format the EpiLoRA page's FP8 base uses, cited there to
the FP8-formats paper): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
no infinities; exponent field 15 with mantissa 7 is NaN; the largest finite
magnitude is 1.75 * 2^8 = 448; exponent field 0 encodes subnormals
m * 2^-9.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9            # subnormal: (m / 8) * 2^(1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> exact float64 values (NaN for the two NaN codes)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# finite non-negative codes sorted by value; used by the encoder below
_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.int64)   # 0x00 .. 0x7E, increasing values
_POS_VALS = _E4M3_TABLE[_POS_CODES]


def encode_e4m3(values: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3fn value, ties to the even code, saturating to +-448.

    Written as a search over the 127 finite non-negative magnitudes (obviously
    correct rather than fast).  Zero (and values that round to it) encode to
    +0 / -0 by sign; NaN input is not expected and maps to 0x7F.
    """
    v = np.asarray(values, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint8)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    # index of the largest representable magnitude <= mag
    lo = np.searchsorted(_POS_VALS, mag, side="right") - 1
    lo = np.clip(lo, 0, len(_POS_VALS) - 1)
    hi = np.minimum(lo + 1, len(_POS_VALS) - 1)
    dlo = mag - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    neg = np.signbit(v)
    out[...] = np.where(neg, code | 0x80, code)
    out[np.isnan(v)] = 0x7F
    return out
