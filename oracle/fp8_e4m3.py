"""OCP E4M3FN 8-bit float codec, fp64 and exact (oracle; test infrastructure only).

The PD-engineering page (ybb.press), section 6.2, stores the KV cache as FP8
E4M3 to halve its bytes (the page's "4-bit" is a typo: E4M3 is an 8-bit format
with 4 exponent and 3 mantissa bits).  The bit format used here is the OCP
8-bit floating point specification's E4M3 ("fn": finite, no infinities):

* sign bit s, 4 exponent bits e (bias 7), 3 mantissa bits m;
* e in 1..15: value = (-1)^s * 2^(e-7) * (1 + m/8);
* e == 0: subnormal, value = (-1)^s * m * 2^-9;
* e == 15 and m == 7 (codes 0x7F, 0xFF) is NaN; there is no infinity;
* the largest finite magnitude is 0x7E = 2^8 * 1.75 = 448.

Encoding (the reading this library takes of "quantise the KV cache"):
round to nearest, ties to even mantissa, and saturate finite overflow
(anything of magnitude above 448, including infinities) to +-448.  NaN
encodes as 0x7F with the input's sign bit.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def decode_code(code: int) -> float:
    """Exact value of one E4M3FN code, straight from the field definitions."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)


# All 256 code values, built once by the scalar definition above.
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes 0x00..0x7E in code order; their values increase
# strictly with the code, so code parity equals mantissa parity.
_POS_VALUES = DECODE_TABLE[:0x7F].copy()


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> exact fp64 values (NaN for 0x7F / 0xFF)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x: np.ndarray) -> np.ndarray:
    """fp64-representable values -> E4M3FN codes, RNE, saturating to +-448.

    The magnitude is located between two neighbouring representable values;
    the nearer one wins, and an exact tie goes to the even code.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    nan = np.isnan(x)
    sat = ~nan & (a >= E4M3_MAX)
    reg = ~nan & ~sat
    ar = a[reg]
    # hi = first index whose value is >= a  (0 .. 0x7E)
    hi = np.searchsorted(_POS_VALUES, ar, side="left")
    lo = np.maximum(hi - 1, 0)
    v_hi = _POS_VALUES[hi]
    v_lo = _POS_VALUES[lo]
    d_hi = v_hi - ar
    d_lo = ar - v_lo
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    exact = v_hi == ar
    code = np.where(exact | pick_hi, hi, lo).astype(np.uint8)
    out[reg] = code
    out[sat] = 0x7E
    out[nan] = NAN_CODE
    return out | sign


def quantize(x_f32: np.ndarray, scale_f32: float | np.ndarray) -> np.ndarray:
    """Cache encoding of a KV value: e4m3fn_rne_satfinite(float32(x) / float32(scale)).

    The division is an IEEE fp32 division (correctly rounded), as the kernel's.
    """
    q = np.asarray(x_f32, dtype=np.float32) / np.asarray(scale_f32, dtype=np.float32)
    return encode(q.astype(np.float64))
