"""Number formats used by the oracle: bf16 and OCP FP8 e4m3fn.

e4m3fn, from its bit definition (OCP 8-bit floating point, the "FN" variant:
finite-only, no infinities):
  * bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
  * exponent field 0 encodes subnormals m * 2**-9 (m = 0..7);
  * exponent field e in 1..15 encodes 2**(e-7) * (1 + m/8);
  * the all-ones pattern S.1111.111 (0x7F / 0xFF) is NaN, so the largest
    finite magnitude is 2**8 * 1.75 = 448 (code 0x7E).

The 8-bit KV cache these functions model is the one the vLLM Triton FAv2 PR
page ("[Kernel][Triton][FP8] Adding fp8 and variable length sequence support to
Triton FAv2 kernel", feature list) and the TransformerEngine PR page's support
table describe; the pages do not fix the variant, so the OCP e4m3fn reading
with a per-tensor scale is used.

Quantisation rule (the contract on the stored bytes): the input is widened to
float32, multiplied in float32 by float32(1/scale), then rounded to the nearest
e4m3fn value with ties to the even code, saturating to +-448 (satfinite); NaN
stays NaN with its sign; -0 keeps its sign.

Pinned by tests/test_oracle_formats.py: every finite code against torch's
float8_e4m3fn widening; every bf16 bit pattern times several scales against
torch's narrowing cast wherever that cast is finite, and against the
saturation rule where it is not.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact (a bf16 is the top half of a float32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3fn_value_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9
        else:
            vals[code] = sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return vals


_TABLE = e4m3fn_value_table()
# non-negative finite magnitudes, indexed by code 0..0x7E; strictly increasing
_POS = _TABLE[:0x7F].copy()


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> float64 values (exact)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3fn_encode(x32: np.ndarray) -> np.ndarray:
    """float32 values -> e4m3fn codes: nearest value, ties to even code, satfinite.

    The magnitude is compared, in float64 (exact for float32 inputs), with the
    ordered table of the 127 non-negative finite values: the candidates are the
    two neighbours; the nearer one wins; a tie goes to the even code (whose
    mantissa LSB is 0); magnitudes at or beyond 448 (including infinity) become
    448.
    """
    return e4m3fn_encode_f64(np.asarray(x32, dtype=np.float32).astype(np.float64))


def e4m3fn_encode_f64(x64: np.ndarray) -> np.ndarray:
    """float64 values -> e4m3fn codes by the same rule, deciding on the float64
    value itself (no float32 rounding first)."""
    x = np.asarray(x64, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a_safe = np.where(nan, 0.0, a)
    # index of the first table value >= a  (0..127)
    hi = np.searchsorted(_POS, a_safe, side="left")
    hi_c = np.minimum(hi, 0x7E)
    lo_c = np.maximum(hi - 1, 0)
    d_hi = _POS[hi_c] - a_safe
    d_lo = a_safe - _POS[lo_c]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    code = np.where(pick_hi, hi_c, lo_c)
    code = np.where(a_safe >= _POS[0x7E], 0x7E, code)   # saturate finite / infinite overflow
    code = np.where(hi == 0, 0, code)                    # exact zero
    code = code.astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    code = np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
    return code
