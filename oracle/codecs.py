"""Number formats used by the method, decoded from their closed forms.

TEST INFRASTRUCTURE ONLY (see the package docstring): a CPU reference that
the GPU library never imports.

Formats:

* E2M1 ("NVIDIA FP4 E2M1", [FP4 doc] §2 Weight Format): 1 sign bit, 2
  exponent bits with bias 1, 1 mantissa bit, no infinities or NaN.  The
  largest magnitude is 6 and the smallest non-zero 0.5; magnitudes carry at
  most 2 significand bits ([FP4 doc] §4, tensor-core sub-path, exactness
  argument).  Code 0x8 is negative zero ([Blog], "Bitwise equivalence was
  checked at three levels").
* E4M3 "fn" (the scale bytes of [FP4 doc] §2 and the weight type
  float8e4m3fn of [FP8 doc] §1): 1 sign, 4 exponent bits with bias 7, 3
  mantissa bits, no infinities, NaN only at S.1111.111 (0x7F / 0xFF).  The
  largest finite value is 448 and the smallest subnormal 2^-9 ([FP4 doc] §4
  quotes both in its range argument).
* FP16 / BF16: the activation / output types T of [FP8 doc] §1.  Stored
  here as raw uint16 bit patterns because numpy has no bfloat16.

Decoding is a pure function of the code; the tables are those functions
evaluated on every code.

Encoding (FP32 -> E4M3 "fn", for the optional W8A8 activation path of
[FP8 doc] §6): the nearest finite E4M3 value, ties to the code with an even
mantissa, magnitudes beyond 448 saturated to 448, NaN to NaN.  The pages
write fp8_e4m3(.) without naming a rounding or overflow rule; round to
nearest even with saturation to the largest finite value is the reading
taken (an "fn" format has no infinity to overflow to).
"""

import math

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code (closed form, see module docstring)."""
    sign = (code >> 3) & 1
    exponent = (code >> 1) & 3
    mantissa = code & 1
    if exponent == 0:
        # subnormal: 2^(1 - bias) * (mantissa / 2) with bias 1
        magnitude = 0.5 * mantissa
    else:
        magnitude = math.ldexp(1.0 + 0.5 * mantissa, exponent - 1)
    return -magnitude if sign else magnitude


def e4m3fn_value(byte: int) -> float:
    """Value of an 8-bit E4M3 "fn" code (closed form, see module docstring)."""
    sign = (byte >> 7) & 1
    exponent = (byte >> 3) & 0xF
    mantissa = byte & 7
    if exponent == 0xF and mantissa == 7:
        return math.nan
    if exponent == 0:
        # subnormal: 2^(1 - bias) * (mantissa / 8) with bias 7
        magnitude = math.ldexp(mantissa / 8.0, -6)
    else:
        magnitude = math.ldexp(1.0 + mantissa / 8.0, exponent - 7)
    return -magnitude if sign else magnitude


# Every code evaluated once; indexing these is the decode step.
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3FN_TABLE = np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float64)


# Finite positive E4M3 magnitudes in code order 0x00 .. 0x7E (increasing).
_E4M3_POS = E4M3FN_TABLE[:0x7F]
E4M3_MAX = 448.0


def e4m3fn_encode(x) -> np.ndarray:
    """float values -> E4M3 "fn" codes (uint8): nearest representable value,
    ties to even code, |x| > 448 saturated to 448, NaN -> 0x7F, sign kept
    (-0.0 -> 0x80).  A plain search over the 127 finite magnitudes."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    nan = np.isnan(x)
    m = np.where(nan, 0.0, np.minimum(mag, E4M3_MAX))
    hi = np.searchsorted(_E4M3_POS, m, side="left")      # first magnitude >= m
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = m - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - m
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    sign = np.signbit(x).astype(np.int64) << 7
    out = (code | sign).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), out).astype(np.uint8)


def f32_to_f16_bits(x) -> np.ndarray:
    """float32 -> IEEE binary16 bits, round to nearest even, subnormals kept,
    overflow to +-inf (numpy's conversion)."""
    x32 = np.asarray(x, dtype=np.float32)
    return x32.astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bits: keep the top 16 bits after adding half an
    ulp with ties to even.  NaN maps to the quiet NaN 0x7FC0 with its sign."""
    x32 = np.asarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    quiet_nan = ((u >> 16) & 0x8000) | 0x7FC0
    out = np.where(np.isnan(x32), quiet_nan, rounded)
    return out.astype(np.uint16)


def bits_to_f64(bits, dtype: str) -> np.ndarray:
    """FP16 or BF16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return b.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def activation_to_f64(bits, dtype: str) -> np.ndarray:
    """Activation / bias tensor of type T (given as bits) -> float64."""
    return bits_to_f64(bits, dtype)
