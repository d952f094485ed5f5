"""NVFP4 activation quantization and the W4A4 matmul of the FP4 operator's
native path ([FP4 doc] §6 Native SM120 FP4 x FP4 Path).

TEST INFRASTRUCTURE ONLY (see the package docstring): a CPU reference that
the GPU library never imports.

The pages' native path quantizes the activation A to packed E2M1 codes with
one E4M3 scale per 16-element block (the weight format of [FP4 doc] §2 Weight
Format, without a tensor scale), multiplies the two FP4 operands with FP32
accumulation, adds the bias, and is checked against an activation-quantized
FP4 reference.  The pages name the format but no rule for choosing the block
scale or for rounding.  Readings taken (each also listed in the design notes
of the repository):

* Blocks are 16 consecutive k of one row of A (K % 16 == 0).
* amax = max |a| over the block, a in T (FP16 / BF16, exact).  A NaN in the
  block makes the block's scale NaN.
* Scale code = e4m3(RNE_f32(amax / 6)): 6 is the largest E2M1 magnitude, so
  the block's largest element lands at the top of the E2M1 range.  The
  quotient is an IEEE FP32 division; e4m3() is the E4M3 "fn" encoder of
  codecs.e4m3fn_encode (nearest, ties to even, saturation at 448, NaN kept).
* Element code = e2m1(RNE_f32(a / s)) with s the decoded scale: IEEE FP32
  division; e2m1() is the nearest E2M1 value, ties to the code with an even
  mantissa bit, magnitudes beyond 6 saturated to 6, the sign kept (a
  negative quotient that rounds to zero gives code 0x8).  A zero scale gives
  code 0 for the whole block, and so does a NaN quotient.
* Dequantized activation = e2m1 x e4m3, exact in FP16 and in BF16 (at most
  2 + 4 significand bits; nonzero magnitudes within [2^-10, 2688]); NaN
  where the scale is NaN.
* W4A4 result = the weight-only FP4 result (reference.matmul_fp4_reference)
  with A replaced by its dequantized activation, under the same acceptance
  bound.

[FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
"""

import numpy as np

from . import codecs
from . import reference

BLOCK = 16           # activation elements per E4M3 scale
E2M1_MAX = 6.0       # largest E2M1 magnitude

# Non-negative E2M1 magnitudes in code order 0 .. 7 (increasing).
_E2M1_POS = codecs.E2M1_TABLE[:8]


def e2m1_encode(x) -> np.ndarray:
    """float values -> 4-bit E2M1 codes (uint8): nearest representable value,
    ties to the code with an even mantissa bit (even code), |x| > 6 saturated
    to 6, sign kept (-0.0 and negative values rounding to zero -> 0x8), NaN
    -> 0.  A plain search over the 8 magnitudes."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    m = np.where(nan, 0.0, np.minimum(np.abs(x), E2M1_MAX))
    hi = np.minimum(np.searchsorted(_E2M1_POS, m, side="left"), 7)  # first magnitude >= m
    lo = np.maximum(hi - 1, 0)
    d_lo = m - _E2M1_POS[lo]
    d_hi = _E2M1_POS[hi] - m
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    sign = np.signbit(x).astype(np.int64) << 3
    out = (code | sign).astype(np.uint8)
    return np.where(nan, np.uint8(0), out).astype(np.uint8)


def quantize_activation_nvfp4(A_bits, dtype: str):
    """A (T bits [M, K], K % 16 == 0) -> (codes uint8 [M, K/2] packed two per
    byte, low nibble = even k; scales uint8 [M, K/16] E4M3 bytes)."""
    A_bits = np.asarray(A_bits, dtype=np.uint16)
    M, K = A_bits.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    a64 = codecs.activation_to_f64(A_bits, dtype).reshape(M, K // BLOCK, BLOCK)
    a32 = a64.astype(np.float32)                      # exact: a is a T value
    has_nan = np.isnan(a32).any(axis=2)
    amax = np.where(has_nan, np.float32(np.nan), np.abs(a32).max(axis=2, initial=np.float32(0)))
    scale_codes = codecs.e4m3fn_encode(amax.astype(np.float32) / np.float32(E2M1_MAX))
    s32 = codecs.E4M3FN_TABLE[scale_codes].astype(np.float32)     # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        q = a32 / s32[:, :, None]                                  # IEEE FP32 division
    codes = e2m1_encode(q)
    codes = np.where((s32 == 0)[:, :, None], np.uint8(0), codes).reshape(M, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale_codes.astype(np.uint8)


def dequant_activation_nvfp4_f64(codes_packed, scales) -> np.ndarray:
    """(codes [M, K/2], scales [M, K/16]) -> e2m1 x e4m3 as float64 [M, K]."""
    codes = reference.unpack_e2m1_codes(np.asarray(codes_packed, dtype=np.uint8), 2 * codes_packed.shape[1])
    s = np.repeat(codecs.E4M3FN_TABLE[np.asarray(scales, dtype=np.uint8)], BLOCK, axis=1)
    return codecs.E2M1_TABLE[codes] * s


def _to_t_bits(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)  # exact for these values
    return codecs.f32_to_bf16_bits(x32) if dtype == "bf16" else codecs.f32_to_f16_bits(x32)


def dequant_activation_nvfp4_bits(codes_packed, scales, dtype: str) -> np.ndarray:
    """The dequantized activation as T bits (exact)."""
    return _to_t_bits(dequant_activation_nvfp4_f64(codes_packed, scales), dtype)


def qdq_activation_nvfp4_bits(A_bits, dtype: str) -> np.ndarray:
    """A -> its NVFP4 quantization, dequantized back to T bits [M, K]."""
    codes, scales = quantize_activation_nvfp4(A_bits, dtype)
    return dequant_activation_nvfp4_bits(codes, scales, dtype)


def matmul_w4a4_reference(A_bits, dtype: str, B_packed, weight_scale, block_size: int, weight_scale_2,
                          bias_bits=None, n_chunk: int = 2048):
    """(Y_ref, S) of the W4A4 path: the weight-only FP4 reference on the
    dequantized NVFP4 activation."""
    A_q = qdq_activation_nvfp4_bits(A_bits, dtype)
    return reference.matmul_fp4_reference(A_q, dtype, B_packed, weight_scale, block_size, weight_scale_2,
                                          bias_bits, n_chunk)
