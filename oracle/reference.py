"""Reference semantics of the weight-only FP4 / FP8 matmul and the FP4 dequant.

TEST INFRASTRUCTURE ONLY (see the package docstring): a CPU reference that
the GPU library never imports.

Every function follows the pages' definitions step by step:

* FP4 ([FP4 doc] §2 Weight Format):
      B_dq[n, k] = e2m1(B[n, k]) * e4m3(weight_scale[n, k / block_size])
                   * weight_scale_2
  B is stored as uint8 [N, K/2]; the low nibble of byte j holds k = 2j and the
  high nibble k = 2j + 1.
* FP8 ([FP8 doc] §2 Tensor and Scale Format):
      B_dq[n, k] = fp8_e4m3(B[n, k]) * b_scale[n, k / block_size]
  and a partial final K block uses the last scale column.
* Both ([FP4 doc] header; [FP8 doc] §2):
      Y[m, n] = sum_k A[m, k] * B_dq[n, k] + bias[n]

Readings where the pages leave a step open (each also listed in the design
notes of the repository):

* The scale column of element k is min(k // block_size, scale_cols - 1).  This
  is the pages' k / block_size for every k of a full block, and it sends the
  K % block_size tail to the last column, whichever of ceil(K/bs) or
  floor(K/bs) columns the caller supplies.  The same rule serves FP4.
* The stored dequant output is RNE_T(RNE_f32(e2m1 * e4m3 * ws2)): the product
  e2m1 * e4m3 is exact, multiplying by the FP32 ws2 rounds once to FP32, and
  the FP32 value is rounded once more to FP16/BF16 (the pages' formula read
  left to right, in the activation type the output takes).
* The matmul result is not unique (accumulation order differs between
  kernels).  The acceptance bound
      tol = 2e-3 * sum_k |A[m,k] * B_dq[n,k]| + 1e-3 * |Y_ref|
  (Y_ref and B_dq exact, float64) bounds the FP32 result before its final
  rounding to T: Y is accepted when it is the FP16/BF16 rounding of some
  value within tol of Y_ref, i.e. RNE_T(Y_ref - tol) <= Y <= RNE_T(Y_ref +
  tol).  The bound is stated for FP32 accumulation followed by FP16/BF16
  output rounding; BF16 alone rounds by up to 2^-8 |Y|, more than
  tol when few terms of one sign (or the bias) dominate, so the rounding is
  taken outside the bound rather than inside it.
"""

import numpy as np

from .codecs import (
    E2M1_TABLE,
    E4M3FN_TABLE,
    e4m3fn_encode,
    activation_to_f64,
    bits_to_f64,
    f32_to_bf16_bits,
    f32_to_f16_bits,
)


def unpack_e2m1_codes(B_packed: np.ndarray, K: int) -> np.ndarray:
    """uint8 [N, K/2] -> E2M1 codes uint8 [N, K]; low nibble = even k
    ([FP4 doc] §2 Weight Format)."""
    B_packed = np.asarray(B_packed, dtype=np.uint8)
    N = B_packed.shape[0]
    if K % 2 != 0 or B_packed.shape[1] != K // 2:
        raise ValueError("B must be [N, K/2] with K even")
    codes = np.empty((N, K), dtype=np.uint8)
    codes[:, 0::2] = B_packed & 0x0F
    codes[:, 1::2] = B_packed >> 4
    return codes


def scale_column(K: int, block_size: int, scale_cols: int) -> np.ndarray:
    """Scale column used by each k in [0, K): k // block_size, with the
    partial final block sent to the last column ([FP8 doc] §2)."""
    if block_size < 1 or scale_cols < 1:
        raise ValueError("block_size and scale_cols must be >= 1")
    k = np.arange(K, dtype=np.int64)
    return np.minimum(k // block_size, scale_cols - 1)


def dequant_fp4_f64(B_packed, weight_scale, block_size: int, weight_scale_2, K: int) -> np.ndarray:
    """Exact B_dq of the FP4 op as float64 [N, K] ([FP4 doc] §2).

    e2m1 (2 significand bits) * e4m3 (4 bits) * fp32 ws2 (24 bits) needs at
    most 30 bits, so the float64 product is exact."""
    weight_scale = np.asarray(weight_scale, dtype=np.uint8)
    codes = unpack_e2m1_codes(B_packed, K)
    cols = scale_column(K, block_size, weight_scale.shape[1])
    q = E2M1_TABLE[codes]
    s = E4M3FN_TABLE[weight_scale[:, cols]]
    ws2 = np.float64(np.float32(weight_scale_2))
    return q * s * ws2


def dequant_fp4_output_bits(B_packed, weight_scale, block_size: int, weight_scale_2, K: int,
                            dtype: str) -> np.ndarray:
    """The stored [N, K] FP16/BF16 dequant output, as uint16 bits:
    RNE_T(RNE_f32(e2m1 * e4m3 * ws2))."""
    exact = dequant_fp4_f64(B_packed, weight_scale, block_size, weight_scale_2, K)
    as_f32 = exact.astype(np.float32)  # the one FP32 rounding
    if dtype == "fp16":
        return f32_to_f16_bits(as_f32)
    if dtype == "bf16":
        return f32_to_bf16_bits(as_f32)
    raise ValueError(f"unknown dtype {dtype!r}")


def dequant_fp8_f64(B_fp8, b_scale, block_size: int) -> np.ndarray:
    """Exact B_dq of the FP8 op as float64 [N, K] ([FP8 doc] §2).
    e4m3 (4 bits) * fp32 (24 bits) is exact in float64."""
    B_fp8 = np.asarray(B_fp8, dtype=np.uint8)
    b_scale = np.asarray(b_scale, dtype=np.float32)
    K = B_fp8.shape[1]
    cols = scale_column(K, block_size, b_scale.shape[1])
    return E4M3FN_TABLE[B_fp8] * b_scale[:, cols].astype(np.float64)


def dequant_fp8_output_bits(B_fp8, b_scale, block_size: int, dtype: str) -> np.ndarray:
    """RNE_T(RNE_f32(e4m3 * b_scale)) as uint16 bits: what a one-hot
    activation must produce through the FP8 matmul (single exact term)."""
    as_f32 = dequant_fp8_f64(B_fp8, b_scale, block_size).astype(np.float32)
    if dtype == "fp16":
        return f32_to_f16_bits(as_f32)
    if dtype == "bf16":
        return f32_to_bf16_bits(as_f32)
    raise ValueError(f"unknown dtype {dtype!r}")


def qdq_activation_fp8_bits(A_bits, dtype: str, a_scale) -> np.ndarray:
    """The optional W8A8 activation of [FP8 doc] §6,
        A_deq = fp8_e4m3(A / a_scale) * a_scale,
    as uint16 bits of T, step by step: A (T) -> FP32; divide by the FP32
    a_scale (one FP32 rounding); encode to E4M3 (e4m3fn_encode); decode and
    multiply by a_scale (exact in float64, then one FP32 rounding); round the
    FP32 value to T."""
    a32 = activation_to_f64(A_bits, dtype).astype(np.float32)
    s32 = np.float32(a_scale)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (a32 / s32).astype(np.float32)
    codes = e4m3fn_encode(q)
    deq = (E4M3FN_TABLE[codes] * np.float64(s32)).astype(np.float32)
    if dtype == "fp16":
        return f32_to_f16_bits(deq)
    if dtype == "bf16":
        return f32_to_bf16_bits(deq)
    raise ValueError(f"unknown dtype {dtype!r}")


def _matmul_from_dq(A64: np.ndarray, dq_rows, N: int, bias64, n_chunk: int):
    """Y_ref = A @ B_dq^T + bias and S = |A| @ |B_dq|^T, in float64,
    materialising B_dq a chunk of output columns at a time."""
    M = A64.shape[0]
    Y = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    absA = np.abs(A64)
    for n0 in range(0, N, n_chunk):
        n1 = min(N, n0 + n_chunk)
        dq = dq_rows(n0, n1)
        Y[:, n0:n1] = A64 @ dq.T
        S[:, n0:n1] = absA @ np.abs(dq).T
    if bias64 is not None:
        Y += bias64[None, :]
    return Y, S


def matmul_fp4_reference(A_bits, dtype: str, B_packed, weight_scale, block_size: int,
                         weight_scale_2, bias_bits=None, n_chunk: int = 2048):
    """FP4 weight-only matmul in float64.

    A_bits: uint16 [M, K] (FP16 or BF16 bits), B_packed: uint8 [N, K/2],
    weight_scale: uint8 [N, cols] (E4M3 bytes), weight_scale_2: FP32 scalar,
    bias_bits: uint16 [N] or None.
    Returns (Y_ref, S): Y_ref[m, n] = sum_k A*B_dq + bias and
    S[m, n] = sum_k |A*B_dq| (the scale of the tolerance)."""
    A64 = activation_to_f64(A_bits, dtype)
    B_packed = np.asarray(B_packed, dtype=np.uint8)
    weight_scale = np.asarray(weight_scale, dtype=np.uint8)
    K = A64.shape[1]
    N = B_packed.shape[0]
    bias64 = None if bias_bits is None else bits_to_f64(bias_bits, dtype)

    def dq_rows(n0, n1):
        return dequant_fp4_f64(B_packed[n0:n1], weight_scale[n0:n1], block_size, weight_scale_2, K)

    return _matmul_from_dq(A64, dq_rows, N, bias64, n_chunk)


def matmul_fp8_reference(A_bits, dtype: str, B_fp8, b_scale, block_size: int, bias_bits=None,
                         n_chunk: int = 2048):
    """FP8 weight-only matmul in float64 (same outputs as matmul_fp4_reference)."""
    A64 = activation_to_f64(A_bits, dtype)
    B_fp8 = np.asarray(B_fp8, dtype=np.uint8)
    b_scale = np.asarray(b_scale, dtype=np.float32)
    N = B_fp8.shape[0]
    bias64 = None if bias_bits is None else bits_to_f64(bias_bits, dtype)

    def dq_rows(n0, n1):
        return dequant_fp8_f64(B_fp8[n0:n1], b_scale[n0:n1], block_size)

    return _matmul_from_dq(A64, dq_rows, N, bias64, n_chunk)


def matmul_tolerance(Y_ref: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Bound on the FP32 result: 2e-3 * sum_k|A*B_dq| + 1e-3 * |Y_ref|."""
    return 2e-3 * S + 1e-3 * np.abs(Y_ref)


def _round_to_t(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> float32 -> T (both round to nearest even), back as float64.
    A composition of monotone roundings, so it preserves order."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "fp16":
        bits = f32_to_f16_bits(x32)
    elif dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
    else:
        raise ValueError(dtype)
    return bits_to_f64(bits, dtype)


def check_matmul(Y_bits, dtype: str, Y_ref: np.ndarray, S: np.ndarray) -> dict:
    """Compare a device result (uint16 bits of type T) with the reference.

    Passes when every element Y lies in [RNE_T(Y_ref - tol), RNE_T(Y_ref +
    tol)] (see the module docstring); an element whose reference is NaN must
    be NaN, and one whose reference is a number must not be NaN.  Y must be
    finite unless the rounded band itself reaches +-inf: an FP16 result
    beyond the format's range rounds to +-inf (round to nearest even has no
    saturation), so there +-inf is the correctly rounded value."""
    Y = bits_to_f64(Y_bits, dtype)
    tol = matmul_tolerance(Y_ref, S)
    ref_nan = np.isnan(Y_ref)
    with np.errstate(over="ignore", invalid="ignore"):
        lo = _round_to_t(np.where(ref_nan, 0.0, Y_ref - tol), dtype)
        hi = _round_to_t(np.where(ref_nan, 0.0, Y_ref + tol), dtype)
    err = np.abs(Y - Y_ref)
    finite_ok = np.where(ref_nan, np.isnan(Y), ~np.isnan(Y))
    within = np.where(ref_nan, True, (Y >= lo) & (Y <= hi))
    bad = ~(finite_ok & within)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(ref_nan | (tol == 0), np.where(err == 0, 0.0, np.inf), err / tol)
    ratio = np.where(ref_nan, 0.0, ratio)
    worst = None
    if bad.any():
        i = tuple(int(v) for v in np.argwhere(bad)[0])
        worst = {"index": i, "Y": float(Y[i]), "Y_ref": float(Y_ref[i]), "S": float(S[i]),
                 "tol": float(tol[i]), "lo": float(lo[i]), "hi": float(hi[i])}
    return {
        "ok": bool(not bad.any()),
        "n_bad": int(bad.sum()),
        "max_ratio": float(np.nanmax(ratio)) if ratio.size else 0.0,
        "max_abs_err": float(np.nanmax(np.where(ref_nan, 0.0, err))) if err.size else 0.0,
        "first_bad": worst,
    }
