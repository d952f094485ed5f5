"""Pins of the NVFP4 activation quantizer and the W4A4 reference
(oracle/nvfp4.py) against things other than themselves: hand-derived blocks,
a brute-force nearest-value search, exact round trips, error bounds, block
independence and an exact rational matmul.

[FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation",
§6 Native SM120 FP4 x FP4 Path (packed E2M1 activation, one E4M3 scale per
16 elements, FP4 x FP4 product checked against an activation-quantized
reference).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import codecs, nvfp4, reference as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_activation_blocks.txt")
E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # magnitudes of codes 0 .. 7 ([FP4 doc] §2)


def _golden():
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            head, a, scale, codes, dq = [p.split() for p in line.split("|")]
            yield (head[0], head[1], np.array([int(x, 16) for x in a], dtype=np.uint16), int(scale[0], 16),
                   [int(c, 16) for c in codes], [float(v) for v in dq])


@pytest.mark.parametrize("case", list(_golden()), ids=lambda c: c[0])
def test_golden_blocks(case):
    name, dtype, a, scale, codes, dq = case
    packed, scales = nvfp4.quantize_activation_nvfp4(a.reshape(1, 16), dtype)
    got_codes = ref.unpack_e2m1_codes(packed, 16)[0].tolist()
    assert scales[0, 0] == scale, name
    assert got_codes == codes, name
    vals = nvfp4.dequant_activation_nvfp4_f64(packed, scales)[0]
    for g, w in zip(vals, dq):
        if math.isnan(w):
            assert math.isnan(g), name
        else:
            assert g == w and math.copysign(1.0, g) == math.copysign(1.0, w), name
    bits = nvfp4.qdq_activation_nvfp4_bits(a.reshape(1, 16), dtype)[0]
    back = codecs.bits_to_f64(bits, dtype)
    assert np.array_equal(np.isnan(back), np.isnan(vals))
    assert np.array_equal(back[~np.isnan(back)], vals[~np.isnan(vals)])


def _brute_e2m1(x: float) -> int:
    """Nearest E2M1 code by trying all 16 codes: smallest distance, then the
    even code (even mantissa bit), then the zero whose sign matches x;
    beyond +-6 the nearest value is +-6 anyway."""
    best = None
    for code in range(16):
        v = codecs.e2m1_value(code)
        key = (abs(v - x), code & 1, 0 if (code >> 3) == (1 if math.copysign(1.0, x) < 0 else 0) else 1)
        if best is None or key < best[0]:
            best = (key, code)
    return best[1]


def test_e2m1_encode_matches_brute_force_on_a_dense_grid():
    xs = np.concatenate([np.arange(-8.0, 8.0 + 1e-9, 1.0 / 64.0), [-0.0, 0.0, 1e-30, -1e-30, 7.0, -100.0]])
    got = nvfp4.e2m1_encode(xs)
    want = np.array([_brute_e2m1(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e2m1_encode_ties_go_to_the_even_code():
    # every midpoint between neighbouring magnitudes, both signs
    for lo, hi in zip(E2M1_VALUES[:-1], E2M1_VALUES[1:]):
        mid = (lo + hi) / 2
        c_lo, c_hi = E2M1_VALUES.index(lo), E2M1_VALUES.index(hi)
        even = c_lo if c_lo % 2 == 0 else c_hi
        assert nvfp4.e2m1_encode(mid) == even
        assert nvfp4.e2m1_encode(-mid) == even | 8
        assert nvfp4.e2m1_encode(np.nextafter(mid, 0)) == c_lo
        assert nvfp4.e2m1_encode(np.nextafter(mid, 10)) == c_hi
    assert nvfp4.e2m1_encode(np.inf) == 7 and nvfp4.e2m1_encode(-np.inf) == 15
    assert nvfp4.e2m1_encode(np.nan) == 0


def _representable(rng, M, K, dtype):
    """A whose every 16-block is exactly NVFP4: a random E4M3 scale s (kept
    within the range where 6 s / 6 and every code * s are exact in T) times
    random codes, with one element at +-6 s so that amax / 6 == s."""
    codes = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    codes[:, ::16] = rng.choice([7, 15], size=(M, K // 16))
    lo, hi = (0x18, 0x70) if dtype == "fp16" else (0x08, 0x7E)
    scales = rng.integers(lo, hi, size=(M, K // 16)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales, nvfp4.dequant_activation_nvfp4_bits(packed, scales, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_representable_activations_round_trip(dtype):
    rng = np.random.default_rng(5)
    packed, scales, A = _representable(rng, 6, 128, dtype)
    p2, s2 = nvfp4.quantize_activation_nvfp4(A, dtype)
    assert np.array_equal(s2, scales)
    # codes agree except that +-0 elements may swap zero signs only through
    # the sign of the value, which the round trip keeps
    assert np.array_equal(ref.unpack_e2m1_codes(p2, 128), ref.unpack_e2m1_codes(packed, 128))
    assert np.array_equal(nvfp4.qdq_activation_nvfp4_bits(A, dtype), A)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_quantization_error_bound(dtype):
    """|dq - a| is at most half the E2M1 spacing at the quantized magnitude
    times s (0.25 s below 2, 0.5 s below 4, 1 s up to 6) when a / s is not
    beyond 6; beyond it the element saturates to +-6 s."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((8, 256)) * rng.choice([1e-3, 0.1, 1.0, 30.0, 1e3], size=(8, 1))
    A = codecs.f32_to_bf16_bits(x.astype(np.float32)) if dtype == "bf16" else codecs.f32_to_f16_bits(x.astype(np.float32))
    a = codecs.bits_to_f64(A, dtype)
    packed, scales = nvfp4.quantize_activation_nvfp4(A, dtype)
    dq = nvfp4.dequant_activation_nvfp4_f64(packed, scales)
    s = np.repeat(codecs.E4M3FN_TABLE[scales], 16, axis=1)
    amax_el = np.repeat(np.abs(a).reshape(8, 16, 16).max(axis=2), 16, axis=1)
    # a zero scale only where amax / 6 is below half the smallest E4M3
    # subnormal, and then the block dequantizes to zero
    assert ((s == 0) == (amax_el / 6 < 2 ** -10)).all()
    assert (dq[s == 0] == 0).all()
    live = s > 0
    assert live.mean() > 0.5
    q = np.where(live, np.abs(a) / np.where(live, s, 1.0), 0.0)
    half = np.where(q < 2, 0.25, np.where(q < 4, 0.5, 1.0))
    # the FP32 quotient may sit an ulp from a / s; allow that
    inside = live & (q <= 6)
    assert (np.abs(dq - a)[inside] <= half[inside] * s[inside] * (1 + 2 ** -20)).all()
    sat = live & (q > 6)
    assert (np.abs(dq[sat]) == 6 * s[sat]).all()
    # the scale tracks the block maximum: amax / 6 rounded to E4M3 (relative
    # error at most 2^-4) unless it saturates at 448
    amax = np.abs(a).reshape(8, 16, 16).max(axis=2)
    sb = codecs.E4M3FN_TABLE[scales]
    unsat = amax / 6 <= 448
    assert (np.abs(sb - amax / 6) <= 2 ** -4 * amax / 6 + 2 ** -10)[unsat].all()
    assert (sb[~unsat] == 448).all()


def test_blocks_are_independent():
    rng = np.random.default_rng(2)
    A = codecs.f32_to_bf16_bits(rng.standard_normal((2, 64)).astype(np.float32))
    base = nvfp4.qdq_activation_nvfp4_bits(A, "bf16")
    B = A.copy()
    B[1, 20] = 0x4700  # 32768 in block 1 of row 1
    out = nvfp4.qdq_activation_nvfp4_bits(B, "bf16")
    changed = out != base
    assert changed[1, 16:32].any()
    changed[1, 16:32] = False
    assert not changed.any()


def test_nan_and_infinity_stay_in_their_block():
    A = np.full((1, 48), 0x3F80, dtype=np.uint16)  # 1.0
    A[0, 3] = 0x7FC0   # NaN in block 0
    A[0, 20] = 0x7F80  # +inf in block 1
    packed, scales = nvfp4.quantize_activation_nvfp4(A, "bf16")
    dq = nvfp4.dequant_activation_nvfp4_f64(packed, scales)
    assert np.isnan(dq[0, :16]).all()
    assert scales[0, 1] == 0x7E and dq[0, 20] == 6 * 448.0  # saturated
    assert (dq[0, 16:32][np.arange(16) != 4] == 0).all()    # 1/448 rounds to 0
    assert scales[0, 2] == codecs.e4m3fn_encode(np.float32(1.0) / np.float32(6.0))
    assert not np.isnan(dq[0, 32:]).any()


def _exact_w4a4(A_bits, dtype, B, ws, ws2, bias):
    """Y and S as exact fractions from the decoded NVFP4 activation and the
    weight definition, by plain loops."""
    packed, scales = nvfp4.quantize_activation_nvfp4(A_bits, dtype)
    M, K = A_bits.shape
    N = B.shape[0]
    acodes = ref.unpack_e2m1_codes(packed, K)
    bcodes = ref.unpack_e2m1_codes(B, K)
    Y = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            for k in range(K):
                av = Fraction(codecs.e2m1_value(int(acodes[m, k]))) * Fraction(codecs.e4m3fn_value(int(scales[m, k // 16])))
                bv = (Fraction(codecs.e2m1_value(int(bcodes[n, k]))) *
                      Fraction(codecs.e4m3fn_value(int(ws[n, k // 16]))) * Fraction(float(ws2)))
                Y[m][n] += av * bv
                S[m][n] += abs(av * bv)
            if bias is not None:
                Y[m][n] += Fraction(float(codecs.bits_to_f64(bias[n:n + 1], dtype)[0]))
    return Y, S


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_w4a4_reference_brute_force(dtype):
    rng = np.random.default_rng(9)
    M, N, K = 3, 4, 32
    x = rng.standard_normal((M, K)).astype(np.float32)
    A = codecs.f32_to_bf16_bits(x) if dtype == "bf16" else codecs.f32_to_f16_bits(x)
    B = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    ws = codecs.e4m3fn_encode(rng.uniform(2 ** -6, 4.0, size=(N, K // 16)).astype(np.float32))
    ws2 = np.float32(0.375)
    bias = codecs.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32)) if dtype == "bf16" else \
        codecs.f32_to_f16_bits(rng.standard_normal(N).astype(np.float32))
    Y, S = nvfp4.matmul_w4a4_reference(A, dtype, B, ws, 16, ws2, bias)
    Ye, Se = _exact_w4a4(A, dtype, B, ws, ws2, bias)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(Y[m, n])) - Ye[m][n]) <= K * Fraction(2) ** -52 * Se[m][n] + Fraction(2) ** -60
            assert abs(Fraction(float(S[m, n])) - Se[m][n]) <= K * Fraction(2) ** -52 * Se[m][n]


def test_w4a4_equals_weight_only_on_representable_activations():
    rng = np.random.default_rng(4)
    _, _, A = _representable(rng, 5, 64, "bf16")
    B = rng.integers(0, 256, size=(7, 32)).astype(np.uint8)
    ws = codecs.e4m3fn_encode(rng.uniform(2 ** -6, 4.0, size=(7, 4)).astype(np.float32))
    Y1, S1 = nvfp4.matmul_w4a4_reference(A, "bf16", B, ws, 16, np.float32(0.5))
    Y2, S2 = ref.matmul_fp4_reference(A, "bf16", B, ws, 16, np.float32(0.5))
    assert np.array_equal(Y1, Y2) and np.array_equal(S1, S2)
