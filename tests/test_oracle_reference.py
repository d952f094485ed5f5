"""Pins of the oracle's dequant and matmul (CPU only).

* unpacking and scale-column choice against the pages' worked examples;
* the stored dequant rounding, exhaustively, against torch float32 arithmetic;
* the matmul against exact rational brute force on tiny shapes, a special
  case that reduces to a library matmul, and invariants any correct
  implementation keeps;
* the tolerance check itself.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs, reference as ref
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


# ------------------------------------------------------------ layout pins

def test_packing_examples_from_page():
    for byte, c_even, c_odd, v_even, v_odd in _rows("packing_examples.txt"):
        B = np.array([[int(byte, 16)]], dtype=np.uint8)
        codes = ref.unpack_e2m1_codes(B, 2)
        assert codes[0, 0] == int(c_even) and codes[0, 1] == int(c_odd)
        vals = codecs.E2M1_TABLE[codes[0]]
        for got, want in zip(vals, (v_even, v_odd)):
            w = float(want)
            assert got == w and np.signbit(got) == want.startswith("-")


def test_unpack_inverts_packing_on_all_bytes():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, size=(7, 64), dtype=np.uint8)
    packed = np.zeros((7, 32), dtype=np.uint8)
    for j in range(32):
        packed[:, j] = codes[:, 2 * j] | (codes[:, 2 * j + 1] << 4)
    assert np.array_equal(ref.unpack_e2m1_codes(packed, 64), codes)
    allbytes = np.arange(256, dtype=np.uint8)[None, :]
    c = ref.unpack_e2m1_codes(allbytes, 512)
    for b in range(256):
        assert (c[0, 2 * b] | (c[0, 2 * b + 1] << 4)) == b


def test_scale_column_examples_from_pages():
    for K, bs, cols, k, want in _rows("block_examples.txt"):
        col = ref.scale_column(int(K), int(bs), int(cols))
        assert col[int(k)] == int(want), (K, bs, cols, k)


def test_scale_column_rejects_bad_args():
    with pytest.raises(ValueError):
        ref.scale_column(32, 0, 2)
    with pytest.raises(ValueError):
        ref.scale_column(32, 16, 0)


# ------------------------------------------------------------ dequant pins

WS2_SET = [1.0, 2.0 ** -8, 0.01, 3.0, 32.0, 2.0 ** -130]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("ws2", WS2_SET)
def test_dequant_exhaustive_byte_by_scale_vs_torch_f32(dtype, ws2):
    """Every packed byte x every scale byte: the stored output equals torch's
    float32 (e2m1 * e4m3) * ws2 rounded to T."""
    ws2_32 = np.float32(ws2)
    B = np.tile(np.arange(256, dtype=np.uint8), (256, 1))         # row n: all 256 bytes
    ws = np.arange(256, dtype=np.uint8)[:, None]                    # row n: scale byte n
    got = ref.dequant_fp4_output_bits(B, ws, 512, ws2_32, 512, dtype)
    q = torch.from_numpy(codecs.E2M1_TABLE[ref.unpack_e2m1_codes(B, 512)]).to(torch.float32)
    s = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)[:, None]
    prod = (q * s) * torch.tensor(ws2_32)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    want = prod.to(tdt).view(torch.int16).numpy().view(np.uint16)
    nan = torch.isnan(prod).numpy()
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7C00 if dtype == "fp16" else got[nan] & 0x7F80) != 0)


def test_dequant_rounding_order_at_fp32():
    """The single FP32 rounding is of (e2m1 * e4m3) * ws2, the page's formula
    read left to right; folding ws2 into the scale first rounds twice and
    differs for a non-power-of-two ws2 (0.01f here)."""
    ws2 = np.float32(0.01)
    B = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    ws = np.arange(256, dtype=np.uint8)[:, None]
    got32 = ref.dequant_fp4_f64(B, ws, 512, ws2, 512).astype(np.float32)
    q = torch.from_numpy(codecs.E2M1_TABLE[ref.unpack_e2m1_codes(B, 512)]).to(torch.float32)
    s = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)[:, None]
    left = ((q * s) * torch.tensor(ws2)).numpy()
    folded = (q * (s * torch.tensor(ws2))).numpy()
    fin = np.isfinite(left)
    assert np.array_equal(got32[fin], left[fin])
    assert np.any(folded[fin] != left[fin])


def test_dequant_double_rounding_witnesses():
    """Hand-derived inputs whose stored value needs the FP32 step."""
    for dtype, byte, sbyte, wbits, want, straight in _rows("double_rounding.txt"):
        ws2 = np.array([int(wbits, 16)], dtype=np.uint32).view(np.float32)[0]
        B = np.array([[int(byte, 16)]], dtype=np.uint8)
        ws = np.array([[int(sbyte, 16)]], dtype=np.uint8)
        got = ref.dequant_fp4_output_bits(B, ws, 16, ws2, 2, dtype)
        assert got[0, 0] == int(want, 16) and got[0, 0] != int(straight, 16)


def test_dequant_fp8_output_bits_vs_torch():
    rng = np.random.default_rng(3)
    B = rng.integers(0, 256, size=(16, 256), dtype=np.uint8)
    bsc = rng.uniform(1e-3, 10, size=(16, 2)).astype(np.float32)
    got = ref.dequant_fp8_output_bits(B, bsc, 128, "bf16")
    q = torch.from_numpy(B).view(torch.float8_e4m3fn).to(torch.float32)
    s = torch.from_numpy(np.repeat(bsc, 128, axis=1))
    prod = q * s
    want = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = torch.isnan(prod).numpy()
    assert np.array_equal(got[~nan], want[~nan])


# ------------------------------------------------------------ matmul pins

def _brute_fp4(p):
    """Exact rational Y and S = sum_k |A * B_dq| for an Fp4Problem, with
    explicit loops."""
    A = codecs.bits_to_f64(p.A, p.dtype)
    bias = None if p.bias is None else codecs.bits_to_f64(p.bias, p.dtype)
    cols = p.weight_scale.shape[1]
    ws2 = Fraction(float(np.float32(p.weight_scale_2)))
    Y = [[Fraction(0)] * p.N for _ in range(p.M)]
    S = [[Fraction(0)] * p.N for _ in range(p.M)]
    for m in range(p.M):
        for n in range(p.N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(p.K):
                byte = int(p.B[n, k // 2])
                code = byte & 0xF if k % 2 == 0 else byte >> 4
                col = k // p.block_size
                if col > cols - 1:
                    col = cols - 1
                q = Fraction(codecs.e2m1_value(code))
                s = Fraction(codecs.e4m3fn_value(int(p.weight_scale[n, col])))
                term = Fraction(float(A[m, k])) * q * s * ws2
                acc += term
                mag += abs(term)
            if bias is not None:
                acc += Fraction(float(bias[n]))
            Y[m][n] = acc
            S[m][n] = mag
    return Y, S


def _brute_fp8(p):
    A = codecs.bits_to_f64(p.A, p.dtype)
    bias = None if p.bias is None else codecs.bits_to_f64(p.bias, p.dtype)
    cols = p.b_scale.shape[1]
    Y = [[Fraction(0)] * p.N for _ in range(p.M)]
    S = [[Fraction(0)] * p.N for _ in range(p.M)]
    for m in range(p.M):
        for n in range(p.N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(p.K):
                col = min(k // p.block_size, cols - 1)
                q = Fraction(codecs.e4m3fn_value(int(p.B[n, k])))
                term = Fraction(float(A[m, k])) * q * Fraction(float(p.b_scale[n, col]))
                acc += term
                mag += abs(term)
            if bias is not None:
                acc += Fraction(float(bias[n]))
            Y[m][n] = acc
            S[m][n] = mag
    return Y, S


def _close(Y, S, exact, K):
    """The oracle's Y and S against the exact rationals: Y within float64
    accumulation error; S (the scale of every tolerance) likewise, so a slip
    that inflates or shrinks it fails here."""
    exact_Y, exact_S = exact
    for m in range(Y.shape[0]):
        for n in range(Y.shape[1]):
            err = abs(Fraction(float(Y[m, n])) - exact_Y[m][n])
            assert err <= Fraction(K + 2) * Fraction(2.0 ** -52) * (exact_S[m][n] + abs(exact_Y[m][n])), (m, n)
            s_err = abs(Fraction(float(S[m, n])) - exact_S[m][n])
            assert s_err <= Fraction(K) * Fraction(2.0 ** -52) * exact_S[m][n], ("S", m, n)


FP4_TINY = [
    # M, N, K, bs, partial, dtype
    (1, 3, 32, 16, "ceil", "bf16"),
    (3, 4, 64, 32, "ceil", "fp16"),
    (2, 4, 40, 16, "ceil", "bf16"),
    (2, 4, 40, 16, "floor", "bf16"),
    (2, 3, 30, 15, "ceil", "fp16"),
    (1, 2, 18, 5, "floor", "bf16"),
    (3, 2, 14, 3, "ceil", "fp16"),
    (2, 2, 8, 1, "ceil", "bf16"),
]


@pytest.mark.parametrize("M,N,K,bs,partial,dtype", FP4_TINY)
def test_fp4_matmul_vs_exact_brute_force(M, N, K, bs, partial, dtype):
    p = workloads.make_fp4(M, N, K, bs, dtype, seed=M * 100 + N * 10 + K, a_dist="uniform",
                           scale_range=(2.0 ** -9, 448.0), ws2=0.37, with_bias=True, partial=partial)
    Y, S = ref.matmul_fp4_reference(p.A, p.dtype, p.B, p.weight_scale, bs, p.weight_scale_2, p.bias)
    _close(Y, S, _brute_fp4(p), K)


FP8_TINY = [
    (1, 3, 64, 32, "ceil", "bf16"),
    (2, 3, 208, 128, "ceil", "bf16"),
    (2, 3, 208, 128, "floor", "fp16"),
    (3, 2, 37, 16, "ceil", "fp16"),
    (2, 2, 37, 16, "floor", "bf16"),
]


@pytest.mark.parametrize("M,N,K,bs,partial,dtype", FP8_TINY)
def test_fp8_matmul_vs_exact_brute_force(M, N, K, bs, partial, dtype):
    p = workloads.make_fp8(M, N, K, bs, dtype, seed=M + N + K, a_dist="uniform",
                           scale_range=(1e-3, 10.0), with_bias=True, partial=partial)
    Y, S = ref.matmul_fp8_reference(p.A, p.dtype, p.B, p.b_scale, bs, p.bias)
    _close(Y, S, _brute_fp8(p), K)


def test_fp8_partial_final_block_uses_last_column():
    """K = 208, bs = 128: the 80 tail values use column 1 when two columns
    are given and column 0 when one is given ([FP8 doc] §2)."""
    K, bs = 208, 128
    B = np.full((1, K), 0x38, dtype=np.uint8)          # every weight 1.0
    A = np.zeros((1, K), dtype=np.uint16)
    A[0, 150] = 0x3F80                                   # bf16 1.0 at a tail position
    two = np.array([[2.0, 8.0]], dtype=np.float32)
    one = np.array([[2.0]], dtype=np.float32)
    Y2, _ = ref.matmul_fp8_reference(A, "bf16", B, two, bs)
    Y1, _ = ref.matmul_fp8_reference(A, "bf16", B, one, bs)
    assert Y2[0, 0] == 8.0 and Y1[0, 0] == 2.0


def test_fp4_partial_final_block_uses_last_column():
    K, bs = 40, 16
    B = np.full((1, K // 2), 0x22, dtype=np.uint8)       # every weight code 2 = 1.0
    A = np.zeros((1, K), dtype=np.uint16)
    A[0, 35] = 0x3F80
    three = np.array([[0x38, 0x40, 0x48]], dtype=np.uint8)   # 1, 2, 4
    two = np.array([[0x38, 0x40]], dtype=np.uint8)
    Y3, _ = ref.matmul_fp4_reference(A, "bf16", B, three, bs, 1.0)
    Y2, _ = ref.matmul_fp4_reference(A, "bf16", B, two, bs, 1.0)
    assert Y3[0, 0] == 4.0 and Y2[0, 0] == 2.0


def test_tolerance_scale_hand_computed_fp4():
    """A worked example computed by hand, for Y and S = sum_k |A * B_dq|.

    Codes 0x2, 0xB, 0x7, 0x9 are E2M1 1.0, -1.5, 6.0, -0.5 ([FP4 doc] §2);
    packed low nibble first: bytes 0xB2, 0x97.  One block of 4 with scale byte
    0x40 (E4M3 2.0) and ws2 = 0.5, so B_dq = (1, -1.5, 6, -0.5).  A (bf16) =
    (1, -2, 0.5, 3): the products are 1, 3, 3, -1.5, so Y = 5.5 and S = 8.5."""
    A = np.array([[0x3F80, 0xC000, 0x3F00, 0x4040]], dtype=np.uint16)
    B = np.array([[0xB2, 0x97]], dtype=np.uint8)
    ws = np.array([[0x40]], dtype=np.uint8)
    Y, S = ref.matmul_fp4_reference(A, "bf16", B, ws, 4, 0.5)
    assert Y[0, 0] == 5.5 and S[0, 0] == 8.5
    tol = ref.matmul_tolerance(Y, S)
    assert tol[0, 0] == 2e-3 * 8.5 + 1e-3 * 5.5


def test_tolerance_scale_hand_computed_fp8():
    """FP8 worked example: E4M3 bytes 0x38 (1.0), 0xC0 (-2.0), 0x30 (0.5) with
    FP32 block scales 4.0 (k 0-1, block 2) and 0.25 (k 2); A (fp16) = (0.5,
    1.5, -8): B_dq = (4, -8, 0.125), products 2, -12, -1, so Y = -11 and S =
    15 ([FP8 doc] §2, partial final block with its own column)."""
    A = np.array([[0x3800, 0x3E00, 0xC800]], dtype=np.uint16)
    B = np.array([[0x38, 0xC0, 0x30]], dtype=np.uint8)
    bs = np.array([[4.0, 0.25]], dtype=np.float32)
    Y, S = ref.matmul_fp8_reference(A, "fp16", B, bs, 2)
    assert Y[0, 0] == -11.0 and S[0, 0] == 15.0


def test_unit_scales_reduce_to_library_matmul():
    """All scale bytes 0x38 (= 1.0) and ws2 = 1: B_dq is the E2M1 values and
    Y_ref is an ordinary float64 matmul."""
    p = workloads.make_fp4(5, 33, 96, 16, "bf16", seed=9, with_bias=False)
    ws = np.full_like(p.weight_scale, 0x38)
    Y, _ = ref.matmul_fp4_reference(p.A, p.dtype, p.B, ws, 16, 1.0)
    A = torch.from_numpy(p.A.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    lo = torch.from_numpy((p.B & 0xF).astype(np.int64))
    hi = torch.from_numpy((p.B >> 4).astype(np.int64))
    codes = torch.stack([lo, hi], dim=2).reshape(p.N, p.K)
    # decode through torch's own FP4 dtype is unavailable on CPU, so build the
    # E2M1 magnitudes from sign / exponent / mantissa with torch ops
    sign = 1 - 2 * ((codes >> 3) & 1)
    e = (codes >> 1) & 3
    mbit = codes & 1
    mag = torch.where(e == 0, 0.5 * mbit, torch.pow(2.0, (e - 1).double()) * (1 + 0.5 * mbit))
    W = (sign * mag).double()
    want = torch.matmul(A, W.T).numpy()
    np.testing.assert_allclose(Y, want, rtol=1e-12, atol=1e-12)


def _fp4_y(p, **over):
    args = dict(A=p.A, B=p.B, ws=p.weight_scale, ws2=p.weight_scale_2, bias=p.bias)
    args.update(over)
    return ref.matmul_fp4_reference(args["A"], p.dtype, args["B"], args["ws"], p.block_size,
                                    args["ws2"], args["bias"])[0]


def test_invariant_k_block_permutation():
    p = workloads.make_fp4(3, 17, 128, 16, "bf16", seed=11, with_bias=True)
    Y = _fp4_y(p)
    perm = np.random.default_rng(0).permutation(128 // 16)
    kperm = np.concatenate([np.arange(b * 16, b * 16 + 16) for b in perm])
    bperm = np.concatenate([np.arange(b * 8, b * 8 + 8) for b in perm])
    Yp = _fp4_y(p, A=p.A[:, kperm], B=p.B[:, bperm], ws=p.weight_scale[:, perm])
    np.testing.assert_allclose(Yp, Y, rtol=1e-12, atol=1e-12)


def test_invariant_sign_flip_negates():
    p = workloads.make_fp4(2, 9, 64, 16, "fp16", seed=12, with_bias=False)
    Y = _fp4_y(p)
    Yn = _fp4_y(p, B=p.B ^ np.uint8(0x88))
    assert np.array_equal(Yn, -Y)


def test_invariant_ws2_doubling_and_bias_shift():
    p = workloads.make_fp4(2, 9, 64, 16, "bf16", seed=13, with_bias=True)
    Y0 = _fp4_y(p, bias=None)
    Y2 = _fp4_y(p, bias=None, ws2=np.float32(2 * p.weight_scale_2))
    assert np.array_equal(Y2, 2 * Y0)
    Yb = _fp4_y(p)
    np.testing.assert_array_equal(Yb - Y0, np.broadcast_to(codecs.bits_to_f64(p.bias, "bf16"), Y0.shape))


def test_fp8_matches_fp4_when_weights_coincide():
    """An FP8 weight whose E4M3 codes are E2M1 values, with b_scale = e4m3
    scale * ws2, gives the same Y as the FP4 op (the two definitions agree)."""
    p = workloads.make_fp4(2, 5, 64, 16, "bf16", seed=14, with_bias=True)
    codes = ref.unpack_e2m1_codes(p.B, p.K)
    vals = codecs.E2M1_TABLE[codes]
    B8 = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bsc = (codecs.E4M3FN_TABLE[p.weight_scale] * np.float64(p.weight_scale_2)).astype(np.float32)
    Y4, _ = ref.matmul_fp4_reference(p.A, "bf16", p.B, p.weight_scale, 16, p.weight_scale_2, p.bias)
    Y8, _ = ref.matmul_fp8_reference(p.A, "bf16", B8, bsc, 16, p.bias)
    np.testing.assert_allclose(Y8, Y4, rtol=1e-12, atol=1e-12)


def test_chunking_does_not_change_result():
    p = workloads.make_fp4(2, 37, 64, 16, "bf16", seed=15, with_bias=True)
    a = ref.matmul_fp4_reference(p.A, "bf16", p.B, p.weight_scale, 16, p.weight_scale_2, p.bias, n_chunk=5)
    b = ref.matmul_fp4_reference(p.A, "bf16", p.B, p.weight_scale, 16, p.weight_scale_2, p.bias, n_chunk=4096)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------ tolerance

def test_check_matmul_accepts_exact_and_rejects_perturbed():
    p = workloads.make_fp4(3, 40, 256, 16, "bf16", seed=16, with_bias=True)
    Y, S = ref.matmul_fp4_reference(p.A, "bf16", p.B, p.weight_scale, 16, p.weight_scale_2, p.bias)
    exact_bits = codecs.f32_to_bf16_bits(Y.astype(np.float32))
    assert ref.check_matmul(exact_bits, "bf16", Y, S)["ok"]
    tol = ref.matmul_tolerance(Y, S)
    bad = exact_bits.copy()
    # one BF16 step beyond the rounding of Y_ref + tol
    hi_bits = codecs.f32_to_bf16_bits(np.float32(Y[1, 7] + tol[1, 7]))
    bad[1, 7] = hi_bits + 1 if Y[1, 7] + tol[1, 7] > 0 else hi_bits - 1
    r = ref.check_matmul(bad, "bf16", Y, S)
    assert not r["ok"] and r["n_bad"] == 1 and r["first_bad"]["index"] == (1, 7)
    nan_bits = exact_bits.copy()
    nan_bits[0, 0] = 0x7FC0
    assert not ref.check_matmul(nan_bits, "bf16", Y, S)["ok"]


def test_check_matmul_takes_output_rounding_outside_the_bound():
    """Y_ref = 1 + 2^-8 + 2^-12 with S = |Y_ref|: tol = 3e-3 * Y_ref is less
    than the BF16 rounding error of Y_ref itself (about 2^-8), yet
    RNE_bf16(Y_ref) must pass; the next BF16 value above must fail, and so
    must the next one below RNE_bf16(Y_ref - tol)."""
    y = 1 + 2.0 ** -8 + 2.0 ** -12
    Y = np.array([[y]])
    S = np.array([[y]])
    rounded = codecs.f32_to_bf16_bits(np.float32(y))            # 0x3F81 (1.0078125)
    assert rounded[()] == 0x3F81
    assert abs(1.0078125 - y) > ref.matmul_tolerance(Y, S)[0, 0]
    assert ref.check_matmul(np.array([[0x3F81]], np.uint16), "bf16", Y, S)["ok"]
    assert not ref.check_matmul(np.array([[0x3F82]], np.uint16), "bf16", Y, S)["ok"]
    assert ref.check_matmul(np.array([[0x3F80]], np.uint16), "bf16", Y, S)["ok"]   # 1.0 = RNE(y - tol)
    assert not ref.check_matmul(np.array([[0x3F7F]], np.uint16), "bf16", Y, S)["ok"]


def test_tolerance_constants():
    """2e-3 of sum|A*B_dq| plus 1e-3 of |Y_ref|, at a hand-checked point."""
    tol = ref.matmul_tolerance(np.array([[-1.0, 0.0]]), np.array([[10.0, 0.0]]))
    assert abs(tol[0, 0] - 0.021) < 1e-15 and tol[0, 1] == 0.0
    Y = np.array([[1.0]])
    S = np.array([[100.0]])
    # tolerance 0.201: 1.1875 (err 0.1875) passes, 1.25 (err 0.25) fails
    assert ref.check_matmul(np.array([[0x3F98]], dtype=np.uint16), "bf16", Y, S)["ok"]
    assert not ref.check_matmul(np.array([[0x3FA0]], dtype=np.uint16), "bf16", Y, S)["ok"]


def test_check_matmul_fp16_overflow_reading():
    """FP32 -> FP16 rounds to nearest even and overflows to +-inf (no
    saturation).  Values from 65520 up round to +inf.  Y_ref = 70000 with S =
    70000 (tol = 210): the whole band rounds to +inf, so +inf passes and the
    largest finite value 65504 fails; Y_ref = 65400 (tol = 196.2): the band
    [65203.8, 65596.2] rounds to [65216, +inf], so 65216, 65504 and +inf
    pass, and 65184, -inf and NaN fail."""
    INF, MAXF = 0x7C00, 0x7BFF
    Y, S = np.array([[70000.0]]), np.array([[70000.0]])
    assert ref.check_matmul(np.array([[INF]], np.uint16), "fp16", Y, S)["ok"]
    assert not ref.check_matmul(np.array([[MAXF]], np.uint16), "fp16", Y, S)["ok"]
    Y, S = np.array([[65400.0]]), np.array([[65400.0]])
    assert ref.check_matmul(np.array([[MAXF]], np.uint16), "fp16", Y, S)["ok"]
    assert ref.check_matmul(np.array([[INF]], np.uint16), "fp16", Y, S)["ok"]
    assert ref.check_matmul(np.array([[0x7BF6]], np.uint16), "fp16", Y, S)["ok"]      # 65216
    assert not ref.check_matmul(np.array([[0x7BF5]], np.uint16), "fp16", Y, S)["ok"]  # 65184
    assert not ref.check_matmul(np.array([[0xFC00]], np.uint16), "fp16", Y, S)["ok"]  # -inf
    assert not ref.check_matmul(np.array([[0x7E00]], np.uint16), "fp16", Y, S)["ok"]  # NaN
    # a finite band still rejects +-inf
    Y, S = np.array([[1.0]]), np.array([[1.0]])
    assert not ref.check_matmul(np.array([[INF]], np.uint16), "fp16", Y, S)["ok"]


def test_check_matmul_nan_reference():
    Y = np.array([[np.nan, 1.0]])
    S = np.array([[1.0, 1.0]])
    assert ref.check_matmul(np.array([[0x7FC0, 0x3F80]], dtype=np.uint16), "bf16", Y, S)["ok"]
    assert not ref.check_matmul(np.array([[0x3F80, 0x3F80]], dtype=np.uint16), "bf16", Y, S)["ok"]


# ---------------------------------------------------------------------------
# Optional W8A8 activation quantize/dequantize ([FP8 doc] §6)
# ---------------------------------------------------------------------------

def _all_bits():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("a_scale", [1.0, 0.0625, 0.37, 3.0e-3, 7.5])
def test_qdq_matches_torch_fp8_round_trip(dtype, a_scale):
    """Every T bit pattern through QDQ vs torch's own float8_e4m3fn casts,
    on inputs whose quotient stays within +-448 (torch does not saturate)."""
    bits = _all_bits()
    x = ref.activation_to_f64(bits, dtype)
    q = (x.astype(np.float32) / np.float32(a_scale)).astype(np.float32)
    keep = np.isfinite(q) & (np.abs(q) <= 448)
    ours = ref.qdq_activation_fp8_bits(bits[keep], dtype, a_scale)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    t = torch.from_numpy(q[keep]).to(torch.float8_e4m3fn).to(torch.float32)
    t = (t * torch.tensor(a_scale, dtype=torch.float32)).to(tdt)
    lib = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_qdq_saturates_and_keeps_nan(dtype):
    a_scale = 0.5
    vals = np.array([300.0, -300.0, 224.0, 240.0, 1e4], dtype=np.float32)
    bits = codecs.f32_to_f16_bits(vals) if dtype == "fp16" else codecs.f32_to_bf16_bits(vals)
    out = ref.activation_to_f64(ref.qdq_activation_fp8_bits(bits, dtype, a_scale), dtype)
    assert np.array_equal(out, [224.0, -224.0, 224.0, 224.0, 224.0])   # 448 * 0.5
    nan_bits = np.array([0x7E00 if dtype == "fp16" else 0x7FC0], dtype=np.uint16)
    assert np.isnan(ref.activation_to_f64(
        ref.qdq_activation_fp8_bits(nan_bits, dtype, a_scale), dtype)).all()


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_qdq_fixes_values_already_on_the_scaled_grid(dtype):
    """A = code * a_scale with a power-of-two a_scale: QDQ is the identity;
    and QDQ is idempotent for any power-of-two scale."""
    a_scale = 2.0 ** -3
    c = np.arange(256)
    v = codecs.E4M3FN_TABLE[c]
    v = v[np.isfinite(v)] * a_scale
    bits = codecs.f32_to_f16_bits(v) if dtype == "fp16" else codecs.f32_to_bf16_bits(v)
    assert np.array_equal(ref.activation_to_f64(bits, dtype), v)   # exact in T
    out = ref.qdq_activation_fp8_bits(bits, dtype, a_scale)
    assert np.array_equal(out, bits)
    once = ref.qdq_activation_fp8_bits(_all_bits(), dtype, 4.0)
    twice = ref.qdq_activation_fp8_bits(once, dtype, 4.0)
    fin = np.isfinite(ref.activation_to_f64(once, dtype))
    assert np.array_equal(once[fin], twice[fin])


def test_qdq_error_within_e4m3_half_ulp():
    """|QDQ(a) - a| <= 2^-4 |a| for normal-range quotients (3 mantissa bits),
    <= 2^-10 * a_scale in the subnormal range; every output is code * a_scale."""
    rng = np.random.default_rng(3)
    a = rng.standard_normal(200_000).astype(np.float32)
    bits = codecs.f32_to_bf16_bits(a)
    x = ref.activation_to_f64(bits, "bf16")
    for a_scale in (0.01, 0.05):
        y = ref.activation_to_f64(ref.qdq_activation_fp8_bits(bits, "bf16", a_scale), "bf16")
        q = np.abs(x) / a_scale
        bound = np.where(q >= 2.0 ** -6, 2.0 ** -4 * np.abs(x), 2.0 ** -10 * a_scale)
        # one more BF16 rounding of the result: half an ulp of |y| (2^-9 relative)
        bound = bound + 2.0 ** -8 * np.abs(y)
        assert np.all(np.abs(y - x) <= bound * (1 + 1e-12))
