"""GPU parity of the W4A4 path ([FP4 doc] "MatMulBlockQuantizedFp4Weight -
CUDA Operator Documentation" §6, Native SM120 FP4 x FP4 Path): the NVFP4
activation quantizer (codes, scales and the dequantized activation) bit for
bit against the oracle, on random activations and on blocks built to hit
every rounding tie, zero, NaN, infinity and saturation case, through both
kernel paths; fp4w_matmul_w4a4 against the oracle's quantized-activation
reference, and bit-identical to the two library calls it is made of."""

import numpy as np
import pytest
import torch

import fp8_weight_only_fp4w_amd as fw
import workloads
from oracle import codecs, nvfp4
from gpu_helpers import (ORACLE_N_CHUNK, TORCH_DT, assert_bits_equal, assert_dequant_equal, assert_parity,
                         bits_to_dev, dev_to_bits, fp4_device, require_gpu, u8)

pytestmark = pytest.mark.gpu

# E2M1 magnitudes and the midpoints between neighbours
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
MIDS = [(a + b) / 2 for a, b in zip(E2M1[:-1], E2M1[1:])]


def _to_bits(x, dtype):
    x32 = np.asarray(x, dtype=np.float32)
    return codecs.f32_to_bf16_bits(x32) if dtype == "bf16" else codecs.f32_to_f16_bits(x32)


def _random(M, K, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * rng.choice([1e-2, 0.3, 1.0, 7.0, 200.0], size=(M, 1))
    x[:, ::37] *= 20.0  # outliers: some blocks with one large element
    return _to_bits(x, dtype)


def _adversarial(dtype):
    """Blocks whose quotients a / s land exactly on E2M1 values and ties
    (s = 1 and s = 11/64), plus blocks with NaN, +-inf, zeros, -0, values
    below the E4M3 range and values that saturate the scale."""
    rows = []
    for s in (1.0, 11.0 / 64.0):
        # 1 + 7 ties + 6 exact values + -0 + a negative value rounding to -0
        vals = [6.0 * s] + [m * s for m in MIDS] + [v * s for v in E2M1[1:7]] + [-0.0, -0.1 * s]
        rows.append(vals[:16])
        rows.append([-v for v in vals[:16]])
        # just above / below each tie
        up = [6.0 * s] + [np.nextafter(np.float32(m * s), np.float32(10)) for m in MIDS] + [0.0] * 8
        dn = [6.0 * s] + [np.nextafter(np.float32(m * s), np.float32(0)) for m in MIDS] + [0.0] * 8
        rows.append(up[:16])
        rows.append(dn[:16])
    rows.append([np.nan, 1.0] + [0.5] * 14)
    rows.append([np.inf, 1.0, -3.0] + [0.0] * 13)
    rows.append([-np.inf, 1.0] + [0.0] * 14)
    rows.append([0.0] * 16)
    rows.append([-0.0] * 16)
    rows.append([2.0 ** -12, -2.0 ** -13] + [0.0] * 14)     # scale underflows to 0
    rows.append([3000.0, 448.0, -100.0] + [1.0] * 13)       # scale saturates at 448
    rows.append([2.0 ** -9 * 6, 2.0 ** -9 * 3, 2.0 ** -10] + [0.0] * 13)   # subnormal scale
    x = np.array(rows, dtype=np.float64)
    return _to_bits(x.reshape(1, -1), dtype)


def _check_quant(A_bits, dtype, d_A, path, what):
    M, K = A_bits.shape
    codes_w, scales_w = nvfp4.quantize_activation_nvfp4(A_bits, dtype)
    codes, scales = fw.fp4w_quantize_activation(d_A, path=path)
    out = fw.fp4w_qdq_activation(d_A, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy().reshape(M, K // 16), scales_w), f"{what}: scales"
    got_c = codes.cpu().numpy().reshape(M, K // 2)
    if not np.array_equal(got_c, codes_w):
        bad = np.argwhere(got_c != codes_w)[:4]
        raise AssertionError(f"{what}: codes differ at {bad.tolist()}")
    want = nvfp4.dequant_activation_nvfp4_bits(codes_w, scales_w, dtype)
    assert_dequant_equal(dev_to_bits(out).reshape(M, K), want, dtype, f"{what}: qdq")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,K", [(1, 16), (3, 48), (7, 5120), (64, 4096), (257, 1040)])
def test_quantize_and_qdq_bit_exact(M, K, dtype):
    require_gpu()
    A = _random(M, K, dtype, seed=M * 31 + K)
    d = bits_to_dev(A, dtype)
    _check_quant(A, dtype, d, fw.PATH_AUTO, f"auto M{M} K{K}")
    _check_quant(A, dtype, d, fw.PATH_NVFP4_GENERIC, f"generic M{M} K{K}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_adversarial_blocks_bit_exact(dtype):
    require_gpu()
    A = _adversarial(dtype)
    d = bits_to_dev(A, dtype)
    _check_quant(A, dtype, d, fw.PATH_NVFP4_VEC, "vec")
    _check_quant(A, dtype, d, fw.PATH_NVFP4_GENERIC, "generic")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_every_bit_pattern_in_a_unit_block(dtype):
    """Every FP16 / BF16 pattern as the 15 small elements of a block whose
    16th element fixes the scale at 1 (amax 6) or saturates it."""
    require_gpu()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for anchor in (6.0, 1.0e4 if dtype == "bf16" else 3.0e4):
        pad = (-len(bits)) % 15
        body = np.concatenate([bits, np.zeros(pad, np.uint16)]).reshape(-1, 15)
        A = np.concatenate([np.full((body.shape[0], 1), _to_bits(np.array([anchor]), dtype)[0], np.uint16), body],
                           axis=1).reshape(1, -1)
        d = bits_to_dev(A, dtype)
        _check_quant(A, dtype, d, fw.PATH_AUTO, f"anchor {anchor}")


def test_unaligned_views_take_the_generic_kernel():
    require_gpu()
    A = _random(4, 64, "bf16", seed=3)
    big = torch.zeros(4 * 64 + 1, dtype=torch.bfloat16, device="cuda")
    big[1:] = bits_to_dev(A.reshape(-1), "bf16")
    view = big[1:].view(4, 64)  # 2-byte aligned
    with pytest.raises(fw.FP4WError):
        fw.fp4w_qdq_activation(view, path=fw.PATH_NVFP4_VEC)
    _check_quant(A, "bf16", view, fw.PATH_AUTO, "unaligned")


def test_qdq_in_place():
    require_gpu()
    A = _random(5, 256, "fp16", seed=8)
    d = bits_to_dev(A, "fp16")
    fw.fp4w_qdq_activation(d, out=d)
    torch.cuda.synchronize()
    assert_dequant_equal(dev_to_bits(d), nvfp4.qdq_activation_nvfp4_bits(A, "fp16"), "fp16", "in place")


W4A4_CASES = [
    # M, N, K, dtype, bias: GEMV, skinny and GEMM paths of the matmul; at
    # M <= 8 and M * K <= 24576 the GEMV quantize-dequantizes its LDS copy of
    # A itself (a last partial 128-k window at K = 480; M = 6, K = 4096 at
    # that limit); M = 7, K = 5120 is past it, and at K = 17440 the
    # activations do not fit in LDS: the separate QDQ runs first
    (1, 300, 256, "bf16", True),
    (4, 1000, 512, "fp16", False),
    (2, 200, 480, "fp16", False),
    (6, 300, 4096, "bf16", False),
    (7, 260, 5120, "bf16", True),
    (8, 1100, 1024, "fp16", True),
    (4, 100, 17440, "bf16", False),
    (8, 64, 17440, "fp16", True),
    (40, 777, 1024, "bf16", True),
    (300, 700, 640, "fp16", True),
    (513, 1024, 128, "bf16", False),
]


@pytest.mark.parametrize("M,N,K,dtype,bias", W4A4_CASES)
def test_w4a4_matmul_parity(M, N, K, dtype, bias):
    require_gpu()
    p = workloads.make_fp4(M, N, K, 16, dtype, seed=M + N + K, with_bias=bias)
    Y_ref, S = nvfp4.matmul_w4a4_reference(p.A, dtype, p.B, p.weight_scale, 16, p.weight_scale_2, p.bias,
                                           n_chunk=ORACLE_N_CHUNK)
    d = fp4_device(p)
    work = torch.empty_like(d["A"])
    Y = fw.fp4w_matmul_w4a4(d["A"], d["B"], d["ws"], d["ws2"], d["bias"], 16, workspace=work)
    torch.cuda.synchronize()
    Yb = dev_to_bits(Y)
    assert_parity(Yb, dtype, Y_ref, S, f"w4a4 M{M} N{N} K{K}")
    # bit-identical to the two calls it is made of
    q = fw.fp4w_qdq_activation(d["A"])
    Y2 = fw.fp4w_matmul(q, d["B"], d["ws"], d["ws2"], d["bias"], 16)
    torch.cuda.synchronize()
    assert_bits_equal(Yb, dev_to_bits(Y2), "w4a4 == qdq + matmul")
    assert_bits_equal(dev_to_bits(work), dev_to_bits(q), "workspace holds the quantized activation")


@pytest.mark.parametrize("M", [12, 3])  # skinny; GEMV (in place: the separate QDQ, then the GEMV)
def test_w4a4_in_place_workspace(M):
    require_gpu()
    p = workloads.make_fp4(M, 256, 512, 16, "bf16", seed=21, with_bias=True)
    Y_ref, S = nvfp4.matmul_w4a4_reference(p.A, "bf16", p.B, p.weight_scale, 16, p.weight_scale_2, p.bias)
    d = fp4_device(p)
    Y = fw.fp4w_matmul_w4a4(d["A"], d["B"], d["ws"], d["ws2"], d["bias"], 16, workspace=d["A"])
    torch.cuda.synchronize()
    assert_parity(dev_to_bits(Y), "bf16", Y_ref, S, "w4a4 in place")
    assert_dequant_equal(dev_to_bits(d["A"]), nvfp4.qdq_activation_nvfp4_bits(p.A, "bf16"), "bf16", "A overwritten")


def test_w4a4_prefill_workload_sampled_rows():
    """The FP4 prefill workload (M = 8192, N = 17408, K = 5120) through the
    W4A4 path; 16 sampled rows against the oracle."""
    require_gpu()
    w = workloads.WORKLOADS["fp4_prefill"]
    p = w.make()
    d = fp4_device(p)
    Y = fw.fp4w_matmul_w4a4(d["A"], d["B"], d["ws"], d["ws2"], None, 16)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 4097, 6000, 8190, 8191, 17, 300, 511, 1024, 2047, 3333, 5555, 7777])
    Y_ref, S = nvfp4.matmul_w4a4_reference(p.A[rows], "bf16", p.B, p.weight_scale, 16, p.weight_scale_2, None,
                                           n_chunk=ORACLE_N_CHUNK)
    assert_parity(dev_to_bits(Y[torch.from_numpy(rows).cuda()]), "bf16", Y_ref, S, "w4a4 prefill rows")
