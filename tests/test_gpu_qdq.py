"""GPU parity of the optional W8A8 activation path ([FP8 doc] §6,
"MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"):
fp8w_qdq_activation against the oracle, bit for bit, on every FP16 / BF16
bit pattern; fp8w_matmul_w8a8 against the oracle's QDQ followed by its
matmul, to the matmul tolerance, and bit-identical to the two library calls
it is made of."""

import numpy as np
import pytest
import torch

import fp8_weight_only_fp4w_amd as fw
import workloads
from oracle import reference as ref
from gpu_helpers import (assert_bits_equal, assert_dequant_equal, assert_parity, bits_to_dev,
                         dev_to_bits, fp8_device, require_gpu)

pytestmark = pytest.mark.gpu

# unit scale, powers of two, awkward values, scales that send most inputs
# into saturation (2^-20) or into the E4M3 subnormal range / to zero (1000)
SCALES = [1.0, 0.0625, 0.37, 3.0e-3, 7.5, 2.0 ** -20, 1000.0, 0.0117]


def _scale(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def _all_bits():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_qdq_every_bit_pattern_bit_exact(dtype):
    require_gpu()
    bits = _all_bits()
    A = bits_to_dev(bits.reshape(8192, 8), dtype)
    for s in SCALES:
        want = ref.qdq_activation_fp8_bits(bits, dtype, s).reshape(8192, 8)
        sc = _scale(s)
        for path in (fw.PATH_AUTO, fw.PATH_QDQ_VEC, fw.PATH_QDQ_GENERIC):
            got = dev_to_bits(fw.fp8w_qdq_activation(A, sc, path=path))
            assert_dequant_equal(got, want, dtype, f"qdq {dtype} a_scale={s} path={path}")
        # in place
        A2 = A.clone()
        fw.fp8w_qdq_activation(A2, sc, out=A2)
        torch.cuda.synchronize()
        assert_dequant_equal(dev_to_bits(A2), want, dtype, f"qdq in place {dtype} a_scale={s}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_qdq_ragged_and_unaligned(dtype):
    require_gpu()
    rng = np.random.default_rng(21)
    bits = rng.integers(0, 65536, size=3 * 8 * 1000 + 5, dtype=np.uint32).astype(np.uint16)
    s = 0.0117
    want = ref.qdq_activation_fp8_bits(bits, dtype, s)
    # ragged count (not a multiple of 8): AUTO takes the generic kernel
    assert fw.fp4w_select_path(fw.OP_FP8_QDQ, 1, 0, bits.size, 1, 1) == fw.PATH_QDQ_GENERIC
    A = bits_to_dev(bits.reshape(1, -1), dtype)
    got = dev_to_bits(fw.fp8w_qdq_activation(A, _scale(s)))
    assert_dequant_equal(got.ravel(), want, dtype, "ragged")
    # a multiple of 8 at an address 2 bytes past a 16-byte boundary
    n = 8 * 1000
    buf = bits_to_dev(np.concatenate([[0], bits[:n]]).astype(np.uint16), dtype)
    view = buf[1:].view(8 * 10, 100)
    assert view.data_ptr() % 16 != 0
    got = dev_to_bits(fw.fp8w_qdq_activation(view, _scale(s)))
    assert_dequant_equal(got.ravel(), want[:n], dtype, "unaligned")


def test_qdq_empty_is_noop():
    require_gpu()
    A = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    assert fw.fp8w_qdq_activation(A, _scale(1.0)).shape == (0, 64)


def _calibrated_scale(A_bits, dtype):
    """Per-tensor a_scale = amax(|A|) / 448 (FP32), the usual static calibration."""
    a = ref.activation_to_f64(A_bits, dtype)
    return float(np.float32(np.max(np.abs(a))) / np.float32(448.0))


W8A8_CASES = [
    # M, N, K, bs, dtype, bias  -- GEMV (M <= 8), GEMM, generic
    (1, 300, 512, 128, "bf16", True),
    (4, 1000, 1024, 128, "fp16", False),
    (8, 777, 640, 128, "bf16", True),
    (16, 4096, 4096, 128, "bf16", False),   # the pages' W8A8 profiling shape ([FP8 doc] §7)
    (300, 700, 640, 64, "fp16", True),
    (5, 40, 208, 128, "bf16", True),        # K % 128 != 0: generic matmul
]


@pytest.mark.parametrize("M,N,K,bs,dtype,bias", W8A8_CASES)
def test_w8a8_matmul_parity(M, N, K, bs, dtype, bias):
    require_gpu()
    p = workloads.make_fp8(M, N, K, bs, dtype, seed=M * 3 + N + K, with_bias=bias)
    s = _calibrated_scale(p.A, dtype)
    Aq = ref.qdq_activation_fp8_bits(p.A, dtype, s)
    Y_ref, S = ref.matmul_fp8_reference(Aq, dtype, p.B, p.b_scale, bs, p.bias)
    d = fp8_device(p)
    sc = _scale(s)
    work = torch.empty_like(d["A"])
    Y = fw.fp8w_matmul_w8a8(d["A"], d["B"], d["bs"], sc, d["bias"], bs, workspace=work)
    torch.cuda.synchronize()
    Yb = dev_to_bits(Y)
    assert_bits_equal(dev_to_bits(work), Aq, f"w8a8 workspace M{M} N{N} K{K}")
    assert_parity(Yb, dtype, Y_ref, S, f"w8a8 M{M} N{N} K{K}")
    # the same two steps through the separate entry points: identical bits
    Y2 = fw.fp8w_matmul(fw.fp8w_qdq_activation(d["A"], sc), d["B"], d["bs"], d["bias"], bs)
    torch.cuda.synchronize()
    assert_bits_equal(dev_to_bits(Y2), Yb, "w8a8 vs qdq + fp8w_matmul")
    # in place (workspace = A)
    A_in = d["A"].clone()
    Y3 = fw.fp8w_matmul_w8a8(A_in, d["B"], d["bs"], sc, d["bias"], bs, workspace=A_in)
    torch.cuda.synchronize()
    assert_bits_equal(dev_to_bits(Y3), Yb, "w8a8 in place")


def test_w8a8_fp8_gemv_workload():
    """The FP8 GEMV workload (M=4, N=17408, K=5120, block 128) in W8A8 mode."""
    require_gpu()
    p = workloads.WORKLOADS["fp8_gemv"].make(M=4)
    s = _calibrated_scale(p.A, p.dtype)
    Aq = ref.qdq_activation_fp8_bits(p.A, p.dtype, s)
    Y_ref, S = ref.matmul_fp8_reference(Aq, p.dtype, p.B, p.b_scale, p.block_size, p.bias)
    d = fp8_device(p)
    Y = fw.fp8w_matmul_w8a8(d["A"], d["B"], d["bs"], _scale(s), d["bias"], p.block_size)
    torch.cuda.synchronize()
    assert_parity(dev_to_bits(Y), p.dtype, Y_ref, S, "w8a8 fp8_gemv M=4")
