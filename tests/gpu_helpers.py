"""Shared helpers of the GPU parity tests: move seeded problems to the device,
run the library through its Python binding (the C ABI), compare with the
oracle."""

import numpy as np
import torch

import fp8_weight_only_fp4w_amd as fw
from oracle import codecs, reference as ref

TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    fw.load_library()  # raises if the HIP library is missing: no fallback exists


def bits_to_dev(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[dtype]).to(device)


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def fp4_device(p):
    return dict(
        A=bits_to_dev(p.A, p.dtype), B=u8(p.B), ws=u8(p.weight_scale),
        ws2=torch.tensor([p.weight_scale_2], dtype=torch.float32, device="cuda"),
        bias=None if p.bias is None else bits_to_dev(p.bias, p.dtype),
    )


def fp8_device(p):
    return dict(
        A=bits_to_dev(p.A, p.dtype), B=u8(p.B), bs=torch.from_numpy(p.b_scale).to("cuda"),
        bias=None if p.bias is None else bits_to_dev(p.bias, p.dtype),
    )


def run_fp4(p, d=None, path=fw.PATH_AUTO):
    d = d or fp4_device(p)
    Y = fw.fp4w_matmul(d["A"], d["B"], d["ws"], d["ws2"], d["bias"], p.block_size, path=path)
    torch.cuda.synchronize()
    return dev_to_bits(Y)


def run_fp8(p, d=None, path=fw.PATH_AUTO):
    d = d or fp8_device(p)
    Y = fw.fp8w_matmul(d["A"], d["B"], d["bs"], d["bias"], p.block_size, path=path)
    torch.cuda.synchronize()
    return dev_to_bits(Y)


# Output columns per oracle chunk: small chunks keep the float64 dequant of a
# chunk in the host caches (the arithmetic is the same for any chunk size).
ORACLE_N_CHUNK = 256


def ref_fp4(p, rows=None):
    A = p.A if rows is None else p.A[rows]
    return ref.matmul_fp4_reference(A, p.dtype, p.B, p.weight_scale, p.block_size, p.weight_scale_2, p.bias,
                                    n_chunk=ORACLE_N_CHUNK)


def ref_fp8(p, rows=None):
    A = p.A if rows is None else p.A[rows]
    return ref.matmul_fp8_reference(A, p.dtype, p.B, p.b_scale, p.block_size, p.bias, n_chunk=ORACLE_N_CHUNK)


def assert_parity(Y_bits, dtype, Y_ref, S, what=""):
    r = ref.check_matmul(Y_bits, dtype, Y_ref, S)
    assert r["ok"], (f"{what}: {r['n_bad']} of {Y_bits.size} outside tolerance, worst err/tol "
                     f"{r['max_ratio']:.3g}, first {r['first_bad']}")
    return r


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what="", zero_sign=True):
    """Bit equality of uint16 patterns; with zero_sign=False, +0 == -0."""
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    assert got.shape == want.shape
    eq = got == want
    if not zero_sign:
        eq |= ((got & 0x7FFF) == 0) & ((want & 0x7FFF) == 0)
    bad = ~eq
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {got.size} differ, first at {idx.tolist()}: "
                             f"got {[hex(int(got[tuple(i)])) for i in idx]} want {[hex(int(want[tuple(i)])) for i in idx]}")


def is_nan_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, np.uint16)
    if dtype == "fp16":
        return ((x & 0x7C00) == 0x7C00) & ((x & 0x03FF) != 0)
    return ((x & 0x7F80) == 0x7F80) & ((x & 0x007F) != 0)


def assert_dequant_equal(got, want, dtype, what=""):
    """Bit-exact dequant comparison: +0 and -0 differ, any NaN equals any NaN."""
    nan_g, nan_w = is_nan_bits(got, dtype), is_nan_bits(want, dtype)
    assert np.array_equal(nan_g, nan_w), f"{what}: NaN positions differ"
    assert_bits_equal(np.where(nan_w, 0, got), np.where(nan_w, 0, want), what)
