"""Python binding of libfp4w: block-scaled weight-only FP4 / FP8 matmul on
AMD MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libfp4w.so; torch supplies device memory and the current stream.
There is no fallback: if the library is missing, every call raises.

The functions carry the C ABI's names (include/fp4w.h):

* ``fp4w_matmul(A, B, weight_scale, weight_scale_2, bias=None, block_size=16)``
  Y = A * dequant(B)^T (+ bias), B packed E2M1 [N, K/2] (low nibble = even k),
  weight_scale E4M3 bytes [N, cols], weight_scale_2 a 1-element FP32 device
  tensor ("MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation" §2).
* ``fp8w_matmul(A, B, b_scale, bias=None, block_size=128)``: B E4M3 [N, K],
  b_scale FP32 [N, cols] ("MatMulBlockQuantizedFp8Weight - CUDA Operator
  Documentation" §2).
* ``fp4w_dequant(B, weight_scale, weight_scale_2, block_size=16, dtype=...)``:
  the [N, K] FP16/BF16 expansion of B.
* ``fp8w_dequant(B, b_scale, block_size=128, dtype=...)``: the [N, K]
  FP16/BF16 expansion of FP8 weights (FP8 document §5, step 1).
* ``fp8w_qdq_activation(A, a_scale)``: fp8_e4m3(A / a_scale) * a_scale in A's
  dtype, the activation step of the FP8 operator's optional W8A8 mode (FP8
  document §6).
* ``fp8w_matmul_w8a8(A, B, b_scale, a_scale, bias=None, block_size=128)``:
  that step into a workspace, then ``fp8w_matmul`` on it.
* ``fp4w_quantize_activation(A)``: (codes [M, K/2], scales [M, K/16]), the
  NVFP4 activation of the FP4 operator's native FP4 x FP4 path (FP4 document
  §6, Native SM120 FP4 x FP4 Path); ``fp4w_qdq_activation(A)``: the same,
  decoded back to A's dtype.
* ``fp4w_matmul_w4a4(A, B, weight_scale, weight_scale_2, bias=None,
  block_size=16)``: that activation times the FP4 weights (W4A4);
  ``fp4w_matmul_w4a4_noalloc(...)``: the same with the activation staged in
  the library's own device scratch, for callers that cannot allocate.

A keeps any leading dimensions; Y has A's leading dimensions, last dimension
N and A's dtype.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4w.so")

# status codes (fp4w_status)
OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_BLOCK, ERR_PATH, ERR_LAUNCH, ERR_ALIAS = 0, -1, -2, -3, -4, -5, -6, -7
# kernel paths (fp4w_path)
PATH_AUTO, PATH_NONE = 0, 1
PATH_FP4_GEMV, PATH_FP4_GEMM, PATH_FP4_GENERIC = 2, 3, 4
PATH_FP8_GEMV, PATH_FP8_GEMM, PATH_FP8_GENERIC = 5, 6, 7
PATH_DEQUANT_VEC, PATH_DEQUANT_GENERIC = 8, 9
PATH_QDQ_VEC, PATH_QDQ_GENERIC = 10, 11
PATH_FP4_SKINNY, PATH_FP8_SKINNY = 12, 13
PATH_FP8_DEQUANT_VEC, PATH_FP8_DEQUANT_GENERIC = 14, 15
PATH_NVFP4_VEC, PATH_NVFP4_GENERIC = 16, 17
# operations (fp4w_op)
OP_FP4_MATMUL, OP_FP8_MATMUL, OP_FP4_DEQUANT, OP_FP8_QDQ, OP_FP8_DEQUANT, OP_NVFP4_ACT = 0, 1, 2, 3, 4, 5
# dtypes (fp4w_dtype)
F16, BF16 = 0, 1

EXPORTED = (
    "fp4w_matmul", "fp4w_matmul_ex", "fp8w_matmul", "fp8w_matmul_ex", "fp4w_dequant",
    "fp4w_dequant_ex", "fp8w_dequant", "fp8w_dequant_ex", "fp8w_qdq_activation", "fp8w_qdq_activation_ex", "fp8w_matmul_w8a8",
    "fp4w_quantize_activation", "fp4w_quantize_activation_ex", "fp4w_qdq_activation", "fp4w_qdq_activation_ex",
    "fp4w_matmul_w4a4", "fp4w_matmul_w4a4_noalloc",
    "fp4w_select_path", "fp4w_status_string", "fp4w_path_name",
)


class FP4WError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fp4w_status_string(status)} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfp4w.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m fp8_weight_only_fp4w_amd.build`")
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.fp4w_matmul_ex.argtypes = [vp, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp, i32, vp, i32]
    lib.fp4w_matmul_ex.restype = i32
    lib.fp4w_matmul.argtypes = [vp, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp, i32, vp]
    lib.fp4w_matmul.restype = i32
    lib.fp8w_matmul_ex.argtypes = [vp, i64, i64, vp, i64, vp, i64, i64, vp, vp, i32, vp, i32]
    lib.fp8w_matmul_ex.restype = i32
    lib.fp8w_matmul.argtypes = [vp, i64, i64, vp, i64, vp, i64, i64, vp, vp, i32, vp]
    lib.fp8w_matmul.restype = i32
    lib.fp4w_dequant_ex.argtypes = [vp, i64, i64, vp, i64, i64, vp, vp, i32, vp, i32]
    lib.fp4w_dequant_ex.restype = i32
    lib.fp4w_dequant.argtypes = [vp, i64, i64, vp, i64, i64, vp, vp, i32, vp]
    lib.fp4w_dequant.restype = i32
    lib.fp8w_dequant_ex.argtypes = [vp, i64, i64, vp, i64, i64, vp, i32, vp, i32]
    lib.fp8w_dequant_ex.restype = i32
    lib.fp8w_dequant.argtypes = [vp, i64, i64, vp, i64, i64, vp, i32, vp]
    lib.fp8w_dequant.restype = i32
    lib.fp8w_qdq_activation_ex.argtypes = [vp, i64, i64, vp, vp, i32, vp, i32]
    lib.fp8w_qdq_activation_ex.restype = i32
    lib.fp8w_qdq_activation.argtypes = [vp, i64, i64, vp, vp, i32, vp]
    lib.fp8w_qdq_activation.restype = i32
    lib.fp8w_matmul_w8a8.argtypes = [vp, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp, vp, i32, vp]
    lib.fp8w_matmul_w8a8.restype = i32
    lib.fp4w_quantize_activation_ex.argtypes = [vp, i64, i64, vp, vp, i32, vp, i32]
    lib.fp4w_quantize_activation_ex.restype = i32
    lib.fp4w_quantize_activation.argtypes = [vp, i64, i64, vp, vp, i32, vp]
    lib.fp4w_quantize_activation.restype = i32
    lib.fp4w_qdq_activation_ex.argtypes = [vp, i64, i64, vp, i32, vp, i32]
    lib.fp4w_qdq_activation_ex.restype = i32
    lib.fp4w_qdq_activation.argtypes = [vp, i64, i64, vp, i32, vp]
    lib.fp4w_qdq_activation.restype = i32
    lib.fp4w_matmul_w4a4.argtypes = [vp, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp, vp, i32, vp]
    lib.fp4w_matmul_w4a4.restype = i32
    lib.fp4w_matmul_w4a4_noalloc.argtypes = [vp, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp, i32, vp]
    lib.fp4w_matmul_w4a4_noalloc.restype = i32
    lib.fp4w_select_path.argtypes = [i32, i64, i64, i64, i64, i64]
    lib.fp4w_select_path.restype = i32
    lib.fp4w_status_string.argtypes = [i32]
    lib.fp4w_status_string.restype = ctypes.c_char_p
    lib.fp4w_path_name.argtypes = [i32]
    lib.fp4w_path_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fp4w_status_string(status: int) -> str:
    return load_library().fp4w_status_string(int(status)).decode()


def fp4w_path_name(path: int) -> str:
    return load_library().fp4w_path_name(int(path)).decode()


def fp4w_select_path(op: int, M: int, N: int, K: int, block_size: int, scale_cols: int) -> int:
    return int(load_library().fp4w_select_path(op, M, N, K, block_size, scale_cols))


# ---------------------------------------------------------------- marshalling

def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return BF16
    if t == torch.float16:
        return F16
    raise TypeError(f"activation dtype must be float16 or bfloat16, got {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _bytes(t: torch.Tensor) -> torch.Tensor:
    """uint8 view of a uint8 / float8_e4m3fn tensor."""
    if t.dtype == torch.uint8:
        return t
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    raise TypeError(f"expected uint8 or float8_e4m3fn bytes, got {t.dtype}")


def _need(t: torch.Tensor, name: str, device: torch.device):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, what: str):
    if status != OK:
        raise FP4WError(status, what)


def fp4w_matmul(A: torch.Tensor, B: torch.Tensor, weight_scale: torch.Tensor,
                weight_scale_2: torch.Tensor, bias: torch.Tensor = None, block_size: int = 16,
                out: torch.Tensor = None, path: int = PATH_AUTO) -> torch.Tensor:
    lib = load_library()
    dev = A.device
    B, weight_scale = _bytes(B), _bytes(weight_scale)
    K = A.shape[-1]
    M = A.numel() // K if K else int(torch.tensor(A.shape[:-1]).prod().item())
    N = B.shape[0]
    if B.dim() != 2 or B.shape[1] * 2 != K:
        raise ValueError(f"B must be [N, K/2] = [N, {K // 2}], got {tuple(B.shape)}")
    if weight_scale.dim() != 2 or weight_scale.shape[0] != N:
        raise ValueError("weight_scale must be [N, scale_cols]")
    if weight_scale_2.dtype != torch.float32 or weight_scale_2.numel() != 1:
        raise ValueError("weight_scale_2 must be a 1-element float32 tensor")
    for t, name in ((A, "A"), (B, "B"), (weight_scale, "weight_scale"), (weight_scale_2, "weight_scale_2")):
        _need(t, name, dev)
    if bias is not None:
        _need(bias, "bias", dev)
        if bias.dtype != A.dtype or bias.numel() != N:
            raise ValueError("bias must be [N] with A's dtype")
    if out is None:
        out = torch.empty(*A.shape[:-1], N, dtype=A.dtype, device=dev)
    _need(out, "out", dev)
    st = lib.fp4w_matmul_ex(_ptr(A), M, K, _ptr(B), N, _ptr(weight_scale), weight_scale.shape[1],
                            block_size, _ptr(weight_scale_2), _ptr(bias), _ptr(out),
                            _dtype_code(A.dtype), _stream(dev), path)
    _check(st, "fp4w_matmul")
    return out


def fp8w_matmul(A: torch.Tensor, B: torch.Tensor, b_scale: torch.Tensor, bias: torch.Tensor = None,
                block_size: int = 128, out: torch.Tensor = None, path: int = PATH_AUTO) -> torch.Tensor:
    lib = load_library()
    dev = A.device
    B = _bytes(B)
    K = A.shape[-1]
    M = A.numel() // K if K else int(torch.tensor(A.shape[:-1]).prod().item())
    N = B.shape[0]
    if B.dim() != 2 or B.shape[1] != K:
        raise ValueError(f"B must be [N, K] = [N, {K}], got {tuple(B.shape)}")
    if b_scale.dtype != torch.float32 or b_scale.dim() != 2 or b_scale.shape[0] != N:
        raise ValueError("b_scale must be float32 [N, scale_cols]")
    for t, name in ((A, "A"), (B, "B"), (b_scale, "b_scale")):
        _need(t, name, dev)
    if bias is not None:
        _need(bias, "bias", dev)
        if bias.dtype != A.dtype or bias.numel() != N:
            raise ValueError("bias must be [N] with A's dtype")
    if out is None:
        out = torch.empty(*A.shape[:-1], N, dtype=A.dtype, device=dev)
    _need(out, "out", dev)
    st = lib.fp8w_matmul_ex(_ptr(A), M, K, _ptr(B), N, _ptr(b_scale), b_scale.shape[1], block_size,
                            _ptr(bias), _ptr(out), _dtype_code(A.dtype), _stream(dev), path)
    _check(st, "fp8w_matmul")
    return out


def fp4w_dequant(B: torch.Tensor, weight_scale: torch.Tensor, weight_scale_2: torch.Tensor,
                 block_size: int = 16, dtype: torch.dtype = torch.bfloat16, out: torch.Tensor = None,
                 path: int = PATH_AUTO) -> torch.Tensor:
    lib = load_library()
    dev = B.device
    B, weight_scale = _bytes(B), _bytes(weight_scale)
    N, K = B.shape[0], 2 * B.shape[1]
    for t, name in ((B, "B"), (weight_scale, "weight_scale"), (weight_scale_2, "weight_scale_2")):
        _need(t, name, dev)
    if weight_scale_2.dtype != torch.float32 or weight_scale_2.numel() != 1:
        raise ValueError("weight_scale_2 must be a 1-element float32 tensor")
    if out is None:
        out = torch.empty(N, K, dtype=dtype, device=dev)
    _need(out, "out", dev)
    st = lib.fp4w_dequant_ex(_ptr(B), N, K, _ptr(weight_scale), weight_scale.shape[1], block_size,
                             _ptr(weight_scale_2), _ptr(out), _dtype_code(out.dtype), _stream(dev), path)
    _check(st, "fp4w_dequant")
    return out


def _scalar_f32(t: torch.Tensor, name: str):
    if t.dtype != torch.float32 or t.numel() != 1:
        raise ValueError(f"{name} must be a 1-element float32 tensor")


def fp8w_qdq_activation(A: torch.Tensor, a_scale: torch.Tensor, out: torch.Tensor = None,
                        path: int = PATH_AUTO) -> torch.Tensor:
    """fp8_e4m3(A / a_scale) * a_scale in A's dtype; ``out`` may be ``A``."""
    lib = load_library()
    dev = A.device
    K = A.shape[-1] if A.dim() else 1
    M = A.numel() // K if K else 0
    _need(A, "A", dev)
    _need(a_scale, "a_scale", dev)
    _scalar_f32(a_scale, "a_scale")
    if out is None:
        out = torch.empty_like(A)
    _need(out, "out", dev)
    if out.shape != A.shape or out.dtype != A.dtype:
        raise ValueError("out must have A's shape and dtype")
    st = lib.fp8w_qdq_activation_ex(_ptr(A), M, K, _ptr(a_scale), _ptr(out),
                                    _dtype_code(A.dtype), _stream(dev), path)
    _check(st, "fp8w_qdq_activation")
    return out


def fp8w_matmul_w8a8(A: torch.Tensor, B: torch.Tensor, b_scale: torch.Tensor, a_scale: torch.Tensor,
                     bias: torch.Tensor = None, block_size: int = 128, out: torch.Tensor = None,
                     workspace: torch.Tensor = None) -> torch.Tensor:
    """fp8w_matmul on fp8_e4m3(A / a_scale) * a_scale.  ``workspace`` (A's shape
    and dtype, or ``A`` itself to quantize in place) receives the quantized
    activation; it is allocated here when not given."""
    lib = load_library()
    dev = A.device
    B = _bytes(B)
    K = A.shape[-1]
    M = A.numel() // K if K else int(torch.tensor(A.shape[:-1]).prod().item())
    N = B.shape[0]
    if B.dim() != 2 or B.shape[1] != K:
        raise ValueError(f"B must be [N, K] = [N, {K}], got {tuple(B.shape)}")
    if b_scale.dtype != torch.float32 or b_scale.dim() != 2 or b_scale.shape[0] != N:
        raise ValueError("b_scale must be float32 [N, scale_cols]")
    _scalar_f32(a_scale, "a_scale")
    for t, name in ((A, "A"), (B, "B"), (b_scale, "b_scale"), (a_scale, "a_scale")):
        _need(t, name, dev)
    if bias is not None:
        _need(bias, "bias", dev)
        if bias.dtype != A.dtype or bias.numel() != N:
            raise ValueError("bias must be [N] with A's dtype")
    if workspace is None:
        workspace = torch.empty_like(A)
    _need(workspace, "workspace", dev)
    if workspace.shape != A.shape or workspace.dtype != A.dtype:
        raise ValueError("workspace must have A's shape and dtype")
    if out is None:
        out = torch.empty(*A.shape[:-1], N, dtype=A.dtype, device=dev)
    _need(out, "out", dev)
    st = lib.fp8w_matmul_w8a8(_ptr(A), M, K, _ptr(B), N, _ptr(b_scale), b_scale.shape[1], block_size,
                              _ptr(a_scale), _ptr(bias), _ptr(workspace), _ptr(out),
                              _dtype_code(A.dtype), _stream(dev))
    _check(st, "fp8w_matmul_w8a8")
    return out


def fp8w_dequant(B: torch.Tensor, b_scale: torch.Tensor, block_size: int = 128,
                 dtype: torch.dtype = torch.bfloat16, out: torch.Tensor = None,
                 path: int = PATH_AUTO) -> torch.Tensor:
    lib = load_library()
    dev = B.device
    B = _bytes(B)
    N, K = B.shape
    for t, name in ((B, "B"), (b_scale, "b_scale")):
        _need(t, name, dev)
    if b_scale.dtype != torch.float32 or b_scale.dim() != 2 or b_scale.shape[0] != N:
        raise ValueError("b_scale must be float32 [N, scale_cols]")
    if out is None:
        out = torch.empty(N, K, dtype=dtype, device=dev)
    _need(out, "out", dev)
    st = lib.fp8w_dequant_ex(_ptr(B), N, K, _ptr(b_scale), b_scale.shape[1], block_size, _ptr(out),
                             _dtype_code(out.dtype), _stream(dev), path)
    _check(st, "fp8w_dequant")
    return out


def _rows_k(A: torch.Tensor):
    K = A.shape[-1] if A.dim() else 1
    return (A.numel() // K if K else 0), K


def fp4w_quantize_activation(A: torch.Tensor, codes: torch.Tensor = None, scales: torch.Tensor = None,
                             path: int = PATH_AUTO):
    """NVFP4 activation: (codes uint8 [..., K/2], scales uint8 [..., K/16])."""
    lib = load_library()
    dev = A.device
    M, K = _rows_k(A)
    _need(A, "A", dev)
    if codes is None:
        codes = torch.empty(*A.shape[:-1], K // 2, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(*A.shape[:-1], K // 16, dtype=torch.uint8, device=dev)
    for t, name, n in ((codes, "codes", K // 2), (scales, "scales", K // 16)):
        _need(t, name, dev)
        if t.dtype != torch.uint8 or t.numel() != M * n:
            raise ValueError(f"{name} must be uint8 with {M * n} elements")
    st = lib.fp4w_quantize_activation_ex(_ptr(A), M, K, _ptr(codes), _ptr(scales), _dtype_code(A.dtype),
                                         _stream(dev), path)
    _check(st, "fp4w_quantize_activation")
    return codes, scales


def fp4w_qdq_activation(A: torch.Tensor, out: torch.Tensor = None, path: int = PATH_AUTO) -> torch.Tensor:
    """The NVFP4 activation decoded back to A's dtype; ``out`` may be ``A``."""
    lib = load_library()
    dev = A.device
    M, K = _rows_k(A)
    _need(A, "A", dev)
    if out is None:
        out = torch.empty_like(A)
    _need(out, "out", dev)
    if out.shape != A.shape or out.dtype != A.dtype:
        raise ValueError("out must have A's shape and dtype")
    st = lib.fp4w_qdq_activation_ex(_ptr(A), M, K, _ptr(out), _dtype_code(A.dtype), _stream(dev), path)
    _check(st, "fp4w_qdq_activation")
    return out


def fp4w_matmul_w4a4(A: torch.Tensor, B: torch.Tensor, weight_scale: torch.Tensor,
                     weight_scale_2: torch.Tensor, bias: torch.Tensor = None, block_size: int = 16,
                     out: torch.Tensor = None, workspace: torch.Tensor = None) -> torch.Tensor:
    """W4A4: fp4w_matmul on the NVFP4 activation of A.  ``workspace`` (A's
    shape and dtype, or ``A`` itself) receives that activation; it is
    allocated here when not given."""
    lib = load_library()
    dev = A.device
    B, weight_scale = _bytes(B), _bytes(weight_scale)
    K = A.shape[-1]
    M = A.numel() // K if K else int(torch.tensor(A.shape[:-1]).prod().item())
    N = B.shape[0]
    if B.dim() != 2 or B.shape[1] * 2 != K:
        raise ValueError(f"B must be [N, K/2] = [N, {K // 2}], got {tuple(B.shape)}")
    if weight_scale.dim() != 2 or weight_scale.shape[0] != N:
        raise ValueError("weight_scale must be [N, scale_cols]")
    _scalar_f32(weight_scale_2, "weight_scale_2")
    for t, name in ((A, "A"), (B, "B"), (weight_scale, "weight_scale"), (weight_scale_2, "weight_scale_2")):
        _need(t, name, dev)
    if bias is not None:
        _need(bias, "bias", dev)
        if bias.dtype != A.dtype or bias.numel() != N:
            raise ValueError("bias must be [N] with A's dtype")
    if workspace is None:
        workspace = torch.empty_like(A)
    _need(workspace, "workspace", dev)
    if workspace.shape != A.shape or workspace.dtype != A.dtype:
        raise ValueError("workspace must have A's shape and dtype")
    if out is None:
        out = torch.empty(*A.shape[:-1], N, dtype=A.dtype, device=dev)
    _need(out, "out", dev)
    st = lib.fp4w_matmul_w4a4(_ptr(A), M, K, _ptr(B), N, _ptr(weight_scale), weight_scale.shape[1], block_size,
                              _ptr(weight_scale_2), _ptr(bias), _ptr(workspace), _ptr(out),
                              _dtype_code(A.dtype), _stream(dev))
    _check(st, "fp4w_matmul_w4a4")
    return out


STATIC_SCRATCH_BYTES = 32 * 1024 * 1024  # FP4W_STATIC_SCRATCH_BYTES


def fp4w_matmul_w4a4_noalloc(A: torch.Tensor, B: torch.Tensor, weight_scale: torch.Tensor,
                             weight_scale_2: torch.Tensor, bias: torch.Tensor = None, block_size: int = 16,
                             out: torch.Tensor = None) -> torch.Tensor:
    """fp4w_matmul_w4a4 with the activation staged in the library's own
    device scratch (STATIC_SCRATCH_BYTES per device) instead of a workspace:
    the C call allocates nothing.  Calls that overlap on one device race on
    that scratch.  ``out`` is allocated here when not given."""
    lib = load_library()
    dev = A.device
    B, weight_scale = _bytes(B), _bytes(weight_scale)
    K = A.shape[-1]
    M = A.numel() // K if K else int(torch.tensor(A.shape[:-1]).prod().item())
    N = B.shape[0]
    if B.dim() != 2 or B.shape[1] * 2 != K:
        raise ValueError(f"B must be [N, K/2] = [N, {K // 2}], got {tuple(B.shape)}")
    if weight_scale.dim() != 2 or weight_scale.shape[0] != N:
        raise ValueError("weight_scale must be [N, scale_cols]")
    _scalar_f32(weight_scale_2, "weight_scale_2")
    for t, name in ((A, "A"), (B, "B"), (weight_scale, "weight_scale"), (weight_scale_2, "weight_scale_2")):
        _need(t, name, dev)
    if bias is not None:
        _need(bias, "bias", dev)
        if bias.dtype != A.dtype or bias.numel() != N:
            raise ValueError("bias must be [N] with A's dtype")
    if out is None:
        out = torch.empty(*A.shape[:-1], N, dtype=A.dtype, device=dev)
    _need(out, "out", dev)
    st = lib.fp4w_matmul_w4a4_noalloc(_ptr(A), M, K, _ptr(B), N, _ptr(weight_scale), weight_scale.shape[1],
                                      block_size, _ptr(weight_scale_2), _ptr(bias), _ptr(out),
                                      _dtype_code(A.dtype), _stream(dev))
    _check(st, "fp4w_matmul_w4a4_noalloc")
    return out
