"""C-ABI tests that need no GPU: the library loads, exports every function
include/fp4w.h declares, validates arguments before touching the device and
reports the dispatch path.  No call here reaches a kernel launch."""

import ctypes
import os
import re

import pytest

import fp8_weight_only_fp4w_amd as fw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4w.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(fp4w_\w+|fp8w_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("fp4w_matmul", "fp8w_matmul", "fp4w_dequant", "fp4w_status_string",
                     "fp4w_select_path"):
        assert required in names
    assert sorted(fw.EXPORTED) == names


def test_library_exports_every_declared_symbol():
    lib = fw.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_hbm_probe_library_exports_its_entry_point():
    # the bench's read-stream probe is built beside the matmul library and
    # exports nothing but its two entry points
    import ctypes
    import os
    import subprocess
    path = os.path.join(os.path.dirname(fw.LIB_PATH), "libhbmprobe.so")
    assert os.path.exists(path), "build() also builds libhbmprobe.so"
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "hbm_read_probe")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines() if " T " in line)
    assert exported == ["hbm_lds_stream_probe", "hbm_read_probe"], exported


def test_mfma_probe_library_exports_its_entry_point():
    # the bench's MFMA-rate probe, likewise, with arguments checked before
    # any launch (no GPU is used here)
    import ctypes
    import os
    import subprocess
    path = os.path.join(os.path.dirname(fw.LIB_PATH), "libmfmaprobe.so")
    assert os.path.exists(path), "build() also builds libmfmaprobe.so"
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines() if " T " in line)
    assert exported == ["mfma_peak_probe"], exported
    lib = ctypes.CDLL(path)
    f = lib.mfma_peak_probe
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int64
    sink = ctypes.c_void_p(0x100000)
    assert f(256, 3, 10, 1, 0, 0, sink, None) == 0      # waves must be 1 or 2
    assert f(0, 1, 10, 1, 0, 0, sink, None) == 0        # grid
    assert f(256, 1, 0, 1, 0, 0, sink, None) == 0       # iters
    assert f(256, 1, 10, 1, 0, 0, None, None) == 0      # sink


def test_status_and_path_strings():
    assert fw.fp4w_status_string(fw.OK) == "ok"
    for st in (fw.ERR_NULL, fw.ERR_SHAPE, fw.ERR_DTYPE, fw.ERR_BLOCK, fw.ERR_PATH, fw.ERR_LAUNCH, fw.ERR_ALIAS):
        assert fw.fp4w_status_string(st) not in ("ok", "unknown status")
    assert fw.fp4w_status_string(12345) == "unknown status"
    assert fw.fp4w_path_name(fw.PATH_FP4_GEMV) == "fp4_gemv"
    assert fw.fp4w_path_name(99) == "unknown"


# -------------------------------------------------------------- dispatch

def sel(op, M, N, K, bs, cols=None):
    if cols is None:
        cols = -(-K // bs) if (K and bs > 0) else 1
    return fw.fp4w_select_path(op, M, N, K, bs, cols)


def test_dispatch_fp4():
    F = fw.OP_FP4_MATMUL
    # decode GEMV for small M with the fast predicate
    for M in (1, 2, 4, 8):
        assert sel(F, M, 5120, 5120, 16) == fw.PATH_FP4_GEMV
    assert sel(F, 1, 256, 512, 16) == fw.PATH_FP4_GEMV
    # skinny matmul for 8 < M <= 64, prefill GEMM above
    assert sel(F, 9, 5120, 5120, 16) == fw.PATH_FP4_SKINNY
    assert sel(F, 64, 5120, 5120, 16) == fw.PATH_FP4_SKINNY
    assert sel(F, 65, 5120, 5120, 16) == fw.PATH_FP4_GEMM
    # above 32 rows a wide N (>= 16384) takes the GEMM, which then fills the GPU
    assert sel(F, 32, 17408, 5120, 16) == fw.PATH_FP4_SKINNY
    assert sel(F, 33, 17408, 5120, 16) == fw.PATH_FP4_GEMM
    assert sel(F, 64, 16384, 4096, 16) == fw.PATH_FP4_GEMM
    assert sel(F, 64, 16383, 4096, 16) == fw.PATH_FP4_SKINNY
    assert sel(F, 16, 5120, 5184, 16) == fw.PATH_FP4_GEMM       # K % 128 != 0, K % 64 == 0
    assert sel(F, 8192, 17408, 5120, 16) == fw.PATH_FP4_GEMM
    # outside the fast predicates -> generic ([Blog] "Existing FP4 tests did not
    # reach the prefill kernel": every leaf must be reachable and tested)
    assert sel(F, 4, 64, 48, 16) == fw.PATH_FP4_GENERIC        # K % 32 != 0
    assert sel(F, 4, 64, 464, 16) == fw.PATH_FP4_GENERIC       # K % 32 != 0
    # the GEMV takes K % 32 == 0 ([FP4 doc] §3): a last window of 32, 64 or 96 k
    assert sel(F, 4, 64, 192, 16) == fw.PATH_FP4_GEMV
    assert sel(F, 3, 1000, 480, 16) == fw.PATH_FP4_GEMV
    assert sel(F, 8, 64, 32, 16) == fw.PATH_FP4_GEMV
    assert sel(F, 4, 64, 64, 32) == fw.PATH_FP4_GENERIC        # block_size != 16
    assert sel(F, 4, 64, 30, 15) == fw.PATH_FP4_GENERIC        # odd block size
    assert sel(F, 100, 64, 96, 16) == fw.PATH_FP4_GENERIC      # K % 64 != 0 for GEMM
    assert sel(F, 3, 64, 0, 16) == fw.PATH_FP4_GENERIC         # K == 0: Y = bias
    # empty output
    assert sel(F, 0, 64, 64, 16) == fw.PATH_NONE
    assert sel(F, 5, 0, 64, 16) == fw.PATH_NONE


def test_dispatch_fp8():
    F = fw.OP_FP8_MATMUL
    assert sel(F, 4, 17408, 5120, 128) == fw.PATH_FP8_GEMV
    assert sel(F, 8192, 17408, 5120, 128) == fw.PATH_FP8_GEMM
    assert sel(F, 16, 4096, 4096, 128) == fw.PATH_FP8_SKINNY
    assert sel(F, 32, 4096, 4096, 128) == fw.PATH_FP8_SKINNY
    assert sel(F, 65, 4096, 4096, 128) == fw.PATH_FP8_GEMM
    assert sel(F, 16, 4096, 4096, 64) == fw.PATH_FP8_GEMM         # skinny needs bs % 128
    assert sel(F, 64, 256, 256, 64) == fw.PATH_FP8_GEMM
    # the GEMV takes block_size % 64 == 0 and K % 16 == 0 ([FP8 doc] §3-4)
    assert sel(F, 4, 256, 256, 64) == fw.PATH_FP8_GEMV
    assert sel(F, 4, 256, 208, 128) == fw.PATH_FP8_GEMV
    assert sel(F, 4, 256, 256, 32) == fw.PATH_FP8_GENERIC      # block_size % 64 != 0
    assert sel(F, 4, 256, 200, 64) == fw.PATH_FP8_GENERIC      # K % 16 != 0
    assert sel(F, 64, 256, 208, 128) == fw.PATH_FP8_GENERIC
    assert sel(F, 3, 256, 37, 16) == fw.PATH_FP8_GENERIC       # odd K is legal for FP8
    assert sel(F, 0, 256, 256, 128) == fw.PATH_NONE


def test_dispatch_dequant():
    F = fw.OP_FP4_DEQUANT
    assert sel(F, 0, 17408, 5120, 16) == fw.PATH_DEQUANT_VEC
    assert sel(F, 0, 64, 40, 8) == fw.PATH_DEQUANT_VEC
    assert sel(F, 0, 64, 30, 15) == fw.PATH_DEQUANT_GENERIC    # odd block size
    assert sel(F, 0, 64, 12, 4) == fw.PATH_DEQUANT_GENERIC     # K % 8 != 0
    assert sel(F, 0, 0, 64, 16) == fw.PATH_NONE
    assert sel(F, 0, 64, 0, 16) == fw.PATH_NONE


def test_select_path_rejects_illegal_shapes():
    F = fw.OP_FP4_MATMUL
    assert sel(F, 1, 16, 33, 16) == fw.ERR_SHAPE             # odd K for FP4
    assert sel(F, -1, 16, 32, 16) == fw.ERR_SHAPE
    assert sel(F, 1, 16, 32, 0) == fw.ERR_BLOCK
    assert sel(F, 1, 16, 32, 16, cols=3) == fw.ERR_SHAPE     # wrong scale_cols
    assert sel(F, 1, 16, 40, 16, cols=2) == fw.PATH_FP4_GENERIC  # floor(40/16) with partial block
    assert sel(F, 1, 16, 32, 16, cols=1) == fw.ERR_SHAPE     # floor only allowed for partial blocks
    assert sel(fw.OP_FP8_MATMUL, 1, 16, 33, 16) == fw.PATH_FP8_GENERIC
    assert fw.fp4w_select_path(7, 1, 1, 2, 1, 2) == fw.ERR_PATH


# -------------------------------------------------------------- validation (no launch)

def _fp4(lib, A=1, M=1, K=32, B=1, N=16, ws=1, cols=2, bs=16, ws2=1, bias=None, Y=1, dtype=fw.BF16, path=0):
    vp = ctypes.c_void_p
    return lib.fp4w_matmul_ex(vp(A), M, K, vp(B), N, vp(ws), cols, bs, vp(ws2), vp(bias), vp(Y), dtype,
                              None, path)


def test_validation_errors_return_before_launch():
    lib = fw.load_library()
    # fake, distinct, non-overlapping "device" addresses: every case below must
    # be rejected before any HIP call is made
    base = dict(A=0x100000, B=0x200000, ws=0x300000, ws2=0x400000, Y=0x500000)
    assert _fp4(lib, **{**base, "K": 33}) == fw.ERR_SHAPE
    assert _fp4(lib, **{**base, "bs": 0}) == fw.ERR_BLOCK
    assert _fp4(lib, **{**base, "dtype": 7}) == fw.ERR_DTYPE
    assert _fp4(lib, **{**base, "cols": 5}) == fw.ERR_SHAPE
    assert _fp4(lib, **{**base, "M": -1}) == fw.ERR_SHAPE
    assert _fp4(lib, **{**base, "A": 0}) == fw.ERR_NULL
    assert _fp4(lib, **{**base, "B": 0}) == fw.ERR_NULL
    assert _fp4(lib, **{**base, "ws": 0}) == fw.ERR_NULL
    assert _fp4(lib, **{**base, "ws2": 0}) == fw.ERR_NULL
    assert _fp4(lib, **{**base, "Y": 0}) == fw.ERR_NULL
    assert _fp4(lib, **{**base, "Y": 0x100000 + 8}) == fw.ERR_ALIAS       # Y inside A
    assert _fp4(lib, **{**base, "path": fw.PATH_FP8_GEMV}) == fw.ERR_PATH  # wrong family
    assert _fp4(lib, **{**base, "M": 9, "path": fw.PATH_FP4_GEMV}) == fw.ERR_PATH  # M > 8
    assert _fp4(lib, **{**base, "A": 0x100002, "path": fw.PATH_FP4_GEMV}) == fw.ERR_PATH  # unaligned


def test_empty_output_is_ok_without_pointers():
    lib = fw.load_library()
    assert _fp4(lib, A=0, B=0, ws=0, ws2=0, Y=0, M=0) == fw.OK
    assert _fp4(lib, A=0, B=0, ws=0, ws2=0, Y=0, N=0) == fw.OK
    vp = ctypes.c_void_p
    assert lib.fp4w_dequant(None, 0, 32, None, 2, 16, None, None, fw.BF16, None) == fw.OK
    assert lib.fp8w_matmul(None, 0, 128, None, 16, None, 1, 128, None, None, fw.BF16, None) == fw.OK


def test_fp8_and_dequant_validation():
    lib = fw.load_library()
    vp = ctypes.c_void_p
    A, B, S, Y = vp(0x100000), vp(0x200000), vp(0x300000), vp(0x500000)
    assert lib.fp8w_matmul(A, 1, 128, B, 16, S, 2, 128, None, Y, fw.BF16, None) == fw.ERR_SHAPE
    assert lib.fp8w_matmul(A, 1, 128, B, 16, S, 1, 0, None, Y, fw.BF16, None) == fw.ERR_BLOCK
    assert lib.fp8w_matmul(A, 1, 128, None, 16, S, 1, 128, None, Y, fw.BF16, None) == fw.ERR_NULL
    assert lib.fp4w_dequant(B, 16, 31, S, 2, 16, vp(0x400000), Y, fw.BF16, None) == fw.ERR_SHAPE
    assert lib.fp4w_dequant(B, 16, 32, S, 2, 16, None, Y, fw.BF16, None) == fw.ERR_NULL
    assert lib.fp4w_dequant(B, 16, 32, S, 2, 16, vp(0x400000), vp(0x200000), fw.BF16, None) == fw.ERR_ALIAS
    assert lib.fp4w_dequant_ex(B, 16, 12, S, 3, 4, vp(0x400000), Y, fw.BF16, None,
                               fw.PATH_DEQUANT_VEC) == fw.ERR_PATH


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.reload(fw)
    try:
        mod._lib = None
        with pytest.raises(RuntimeError):
            mod.load_library(str(tmp_path / "missing.so"))
    finally:
        importlib.reload(fw)


def test_dispatch_and_validation_qdq():
    Q = fw.OP_FP8_QDQ
    assert fw.fp4w_select_path(Q, 4, 0, 5120, 1, 1) == fw.PATH_QDQ_VEC
    assert fw.fp4w_select_path(Q, 3, 0, 7, 1, 1) == fw.PATH_QDQ_GENERIC      # 21 elements
    assert fw.fp4w_select_path(Q, 0, 0, 64, 1, 1) == fw.PATH_NONE
    assert fw.fp4w_select_path(Q, -1, 0, 64, 1, 1) == fw.ERR_SHAPE
    assert fw.fp4w_path_name(fw.PATH_QDQ_VEC) == "qdq_vec"
    lib = fw.load_library()
    vp = ctypes.c_void_p
    A, S, O = vp(0x100000), vp(0x300000), vp(0x500000)
    q = lib.fp8w_qdq_activation_ex
    assert q(A, 4, 64, S, O, 7, None, 0) == fw.ERR_DTYPE
    assert q(A, -4, 64, S, O, fw.BF16, None, 0) == fw.ERR_SHAPE
    assert q(None, 4, 64, S, O, fw.BF16, None, 0) == fw.ERR_NULL
    assert q(A, 4, 64, None, O, fw.BF16, None, 0) == fw.ERR_NULL
    assert q(A, 4, 64, S, None, fw.BF16, None, 0) == fw.ERR_NULL
    assert q(A, 4, 64, S, vp(0x100000 + 16), fw.BF16, None, 0) == fw.ERR_ALIAS   # partial overlap
    assert q(A, 4, 64, S, vp(0x300000 - 8), fw.BF16, None, 0) == fw.ERR_ALIAS    # out over a_scale
    assert q(A, 3, 7, S, O, fw.BF16, None, fw.PATH_QDQ_VEC) == fw.ERR_PATH        # 21 % 8 != 0
    assert q(vp(0x100002), 4, 64, S, O, fw.BF16, None, fw.PATH_QDQ_VEC) == fw.ERR_PATH  # unaligned
    assert q(A, 4, 64, S, O, fw.BF16, None, fw.PATH_FP8_GEMV) == fw.ERR_PATH     # not a QDQ path
    assert q(None, 0, 64, None, None, fw.BF16, None, 0) == fw.OK                  # empty: no launch
    assert q(None, 4, 0, None, None, fw.F16, None, fw.PATH_QDQ_GENERIC) == fw.OK


def test_w8a8_validation_before_any_launch():
    lib = fw.load_library()
    vp = ctypes.c_void_p
    A, B, S, AS, W, Y = (vp(x) for x in (0x100000, 0x200000, 0x300000, 0x380000, 0x400000, 0x500000))
    m = lib.fp8w_matmul_w8a8
    # M=4, K=256, N=16, bs=128, cols=2
    assert m(A, 4, 256, B, 16, S, 3, 128, AS, None, W, Y, fw.BF16, None) == fw.ERR_SHAPE
    assert m(A, 4, 256, B, 16, S, 2, 128, None, None, W, Y, fw.BF16, None) == fw.ERR_NULL
    assert m(A, 4, 256, B, 16, S, 2, 128, AS, None, None, Y, fw.BF16, None) == fw.ERR_NULL
    assert m(None, 4, 256, B, 16, S, 2, 128, AS, None, W, Y, fw.BF16, None) == fw.ERR_NULL
    assert m(A, 4, 256, B, 16, S, 2, 128, AS, None, vp(0x100000 + 32), Y, fw.BF16, None) == fw.ERR_ALIAS
    assert m(A, 4, 256, B, 16, S, 2, 128, AS, None, W, vp(0x400000 + 64), fw.BF16, None) == fw.ERR_ALIAS
    assert m(A, 4, 256, B, 16, S, 2, 128, AS, None, W, vp(0x100000 + 64), fw.BF16, None) == fw.ERR_ALIAS
    assert m(A, 4, 256, B, 16, S, 2, 128, AS, None, vp(0x200000 + 64), Y, fw.BF16, None) == fw.ERR_ALIAS
    assert m(A, 4, 256, B, 16, S, 2, 128, AS, None, W, Y, 9, None) == fw.ERR_DTYPE
    assert m(None, 0, 256, None, 16, None, 2, 128, None, None, None, None, fw.BF16, None) == fw.OK


def test_dispatch_and_validation_fp8_dequant():
    F = fw.OP_FP8_DEQUANT
    assert sel(F, 0, 17408, 5120, 128) == fw.PATH_FP8_DEQUANT_VEC
    assert sel(F, 0, 64, 208, 16) == fw.PATH_FP8_DEQUANT_VEC
    assert sel(F, 0, 64, 37, 16) == fw.PATH_FP8_DEQUANT_GENERIC      # K % 16 != 0 (odd K is legal)
    assert sel(F, 0, 64, 256, 24) == fw.PATH_FP8_DEQUANT_GENERIC     # block_size % 16 != 0
    assert sel(F, 0, 0, 256, 128) == fw.PATH_NONE
    lib = fw.load_library()
    vp = ctypes.c_void_p
    B, S, O = vp(0x100000), vp(0x300000), vp(0x500000)
    d = lib.fp8w_dequant_ex
    assert d(B, 16, 256, S, 3, 128, O, fw.BF16, None, 0) == fw.ERR_SHAPE
    assert d(B, 16, 256, S, 2, 0, O, fw.BF16, None, 0) == fw.ERR_BLOCK
    assert d(B, 16, 256, None, 2, 128, O, fw.BF16, None, 0) == fw.ERR_NULL
    assert d(B, 16, 256, S, 2, 128, vp(0x100000 + 64), fw.BF16, None, 0) == fw.ERR_ALIAS
    assert d(B, 16, 256, S, 2, 128, O, 5, None, 0) == fw.ERR_DTYPE
    assert d(B, 16, 37, S, 3, 16, O, fw.BF16, None, fw.PATH_FP8_DEQUANT_VEC) == fw.ERR_PATH
    assert d(B, 16, 256, S, 2, 128, O, fw.BF16, None, fw.PATH_DEQUANT_VEC) == fw.ERR_PATH
    assert d(None, 0, 256, None, 2, 128, None, fw.BF16, None, 0) == fw.OK


def test_dispatch_and_validation_nvfp4_activation():
    Q = fw.OP_NVFP4_ACT
    assert fw.fp4w_select_path(Q, 8192, 0, 5120, 1, 1) == fw.PATH_NVFP4_VEC
    assert fw.fp4w_select_path(Q, 0, 0, 64, 1, 1) == fw.PATH_NONE
    assert fw.fp4w_select_path(Q, 4, 0, 40, 1, 1) == fw.ERR_SHAPE           # K % 16 != 0
    assert fw.fp4w_select_path(Q, -1, 0, 64, 1, 1) == fw.ERR_SHAPE
    assert fw.fp4w_path_name(fw.PATH_NVFP4_VEC) == "nvfp4_vec"
    assert fw.fp4w_path_name(fw.PATH_NVFP4_GENERIC) == "nvfp4_generic"
    lib = fw.load_library()
    vp = ctypes.c_void_p
    A, C, S, O = vp(0x100000), vp(0x300000), vp(0x380000), vp(0x500000)   # A: 4 x 64 bf16 = 512 B
    q = lib.fp4w_quantize_activation_ex
    assert q(A, 4, 64, C, S, 7, None, 0) == fw.ERR_DTYPE
    assert q(A, 4, 40, C, S, fw.BF16, None, 0) == fw.ERR_SHAPE
    assert q(A, -4, 64, C, S, fw.BF16, None, 0) == fw.ERR_SHAPE
    assert q(None, 4, 64, C, S, fw.BF16, None, 0) == fw.ERR_NULL
    assert q(A, 4, 64, None, S, fw.BF16, None, 0) == fw.ERR_NULL
    assert q(A, 4, 64, C, None, fw.BF16, None, 0) == fw.ERR_NULL
    assert q(A, 4, 64, vp(0x100000 + 256), S, fw.BF16, None, 0) == fw.ERR_ALIAS     # codes inside A
    assert q(A, 4, 64, C, vp(0x100000 + 500), fw.BF16, None, 0) == fw.ERR_ALIAS     # scales inside A
    assert q(A, 4, 64, C, vp(0x300000 + 64), fw.BF16, None, 0) == fw.ERR_ALIAS      # scales inside codes
    assert q(vp(0x100002), 4, 64, C, S, fw.BF16, None, fw.PATH_NVFP4_VEC) == fw.ERR_PATH   # unaligned A
    assert q(A, 4, 64, vp(0x300004), S, fw.BF16, None, fw.PATH_NVFP4_VEC) == fw.ERR_PATH   # codes % 8
    assert q(A, 4, 64, C, S, fw.BF16, None, fw.PATH_QDQ_VEC) == fw.ERR_PATH        # not an NVFP4 path
    assert q(None, 0, 64, None, None, fw.BF16, None, 0) == fw.OK                    # empty: no launch
    d = lib.fp4w_qdq_activation_ex
    assert d(A, 4, 40, O, fw.BF16, None, 0) == fw.ERR_SHAPE
    assert d(A, 4, 64, None, fw.BF16, None, 0) == fw.ERR_NULL
    assert d(A, 4, 64, vp(0x100000 + 32), fw.BF16, None, 0) == fw.ERR_ALIAS         # partial overlap
    assert d(A, 4, 64, vp(0x500008), fw.F16, None, fw.PATH_NVFP4_VEC) == fw.ERR_PATH  # out % 16
    assert d(None, 4, 0, None, fw.F16, None, fw.PATH_NVFP4_GENERIC) == fw.OK


def test_w4a4_validation_before_any_launch():
    lib = fw.load_library()
    vp = ctypes.c_void_p
    A, B, S, W2, W, Y = (vp(x) for x in (0x100000, 0x200000, 0x300000, 0x380000, 0x400000, 0x500000))
    m = lib.fp4w_matmul_w4a4
    # M=4, K=256, N=16, bs=16, cols=16
    assert m(A, 4, 256, B, 16, S, 15, 16, W2, None, W, Y, fw.BF16, None) == fw.ERR_SHAPE
    assert m(A, 4, 40, B, 16, S, 3, 16, W2, None, W, Y, fw.BF16, None) == fw.ERR_SHAPE    # K % 16
    assert m(A, 4, 256, B, 16, S, 16, 16, None, None, W, Y, fw.BF16, None) == fw.ERR_NULL
    assert m(A, 4, 256, B, 16, S, 16, 16, W2, None, None, Y, fw.BF16, None) == fw.ERR_NULL
    assert m(None, 4, 256, B, 16, S, 16, 16, W2, None, W, Y, fw.BF16, None) == fw.ERR_NULL
    assert m(A, 4, 256, B, 16, S, 16, 16, W2, None, vp(0x100000 + 32), Y, fw.BF16, None) == fw.ERR_ALIAS
    assert m(A, 4, 256, B, 16, S, 16, 16, W2, None, W, vp(0x400000 + 64), fw.BF16, None) == fw.ERR_ALIAS
    assert m(A, 4, 256, B, 16, S, 16, 16, W2, None, W, vp(0x100000 + 64), fw.BF16, None) == fw.ERR_ALIAS
    assert m(A, 4, 256, B, 16, S, 16, 16, W2, None, vp(0x200000 + 64), Y, fw.BF16, None) == fw.ERR_ALIAS
    assert m(A, 4, 256, B, 16, S, 16, 16, W2, None, vp(0x380000 - 64), Y, fw.BF16, None) == fw.ERR_ALIAS
    assert m(A, 4, 256, B, 16, S, 16, 16, W2, None, W, Y, 9, None) == fw.ERR_DTYPE
    assert m(None, 0, 256, None, 16, None, 16, 16, None, None, None, None, fw.BF16, None) == fw.OK


def test_w4a4_noalloc_validation_before_any_launch():
    """The allocation-free W4A4 entry point validates like fp4w_matmul_w4a4
    and rejects activations larger than its scratch before it touches the
    device (no GPU is used here)."""
    lib = fw.load_library()
    vp = ctypes.c_void_p
    A, B, S, W2, Y = (vp(x) for x in (0x100000, 0x200000, 0x300000, 0x380000, 0x500000))
    m = lib.fp4w_matmul_w4a4_noalloc
    assert m(A, 4, 256, B, 16, S, 15, 16, W2, None, Y, fw.BF16, None) == fw.ERR_SHAPE   # scale_cols
    assert m(A, 4, 40, B, 16, S, 3, 16, W2, None, Y, fw.BF16, None) == fw.ERR_SHAPE     # K % 16
    assert m(None, 4, 256, B, 16, S, 16, 16, W2, None, Y, fw.BF16, None) == fw.ERR_NULL
    assert m(A, 4, 256, B, 16, S, 16, 16, None, None, Y, fw.BF16, None) == fw.ERR_NULL
    assert m(A, 4, 256, B, 16, S, 16, 16, W2, None, vp(0x100000 + 64), fw.BF16, None) == fw.ERR_ALIAS
    assert m(A, 4, 256, B, 16, S, 16, 16, W2, None, Y, 9, None) == fw.ERR_DTYPE
    assert m(None, 0, 256, None, 16, None, 16, 16, None, None, None, fw.BF16, None) == fw.OK
    # M * K * 2 beyond the scratch: one row past it
    K = 8192
    rows = fw.STATIC_SCRATCH_BYTES // (2 * K)
    big_B, big_S = vp(0x10000000), vp(0x30000000)
    big_Y = vp(0x40000000)
    assert m(A, rows + 1, K, big_B, 16, big_S, K // 16, 16, W2, None, big_Y, fw.BF16, None) == fw.ERR_SHAPE
