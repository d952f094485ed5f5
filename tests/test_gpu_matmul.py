"""GPU parity of fp4w_matmul / fp8w_matmul against the oracle.

Acceptance (results are not unique: the accumulation order differs between
kernels) is element by element
    |Y - Y_ref| <= 2e-3 * sum_k |A * B_dq| + 1e-3 * |Y_ref|.
One-hot activations make each output a single exact product, so there the
kernels must match the oracle bit for bit (+0 and -0 aside); this also probes
which lane owns which row and column ([FP4 doc] §4 and [FP8 doc] §4.1 describe
the same probe for the CUDA fragments).

Every dispatch leaf is reached and forced where it applies ([Blog], "Existing
FP4 tests did not reach the prefill kernel").
"""

import numpy as np
import pytest
import torch

import fp8_fold_cases
import fp8_weight_only_fp4w_amd as fw
import workloads
from oracle import codecs, reference as ref
from gpu_helpers import (assert_bits_equal, assert_parity, bits_to_dev, dev_to_bits, fp4_device,
                         fp8_device, ref_fp4, ref_fp8, require_gpu, run_fp4, run_fp8, u8)

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------- FP4

FP4_CASES = [
    # M, N, K, bs, dtype, bias, partial, paths to force (besides AUTO)
    (1, 16, 128, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMV, fw.PATH_FP4_GENERIC]),
    # K % 128 != 0: the GEMV's last window holds 96, 64 or 32 k (scale bytes
    # past the row masked), against the generic kernel
    (3, 1000, 480, 16, "fp16", True, "ceil", [fw.PATH_FP4_GEMV, fw.PATH_FP4_GENERIC]),
    (8, 300, 320, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMV]),
    (1, 77, 32, 16, "bf16", False, "ceil", [fw.PATH_FP4_GEMV]),
    (5, 4100, 5152, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMV]),
    (4, 300, 17440, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMV]),  # streamed activations, 137 windows
    # M = 5 .. 8 (row pairs) with streamed activations, one with a last window of 32 k
    (8, 300, 17440, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMV]),
    (6, 200, 12320, 16, "fp16", False, "ceil", [fw.PATH_FP4_GEMV]),
    # streamed activations with several tile groups per workgroup (N = 5120:
    # 320 tiles on 160 workgroups)
    (4, 5120, 17408, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMV]),
    (7, 4500, 9024, 16, "fp16", True, "ceil", [fw.PATH_FP4_GEMV]),
    (3, 1000, 25600, 16, "bf16", False, "ceil", [fw.PATH_FP4_GEMV]),
    (8, 777, 1024, 16, "bf16", False, "ceil", [fw.PATH_FP4_GEMV, fw.PATH_FP4_GEMM]),
    (5, 65590, 128, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMV]),  # 2 tiles per wave, ragged N
    (9, 300, 128, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMM, fw.PATH_FP4_GENERIC]),
    # GEMM tiles are 256 x 256; a last round of at most half the CUs' worth
    # of tiles runs as 256 x 128 halves.  Ragged M and N in 2 x 3 tiles (all
    # halves, the last column's second half past N); one tile row past M.
    (300, 700, 640, 16, "fp16", True, "ceil", [fw.PATH_FP4_GEMM]),
    (513, 256, 64, 16, "bf16", False, "ceil", [fw.PATH_FP4_GEMM]),
    # 3 x 8 = 24 tiles, an odd number of K steps; the last column tile takes
    # the element-wise epilogue, the others the 16-byte one
    (700, 1800, 448, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMM]),
    # 2 x 70 = 140 tiles: more than half of 256 CUs, all whole tiles (the XCD
    # tile remap is active: 140 % 8 != 0 leaves it off, so also below)
    (300, 17920, 128, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMM]),
    # 3 x 102 = 306 tiles: 256 whole ones (grid a multiple of 8: XCD remap
    # on) and 50 as halves, among them the ragged last tile column
    (600, 26012, 192, 16, "fp16", True, "ceil", [fw.PATH_FP4_GEMM]),
    # M <= 128 takes 128-row tiles: 300 of them, 256 whole and 44 halves
    (128, 76760, 64, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMM]),
    (97, 2000, 320, 16, "fp16", False, "ceil", [fw.PATH_FP4_GEMM]),
    # K steps of 64 through the GEMM's step loop (six steps at a time while
    # eight remain, then single steps, then the last two, which issue no
    # loads): 13 = 6 + 5 + 2, 14 = 2 x 6 + 2, 15 = 2 x 6 + 1 + 2, 9 = 6 + 1 + 2
    (300, 600, 832, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMM]),
    (260, 300, 896, 16, "fp16", True, "ceil", [fw.PATH_FP4_GEMM]),
    (129, 520, 960, 16, "bf16", False, "ceil", [fw.PATH_FP4_GEMM]),
    (100, 700, 576, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMM]),
    # skinny kernel: 1, 2 and 4 row tiles, ragged M and N, one window per
    # wave (K = 128), long K, the persistent loop over many tiles
    (9, 300, 256, 16, "bf16", True, "ceil", [fw.PATH_FP4_SKINNY, fw.PATH_FP4_GEMM]),
    (16, 1000, 1024, 16, "fp16", True, "ceil", [fw.PATH_FP4_SKINNY]),
    (17, 777, 640, 16, "bf16", False, "ceil", [fw.PATH_FP4_SKINNY, fw.PATH_FP4_GENERIC]),
    (33, 4100, 512, 16, "fp16", True, "ceil", [fw.PATH_FP4_SKINNY]),
    (64, 256, 5120, 16, "bf16", True, "ceil", [fw.PATH_FP4_SKINNY, fw.PATH_FP4_GEMM]),
    (1, 40, 128, 16, "bf16", True, "ceil", [fw.PATH_FP4_SKINNY]),
    (5, 65590, 256, 16, "fp16", False, "ceil", [fw.PATH_FP4_SKINNY]),
    # 32 < M <= 64 with N >= 16384: AUTO takes the 128-row-tile GEMM (ragged N)
    (40, 16400, 256, 16, "bf16", True, "ceil", [fw.PATH_FP4_SKINNY]),
    (40, 96, 96, 16, "bf16", True, "ceil", [fw.PATH_FP4_GENERIC]),  # K % 64 != 0
    (6, 50, 40, 16, "fp16", True, "floor", [fw.PATH_FP4_GENERIC]),  # partial block, floor cols
    (4, 33, 30, 15, "bf16", True, "ceil", [fw.PATH_FP4_GENERIC]),   # odd block size
    (12, 20, 18, 5, "fp16", False, "floor", [fw.PATH_FP4_GENERIC]),
    (2, 64, 64, 32, "bf16", True, "ceil", [fw.PATH_FP4_GENERIC]),   # block size 32
    # GEMV activation modes: K = 17536 (137 windows, odd: the last unit has one
    # window) does not fit in LDS, so the activations stream from L2; two row
    # halves streamed; 6 rows x 41 windows fit only beside the shallow ring
    (4, 300, 17536, 16, "bf16", True, "ceil", [fw.PATH_FP4_GEMV]),
    (8, 100, 17408, 16, "fp16", True, "ceil", [fw.PATH_FP4_GEMV]),
    (6, 200, 5248, 16, "bf16", False, "ceil", [fw.PATH_FP4_GEMV]),
    # many tile groups per persistent workgroup, with a K split that pads
    # (10 windows = 5 two-window units)
    (3, 70000, 1280, 16, "fp16", True, "ceil", [fw.PATH_FP4_GEMV]),
]


@pytest.mark.parametrize("M,N,K,bs,dtype,bias,partial,paths", FP4_CASES)
def test_fp4_matmul_parity(M, N, K, bs, dtype, bias, partial, paths):
    require_gpu()
    p = workloads.make_fp4(M, N, K, bs, dtype, seed=M * 7 + N * 3 + K, with_bias=bias, partial=partial)
    Y_ref, S = ref_fp4(p)
    d = fp4_device(p)
    for path in [fw.PATH_AUTO] + paths:
        assert_parity(run_fp4(p, d, path), dtype, Y_ref, S, f"fp4 M{M} N{N} K{K} path {path}")


def _one_hot_fp4(M, N, K, dtype, seed):
    """Row m of A is one-hot at k_m (value 1.0): Y[m, n] = RNE_T(RNE_f32(B_dq
    product at (n, k_m))) exactly."""
    p = workloads.make_fp4(M, N, K, 16, dtype, seed=seed, scale_range=(2.0 ** -9, 448.0), ws2=0.01,
                           with_bias=False)
    rng = np.random.default_rng(seed)
    ks = rng.choice(K, size=M, replace=False)
    one = 0x3F80 if dtype == "bf16" else 0x3C00
    p.A[:] = 0
    p.A[np.arange(M), ks] = one
    want = ref.dequant_fp4_output_bits(p.B, p.weight_scale, 16, p.weight_scale_2, K, dtype)[:, ks].T
    return p, want


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K,path", [
    (8, 64, 256, fw.PATH_FP4_GEMV), (5, 48, 128, fw.PATH_FP4_GEMV), (1, 32, 4096, fw.PATH_FP4_GEMV),
    (8, 64, 480, fw.PATH_FP4_GEMV), (3, 40, 160, fw.PATH_FP4_GEMV),
    (8, 300, 512, fw.PATH_FP4_GEMM), (64, 512, 1024, fw.PATH_FP4_GEMM), (16, 40, 96, fw.PATH_FP4_GENERIC),
    (13, 80, 512, fw.PATH_FP4_SKINNY), (64, 48, 1024, fw.PATH_FP4_SKINNY),
])
def test_fp4_one_hot_probe_bit_exact(M, N, K, path, dtype):
    require_gpu()
    p, want = _one_hot_fp4(M, N, K, dtype, seed=M + N + K)
    got = run_fp4(p, path=path)
    assert_bits_equal(got, want, f"one-hot fp4 path {path}", zero_sign=False)


@pytest.mark.parametrize("M,N,K,path", [
    (4, 64, 256, fw.PATH_FP4_GEMV), (8, 64, 256, fw.PATH_FP4_GEMV), (24, 64, 256, fw.PATH_FP4_SKINNY),
    (130, 520, 256, fw.PATH_FP4_GEMM),
    (4, 64, 256, fw.PATH_FP4_GENERIC),
])
def test_fp4_fp16_overflow_rounds_to_inf(M, N, K, path):
    """FP16 outputs beyond 65504 round to +-inf (round to nearest even, no
    saturation): activations of 1000, E2M1 weights of +-6 with scale 448 and
    ws2 = 1 give column sums far beyond the FP16 range, while the columns
    with mixed weights stay finite."""
    require_gpu()
    p = workloads.make_fp4(M, N, K, 16, "fp16", seed=M + N, with_bias=False)
    p.A[:] = 0x63D0                                          # fp16 1000.0
    rng = np.random.default_rng(M)
    big = rng.random(N) < 0.5
    sign = np.where(rng.random(N) < 0.5, 0x8, 0x0)
    code = (0x7 | sign).astype(np.uint8)                      # +-6
    p.B[big] = (code[big, None] | (code[big, None] << 4))
    p.weight_scale[big] = 0x7E                                # E4M3 448
    p.weight_scale[~big] = 0x08                               # E4M3 2^-6: those sums stay finite
    p.weight_scale_2 = np.float32(1.0)
    Y_ref, S = ref_fp4(p)
    got = run_fp4(p, path=path)
    inf = (got & 0x7FFF) == 0x7C00
    assert inf[:, big].all() and not inf[:, ~big].any()
    assert_parity(got, "fp16", Y_ref, S, f"fp16 overflow path {path}")


@pytest.mark.parametrize("M", [4, 7])
@pytest.mark.parametrize("K", [480, 352, 160])
def test_fp4_gemv_partial_window_masks_next_row_scales(K, M):
    """K % 128 != 0: the last 128-k window of a row reads scale bytes past the
    row's last column, which belong to the next row.  Every odd row's first
    8 scale bytes hold the E4M3 NaN code 0x7F: the odd rows' outputs are NaN
    (their own scales), and the even rows' must not be touched by them."""
    require_gpu()
    p = workloads.make_fp4(M, 96, K, 16, "bf16", seed=K + M, with_bias=True)
    p.weight_scale[1::2, :8] = 0x7F
    Y_ref, S = ref_fp4(p)
    assert np.isnan(Y_ref[:, 1::2]).all() and np.isfinite(Y_ref[:, 0::2]).all()
    for path in (fw.PATH_FP4_GEMV, fw.PATH_FP4_GENERIC):
        assert_parity(run_fp4(p, path=path), "bf16", Y_ref, S, f"fp4 K={K} NaN scales path {path}")


def test_fp4_k_zero_gives_bias():
    require_gpu()
    for dtype in ("bf16", "fp16"):
        A = torch.zeros((3, 0), dtype=torch.bfloat16 if dtype == "bf16" else torch.float16, device="cuda")
        bias = torch.randn(5, device="cuda").to(A.dtype)
        Y = fw.fp4w_matmul(A, torch.zeros((5, 0), dtype=torch.uint8, device="cuda"),
                           torch.zeros((5, 0), dtype=torch.uint8, device="cuda"),
                           torch.ones(1, device="cuda"), bias, 16)
        Y0 = fw.fp4w_matmul(A, torch.zeros((5, 0), dtype=torch.uint8, device="cuda"),
                            torch.zeros((5, 0), dtype=torch.uint8, device="cuda"),
                            torch.ones(1, device="cuda"), None, 16)
        torch.cuda.synchronize()
        assert torch.equal(Y, bias.expand(3, 5))
        assert torch.equal(Y0, torch.zeros_like(Y0))


def test_empty_outputs_are_noops():
    require_gpu()
    A = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    Y = fw.fp4w_matmul(A, torch.zeros((16, 32), dtype=torch.uint8, device="cuda"),
                       torch.zeros((16, 4), dtype=torch.uint8, device="cuda"), torch.ones(1, device="cuda"))
    assert Y.shape == (0, 16)
    A = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    Y = fw.fp4w_matmul(A, torch.zeros((0, 32), dtype=torch.uint8, device="cuda"),
                       torch.zeros((0, 4), dtype=torch.uint8, device="cuda"), torch.ones(1, device="cuda"))
    assert Y.shape == (4, 0)
    torch.cuda.synchronize()


def test_leading_dims_and_determinism():
    require_gpu()
    p = workloads.make_fp4(6, 256, 512, 16, "bf16", seed=3, with_bias=True)
    d = fp4_device(p)
    A3 = d["A"].view(2, 3, 512)
    Y3 = fw.fp4w_matmul(A3, d["B"], d["ws"], d["ws2"], d["bias"])
    Y3b = fw.fp4w_matmul(A3, d["B"], d["ws"], d["ws2"], d["bias"])
    torch.cuda.synchronize()
    assert Y3.shape == (2, 3, 256)
    assert torch.equal(Y3.view(torch.int16), Y3b.view(torch.int16))
    Y_ref, S = ref_fp4(p)
    assert_parity(dev_to_bits(Y3.reshape(6, 256)), "bf16", Y_ref, S, "leading dims")


def test_gemm_determinism_and_gemv_vs_gemm_agree():
    require_gpu()
    p = workloads.make_fp4(8, 512, 1024, 16, "bf16", seed=4, with_bias=True)
    d = fp4_device(p)
    a = run_fp4(p, d, fw.PATH_FP4_GEMM)
    b = run_fp4(p, d, fw.PATH_FP4_GEMM)
    assert np.array_equal(a, b)
    g = run_fp4(p, d, fw.PATH_FP4_GEMV)
    Y_ref, S = ref_fp4(p)
    assert_parity(a, "bf16", Y_ref, S, "gemm")
    assert_parity(g, "bf16", Y_ref, S, "gemv")


# ----------------------------------------------------------------- FP8

FP8_CASES = [
    (4, 300, 512, 128, "bf16", False, "ceil", [fw.PATH_FP8_GEMV, fw.PATH_FP8_GENERIC]),
    (1, 1000, 1280, 256, "fp16", True, "ceil", [fw.PATH_FP8_GEMV]),
    (7, 64, 384, 256, "bf16", True, "floor", [fw.PATH_FP8_GEMV, fw.PATH_FP8_GENERIC]),  # partial block
    (300, 520, 640, 128, "bf16", True, "ceil", [fw.PATH_FP8_GEMM]),
    (700, 1800, 448, 64, "fp16", False, "ceil", [fw.PATH_FP8_GEMM]),  # 24 tiles, ragged, odd K steps
    (12, 300, 512, 128, "bf16", True, "ceil", [fw.PATH_FP8_SKINNY, fw.PATH_FP8_GEMM]),
    (40, 1000, 640, 256, "fp16", False, "floor", [fw.PATH_FP8_SKINNY]),  # partial block, 3 row tiles
    (64, 100, 384, 384, "bf16", True, "ceil", [fw.PATH_FP8_SKINNY, fw.PATH_FP8_GENERIC]),
    (3, 50, 256, 128, "fp16", True, "ceil", [fw.PATH_FP8_SKINNY]),
    (20, 20000, 1024, 128, "bf16", False, "ceil", [fw.PATH_FP8_SKINNY]),
    (64, 256, 448, 64, "fp16", False, "ceil", [fw.PATH_FP8_GEMM]),
    (33, 100, 320, 128, "bf16", True, "floor", [fw.PATH_FP8_GEMM, fw.PATH_FP8_GENERIC]),  # partial block
    # GEMV: K % 128 != 0 (a last window of 80 k), block size 64 (two scale
    # blocks per 128-k window), partial final blocks in both column counts
    (5, 40, 208, 128, "bf16", True, "ceil", [fw.PATH_FP8_GEMV, fw.PATH_FP8_GENERIC]),
    (5, 40, 208, 128, "fp16", True, "floor", [fw.PATH_FP8_GEMV, fw.PATH_FP8_GENERIC]),
    (4, 1000, 512, 64, "bf16", True, "ceil", [fw.PATH_FP8_GEMV]),
    (8, 300, 5136, 64, "fp16", False, "ceil", [fw.PATH_FP8_GEMV]),
    (3, 500, 4000, 192, "bf16", True, "floor", [fw.PATH_FP8_GEMV]),
    (4, 300, 17424, 64, "bf16", True, "ceil", [fw.PATH_FP8_GEMV]),  # streamed activations
    (3, 21, 37, 16, "bf16", True, "ceil", [fw.PATH_FP8_GENERIC]),
    # GEMV activation modes: streamed from L2 (K = 17408), shallow ring (8 rows)
    (4, 300, 17408, 128, "bf16", True, "ceil", [fw.PATH_FP8_GEMV]),
    (8, 200, 5120, 128, "fp16", False, "ceil", [fw.PATH_FP8_GEMV]),
    # streamed activations, 137 windows (the K split pads), several tile
    # groups per workgroup
    (4, 5000, 17536, 128, "bf16", True, "ceil", [fw.PATH_FP8_GEMV]),
]


@pytest.mark.parametrize("M,N,K,bs,dtype,bias,partial,paths", FP8_CASES)
def test_fp8_matmul_parity(M, N, K, bs, dtype, bias, partial, paths):
    require_gpu()
    p = workloads.make_fp8(M, N, K, bs, dtype, seed=M + N + K, with_bias=bias, partial=partial)
    Y_ref, S = ref_fp8(p)
    d = fp8_device(p)
    for path in [fw.PATH_AUTO] + paths:
        assert_parity(run_fp8(p, d, path), dtype, Y_ref, S, f"fp8 M{M} N{N} K{K} path {path}")


@pytest.mark.parametrize("M,N,K,bs,path", [
    (8, 64, 512, 128, fw.PATH_FP8_GEMV), (3, 40, 384, 256, fw.PATH_FP8_GEMV),
    (8, 64, 512, 64, fw.PATH_FP8_GEMV), (4, 40, 208, 64, fw.PATH_FP8_GEMV),
    (16, 300, 512, 128, fw.PATH_FP8_GEMM), (40, 64, 208, 128, fw.PATH_FP8_GENERIC),
    (24, 64, 512, 128, fw.PATH_FP8_SKINNY), (50, 33, 640, 128, fw.PATH_FP8_SKINNY),
])
def test_fp8_one_hot_probe_bit_exact(M, N, K, bs, path):
    require_gpu()
    p = workloads.make_fp8(M, N, K, bs, "bf16", seed=M * N, scale_range=(1e-3, 10.0))
    ks = np.random.default_rng(M).choice(K, size=M, replace=False)
    p.A[:] = 0
    p.A[np.arange(M), ks] = 0x3F80
    want = ref.dequant_fp8_output_bits(p.B, p.b_scale, bs, "bf16")[:, ks].T
    got = run_fp8(p, path=path)
    assert_bits_equal(got, want, f"one-hot fp8 path {path}", zero_sign=False)


@pytest.mark.parametrize("K,bs", [(208, 128), (144, 64), (5136, 64)])
def test_fp8_gemv_partial_window_masks_next_row_weights(K, bs):
    """K % 128 != 0: the last 128-k window of a weight row reads the bytes
    past the row, which are the next row's first E4M3 codes.  Every odd row
    starts with 64 NaN codes (0x7F): the odd rows' outputs are NaN (their own
    codes), and the even rows' outputs must stay finite and within tolerance
    (the kernel zeroes the bytes past K before decoding them)."""
    require_gpu()
    p = workloads.make_fp8(4, 96, K, bs, "bf16", seed=K, with_bias=True)
    p.B[1::2, :64] = 0x7F
    Y_ref, S = ref_fp8(p)
    assert np.isnan(Y_ref[:, 1::2]).all() and np.isfinite(Y_ref[:, 0::2]).all()
    for path in (fw.PATH_FP8_GEMV, fw.PATH_FP8_GENERIC):
        assert_parity(run_fp8(p, path=path), "bf16", Y_ref, S, f"fp8 K={K} bs={bs} NaN next-row codes path {path}")


@pytest.mark.parametrize("M,K,row_powers,paths", [
    (4, 768, False, [fw.PATH_FP8_GEMV, fw.PATH_FP8_SKINNY, fw.PATH_FP8_GENERIC]),
    (40, 5120, False, [fw.PATH_FP8_SKINNY, fw.PATH_FP8_GEMM]),
    (300, 768, True, [fw.PATH_FP8_GEMM, fw.PATH_FP8_GENERIC]),
    (256, 5120, True, [fw.PATH_FP8_GEMM]),
])
def test_fp8_block_scale_exact_on_fold_breaking_inputs(M, K, row_powers, paths):
    """Inputs on which multiplying RNE_bf16(e4m3 * b_scale) instead of the
    exact B_dq fails every element (pinned on the CPU by
    test_fp8_fold_witness.py): each FP8 kernel must apply the FP32 block scale
    to an FP32 block sum ([FP8 doc] §2)."""
    require_gpu()
    A, B, s = fp8_fold_cases.fold_breaking_problem(M, K, n_cols=16, row_powers=row_powers)
    p = workloads.Fp8Problem(M, B.shape[0], K, 128, "bf16", A, B, s, None)
    Y_ref, S = ref_fp8(p)
    d = fp8_device(p)
    for path in [fw.PATH_AUTO] + paths:
        assert_parity(run_fp8(p, d, path), "bf16", Y_ref, S, f"fp8 fold-breaking M{M} K{K} path {path}")


@pytest.mark.parametrize("fp8", [False, True])
def test_gemm_activations_past_2gib(fp8):
    """M x K x 2 bytes of activations beyond 2^31 (offsets are relative to
    each tile's first row): sampled rows, including those on both sides of
    the 2 GiB boundary, against the oracle."""
    require_gpu()
    K, N = 1024, 300
    M = (1 << 31) // (2 * K) + 333
    g = torch.Generator(device="cuda").manual_seed(21)
    A = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M), (1 << 20) + np.arange(-8, 8),
                                     np.random.default_rng(21).integers(0, M, 32)]))
    A_rows = dev_to_bits(A[torch.from_numpy(rows).cuda()])
    if fp8:
        p = workloads.make_fp8(1, N, K, 128, "bf16", seed=22, with_bias=True)
        d = fp8_device(p)
        Y = fw.fp8w_matmul(A, d["B"], d["bs"], d["bias"], 128, path=fw.PATH_FP8_GEMM)
        Y_ref, S = ref.matmul_fp8_reference(A_rows, "bf16", p.B, p.b_scale, 128, p.bias)
    else:
        p = workloads.make_fp4(1, N, K, 16, "bf16", seed=22, with_bias=True)
        d = fp4_device(p)
        Y = fw.fp4w_matmul(A, d["B"], d["ws"], d["ws2"], d["bias"], 16, path=fw.PATH_FP4_GEMM)
        Y_ref, S = ref.matmul_fp4_reference(A_rows, "bf16", p.B, p.weight_scale, 16, p.weight_scale_2, p.bias)
    got = dev_to_bits(Y[torch.from_numpy(rows).cuda()])
    del A, Y
    torch.cuda.empty_cache()
    assert_parity(got, "bf16", Y_ref, S, f"gemm past 2 GiB fp8={fp8}")


# ----------------------------------------------------------------- the five workloads

def _sample_rows(M, seed, n_rand=32):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M), rng.integers(0, M, n_rand)]))


def test_workload_fp4_gemv_small():
    require_gpu()
    p = workloads.WORKLOADS["fp4_gemv_small"].make()
    Y_ref, S = ref_fp4(p)
    Y = run_fp4(p)
    r = assert_parity(Y, "fp16", Y_ref, S, "fp4_gemv_small")
    # soft expectation: FP16 output rounding dominates the relative error
    y = codecs.bits_to_f64(Y, "fp16")
    big = np.abs(Y_ref) >= 1e-2 * np.abs(Y_ref).max()
    rel = np.max(np.abs(y[big] - Y_ref[big]) / np.abs(Y_ref[big]))
    assert rel < 2 ** -10, rel


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_workload_fp4_gemv_decode(M):
    require_gpu()
    p = workloads.WORKLOADS["fp4_gemv_decode"].make(M=M)
    Y_ref, S = ref_fp4(p)
    assert_parity(run_fp4(p), "bf16", Y_ref, S, f"fp4_gemv_decode M={M}")


def test_workload_fp4_prefill_sampled_rows():
    require_gpu()
    w = workloads.WORKLOADS["fp4_prefill"]
    p = w.make()
    rows = _sample_rows(p.M, 11)
    Y = run_fp4(p)
    Y_ref, S = ref_fp4(p, rows)
    assert_parity(Y[rows], "bf16", Y_ref, S, "fp4_prefill sampled rows")


def test_workload_fp8_gemv_and_prefill():
    require_gpu()
    w = workloads.WORKLOADS["fp8_gemv"]
    p = w.make(M=4)
    Y_ref, S = ref_fp8(p)
    assert_parity(run_fp8(p), "bf16", Y_ref, S, "fp8_gemv M=4")
    p8k = w.make(M=8192)
    rows = _sample_rows(p8k.M, 12)
    Y = run_fp8(p8k)
    Y_ref, S = ref_fp8(p8k, rows)
    assert_parity(Y[rows], "bf16", Y_ref, S, "fp8 prefill sampled rows")


def test_workload_fp4_gemv_wide_full_output():
    """The wide-output GEMV (M=4, N=152064, K=5120) on every output column."""
    require_gpu()
    p = workloads.WORKLOADS["fp4_gemv_wide"].make()
    Y = run_fp4(p)
    Y_ref, S = ref_fp4(p)
    assert_parity(Y, "bf16", Y_ref, S, "fp4_gemv_wide full output")
