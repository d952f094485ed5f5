"""A seeded sweep of shapes through the default dispatch of fp4w_matmul and
fp8w_matmul, each against the oracle on the full output: M across the GEMV,
skinny and GEMM ranges, ragged N, K with and without whole 32-k, 128-k and
scale blocks, block sizes off the fast paths' values (which the generic
kernels take), both scale-column rules, both activation types, with and
without bias.  The cases are drawn once from a fixed seed, so the set is the
same on every run."""

import numpy as np
import pytest

import workloads
from gpu_helpers import assert_parity, ref_fp4, ref_fp8, require_gpu, run_fp4, run_fp8

pytestmark = pytest.mark.gpu

MAX_MACS = 3e7  # keeps the oracle at well under a second per case


def _draw_m(rng):
    r = rng.random()
    if r < 0.5:
        return int(rng.integers(1, 9))     # decode GEMV
    if r < 0.8:
        return int(rng.integers(9, 65))    # skinny
    return int(rng.integers(65, 300))      # GEMM


def _draw_k(rng, quantum, kmax):
    return quantum * int(rng.integers(1, max(1, kmax // quantum) + 1))


def _cases(kind, count, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        M = _draw_m(rng)
        N = int(rng.integers(1, 1600))
        kmax = int(min(12000, MAX_MACS // (M * N)))
        if kind == "fp4":
            K = _draw_k(rng, int(rng.choice([2, 16, 32, 128])), kmax)
            bs = 16 if rng.random() < 0.75 else int(rng.choice([7, 8, 24, 32]))
        else:
            K = _draw_k(rng, int(rng.choice([1, 16, 64, 128])), kmax)
            bs = int(rng.choice([128, 128, 64, 16, 256, 48, 5]))
        if M * N * K > MAX_MACS:
            continue
        partial = "floor" if (K % bs != 0 and K // bs >= 1 and rng.random() < 0.5) else "ceil"
        dtype = "bf16" if rng.random() < 0.5 else "fp16"
        bias = bool(rng.random() < 0.5)
        out.append((M, N, K, bs, dtype, bias, partial))
    return out


FP4_SWEEP = _cases("fp4", 96, 20261202)
FP8_SWEEP = _cases("fp8", 64, 20261203)


@pytest.mark.parametrize("M,N,K,bs,dtype,bias,partial", FP4_SWEEP)
def test_fp4_sweep(M, N, K, bs, dtype, bias, partial):
    require_gpu()
    p = workloads.make_fp4(M, N, K, bs, dtype, seed=M * 7 + N * 3 + K, with_bias=bias, partial=partial)
    Y_ref, S = ref_fp4(p)
    assert_parity(run_fp4(p), dtype, Y_ref, S, f"fp4 sweep M{M} N{N} K{K} bs{bs} {dtype} {partial}")


@pytest.mark.parametrize("M,N,K,bs,dtype,bias,partial", FP8_SWEEP)
def test_fp8_sweep(M, N, K, bs, dtype, bias, partial):
    require_gpu()
    p = workloads.make_fp8(M, N, K, bs, dtype, seed=M * 5 + N * 11 + K, with_bias=bias, partial=partial)
    Y_ref, S = ref_fp8(p)
    assert_parity(run_fp8(p), dtype, Y_ref, S, f"fp8 sweep M{M} N{N} K{K} bs{bs} {dtype} {partial}")
