"""CPU pin of the adversarial FP8 inputs (tests/fp8_fold_cases.py): on every
element, a kernel that folds the FP32 block scale into BF16 weights fails the
acceptance check, while the exact result passes.  This is what gives the GPU
test on the same inputs (test_gpu_matmul.py) its power to tell the two apart
([FP8 doc] §2: B_dq = e4m3 * b_scale, b_scale FP32)."""

import numpy as np
import pytest

import fp8_fold_cases as fc
from oracle import codecs, reference as ref


@pytest.mark.parametrize("M,K,row_powers", [(4, 768, False), (300, 768, True), (256, 5120, True)])
def test_fold_fails_exact_passes(M, K, row_powers):
    A, B, s = fc.fold_breaking_problem(M, K, n_cols=16, row_powers=row_powers)
    assert B.shape == (16, K) and (B > 0).all() and (B < 0x7F).all()
    assert fc.fold_fails(A, B, s, 128).all()
    Y_ref, S = ref.matmul_fp8_reference(A, "bf16", B, s, 128)
    exact_bits = codecs.f32_to_bf16_bits(Y_ref.astype(np.float32))
    assert ref.check_matmul(exact_bits, "bf16", Y_ref, S)["ok"]
