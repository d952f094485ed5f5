"""Adversarial FP8 inputs: columns on which folding the FP32 block scale into a
BF16 operand leaves the acceptance band.

[FP8 doc] §2 defines B_dq = e4m3 * b_scale with an FP32 b_scale.  A kernel
that multiplies RNE_bf16(RNE_f32(e4m3 * b_scale)) instead of B_dq rounds each
weight by up to 2^-8 relative.  With positive activations and one code per
column, every product of a column errs in the same direction, so the sum errs
by the same relative amount, which for the codes chosen here exceeds the
3e-3 relative band of a same-sign sum (2e-3 * S + 1e-3 * |Y_ref|, S = Y_ref).

Column n holds one E4M3 code c_n in every k and one b_scale s_n in every
block.  (s_n, c_n) come from seeded candidate scales in [1e-3, 1e-2) (the FP8
workload's range): for each candidate, the positive finite code whose BF16
fold has the largest relative error, kept only when the folded sum fails the
oracle's check.  Every activation row is one power of two repeated (all 1.0,
or per row one of 0.5, 1, 2, 4), so a column's folded sum in row m is
2^e_m * K * fold(c_n): exact in FP32 in any order (8 + 13 significand bits
for K <= 8192), and a power-of-two multiple of row 0's, so it fails the
check in every row when it fails in one.
Test infrastructure: only the tests use it.
"""

import numpy as np

from oracle import codecs, reference as ref

BF16_ONE = 0x3F80


def _fold_f64(codes, s32):
    """RNE_bf16(RNE_f32(e4m3 * s)) as float64."""
    exact = codecs.E4M3FN_TABLE[codes] * np.float64(s32)
    return codecs.bits_to_f64(codecs.f32_to_bf16_bits(exact.astype(np.float32)), "bf16")


def folded_sums(A_bits, B, b_scale, block_size):
    """sum_k A * RNE_bf16(RNE_f32(e4m3 * b_scale)) in float64 [M, N]: what a
    kernel that folds the scale into BF16 weights accumulates."""
    K = B.shape[1]
    cols = ref.scale_column(K, block_size, b_scale.shape[1])
    W = np.empty(B.shape, dtype=np.float64)
    for n in range(B.shape[0]):
        for j in range(b_scale.shape[1]):
            sel = cols == j
            W[n, sel] = _fold_f64(B[n, sel], b_scale[n, j])
    return codecs.bits_to_f64(A_bits, "bf16") @ W.T


def fold_fails(A_bits, B, b_scale, block_size):
    """Per element: does the folded result (exact sum, one rounding to BF16)
    fail the oracle's check?"""
    Y_ref, S = ref.matmul_fp8_reference(A_bits, "bf16", B, b_scale, block_size)
    F = folded_sums(A_bits, B, b_scale, block_size)
    r = codecs.f32_to_bf16_bits(F.astype(np.float32))
    bad = np.zeros(F.shape, dtype=bool)
    for m in range(F.shape[0]):
        for n in range(F.shape[1]):
            bad[m, n] = not ref.check_matmul(r[m:m + 1, n:n + 1], "bf16", Y_ref[m:m + 1, n:n + 1],
                                             S[m:m + 1, n:n + 1])["ok"]
    return bad


def fold_breaking_problem(M, K, block_size=128, n_cols=16, row_powers=False, seed=0):
    """(A bits [M, K], B [N, K], b_scale [N, K // block_size]): N = n_cols
    columns, on each of which the BF16 fold fails the acceptance check in
    every row.  row_powers: row m of A is 0.5, 1, 2 or 4 (seeded) instead of
    1.0."""
    rng = np.random.default_rng(seed)
    A = np.full((M, K), BF16_ONE, dtype=np.uint16)
    if row_powers:
        A[:] = rng.choice(np.array([0x3F00, BF16_ONE, 0x4000, 0x4080], dtype=np.uint16), size=(M, 1))
    codes = np.arange(1, 0x7F, dtype=np.uint8)  # positive finite E4M3 codes
    cols = K // block_size
    picked_B, picked_s = [], []
    for s in rng.uniform(1e-3, 1e-2, size=4000).astype(np.float32):
        exact = codecs.E4M3FN_TABLE[codes] * np.float64(s)
        rel = (_fold_f64(codes, s) - exact) / exact
        Bn = np.full((1, K), codes[int(np.argmax(rel))], dtype=np.uint8)
        sn = np.full((1, cols), s, dtype=np.float32)
        if fold_fails(np.full((1, K), BF16_ONE, dtype=np.uint16), Bn, sn, block_size).all():
            picked_B.append(Bn)
            picked_s.append(sn)
            if len(picked_B) == n_cols:
                break
    assert len(picked_B) == n_cols, "not enough fold-breaking columns among the candidates"
    return A, np.concatenate(picked_B), np.concatenate(picked_s)
