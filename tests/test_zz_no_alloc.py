"""The allocation-free W4A4 entry point, fp4w_matmul_w4a4_noalloc (the NVFP4
activation staged in the library's own device scratch), against
fp4w_matmul_w4a4 with a caller workspace: bit-identical outputs on calls in a
row, each smaller than the one before, so that every call reads only what it
wrote itself; and a size past the scratch rejected without a launch."""

import numpy as np
import pytest
import torch

import fp8_weight_only_fp4w_amd as fw
import workloads
from gpu_helpers import dev_to_bits, fp4_device, require_gpu

pytestmark = pytest.mark.gpu

# M, N, K, dtype: a prefill-sized call (GEMM), a batched-decode one (skinny),
# then a decode one (GEMV)
CALLS = [
    (300, 1000, 2048, "bf16"),
    (24, 700, 1024, "bf16"),
    (4, 300, 512, "fp16"),
]


def test_noalloc_matches_workspace_variant():
    require_gpu()
    for M, N, K, dtype in CALLS:
        p = workloads.make_fp4(M, N, K, 16, dtype, seed=M + 3 * N + 7 * K, with_bias=True)
        d = fp4_device(p)
        ws = torch.empty_like(d["A"])
        y_ws = fw.fp4w_matmul_w4a4(d["A"], d["B"], d["ws"], d["ws2"], d["bias"], 16, workspace=ws)
        y_na = fw.fp4w_matmul_w4a4_noalloc(d["A"], d["B"], d["ws"], d["ws2"], d["bias"], 16)
        torch.cuda.synchronize()
        a, b = dev_to_bits(y_ws), dev_to_bits(y_na)
        assert np.array_equal(a, b), f"M{M} N{N} K{K} {dtype}: {np.count_nonzero(a != b)} outputs differ"
        # A itself is left as it was: the scratch holds its quantized copy
        assert np.array_equal(dev_to_bits(d["A"]), p.A)


def test_noalloc_rejects_sizes_past_the_scratch():
    require_gpu()
    K = 4096
    M = fw.STATIC_SCRATCH_BYTES // (2 * K) + 1
    A = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(16, K // 2, dtype=torch.uint8, device="cuda")
    S = torch.full((16, K // 16), 0x38, dtype=torch.uint8, device="cuda")
    ws2 = torch.ones(1, dtype=torch.float32, device="cuda")
    out = torch.full((M, 16), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fw.FP4WError) as e:
        fw.fp4w_matmul_w4a4_noalloc(A, B, S, ws2, None, 16, out=out)
    assert e.value.status == fw.ERR_SHAPE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was launched
