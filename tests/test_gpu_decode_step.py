"""GPU checks of the decode-step sequence: 121 back-to-back FP4 GEMV launches
at M = 4 with FP16 activations ("MatMulBlockQuantizedFp4Weight - CUDA
Operator Documentation", §4, tensor-core sub-path, per-step figure), the
sequence the benchmark replays from one HIP graph.

* Each distinct shape of the sequence against the oracle (sampled columns).
* The full-size sequence replayed from a graph, several times with eager
  work and synchronisation between the replays: every replay bit-identical
  to the same launches issued eagerly, and sampled launches of it against
  the oracle.
"""

import numpy as np
import pytest
import torch

import fp8_weight_only_fp4w_amd as fw
import workloads
from gpu_helpers import assert_bits_equal, assert_parity, bits_to_dev, dev_to_bits, ref_fp4, require_gpu

pytestmark = pytest.mark.gpu

M = workloads.DECODE_STEP_M


def _column_subproblem(p, cols):
    return workloads.Fp4Problem(p.M, cols.size, p.K, p.block_size, p.dtype, p.A, p.B[cols],
                                p.weight_scale[cols], p.weight_scale_2, None)


def _cols(N, seed, n=1024):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(256), np.arange(N - 256, N), rng.integers(0, N, n)]))


@pytest.mark.parametrize("N,K", sorted(set(workloads.DECODE_STEP_SHAPES)))
def test_decode_step_shapes_parity(N, K):
    require_gpu()
    p = workloads.make_fp4(M, N, K, 16, "fp16", seed=N + K, a_dist="uniform", with_bias=False)
    d = dict(A=bits_to_dev(p.A, "fp16"), B=torch.from_numpy(p.B).cuda(),
             ws=torch.from_numpy(p.weight_scale).cuda(),
             ws2=torch.tensor([p.weight_scale_2], dtype=torch.float32, device="cuda"))
    assert fw.fp4w_select_path(fw.OP_FP4_MATMUL, M, N, K, 16, K // 16) == fw.PATH_FP4_GEMV
    Y = fw.fp4w_matmul(d["A"], d["B"], d["ws"], d["ws2"], None, 16)
    torch.cuda.synchronize()
    cols = _cols(N, K)
    Y_ref, S = ref_fp4(_column_subproblem(p, cols))
    assert_parity(dev_to_bits(Y)[:, cols], "fp16", Y_ref, S, f"decode step N{N} K{K}")


def test_decode_step_graph_replays_match_eager_and_oracle():
    require_gpu()
    shapes = workloads.DECODE_STEP_SHAPES
    ws2_val = np.float32(2.0 ** -8)
    ws2 = torch.tensor([ws2_val], dtype=torch.float32, device="cuda")
    W = [workloads.fp4_weights_on_device(N, K, 16, seed=7000 + i) for i, (N, K) in enumerate(shapes)]
    A_bits = {K: workloads.activations(np.random.default_rng(K), M, K, "fp16", "uniform")
              for K in sorted({K for _, K in shapes})}
    A = {K: bits_to_dev(b, "fp16") for K, b in A_bits.items()}
    outs = [torch.empty(M, N, dtype=torch.float16, device="cuda") for N, _ in shapes]

    def step():
        for (N, K), (B, ws), o in zip(shapes, W, outs):
            fw.fp4w_matmul(A[K], B, ws, ws2, None, 16, out=o)

    step()
    torch.cuda.synchronize()
    eager = [dev_to_bits(o) for o in outs]

    # a few launches of the eager result against the oracle (sampled columns)
    for i in (0, 1, 2, len(shapes) - 1):
        N, K = shapes[i]
        cols = _cols(N, 100 + i, 512)
        B, ws = W[i]
        p = workloads.Fp4Problem(M, N, K, 16, "fp16", A_bits[K], B.cpu().numpy(), ws.cpu().numpy(), ws2_val, None)
        Y_ref, S = ref_fp4(_column_subproblem(p, cols))
        assert_parity(eager[i][:, cols], "fp16", Y_ref, S, f"decode step launch {i} N{N} K{K}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:  # eager work between replays: poison every output with NaN
            o.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert_bits_equal(dev_to_bits(o), eager[i], f"graph replay {rep}, launch {i} {shapes[i]}")
    del g
