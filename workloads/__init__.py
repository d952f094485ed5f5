"""Seeded synthetic inputs for the weight-only FP4 / FP8 matmul.

This module only draws random inputs; it holds none of the method's
arithmetic (no decoding, scaling or accumulation).  Both the GPU tests /
benchmark and the CPU oracle take their inputs from here, and from nowhere
else.

Activations and biases are returned as raw uint16 bit patterns of type T
(FP16 or BF16), packed FP4 weights as uint8 [N, K/2], FP8 weights as uint8
[N, K], E4M3 block scales as uint8 [N, cols] and FP8 block scales as float32
[N, cols].

Recipe (one numpy Generator per problem, draws in the order
A -> B -> scales -> bias):

* A "bf16 N(0,1)": float32 standard normal, rounded to BF16 (RNE).
* A "fp16 U(-1,1)": float64 uniform, rounded to FP16 (RNE).
* FP4 B: uniform bytes 0..255, so each nibble is uniform over the 16 codes.
* E4M3 scales "U[a, b]": x ~ U[a, b) in float64, encoded to E4M3 with
  torch.float8_e4m3fn (RNE).
* FP8 B "uniform over finite E4M3 codes": uniform over the 254 bytes other
  than the two NaN codes 0x7F and 0xFF.
* FP8 b_scale: float32 U[1e-3, 1e-2].
* bias "N(0, 0.1)": standard deviation 0.1, rounded to T.

Large weight sets that are only timed (the decode-step sequence) are drawn on
the device instead (``fp4_weights_on_device``): torch's seeded device
generator, uniform bytes for B and float32 U[a, b) encoded to E4M3 for the
scales.  Same distributions, different streams of numbers; nothing checks
their products against the oracle.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass
class Fp4Problem:
    M: int
    N: int
    K: int
    block_size: int
    dtype: str                     # "bf16" | "fp16"
    A: np.ndarray                  # uint16 [M, K]
    B: np.ndarray                  # uint8  [N, K/2]
    weight_scale: np.ndarray       # uint8  [N, cols] (E4M3 bytes)
    weight_scale_2: np.float32
    bias: Optional[np.ndarray]     # uint16 [N] or None

    @property
    def scale_cols(self) -> int:
        return int(self.weight_scale.shape[1])


@dataclass
class Fp8Problem:
    M: int
    N: int
    K: int
    block_size: int
    dtype: str
    A: np.ndarray                  # uint16 [M, K]
    B: np.ndarray                  # uint8  [N, K] (E4M3 bytes)
    b_scale: np.ndarray            # float32 [N, cols]
    bias: Optional[np.ndarray]

    @property
    def scale_cols(self) -> int:
        return int(self.b_scale.shape[1])


# ---------------------------------------------------------------- primitives

def _to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp16":
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def activations(rng: np.random.Generator, M: int, K: int, dtype: str, dist: str) -> np.ndarray:
    if dist == "normal":
        x = rng.standard_normal((M, K), dtype=np.float32)
    elif dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=(M, K))
    else:
        raise ValueError(dist)
    return _to_bits(x, dtype)


def fp4_weights(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    return rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)


def fp8_weights(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
    return finite[rng.integers(0, finite.size, size=(N, K))]


def e4m3_scale_bytes(rng: np.random.Generator, N: int, cols: int, lo: float, hi: float) -> np.ndarray:
    x = rng.uniform(lo, hi, size=(N, cols))
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp32_scales(rng: np.random.Generator, N: int, cols: int, lo: float, hi: float) -> np.ndarray:
    return rng.uniform(lo, hi, size=(N, cols)).astype(np.float32)


def bias_bits(rng: np.random.Generator, N: int, dtype: str, std: float = 0.1) -> np.ndarray:
    return _to_bits((std * rng.standard_normal(N)).astype(np.float32), dtype)


def scale_cols_for(K: int, block_size: int, partial: str = "ceil") -> int:
    """Number of scale columns: ceil(K/bs) (the partial block has its own
    column) or floor(K/bs) (the tail reuses the last full block's column)."""
    if partial == "ceil":
        return -(-K // block_size)
    if partial == "floor":
        return max(1, K // block_size)
    raise ValueError(partial)


# ---------------------------------------------------------------- problems

def make_fp4(M: int, N: int, K: int, block_size: int = 16, dtype: str = "bf16", seed: int = 0,
             a_dist: str = "normal", scale_range=(2.0 ** -6, 4.0), ws2: float = 2.0 ** -8,
             with_bias: bool = True, partial: str = "ceil") -> Fp4Problem:
    rng = np.random.default_rng(seed)
    A = activations(rng, M, K, dtype, a_dist)
    B = fp4_weights(rng, N, K)
    cols = scale_cols_for(K, block_size, partial)
    ws = e4m3_scale_bytes(rng, N, cols, *scale_range)
    bias = bias_bits(rng, N, dtype) if with_bias else None
    return Fp4Problem(M, N, K, block_size, dtype, A, B, ws, np.float32(ws2), bias)


def make_fp8(M: int, N: int, K: int, block_size: int = 128, dtype: str = "bf16", seed: int = 0,
             a_dist: str = "normal", scale_range=(1e-3, 1e-2), with_bias: bool = False,
             partial: str = "ceil") -> Fp8Problem:
    rng = np.random.default_rng(seed)
    A = activations(rng, M, K, dtype, a_dist)
    B = fp8_weights(rng, N, K)
    cols = scale_cols_for(K, block_size, partial)
    bs = fp32_scales(rng, N, cols, *scale_range)
    bias = bias_bits(rng, N, dtype) if with_bias else None
    return Fp8Problem(M, N, K, block_size, dtype, A, B, bs, bias)


@dataclass
class Workload:
    """One of the five benchmark workloads, by name, with its sizes."""
    name: str
    op: str                        # "fp4" | "fp8"
    Ms: tuple
    N: int
    K: int
    block_size: int
    dtype: str
    a_dist: str
    scale_range: tuple
    ws2: float = 2.0 ** -8
    with_bias: bool = False
    index: int = 0
    notes: str = field(default="")

    def make(self, M: Optional[int] = None, seed: Optional[int] = None):
        M = self.Ms[0] if M is None else M
        seed = 1000 + self.index if seed is None else seed
        if self.op == "fp4":
            return make_fp4(M, self.N, self.K, self.block_size, self.dtype, seed, self.a_dist,
                            self.scale_range, self.ws2, self.with_bias)
        return make_fp8(M, self.N, self.K, self.block_size, self.dtype, seed, self.a_dist,
                        self.scale_range, self.with_bias)


WORKLOADS = {
    # small FP16 GEMV with a non-power-of-two tensor scale (parity case)
    "fp4_gemv_small": Workload("fp4_gemv_small", "fp4", (1,), 256, 512, 16, "fp16", "uniform",
                               (2.0 ** -4, 4.0), ws2=0.01, with_bias=False, index=0),
    # decode GEMV, N = K = 5120
    "fp4_gemv_decode": Workload("fp4_gemv_decode", "fp4", (1, 2, 4, 8), 5120, 5120, 16, "bf16",
                                "normal", (2.0 ** -6, 4.0), with_bias=True, index=1),
    # prefill GEMM, 8192 tokens, N = 17408, K = 5120
    "fp4_prefill": Workload("fp4_prefill", "fp4", (8192,), 17408, 5120, 16, "bf16", "normal",
                            (2.0 ** -6, 4.0), with_bias=False, index=2),
    # FP8 E4M3 weight GEMV (M = 4) and the same weights at prefill M = 8192
    "fp8_gemv": Workload("fp8_gemv", "fp8", (4, 8192), 17408, 5120, 128, "bf16", "normal",
                         (1e-3, 1e-2), with_bias=False, index=3),
    # wide-output GEMV (lm_head-like), N = 152064
    "fp4_gemv_wide": Workload("fp4_gemv_wide", "fp4", (4,), 152064, 5120, 16, "bf16", "normal",
                              (2.0 ** -6, 4.0), with_bias=False, index=4),
}


def fp4_weights_on_device(N: int, K: int, block_size: int = 16, seed: int = 0,
                          scale_range=(2.0 ** -6, 4.0), device="cuda"):
    """(B uint8 [N, K/2], E4M3 scale bytes uint8 [N, ceil(K/bs)]) drawn on the
    device with a seeded torch generator (see the module docstring)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    B = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=device, generator=g)
    cols = scale_cols_for(K, block_size)
    x = torch.empty(N, cols, dtype=torch.float32, device=device).uniform_(*scale_range, generator=g)
    return B, x.to(torch.float8_e4m3fn).view(torch.uint8)


# A decode step as a sequence of back-to-back FP4 GEMV launches: 121 launches
# at M = 4 with FP16 activations, the launch count and batch of the pages'
# per-step figure ("MatMulBlockQuantizedFp4Weight - CUDA Operator
# Documentation", §4, tensor-core sub-path).  The pages do not give the
# shapes of those launches.  Taken here: 40 repetitions of three projections
# over the widths of the workloads above (5120 -> 5120, 5120 -> 17408,
# 17408 -> 5120), then one more 5120 -> 5120, each launch with weights of its
# own (about 4.6 GB per step, far beyond the last-level cache).
DECODE_STEP_M = 4
DECODE_STEP_SHAPES = tuple([(5120, 5120), (17408, 5120), (5120, 17408)] * 40 + [(5120, 5120)])  # (N, K)
