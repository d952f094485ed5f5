"""CPU oracle for block-scaled weight-only FP4 / FP8 matmul.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
CPU reference of what the GPU library computes.  It exists to check the GPU
path and nothing else: only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it.  The GPU library never calls it
and shares no code with it (no kernels, headers, tables or helpers).

Sources (web pages; cited by title and section throughout):

* [FP4 doc]  "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
             (ONNX Runtime 1.29.0 contrib-op docs).
* [FP8 doc]  "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"
             (ONNX Runtime contrib-op docs).
* [Blog]     "ONNX Runtime #32128 - Why Dequantizing 4-Bit Weights Became the
             Most Expensive Kernel in H200 Prefill" (Part 1 of 3).

Arithmetic: every value the method defines is formed exactly in float64
(E2M1 x E4M3 x FP32 needs at most 2 + 4 + 24 = 30 significand bits) and the
matmul accumulates in float64 with numpy's dgemm.  The only roundings are the
ones the method itself prescribes for the stored FP16/BF16 dequant output.

Pins (tests/test_oracle_*.py, run with -m "not gpu"):

* ``codecs.e4m3fn_value``        all 256 codes vs torch.float8_e4m3fn and the
                                 landmarks the pages print (max 448, 2^-9).
* ``codecs.e2m1_value``          all 16 codes vs the landmarks the pages print
                                 (max 6, min 0.5, 2 significand bits, -0.0 at
                                 code 0x8) plus monotonicity / sign symmetry.
* ``codecs.f32_to_f16_bits`` /
  ``codecs.f32_to_bf16_bits``    exhaustive f16 round trips, all ties, and
                                 torch's independent CPU conversions.
* ``reference.unpack_e2m1_codes`` the page's nibble order (low = even k) on
                                 all 256 bytes.
* ``reference.scale_column``     the pages' block examples (bs 16, bs 15) and
                                 the FP8 partial-final-block rule.
* ``reference.dequant_*``        exhaustive byte x scale-byte x ws2 sweep vs
                                 torch float32 arithmetic.
* ``reference.matmul_*``         exact rational brute force on tiny shapes,
                                 the unit-scale special case vs torch.matmul,
                                 and invariants (K-block permutation, sign
                                 flip, ws2 doubling, bias shift).
* ``reference.matmul_tolerance`` exact result passes, perturbed result fails.
* ``nvfp4.*``                    (the W4A4 path of [FP4 doc] §6) hand-derived
                                 blocks (tests/golden), a brute-force E2M1
                                 nearest-value search, exact round trips of
                                 representable activations, the quantization
                                 error bound, block independence, NaN / inf
                                 confinement, and exact rational W4A4 sums.

No function here is "parity unpinned".
"""

from .codecs import (  # noqa: F401
    E2M1_TABLE,
    E4M3FN_TABLE,
    activation_to_f64,
    e2m1_value,
    e4m3fn_value,
    f32_to_bf16_bits,
    f32_to_f16_bits,
    bits_to_f64,
)
from .reference import (  # noqa: F401
    check_matmul,
    dequant_fp4_f64,
    dequant_fp4_output_bits,
    dequant_fp8_f64,
    dequant_fp8_output_bits,
    matmul_fp4_reference,
    matmul_fp8_reference,
    matmul_tolerance,
    scale_column,
    unpack_e2m1_codes,
)
from .nvfp4 import (  # noqa: F401
    e2m1_encode,
    matmul_w4a4_reference,
    qdq_activation_nvfp4_bits,
    quantize_activation_nvfp4,
)
