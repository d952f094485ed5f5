/*
 * fp4w.h - block-scaled weight-only FP4 / FP8 matmul for AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; the library never allocates, frees or
 * synchronises (fp4w_matmul_w4a4_noalloc uses a device array that is part of
 * the library's code object).  Every call validates its arguments, enqueues its kernel(s) on
 * `stream` (a hipStream_t, NULL = the default stream) and returns.  Faults in a
 * kernel surface at the caller's next synchronisation.
 *
 * Sources, cited by page title and section:
 *   [FP4 doc] "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
 *             (ONNX Runtime 1.29.0 contrib-op docs)
 *   [FP8 doc] "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"
 *   [Blog]    "ONNX Runtime #32128 - Why Dequantizing 4-Bit Weights Became the
 *             Most Expensive Kernel in H200 Prefill"
 *
 * Common conventions
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major
 *     and contiguous.  Scalars passed by pointer (weight_scale_2) are device
 *     pointers too: the kernel reads the value, so no host sync is needed.
 *   - T (dtype) is FP16 or BF16 and is the type of A, bias and Y ([FP8 doc] §1
 *     type constraints; [FP4 doc] §1: Y has A's type).  M is the product of
 *     A's leading dimensions; Y is [M, N].
 *   - Scale column of element k: min(k / block_size, scale_cols - 1).  A
 *     partial final K block therefore uses the last scale column ([FP8 doc]
 *     §2); scale_cols may be ceil(K / block_size) or, when K % block_size != 0,
 *     floor(K / block_size) >= 1.  The same rule applies to FP4.
 *   - M == 0 or N == 0: returns FP4W_OK and launches nothing ([FP4 doc] §3,
 *     empty output).  K == 0: Y = bias, or 0 without bias (an empty sum).
 *   - Y must not overlap any input (FP4W_ERR_ALIAS).
 *   - Unaligned pointers or shapes outside a fast kernel's predicate run the
 *     generic kernel; correctness never depends on the fast path.
 *   - Accumulation is FP32.  The result is rounded once to T (round to
 *     nearest even) after the tensor scale and bias are applied.
 *   - Re-entrant and stateless; calls on different streams may overlap
 *     (except fp4w_matmul_w4a4_noalloc calls on one device, which share that
 *     device's scratch).
 */
#ifndef FP4W_H
#define FP4W_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FP4W_F16 = 0, FP4W_BF16 = 1 } fp4w_dtype;

typedef enum {
  FP4W_OK = 0,
  FP4W_ERR_NULL = -1,   /* a required pointer is NULL */
  FP4W_ERR_SHAPE = -2,  /* negative size, odd K for FP4, bad scale_cols, size overflow */
  FP4W_ERR_DTYPE = -3,  /* dtype is not FP4W_F16 / FP4W_BF16 */
  FP4W_ERR_BLOCK = -4,  /* block_size < 1 */
  FP4W_ERR_PATH = -5,   /* a forced path (the *_ex calls) does not apply to these arguments */
  FP4W_ERR_LAUNCH = -6, /* HIP reported an error when the kernel was enqueued */
  FP4W_ERR_ALIAS = -7   /* the output overlaps an input */
} fp4w_status;

/* Kernel paths.  FP4W_PATH_AUTO picks the fastest applicable one. */
typedef enum {
  FP4W_PATH_AUTO = 0,
  FP4W_PATH_NONE = 1,            /* empty output: nothing launched */
  FP4W_PATH_FP4_GEMV = 2,        /* MFMA decode GEMV: 1 <= M <= 8, block_size 16, K % 32 == 0 */
  FP4W_PATH_FP4_GEMM = 3,        /* fused MFMA prefill GEMM: block_size 16, K % 64 == 0 */
  FP4W_PATH_FP4_GENERIC = 4,     /* any legal FP4 arguments */
  FP4W_PATH_FP8_GEMV = 5,        /* MFMA decode GEMV: 1 <= M <= 8, block_size % 64 == 0, K % 16 == 0 */
  FP4W_PATH_FP8_GEMM = 6,        /* MFMA prefill GEMM: block_size % 64 == 0, K % 64 == 0 */
  FP4W_PATH_FP8_GENERIC = 7,     /* any legal FP8 arguments */
  FP4W_PATH_DEQUANT_VEC = 8,     /* vectorised dequant: K % 8 == 0, block_size % 8 == 0 */
  FP4W_PATH_DEQUANT_GENERIC = 9, /* any legal dequant arguments */
  FP4W_PATH_QDQ_VEC = 10,        /* vectorised activation QDQ: M*K % 8 == 0 */
  FP4W_PATH_QDQ_GENERIC = 11,    /* any legal QDQ arguments */
  FP4W_PATH_FP4_SKINNY = 12,     /* MFMA skinny matmul: 1 <= M <= 64, block_size 16, K % 128 == 0 */
  FP4W_PATH_FP8_SKINNY = 13,     /* MFMA skinny matmul: 1 <= M <= 64, block_size % 128 == 0, K % 128 == 0 */
  FP4W_PATH_FP8_DEQUANT_VEC = 14,    /* vectorised FP8 dequant: K % 16 == 0, block_size % 16 == 0 */
  FP4W_PATH_FP8_DEQUANT_GENERIC = 15, /* any legal FP8 dequant arguments */
  FP4W_PATH_NVFP4_VEC = 16,     /* NVFP4 activation quantize / QDQ, 16-byte loads (aligned pointers) */
  FP4W_PATH_NVFP4_GENERIC = 17  /* any legal NVFP4 activation arguments */
} fp4w_path;

/* Operation selector for fp4w_select_path. */
typedef enum {
  FP4W_OP_FP4_MATMUL = 0,
  FP4W_OP_FP8_MATMUL = 1,
  FP4W_OP_FP4_DEQUANT = 2,
  FP4W_OP_FP8_QDQ = 3, /* fp8w_qdq_activation: only M and K are used */
  FP4W_OP_FP8_DEQUANT = 4, /* fp8w_dequant: M is ignored */
  FP4W_OP_NVFP4_ACT = 5 /* fp4w_quantize_activation / fp4w_qdq_activation: only M and K are used */
} fp4w_op;

/*
 * fp4w_matmul - weight-only FP4 matmul, Y = A * dequant(B)^T (+ bias).
 * [FP4 doc] header and §2 Weight Format:
 *   B_dq[n, k] = e2m1(B[n, k]) * e4m3(weight_scale[n, k / block_size]) * weight_scale_2
 *
 *   A              T[M, K]
 *   B              uint8[N, K/2]: two E2M1 codes per byte, low nibble = even k,
 *                  high nibble = odd k.  K must be even.
 *   weight_scale   uint8[N, scale_cols]: raw E4M3 ("fn") bytes, unswizzled.
 *   weight_scale_2 device float*: FP32 tensor scale.
 *   bias           T[N] or NULL.
 *   Y              T[M, N] (written).
 * Errors: FP4W_ERR_NULL (A, B, weight_scale, weight_scale_2 or Y NULL while
 * M, N > 0), FP4W_ERR_SHAPE, FP4W_ERR_BLOCK, FP4W_ERR_DTYPE, FP4W_ERR_ALIAS,
 * FP4W_ERR_LAUNCH.  Nothing is launched when an error is returned.
 */
int fp4w_matmul(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                const uint8_t* weight_scale, int64_t scale_cols, int64_t block_size,
                const float* weight_scale_2, const void* bias, void* Y, int dtype, void* stream);

/* Same as fp4w_matmul, with the kernel path forced (FP4W_PATH_AUTO, _FP4_GEMV,
 * _FP4_SKINNY, _FP4_GEMM or _FP4_GENERIC).  FP4W_ERR_PATH if the path does not
 * apply. */
int fp4w_matmul_ex(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                   const uint8_t* weight_scale, int64_t scale_cols, int64_t block_size,
                   const float* weight_scale_2, const void* bias, void* Y, int dtype, void* stream,
                   int path);

/*
 * fp8w_matmul - weight-only FP8 matmul ([FP8 doc] §2 Tensor and Scale Format):
 *   Y[m, n] = sum_k A[m, k] * (e4m3(B[n, k]) * b_scale[n, k / block_size]) + bias[n]
 *
 *   A        T[M, K]
 *   B        uint8[N, K]: E4M3 ("fn") bytes.
 *   b_scale  float[N, scale_cols]: FP32 block scales.
 *   bias     T[N] or NULL.   Y  T[M, N].
 * Errors as fp4w_matmul (no evenness rule on K).
 */
int fp8w_matmul(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                const float* b_scale, int64_t scale_cols, int64_t block_size, const void* bias,
                void* Y, int dtype, void* stream);

/* Path-forcing variant (FP4W_PATH_AUTO, _FP8_GEMV, _FP8_SKINNY, _FP8_GEMM,
 * _FP8_GENERIC). */
int fp8w_matmul_ex(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                   const float* b_scale, int64_t scale_cols, int64_t block_size, const void* bias,
                   void* Y, int dtype, void* stream, int path);

/*
 * fp4w_quantize_activation - step 1 of the FP4 operator's native FP4 x FP4
 * (W4A4) path ([FP4 doc] §6 Native SM120 FP4 x FP4 Path): the activation as
 * packed E2M1 codes with one E4M3 scale per 16-element block (NVFP4).  The
 * pages name the format but no rounding rule; this library uses, per block
 * of 16 consecutive k of one row:
 *   scale = e4m3( min( RNE_f32(amax / 6), 448 ) )   (NaN in the block -> NaN, 0x7F)
 *   code  = e2m1( RNE_f32(a / scale) )               (scale == 0 -> code 0)
 * amax = max |a|; both divisions are IEEE FP32 divisions; e4m3 and e2m1 give
 * the nearest value with ties to the even code; e2m1 saturates at 6 and keeps
 * the sign (a negative quotient rounding to zero gives code 0x8); a NaN
 * quotient gives code 0.  Bit-exact.
 *
 *   A       T[M, K], K % 16 == 0.
 *   codes   uint8[M, K/2] (written): two codes per byte, low nibble = even k
 *           (the weight layout of [FP4 doc] §2).
 *   scales  uint8[M, K/16] (written): E4M3 "fn" bytes.
 * M == 0 or K == 0: FP4W_OK, nothing launched.  Errors: FP4W_ERR_NULL,
 * FP4W_ERR_SHAPE (negative sizes, K % 16 != 0, overflow), FP4W_ERR_DTYPE,
 * FP4W_ERR_ALIAS (codes or scales overlap A or each other),
 * FP4W_ERR_LAUNCH.
 */
int fp4w_quantize_activation(const void* A, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                             int dtype, void* stream);

/* Path-forcing variant (FP4W_PATH_AUTO, _NVFP4_VEC, _NVFP4_GENERIC). */
int fp4w_quantize_activation_ex(const void* A, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                                int dtype, void* stream, int path);

/*
 * fp4w_qdq_activation - the same quantization, decoded back to T:
 *   out[m, k] = e2m1(code) * e4m3(scale)
 * which is exact in FP16 and BF16 (at most 6 significand bits; nonzero
 * magnitudes within [2^-10, 2688]); NaN where the block's scale is NaN.
 *
 *   A    T[M, K], K % 16 == 0.
 *   out  T[M, K] (written).  out == A is allowed (in place); any other
 *        overlap with A is FP4W_ERR_ALIAS.
 * Errors as fp4w_quantize_activation.
 */
int fp4w_qdq_activation(const void* A, int64_t M, int64_t K, void* out, int dtype, void* stream);

/* Path-forcing variant (FP4W_PATH_AUTO, _NVFP4_VEC, _NVFP4_GENERIC). */
int fp4w_qdq_activation_ex(const void* A, int64_t M, int64_t K, void* out, int dtype, void* stream,
                           int path);

/*
 * fp4w_matmul_w4a4 - the FP4 operator's native FP4 x FP4 path ([FP4 doc] §6):
 * the activation quantized as above, times the FP4 weights, plus bias,
 * accumulated in FP32 and rounded once to T:
 *   Y[m, n] = sum_k qdq(A)[m, k] * B_dq[n, k] + bias[n]
 * gfx950's scaled MFMA takes power-of-two (E8M0) scales per 32 elements and
 * cannot apply E4M3 scales per 16 exactly, so this runs as A_work =
 * fp4w_qdq_activation(A) (exact in T), then fp4w_matmul(A_work, ...), whose
 * kernels fold the weight scales into exact BF16/FP16 MFMA operands.  Both
 * steps are enqueued on `stream`.  For a decode GEMV (M <= 8) with
 * M x K <= 24576, A and A_work distinct and A 16-byte aligned, the two are
 * one launch: the GEMV quantize-dequantizes its own LDS copy of A (the same
 * values, bit for bit) and writes it to A_work as well.  The pages' guards (block_size 16,
 * K % 32, N % 32, M > 8) choose this path inside their operator; called
 * directly it takes any arguments fp4w_matmul takes with K % 16 == 0.
 *
 *   A_work   T[M, K] caller-owned workspace that receives qdq(A) (the
 *            library allocates nothing).  A_work == A is allowed and
 *            overwrites A; any other overlap with A is FP4W_ERR_ALIAS, as is
 *            an overlap of A_work with B, weight_scale, weight_scale_2, bias
 *            or Y, or of Y with A.
 *   Other arguments and errors as fp4w_matmul; K % 16 != 0 is
 *   FP4W_ERR_SHAPE.  Every argument is validated before anything is
 *   launched.
 */
int fp4w_matmul_w4a4(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                     const uint8_t* weight_scale, int64_t scale_cols, int64_t block_size,
                     const float* weight_scale_2, const void* bias, void* A_work, void* Y, int dtype,
                     void* stream);

/* Size of the library-owned device scratch of fp4w_matmul_w4a4_noalloc. */
#define FP4W_STATIC_SCRATCH_BYTES (32 * 1024 * 1024)

/*
 * fp4w_matmul_w4a4_noalloc - fp4w_matmul_w4a4 for callers that cannot
 * allocate: code under HIP graph capture, serving loops that make no
 * allocations, harnesses that forbid hipMalloc.  The quantized activation
 * goes to a library-owned device array of FP4W_STATIC_SCRATCH_BYTES instead
 * of a caller workspace; the call allocates nothing.
 *
 *   Arguments, results and errors as fp4w_matmul_w4a4 without A_work.
 *   M * K * 2 > FP4W_STATIC_SCRATCH_BYTES is FP4W_ERR_SHAPE.
 *   Each device the library runs on holds its own copy of the array until
 *   the process ends.  Its address is taken on the first call on a device,
 *   with that device current (FP4W_ERR_LAUNCH if HIP cannot provide it).
 *   Every call writes the part it reads before reading it, but all calls on
 *   one device share that device's copy: calls that overlap on one device
 *   (on two streams, or from two threads) race on it, and the caller must
 *   order them.
 */
int fp4w_matmul_w4a4_noalloc(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                             const uint8_t* weight_scale, int64_t scale_cols, int64_t block_size,
                             const float* weight_scale_2, const void* bias, void* Y, int dtype,
                             void* stream);

/*
 * fp4w_dequant - expand packed FP4 weights to T[N, K] ([FP4 doc] §5 step 1;
 * [Blog] vectorised dequant).  out[n, k] = RNE_T(RNE_f32(e2m1 * e4m3 * ws2)):
 * the E2M1 x E4M3 product is exact, the FP32 multiply by weight_scale_2 rounds
 * once, then the FP32 value is rounded to T.  Bit-exact; no FTZ.
 *
 *   B, weight_scale, weight_scale_2: as fp4w_matmul.   out: T[N, K] (written).
 * N == 0 or K == 0: FP4W_OK, nothing launched.
 */
int fp4w_dequant(const uint8_t* B, int64_t N, int64_t K, const uint8_t* weight_scale,
                 int64_t scale_cols, int64_t block_size, const float* weight_scale_2, void* out,
                 int dtype, void* stream);

/* Path-forcing variant (FP4W_PATH_AUTO, _DEQUANT_VEC, _DEQUANT_GENERIC). */
int fp4w_dequant_ex(const uint8_t* B, int64_t N, int64_t K, const uint8_t* weight_scale,
                    int64_t scale_cols, int64_t block_size, const float* weight_scale_2, void* out,
                    int dtype, void* stream, int path);

/*
 * fp8w_dequant - expand FP8 weights to T[N, K], the first step of the FP8
 * operator's default path ([FP8 doc] §5 Default Path, step 1).
 *   out[n, k] = RNE_T(RNE_f32(e4m3(B[n, k]) * b_scale[n, min(k / block_size, scale_cols - 1)]))
 * The E4M3 value is exact in FP32; the product with the FP32 block scale
 * rounds once, then the FP32 value is rounded to T.  Bit-exact; no FTZ.
 *
 *   B, b_scale, scale_cols, block_size: as fp8w_matmul.   out: T[N, K] (written).
 * N == 0 or K == 0: FP4W_OK, nothing launched.  Errors: FP4W_ERR_NULL,
 * FP4W_ERR_SHAPE, FP4W_ERR_BLOCK, FP4W_ERR_DTYPE, FP4W_ERR_ALIAS, FP4W_ERR_LAUNCH.
 */
int fp8w_dequant(const uint8_t* B, int64_t N, int64_t K, const float* b_scale, int64_t scale_cols,
                 int64_t block_size, void* out, int dtype, void* stream);

/* Path-forcing variant (FP4W_PATH_AUTO, _FP8_DEQUANT_VEC, _FP8_DEQUANT_GENERIC). */
int fp8w_dequant_ex(const uint8_t* B, int64_t N, int64_t K, const float* b_scale, int64_t scale_cols,
                    int64_t block_size, void* out, int dtype, void* stream, int path);

/*
 * fp8w_qdq_activation - the activation step of the FP8 operator's optional
 * W8A8 mode ([FP8 doc] §6, Optional W8A8 Activation Path):
 *   out[m, k] = RNE_T( RNE_f32( e4m3( sat( RNE_f32(A[m, k] / a_scale) ) ) * a_scale ) )
 * The quotient is an IEEE FP32 division; e4m3() rounds to nearest even; sat()
 * clamps magnitudes above 448 (the largest finite E4M3 "fn" value) to 448 and
 * keeps NaN; the decoded value times a_scale is rounded once in FP32, then to
 * T.  Bit-exact.
 *
 *   A        T[M, K]
 *   a_scale  device float*: the per-tensor activation scale (expected > 0;
 *            other values just follow the IEEE steps above).
 *   out      T[M, K] (written).  out == A is allowed (in place); any other
 *            overlap with A is FP4W_ERR_ALIAS.
 * M == 0 or K == 0: FP4W_OK, nothing launched.  Errors: FP4W_ERR_NULL,
 * FP4W_ERR_SHAPE, FP4W_ERR_DTYPE, FP4W_ERR_ALIAS, FP4W_ERR_LAUNCH.
 */
int fp8w_qdq_activation(const void* A, int64_t M, int64_t K, const float* a_scale, void* out,
                        int dtype, void* stream);

/* Path-forcing variant (FP4W_PATH_AUTO, _QDQ_VEC, _QDQ_GENERIC). */
int fp8w_qdq_activation_ex(const void* A, int64_t M, int64_t K, const float* a_scale, void* out,
                           int dtype, void* stream, int path);

/*
 * fp8w_matmul_w8a8 - the FP8 operator with its optional a_scale input
 * ([FP8 doc] §3 dispatch chain, whose first step quantizes/dequantizes A when
 * a_scale is present, and §6): A_work = fp8w_qdq_activation(A), then
 * Y = fp8w_matmul(A_work, ...).  Both steps are enqueued on `stream`.
 *
 *   A_work   T[M, K] caller-owned workspace that receives the quantized
 *            activation (the library allocates nothing).  A_work == A is
 *            allowed and overwrites A; any other overlap with A is
 *            FP4W_ERR_ALIAS, as is an overlap of Y with A_work.
 *   a_scale  device float*, as fp8w_qdq_activation.
 *   Other arguments and errors as fp8w_matmul.  Every argument is validated
 *   before anything is launched.
 */
int fp8w_matmul_w8a8(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                     const float* b_scale, int64_t scale_cols, int64_t block_size,
                     const float* a_scale, const void* bias, void* A_work, void* Y, int dtype,
                     void* stream);

/*
 * fp4w_select_path - the path FP4W_PATH_AUTO takes for these sizes, assuming
 * 16-byte-aligned pointers ([FP4 doc] §3 and [FP8 doc] §3 dispatch chains,
 * re-derived for this library).  `op` is an fp4w_op.  For dequant, M is
 * ignored.  Returns an fp4w_path, or a negative fp4w_status for illegal
 * arguments.  Host-only; never touches the GPU.
 */
int fp4w_select_path(int op, int64_t M, int64_t N, int64_t K, int64_t block_size,
                     int64_t scale_cols);

/* Static strings; never NULL. */
const char* fp4w_status_string(int status);
const char* fp4w_path_name(int path);

#ifdef __cplusplus
}
#endif

#endif /* FP4W_H */
