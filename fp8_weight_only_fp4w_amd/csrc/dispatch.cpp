// C ABI entry points: argument validation and kernel-path dispatch.
//
// Plain host C++ (no device code).  The dispatch chain follows the shape of
// [FP4 doc] §3 and [FP8 doc] §3 ("MatMulBlockQuantizedFp4Weight /
// MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation", Dispatch
// Chain): empty output returns at once, small M takes the fused decode GEMV,
// everything else a GEMM.  Unlike the pages' default path, the GEMM here is
// fused (decode into MFMA operands), so no [N, K] scratch copy exists.

#include <limits.h>
#include <stdint.h>

#include "../../include/fp4w.h"
#include "launch.h"

namespace {

using fp4w::Act;
using fp4w::DequantArgs;
using fp4w::Fp8DequantArgs;
using fp4w::MatmulArgs;
using fp4w::Nvfp4Args;
using fp4w::QdqArgs;

// Element counts (M * K, N * K, M * N, N * scale_cols) are capped at 2^60, so
// every byte count derived from them (at most 4 bytes per element) stays
// below 2^63.
constexpr int64_t kMaxElems = int64_t(1) << 60;

bool mul_ok(int64_t a, int64_t b) { return a == 0 || b <= kMaxElems / a; }

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// [lo, lo + bytes) and [lo2, lo2 + bytes2) overlap?
bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (a == nullptr || b == nullptr || abytes <= 0 || bbytes <= 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape rules shared by every op.  Returns FP4W_OK or an error status.
int check_shape(int op, int64_t M, int64_t N, int64_t K, int64_t bs, int64_t cols) {
  if (M < 0 || N < 0 || K < 0 || cols < 0) return FP4W_ERR_SHAPE;
  if (bs < 1) return FP4W_ERR_BLOCK;
  if (op == FP4W_OP_FP4_MATMUL || op == FP4W_OP_FP4_DEQUANT) {
    if (K % 2 != 0) return FP4W_ERR_SHAPE;  // two E2M1 codes per byte ([FP4 doc] §2)
  }
  if (!mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N) || !mul_ok(N, cols)) return FP4W_ERR_SHAPE;
  if (K > 0) {
    // ceil(K/bs) columns, or floor(K/bs) >= 1 when the last block is partial
    const int64_t c_ceil = ceil_div(K, bs), c_floor = K / bs;
    const bool ok = cols == c_ceil || (K % bs != 0 && c_floor >= 1 && cols == c_floor);
    if (!ok) return FP4W_ERR_SHAPE;
  }
  return FP4W_OK;
}

// Sizes the fast kernels address with 32-bit offsets (anything larger takes
// the generic kernel).  GEMV / skinny: one 16-column tile of B and all of A
// inside a buffer descriptor.  GEMM: offsets relative to a workgroup's first
// row of A, B and the scales (128 rows of A, 512 rows of B: K < 2^22), and a
// tile count that fits the grid.
bool streams_fit(int64_t M, int64_t N, int64_t K) {
  return N <= INT_MAX - 16 && K <= (int64_t(1) << 26) && M * K * 2 < (int64_t(1) << 31);
}
bool gemm_fits(int64_t M, int64_t N, int64_t K) {
  return M <= INT_MAX && N <= INT_MAX && K < (int64_t(1) << 22) &&
         ceil_div(M, 128) * ceil_div(N, 256) <= (int64_t(1) << 30);
}

// FP4 GEMV: K % 32 == 0, as the pages' decode path ([FP4 doc] §3, Dispatch
// Chain); a last window of 32, 64 or 96 k has its missing scale bytes masked.
bool fp4_gemv_ok(int64_t M, int64_t N, int64_t K, int64_t bs) {
  return M >= 1 && M <= 8 && bs == 16 && K % 32 == 0 && K > 0 && streams_fit(M, N, K);
}
bool fp4_skinny_ok(int64_t M, int64_t N, int64_t K, int64_t bs) {
  return M >= 1 && M <= 64 && bs == 16 && K % 128 == 0 && K > 0 && streams_fit(M, N, K);
}
bool fp8_skinny_ok(int64_t M, int64_t N, int64_t K, int64_t bs) {
  return M >= 1 && M <= 64 && bs % 128 == 0 && K % 128 == 0 && K > 0 && streams_fit(M, N, K);
}
bool fp4_gemm_ok(int64_t M, int64_t N, int64_t K, int64_t bs) {
  return M >= 1 && bs == 16 && K % 64 == 0 && K > 0 && gemm_fits(M, N, K);
}
// FP8 GEMV: K % 16 == 0 ([FP8 doc] §3-4) and block_size % 64 == 0 (each 64-k
// half of a 128-k window lies in one scale block).
bool fp8_gemv_ok(int64_t M, int64_t N, int64_t K, int64_t bs) {
  return M >= 1 && M <= 8 && bs % 64 == 0 && K % 16 == 0 && K > 0 && streams_fit(M, N, K);
}
bool fp8_gemm_ok(int64_t M, int64_t N, int64_t K, int64_t bs) {
  return M >= 1 && bs % 64 == 0 && K % 64 == 0 && K > 0 && gemm_fits(M, N, K);
}
bool dequant_vec_ok(int64_t N, int64_t K, int64_t bs) {
  return K % 8 == 0 && bs % 8 == 0 && K > 0 && N > 0 && (N * (K / 8)) < (int64_t(1) << 32);
}
bool fp8_dequant_vec_ok(int64_t N, int64_t K, int64_t bs) {
  return K % 16 == 0 && bs % 16 == 0 && K > 0 && N > 0 && (N * (K / 16)) < (int64_t(1) << 32);
}

// Path choice from sizes alone (pointers assumed 16-byte aligned).
int shape_path(int op, int64_t M, int64_t N, int64_t K, int64_t bs) {
  if (op == FP4W_OP_FP4_DEQUANT) {
    if (N == 0 || K == 0) return FP4W_PATH_NONE;
    return dequant_vec_ok(N, K, bs) ? FP4W_PATH_DEQUANT_VEC : FP4W_PATH_DEQUANT_GENERIC;
  }
  if (op == FP4W_OP_FP8_DEQUANT) {
    if (N == 0 || K == 0) return FP4W_PATH_NONE;
    return fp8_dequant_vec_ok(N, K, bs) ? FP4W_PATH_FP8_DEQUANT_VEC : FP4W_PATH_FP8_DEQUANT_GENERIC;
  }
  if (M == 0 || N == 0) return FP4W_PATH_NONE;
  if (op == FP4W_OP_FP4_MATMUL) {
    if (fp4_gemv_ok(M, N, K, bs)) return FP4W_PATH_FP4_GEMV;
    // Above 32 rows the skinny kernel needs its 4-row-tile variant; with
    // N >= 16384 the GEMM then has at least 128 workgroups (128-row tiles,
    // 128-column halves) and is the faster of the two (47.5 against 57-62 us
    // at N = 17408, K = 5120, M = 40..64; 46 against 23 us at N = 5120).
    const bool wide_gemm = M > 32 && N >= 16384 && fp4_gemm_ok(M, N, K, bs);
    if (M > 8 && !wide_gemm && fp4_skinny_ok(M, N, K, bs)) return FP4W_PATH_FP4_SKINNY;
    if (M > 8 && fp4_gemm_ok(M, N, K, bs)) return FP4W_PATH_FP4_GEMM;
    return FP4W_PATH_FP4_GENERIC;
  }
  if (fp8_gemv_ok(M, N, K, bs)) return FP4W_PATH_FP8_GEMV;
  if (M > 8 && fp8_skinny_ok(M, N, K, bs)) return FP4W_PATH_FP8_SKINNY;
  if (M > 8 && fp8_gemm_ok(M, N, K, bs)) return FP4W_PATH_FP8_GEMM;
  return FP4W_PATH_FP8_GENERIC;
}

// Does `path` apply to these arguments, including pointer alignment?
bool path_applies(int path, const MatmulArgs& a) {
  switch (path) {
    case FP4W_PATH_FP4_GEMV:
      return fp4_gemv_ok(a.M, a.N, a.K, a.block_size) && aligned(a.A, 16) && aligned(a.B, 16) &&
             aligned(a.scales, 4) && aligned(a.bias, 2) && aligned(a.Y, 2);
    case FP4W_PATH_FP4_SKINNY:
      return fp4_skinny_ok(a.M, a.N, a.K, a.block_size) && aligned(a.A, 16) && aligned(a.B, 16) &&
             aligned(a.scales, 4) && aligned(a.bias, 2) && aligned(a.Y, 2);
    case FP4W_PATH_FP4_GEMM:
      return fp4_gemm_ok(a.M, a.N, a.K, a.block_size) && aligned(a.A, 16) && aligned(a.B, 16) &&
             aligned(a.scales, 4) && aligned(a.bias, 2) && aligned(a.Y, 2);
    case FP4W_PATH_FP4_GENERIC:
    case FP4W_PATH_FP8_GENERIC:
      return true;
    case FP4W_PATH_FP8_GEMV:
      return fp8_gemv_ok(a.M, a.N, a.K, a.block_size) && aligned(a.A, 16) && aligned(a.B, 16) &&
             aligned(a.scales, 4) && aligned(a.bias, 2) && aligned(a.Y, 2);
    case FP4W_PATH_FP8_SKINNY:
      return fp8_skinny_ok(a.M, a.N, a.K, a.block_size) && aligned(a.A, 16) && aligned(a.B, 16) &&
             aligned(a.scales, 4) && aligned(a.bias, 2) && aligned(a.Y, 2);
    case FP4W_PATH_FP8_GEMM:
      return fp8_gemm_ok(a.M, a.N, a.K, a.block_size) && aligned(a.A, 16) && aligned(a.B, 16) &&
             aligned(a.scales, 4) && aligned(a.bias, 2) && aligned(a.Y, 2);
    default:
      return false;
  }
}

// Validates a matmul call and picks its kernel path.  Returns FP4W_OK with
// *chosen set (FP4W_PATH_NONE when there is nothing to launch), or an error.
int plan_matmul(int op, const MatmulArgs& a, const void* scale_ptr_for_alias,
                int64_t scale_elem_bytes, int path, int* chosen_out) {
  const int dtype = static_cast<int>(a.act);
  if (dtype != FP4W_F16 && dtype != FP4W_BF16) return FP4W_ERR_DTYPE;
  int st = check_shape(op, a.M, a.N, a.K, a.block_size, a.scale_cols);
  if (st != FP4W_OK) return st;
  const bool fp4 = op == FP4W_OP_FP4_MATMUL;
  if (path != FP4W_PATH_AUTO) {
    const bool family_ok = fp4 ? (path == FP4W_PATH_FP4_GEMV || path == FP4W_PATH_FP4_SKINNY ||
                                  path == FP4W_PATH_FP4_GEMM || path == FP4W_PATH_FP4_GENERIC)
                               : (path == FP4W_PATH_FP8_GEMV || path == FP4W_PATH_FP8_SKINNY ||
                                  path == FP4W_PATH_FP8_GEMM || path == FP4W_PATH_FP8_GENERIC);
    if (!family_ok) return FP4W_ERR_PATH;
  }
  *chosen_out = FP4W_PATH_NONE;
  if (a.M == 0 || a.N == 0) return FP4W_OK;  // empty output: nothing to do
  if (a.Y == nullptr) return FP4W_ERR_NULL;
  if (a.K > 0 && (a.A == nullptr || a.B == nullptr || a.scales == nullptr)) return FP4W_ERR_NULL;
  if (fp4 && a.K > 0 && a.ws2 == nullptr) return FP4W_ERR_NULL;

  const int64_t ybytes = a.M * a.N * 2;
  const int64_t bbytes = fp4 ? a.N * (a.K / 2) : a.N * a.K;
  if (overlaps(a.Y, ybytes, a.A, a.M * a.K * 2) || overlaps(a.Y, ybytes, a.B, bbytes) ||
      overlaps(a.Y, ybytes, scale_ptr_for_alias, a.N * a.scale_cols * scale_elem_bytes) ||
      overlaps(a.Y, ybytes, a.bias, a.N * 2) || overlaps(a.Y, ybytes, a.ws2, fp4 ? 4 : 0))
    return FP4W_ERR_ALIAS;

  int chosen = path;
  if (path == FP4W_PATH_AUTO) {
    chosen = shape_path(op, a.M, a.N, a.K, a.block_size);
    if (!path_applies(chosen, a)) chosen = fp4 ? FP4W_PATH_FP4_GENERIC : FP4W_PATH_FP8_GENERIC;
  } else if (!path_applies(path, a)) {
    return FP4W_ERR_PATH;
  }
  *chosen_out = chosen;
  return FP4W_OK;
}

int launch_matmul(int chosen, const MatmulArgs& a) {
  int rc = -1;
  switch (chosen) {
    case FP4W_PATH_NONE: return FP4W_OK;
    case FP4W_PATH_FP4_GEMV: rc = fp4w::launch_fp4_gemv(a); break;
    case FP4W_PATH_FP4_SKINNY: rc = fp4w::launch_fp4_skinny(a); break;
    case FP4W_PATH_FP4_GEMM: rc = fp4w::launch_fp4_gemm(a); break;
    case FP4W_PATH_FP4_GENERIC: rc = fp4w::launch_fp4_generic(a); break;
    case FP4W_PATH_FP8_GEMV: rc = fp4w::launch_fp8_gemv(a); break;
    case FP4W_PATH_FP8_SKINNY: rc = fp4w::launch_fp8_skinny(a); break;
    case FP4W_PATH_FP8_GEMM: rc = fp4w::launch_fp8_gemm(a); break;
    case FP4W_PATH_FP8_GENERIC: rc = fp4w::launch_fp8_generic(a); break;
    default: return FP4W_ERR_PATH;
  }
  return rc == 0 ? FP4W_OK : FP4W_ERR_LAUNCH;
}

int run_matmul(int op, const MatmulArgs& a, const void* scale_ptr_for_alias,
               int64_t scale_elem_bytes, int path) {
  int chosen = FP4W_PATH_NONE;
  const int st = plan_matmul(op, a, scale_ptr_for_alias, scale_elem_bytes, path, &chosen);
  return st != FP4W_OK ? st : launch_matmul(chosen, a);
}

bool qdq_vec_ok(int64_t count) { return count > 0 && count % 8 == 0; }

// Validates a QDQ call and picks its path (FP4W_PATH_NONE: nothing to do).
int plan_qdq(const QdqArgs& q, int64_t M, int64_t K, int path, int* chosen_out) {
  const int dtype = static_cast<int>(q.act);
  if (dtype != FP4W_F16 && dtype != FP4W_BF16) return FP4W_ERR_DTYPE;
  if (M < 0 || K < 0 || !mul_ok(M, K) || !mul_ok(M * K, 2)) return FP4W_ERR_SHAPE;
  if (path != FP4W_PATH_AUTO && path != FP4W_PATH_QDQ_VEC && path != FP4W_PATH_QDQ_GENERIC)
    return FP4W_ERR_PATH;
  *chosen_out = FP4W_PATH_NONE;
  if (M == 0 || K == 0) return FP4W_OK;
  if (q.A == nullptr || q.a_scale == nullptr || q.out == nullptr) return FP4W_ERR_NULL;
  const int64_t bytes = M * K * 2;
  if (q.out != q.A && overlaps(q.out, bytes, q.A, bytes)) return FP4W_ERR_ALIAS;
  if (overlaps(q.out, bytes, q.a_scale, 4)) return FP4W_ERR_ALIAS;
  const bool vec = qdq_vec_ok(M * K) && aligned(q.A, 16) && aligned(q.out, 16);
  int chosen = path;
  if (path == FP4W_PATH_AUTO) chosen = vec ? FP4W_PATH_QDQ_VEC : FP4W_PATH_QDQ_GENERIC;
  if (chosen == FP4W_PATH_QDQ_VEC && !vec) return FP4W_ERR_PATH;
  *chosen_out = chosen;
  return FP4W_OK;
}

int launch_qdq(int chosen, const QdqArgs& q) {
  if (chosen == FP4W_PATH_NONE) return FP4W_OK;
  const int rc = chosen == FP4W_PATH_QDQ_VEC ? fp4w::launch_qdq_vec(q) : fp4w::launch_qdq_generic(q);
  return rc == 0 ? FP4W_OK : FP4W_ERR_LAUNCH;
}

// NVFP4 activation quantization (W4A4 path, [FP4 doc] §6): blocks of 16
// along K.  Validates and picks the path; *chosen_out = FP4W_PATH_NONE when
// there is nothing to do.  packed: codes / scales are written, else out.
bool nvfp4_shape_ok(int64_t M, int64_t K) {
  return M >= 0 && K >= 0 && K % 16 == 0 && mul_ok(M, K) && mul_ok(M * K, 2);
}

int plan_nvfp4(const Nvfp4Args& q, int64_t M, int64_t K, bool packed, int path, int* chosen_out) {
  const int dtype = static_cast<int>(q.act);
  if (dtype != FP4W_F16 && dtype != FP4W_BF16) return FP4W_ERR_DTYPE;
  if (!nvfp4_shape_ok(M, K)) return FP4W_ERR_SHAPE;
  if (path != FP4W_PATH_AUTO && path != FP4W_PATH_NVFP4_VEC && path != FP4W_PATH_NVFP4_GENERIC)
    return FP4W_ERR_PATH;
  *chosen_out = FP4W_PATH_NONE;
  if (M == 0 || K == 0) return FP4W_OK;
  if (q.A == nullptr) return FP4W_ERR_NULL;
  const int64_t abytes = M * K * 2;
  bool vec = aligned(q.A, 16);
  if (packed) {
    if (q.codes == nullptr || q.scales == nullptr) return FP4W_ERR_NULL;
    const int64_t cbytes = M * K / 2, sbytes = M * K / 16;
    if (overlaps(q.codes, cbytes, q.A, abytes) || overlaps(q.scales, sbytes, q.A, abytes) ||
        overlaps(q.codes, cbytes, q.scales, sbytes))
      return FP4W_ERR_ALIAS;
    vec = vec && aligned(q.codes, 8);
  } else {
    if (q.out == nullptr) return FP4W_ERR_NULL;
    if (q.out != q.A && overlaps(q.out, abytes, q.A, abytes)) return FP4W_ERR_ALIAS;
    vec = vec && aligned(q.out, 16);
  }
  int chosen = path;
  if (path == FP4W_PATH_AUTO) chosen = vec ? FP4W_PATH_NVFP4_VEC : FP4W_PATH_NVFP4_GENERIC;
  if (chosen == FP4W_PATH_NVFP4_VEC && !vec) return FP4W_ERR_PATH;
  *chosen_out = chosen;
  return FP4W_OK;
}

int launch_nvfp4(int chosen, const Nvfp4Args& q, bool packed) {
  if (chosen == FP4W_PATH_NONE) return FP4W_OK;
  const bool vec = chosen == FP4W_PATH_NVFP4_VEC;
  const int rc = packed ? fp4w::launch_nvfp4_quantize(q, vec) : fp4w::launch_nvfp4_qdq(q, vec);
  return rc == 0 ? FP4W_OK : FP4W_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fp4w_matmul_ex(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                   const uint8_t* weight_scale, int64_t scale_cols, int64_t block_size,
                   const float* weight_scale_2, const void* bias, void* Y, int dtype, void* stream,
                   int path) {
  MatmulArgs a{A, B, weight_scale, weight_scale_2, bias, Y, M, N, K, block_size, scale_cols,
               static_cast<Act>(dtype), stream};
  return run_matmul(FP4W_OP_FP4_MATMUL, a, weight_scale, 1, path);
}

int fp4w_matmul(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                const uint8_t* weight_scale, int64_t scale_cols, int64_t block_size,
                const float* weight_scale_2, const void* bias, void* Y, int dtype, void* stream) {
  return fp4w_matmul_ex(A, M, K, B, N, weight_scale, scale_cols, block_size, weight_scale_2, bias,
                        Y, dtype, stream, FP4W_PATH_AUTO);
}

int fp8w_matmul_ex(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                   const float* b_scale, int64_t scale_cols, int64_t block_size, const void* bias,
                   void* Y, int dtype, void* stream, int path) {
  MatmulArgs a{A, B, b_scale, nullptr, bias, Y, M, N, K, block_size, scale_cols,
               static_cast<Act>(dtype), stream};
  return run_matmul(FP4W_OP_FP8_MATMUL, a, b_scale, 4, path);
}

int fp8w_matmul(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                const float* b_scale, int64_t scale_cols, int64_t block_size, const void* bias,
                void* Y, int dtype, void* stream) {
  return fp8w_matmul_ex(A, M, K, B, N, b_scale, scale_cols, block_size, bias, Y, dtype, stream,
                        FP4W_PATH_AUTO);
}

int fp8w_qdq_activation_ex(const void* A, int64_t M, int64_t K, const float* a_scale, void* out,
                           int dtype, void* stream, int path) {
  const int64_t count = (M >= 0 && K >= 0 && mul_ok(M, K)) ? M * K : 0;
  QdqArgs q{A, a_scale, out, count, static_cast<Act>(dtype), stream};
  int chosen = FP4W_PATH_NONE;
  const int st = plan_qdq(q, M, K, path, &chosen);
  return st != FP4W_OK ? st : launch_qdq(chosen, q);
}

int fp8w_qdq_activation(const void* A, int64_t M, int64_t K, const float* a_scale, void* out,
                        int dtype, void* stream) {
  return fp8w_qdq_activation_ex(A, M, K, a_scale, out, dtype, stream, FP4W_PATH_AUTO);
}

int fp8w_matmul_w8a8(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                     const float* b_scale, int64_t scale_cols, int64_t block_size,
                     const float* a_scale, const void* bias, void* A_work, void* Y, int dtype,
                     void* stream) {
  // The matmul reads A_work; validate it as the matmul's activation.
  MatmulArgs a{A_work, B, b_scale, nullptr, bias, Y, M, N, K, block_size, scale_cols,
               static_cast<Act>(dtype), stream};
  int mm_path = FP4W_PATH_NONE;
  int st = plan_matmul(FP4W_OP_FP8_MATMUL, a, b_scale, 4, FP4W_PATH_AUTO, &mm_path);
  if (st != FP4W_OK) return st;
  if (mm_path == FP4W_PATH_NONE) return FP4W_OK;  // empty output
  QdqArgs q{A, a_scale, A_work, M * K, static_cast<Act>(dtype), stream};
  int q_path = FP4W_PATH_NONE;
  st = plan_qdq(q, M, K, FP4W_PATH_AUTO, &q_path);
  if (st != FP4W_OK) return st;
  // The weights, scales and bias are only read, but the QDQ step writes
  // A_work: it must not overlap them or Y (checked against Y by plan_matmul).
  // Y must not overlap the original activation or a_scale either.
  const int64_t abytes = M * K * 2;
  if (overlaps(Y, M * N * 2, A, abytes) || overlaps(Y, M * N * 2, a_scale, 4) ||
      overlaps(A_work, abytes, B, N * K) ||
      overlaps(A_work, abytes, b_scale, N * scale_cols * 4) || overlaps(A_work, abytes, bias, N * 2))
    return FP4W_ERR_ALIAS;
  st = launch_qdq(q_path, q);
  if (st != FP4W_OK) return st;
  return launch_matmul(mm_path, a);
}

int fp4w_quantize_activation_ex(const void* A, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                                int dtype, void* stream, int path) {
  const int64_t blocks = nvfp4_shape_ok(M, K) ? M * (K / 16) : 0;
  Nvfp4Args q{A, codes, scales, nullptr, blocks, static_cast<Act>(dtype), stream};
  int chosen = FP4W_PATH_NONE;
  const int st = plan_nvfp4(q, M, K, true, path, &chosen);
  return st != FP4W_OK ? st : launch_nvfp4(chosen, q, true);
}

int fp4w_quantize_activation(const void* A, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                             int dtype, void* stream) {
  return fp4w_quantize_activation_ex(A, M, K, codes, scales, dtype, stream, FP4W_PATH_AUTO);
}

int fp4w_qdq_activation_ex(const void* A, int64_t M, int64_t K, void* out, int dtype, void* stream,
                           int path) {
  const int64_t blocks = nvfp4_shape_ok(M, K) ? M * (K / 16) : 0;
  Nvfp4Args q{A, nullptr, nullptr, out, blocks, static_cast<Act>(dtype), stream};
  int chosen = FP4W_PATH_NONE;
  const int st = plan_nvfp4(q, M, K, false, path, &chosen);
  return st != FP4W_OK ? st : launch_nvfp4(chosen, q, false);
}

int fp4w_qdq_activation(const void* A, int64_t M, int64_t K, void* out, int dtype, void* stream) {
  return fp4w_qdq_activation_ex(A, M, K, out, dtype, stream, FP4W_PATH_AUTO);
}

int fp4w_matmul_w4a4(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                     const uint8_t* weight_scale, int64_t scale_cols, int64_t block_size,
                     const float* weight_scale_2, const void* bias, void* A_work, void* Y, int dtype,
                     void* stream) {
  // The matmul reads A_work; validate it as the matmul's activation.
  MatmulArgs a{A_work, B, weight_scale, weight_scale_2, bias, Y, M, N, K, block_size, scale_cols,
               static_cast<Act>(dtype), stream};
  int mm_path = FP4W_PATH_NONE;
  int st = plan_matmul(FP4W_OP_FP4_MATMUL, a, weight_scale, 1, FP4W_PATH_AUTO, &mm_path);
  if (st != FP4W_OK) return st;
  if (K % 16 != 0) return FP4W_ERR_SHAPE;  // activation blocks of 16
  if (mm_path == FP4W_PATH_NONE) return FP4W_OK;  // empty output
  Nvfp4Args q{A, nullptr, nullptr, A_work, M * (K / 16), static_cast<Act>(dtype), stream};
  int q_path = FP4W_PATH_NONE;
  st = plan_nvfp4(q, M, K, false, FP4W_PATH_AUTO, &q_path);
  if (st != FP4W_OK) return st;
  // The QDQ step writes A_work: it must not overlap the weights, scales,
  // bias or Y (Y against A_work is checked by plan_matmul); Y must not
  // overlap the original activation.
  const int64_t abytes = M * K * 2;
  if (overlaps(Y, M * N * 2, A, abytes) || overlaps(A_work, abytes, B, N * (K / 2)) ||
      overlaps(A_work, abytes, weight_scale, N * scale_cols) || overlaps(A_work, abytes, weight_scale_2, 4) ||
      overlaps(A_work, abytes, bias, N * 2))
    return FP4W_ERR_ALIAS;
  if (mm_path == FP4W_PATH_FP4_GEMV && A_work != A && aligned(A, 16)) {
    // Decode: the GEMV quantize-dequantizes its LDS copy of A itself (and
    // writes it to A_work); 1 = the activations do not fit in LDS.
    MatmulArgs f = a;
    f.A = A;
    const int rc = fp4w::launch_fp4_gemv_w4a4(f, A_work);
    if (rc <= 0) return rc == 0 ? FP4W_OK : FP4W_ERR_LAUNCH;
  }
  st = launch_nvfp4(q_path, q, false);
  if (st != FP4W_OK) return st;
  return launch_matmul(mm_path, a);
}

int fp4w_matmul_w4a4_noalloc(const void* A, int64_t M, int64_t K, const uint8_t* B, int64_t N,
                             const uint8_t* weight_scale, int64_t scale_cols, int64_t block_size,
                             const float* weight_scale_2, const void* bias, void* Y, int dtype,
                             void* stream) {
  static_assert(fp4w::kStaticScratchBytes == FP4W_STATIC_SCRATCH_BYTES, "scratch size");
  // Validate as fp4w_matmul_w4a4 would, with A standing in for the
  // workspace (the scratch overlaps no caller buffer), before the scratch's
  // address is taken.
  MatmulArgs a{A, B, weight_scale, weight_scale_2, bias, Y, M, N, K, block_size, scale_cols,
               static_cast<Act>(dtype), stream};
  int mm_path = FP4W_PATH_NONE;
  int st = plan_matmul(FP4W_OP_FP4_MATMUL, a, weight_scale, 1, FP4W_PATH_AUTO, &mm_path);
  if (st != FP4W_OK) return st;
  if (K % 16 != 0) return FP4W_ERR_SHAPE;
  if (mm_path == FP4W_PATH_NONE) return FP4W_OK;  // empty output
  if (K > 0 && M > FP4W_STATIC_SCRATCH_BYTES / 2 / K) return FP4W_ERR_SHAPE;
  void* work = nullptr;
  if (fp4w::static_scratch(&work) != 0) return FP4W_ERR_LAUNCH;
  return fp4w_matmul_w4a4(A, M, K, B, N, weight_scale, scale_cols, block_size, weight_scale_2, bias, work, Y,
                          dtype, stream);
}

int fp4w_dequant_ex(const uint8_t* B, int64_t N, int64_t K, const uint8_t* weight_scale,
                    int64_t scale_cols, int64_t block_size, const float* weight_scale_2, void* out,
                    int dtype, void* stream, int path) {
  if (dtype != FP4W_F16 && dtype != FP4W_BF16) return FP4W_ERR_DTYPE;
  int st = check_shape(FP4W_OP_FP4_DEQUANT, 0, N, K, block_size, scale_cols);
  if (st != FP4W_OK) return st;
  if (path != FP4W_PATH_AUTO && path != FP4W_PATH_DEQUANT_VEC && path != FP4W_PATH_DEQUANT_GENERIC)
    return FP4W_ERR_PATH;
  if (N == 0 || K == 0) return FP4W_OK;
  if (B == nullptr || weight_scale == nullptr || weight_scale_2 == nullptr || out == nullptr)
    return FP4W_ERR_NULL;
  const int64_t obytes = N * K * 2;
  if (overlaps(out, obytes, B, N * (K / 2)) || overlaps(out, obytes, weight_scale, N * scale_cols) ||
      overlaps(out, obytes, weight_scale_2, 4))
    return FP4W_ERR_ALIAS;
  DequantArgs a{B, weight_scale, weight_scale_2, out, N, K, block_size, scale_cols,
                static_cast<Act>(dtype), stream};
  const bool vec_ok = dequant_vec_ok(N, K, block_size) && aligned(B, 4) && aligned(out, 16);
  int chosen = path;
  if (path == FP4W_PATH_AUTO) chosen = vec_ok ? FP4W_PATH_DEQUANT_VEC : FP4W_PATH_DEQUANT_GENERIC;
  if (chosen == FP4W_PATH_DEQUANT_VEC && !vec_ok) return FP4W_ERR_PATH;
  const int rc = chosen == FP4W_PATH_DEQUANT_VEC ? fp4w::launch_dequant_vec(a)
                                                 : fp4w::launch_dequant_generic(a);
  return rc == 0 ? FP4W_OK : FP4W_ERR_LAUNCH;
}

int fp8w_dequant_ex(const uint8_t* B, int64_t N, int64_t K, const float* b_scale, int64_t scale_cols,
                    int64_t block_size, void* out, int dtype, void* stream, int path) {
  if (dtype != FP4W_F16 && dtype != FP4W_BF16) return FP4W_ERR_DTYPE;
  int st = check_shape(FP4W_OP_FP8_DEQUANT, 0, N, K, block_size, scale_cols);
  if (st != FP4W_OK) return st;
  if (path != FP4W_PATH_AUTO && path != FP4W_PATH_FP8_DEQUANT_VEC && path != FP4W_PATH_FP8_DEQUANT_GENERIC)
    return FP4W_ERR_PATH;
  if (N == 0 || K == 0) return FP4W_OK;
  if (B == nullptr || b_scale == nullptr || out == nullptr) return FP4W_ERR_NULL;
  const int64_t obytes = N * K * 2;
  if (overlaps(out, obytes, B, N * K) || overlaps(out, obytes, b_scale, N * scale_cols * 4))
    return FP4W_ERR_ALIAS;
  Fp8DequantArgs a{B, b_scale, out, N, K, block_size, scale_cols, static_cast<Act>(dtype), stream};
  const bool vec_ok = fp8_dequant_vec_ok(N, K, block_size) && aligned(B, 16) && aligned(out, 16) &&
                      aligned(b_scale, 4);
  int chosen = path;
  if (path == FP4W_PATH_AUTO) chosen = vec_ok ? FP4W_PATH_FP8_DEQUANT_VEC : FP4W_PATH_FP8_DEQUANT_GENERIC;
  if (chosen == FP4W_PATH_FP8_DEQUANT_VEC && !vec_ok) return FP4W_ERR_PATH;
  const int rc = chosen == FP4W_PATH_FP8_DEQUANT_VEC ? fp4w::launch_fp8_dequant_vec(a)
                                                     : fp4w::launch_fp8_dequant_generic(a);
  return rc == 0 ? FP4W_OK : FP4W_ERR_LAUNCH;
}

int fp8w_dequant(const uint8_t* B, int64_t N, int64_t K, const float* b_scale, int64_t scale_cols,
                 int64_t block_size, void* out, int dtype, void* stream) {
  return fp8w_dequant_ex(B, N, K, b_scale, scale_cols, block_size, out, dtype, stream, FP4W_PATH_AUTO);
}

int fp4w_dequant(const uint8_t* B, int64_t N, int64_t K, const uint8_t* weight_scale,
                 int64_t scale_cols, int64_t block_size, const float* weight_scale_2, void* out,
                 int dtype, void* stream) {
  return fp4w_dequant_ex(B, N, K, weight_scale, scale_cols, block_size, weight_scale_2, out, dtype,
                         stream, FP4W_PATH_AUTO);
}

int fp4w_select_path(int op, int64_t M, int64_t N, int64_t K, int64_t block_size,
                     int64_t scale_cols) {
  if (op == FP4W_OP_NVFP4_ACT) {
    if (!nvfp4_shape_ok(M, K)) return FP4W_ERR_SHAPE;
    if (M == 0 || K == 0) return FP4W_PATH_NONE;
    return FP4W_PATH_NVFP4_VEC;
  }
  if (op == FP4W_OP_FP8_QDQ) {
    if (M < 0 || K < 0 || !mul_ok(M, K) || !mul_ok(M * K, 2)) return FP4W_ERR_SHAPE;
    if (M == 0 || K == 0) return FP4W_PATH_NONE;
    return qdq_vec_ok(M * K) ? FP4W_PATH_QDQ_VEC : FP4W_PATH_QDQ_GENERIC;
  }
  if (op != FP4W_OP_FP4_MATMUL && op != FP4W_OP_FP8_MATMUL && op != FP4W_OP_FP4_DEQUANT &&
      op != FP4W_OP_FP8_DEQUANT)
    return FP4W_ERR_PATH;
  const bool dq = op == FP4W_OP_FP4_DEQUANT || op == FP4W_OP_FP8_DEQUANT;
  int st = check_shape(op, dq ? 0 : M, N, K, block_size, scale_cols);
  if (st != FP4W_OK) return st;
  return shape_path(op, M, N, K, block_size);
}

const char* fp4w_status_string(int status) {
  switch (status) {
    case FP4W_OK: return "ok";
    case FP4W_ERR_NULL: return "a required pointer is NULL";
    case FP4W_ERR_SHAPE: return "invalid shape (negative size, odd K for FP4, bad scale_cols or overflow)";
    case FP4W_ERR_DTYPE: return "dtype must be FP4W_F16 or FP4W_BF16";
    case FP4W_ERR_BLOCK: return "block_size must be >= 1";
    case FP4W_ERR_PATH: return "the requested kernel path does not apply to these arguments";
    case FP4W_ERR_LAUNCH: return "HIP reported an error when enqueuing the kernel";
    case FP4W_ERR_ALIAS: return "the output overlaps an input";
    default: return "unknown status";
  }
}

const char* fp4w_path_name(int path) {
  switch (path) {
    case FP4W_PATH_AUTO: return "auto";
    case FP4W_PATH_NONE: return "none";
    case FP4W_PATH_FP4_GEMV: return "fp4_gemv";
    case FP4W_PATH_FP4_GEMM: return "fp4_gemm";
    case FP4W_PATH_FP4_GENERIC: return "fp4_generic";
    case FP4W_PATH_FP8_GEMV: return "fp8_gemv";
    case FP4W_PATH_FP8_GEMM: return "fp8_gemm";
    case FP4W_PATH_FP8_GENERIC: return "fp8_generic";
    case FP4W_PATH_DEQUANT_VEC: return "dequant_vec";
    case FP4W_PATH_DEQUANT_GENERIC: return "dequant_generic";
    case FP4W_PATH_QDQ_VEC: return "qdq_vec";
    case FP4W_PATH_QDQ_GENERIC: return "qdq_generic";
    case FP4W_PATH_FP4_SKINNY: return "fp4_skinny";
    case FP4W_PATH_FP8_SKINNY: return "fp8_skinny";
    case FP4W_PATH_FP8_DEQUANT_VEC: return "fp8_dequant_vec";
    case FP4W_PATH_FP8_DEQUANT_GENERIC: return "fp8_dequant_generic";
    case FP4W_PATH_NVFP4_VEC: return "nvfp4_vec";
    case FP4W_PATH_NVFP4_GENERIC: return "nvfp4_generic";
    default: return "unknown";
  }
}

}  // extern "C"
