// Drives every C-ABI entry point of fp4w.h through its validation and
// dispatch with host buffers standing in for device pointers (nothing is
// dereferenced: the launchers are stubs), for an AddressSanitizer /
// UndefinedBehaviorSanitizer build.  Prints "ok" and exits 0 when every
// status and every chosen kernel matches the expectation.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/fp4w.h"

namespace fp4w {
extern const char* g_last;
extern int g_fused_rc;
}

static int failures = 0;
static void expect(bool ok, const char* what, int line) {
  if (!ok) {
    printf("FAIL line %d: %s\n", line, what);
    ++failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

int main() {
  // Stand-in device addresses, 64 GiB apart so that no claimed extent
  // overlaps another (the dispatcher compares addresses, never dereferences)
  auto fake = [](uint64_t i) { return reinterpret_cast<unsigned char*>(i << 36); };
  unsigned char *A = fake(1), *B = fake(2), *S = fake(3), *Y = fake(4), *W = fake(5);
  float* ws2 = reinterpret_cast<float*>(fake(6));
  const int64_t big = int64_t(1) << 31;
  // FP4: the kernel each shape takes
  struct Case { int64_t M, N, K, bs; const char* want; };
  const Case fp4_cases[] = {
      {4, 5120, 5120, 16, "launch_fp4_gemv"},   {8, 16, 128, 16, "launch_fp4_gemv"},
      {40, 300, 256, 16, "launch_fp4_skinny"},  {100, 300, 256, 16, "launch_fp4_gemm"},
      {100, 300, 96, 16, "launch_fp4_generic"}, {4, 300, 30, 15, "launch_fp4_generic"},
      {3, 1000, 480, 16, "launch_fp4_gemv"},    {3, 1000, 464, 16, "launch_fp4_generic"},
      {100, 300, int64_t(1) << 22, 16, "launch_fp4_generic"},
  };
  for (const Case& c : fp4_cases) {
    fp4w::g_last = "";
    const int64_t cols = (c.K + c.bs - 1) / c.bs;
    const int st = fp4w_matmul(A, c.M, c.K, B, c.N, S, cols, c.bs, ws2, nullptr, Y, FP4W_BF16, nullptr);
    EXPECT(st == FP4W_OK);
    EXPECT(strcmp(fp4w::g_last, c.want) == 0);
  }
  // FP8
  const Case fp8_cases[] = {
      {4, 17408, 5120, 128, "launch_fp8_gemv"}, {40, 300, 512, 128, "launch_fp8_skinny"},
      {300, 520, 640, 128, "launch_fp8_gemm"},  {3, 21, 37, 16, "launch_fp8_generic"},
      {4, 300, 208, 64, "launch_fp8_gemv"},     {4, 300, 256, 32, "launch_fp8_generic"},
  };
  for (const Case& c : fp8_cases) {
    fp4w::g_last = "";
    const int64_t cols = (c.K + c.bs - 1) / c.bs;
    const int st = fp8w_matmul(A, c.M, c.K, B, c.N, reinterpret_cast<const float*>(S), cols, c.bs, nullptr, Y,
                               FP4W_F16, nullptr);
    EXPECT(st == FP4W_OK);
    EXPECT(strcmp(fp4w::g_last, c.want) == 0);
  }
  // empty outputs launch nothing; K == 0 takes the generic kernel (Y = bias)
  fp4w::g_last = "";
  EXPECT(fp4w_matmul(nullptr, 0, 64, B, 16, S, 4, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_OK);
  EXPECT(fp4w_matmul(A, 4, 64, B, 0, S, 4, 16, ws2, nullptr, nullptr, FP4W_BF16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "") == 0);
  EXPECT(fp4w_matmul(A, 3, 0, B, 5, S, 0, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "launch_fp4_generic") == 0);
  // errors, each before anything is launched
  fp4w::g_last = "";
  EXPECT(fp4w_matmul(nullptr, 4, 64, B, 16, S, 4, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_ERR_NULL);
  EXPECT(fp4w_matmul(A, 4, 64, B, 16, S, 4, 16, nullptr, nullptr, Y, FP4W_BF16, nullptr) == FP4W_ERR_NULL);
  EXPECT(fp4w_matmul(A, 4, 63, B, 16, S, 4, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_ERR_SHAPE);
  EXPECT(fp4w_matmul(A, -1, 64, B, 16, S, 4, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_ERR_SHAPE);
  EXPECT(fp4w_matmul(A, 4, 64, B, 16, S, 5, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_ERR_SHAPE);
  EXPECT(fp4w_matmul(A, 4, 64, B, 16, S, 4, 0, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_ERR_BLOCK);
  EXPECT(fp4w_matmul(A, 4, 64, B, 16, S, 4, 16, ws2, nullptr, Y, 7, nullptr) == FP4W_ERR_DTYPE);
  EXPECT(fp4w_matmul(A, 4, 64, B, 16, S, 4, 16, ws2, nullptr, A, FP4W_BF16, nullptr) == FP4W_ERR_ALIAS);
  EXPECT(fp4w_matmul_ex(A, 4, 96, B, 16, S, 6, 16, ws2, nullptr, Y, FP4W_BF16, nullptr, FP4W_PATH_FP4_GEMM) ==
         FP4W_ERR_PATH);
  EXPECT(fp4w_matmul_ex(A, 4, 64, B, 16, S, 4, 16, ws2, nullptr, Y, FP4W_BF16, nullptr, FP4W_PATH_FP8_GEMV) ==
         FP4W_ERR_PATH);
  EXPECT(fp4w_matmul(A + 1, 4, 128, B, 16, S, 8, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_OK);  // unaligned
  EXPECT(strcmp(fp4w::g_last, "launch_fp4_generic") == 0);
  // sizes whose byte counts overflow 64 bits are rejected, not wrapped
  EXPECT(fp4w_matmul(A, big, 64, B, big, S, 4, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_ERR_SHAPE);
  EXPECT(fp4w_matmul(A, int64_t(1) << 40, int64_t(1) << 24, B, 16, S, int64_t(1) << 20, 16, ws2, nullptr, Y,
                     FP4W_BF16, nullptr) == FP4W_ERR_SHAPE);
  EXPECT(fp8w_matmul(A, big, 64, B, big, reinterpret_cast<const float*>(S), 1, 64, nullptr, Y, FP4W_BF16,
                     nullptr) == FP4W_ERR_SHAPE);
  // dequant and QDQ
  EXPECT(fp4w_dequant(B, 128, 256, S, 16, 16, ws2, W, FP4W_F16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "launch_dequant_vec") == 0);
  EXPECT(fp4w_dequant(B, 128, 30, S, 2, 15, ws2, W, FP4W_F16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "launch_dequant_generic") == 0);
  EXPECT(fp8w_dequant(B, 128, 256, reinterpret_cast<const float*>(S), 2, 128, W, FP4W_BF16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "launch_fp8_dequant_vec") == 0);
  EXPECT(fp8w_qdq_activation(A, 4, 64, ws2, A, FP4W_BF16, nullptr) == FP4W_OK);  // in place
  EXPECT(strcmp(fp4w::g_last, "launch_qdq_vec") == 0);
  EXPECT(fp8w_qdq_activation(A, 4, 64, ws2, A + 2, FP4W_BF16, nullptr) == FP4W_ERR_ALIAS);
  EXPECT(fp8w_matmul_w8a8(A, 4, 512, B, 300, reinterpret_cast<const float*>(S), 4, 128, ws2, nullptr, W, Y,
                          FP4W_BF16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "launch_fp8_gemv") == 0);
  // NVFP4 activation and W4A4
  uint8_t* C = reinterpret_cast<uint8_t*>(W);
  EXPECT(fp4w_quantize_activation(A, 4, 64, C, C + 128, FP4W_BF16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "launch_nvfp4_quantize_vec") == 0);
  EXPECT(fp4w_quantize_activation(A + 1, 4, 64, C, C + 128, FP4W_BF16, nullptr) == FP4W_OK);  // unaligned
  EXPECT(strcmp(fp4w::g_last, "launch_nvfp4_quantize_generic") == 0);
  EXPECT(fp4w_quantize_activation(A, 4, 64, C, C + 64, FP4W_BF16, nullptr) == FP4W_ERR_ALIAS);
  EXPECT(fp4w_qdq_activation(A, 4, 64, A, FP4W_F16, nullptr) == FP4W_OK);  // in place
  EXPECT(strcmp(fp4w::g_last, "launch_nvfp4_qdq_vec") == 0);
  EXPECT(fp4w_qdq_activation(A, 4, 48, A, FP4W_F16, nullptr) == FP4W_OK);
  EXPECT(fp4w_qdq_activation(A, 4, 40, A, FP4W_F16, nullptr) == FP4W_ERR_SHAPE);
  EXPECT(fp4w_quantize_activation(A, big, big, C, C + 128, FP4W_BF16, nullptr) == FP4W_ERR_SHAPE);
  EXPECT(fp4w_matmul_w4a4(A, 4, 512, B, 300, S, 32, 16, ws2, nullptr, W, Y, FP4W_BF16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "launch_fp4_gemv_w4a4") == 0);  // decode: the QDQ fused into the GEMV
  fp4w::g_fused_rc = 1;  // A too large for the GEMV's LDS copy: separate QDQ, then the GEMV
  EXPECT(fp4w_matmul_w4a4(A, 4, 512, B, 300, S, 32, 16, ws2, nullptr, W, Y, FP4W_BF16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "launch_fp4_gemv") == 0);
  fp4w::g_fused_rc = 0;
  EXPECT(fp4w_matmul_w4a4(A, 4, 512, B, 300, S, 32, 16, ws2, nullptr, A, Y, FP4W_BF16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "launch_fp4_gemv") == 0);  // in place: separate QDQ, then the GEMV
  EXPECT(fp4w_matmul_w4a4(A, 4, 520, B, 300, S, 33, 16, ws2, nullptr, W, Y, FP4W_BF16, nullptr) ==
         FP4W_ERR_SHAPE);
  // the allocation-free variant: same dispatch, the library's scratch as the
  // workspace, sizes past the scratch rejected before anything is launched
  fp4w::g_last = "";
  EXPECT(fp4w_matmul_w4a4_noalloc(A, 4, 512, B, 300, S, 32, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_OK);
  EXPECT(strcmp(fp4w::g_last, "launch_fp4_gemv_w4a4") == 0);
  fp4w::g_last = "";
  EXPECT(fp4w_matmul_w4a4_noalloc(A, 4096, 8192, B, 300, S, 512, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) ==
         FP4W_ERR_SHAPE);  // 64 MiB of activation > FP4W_STATIC_SCRATCH_BYTES
  EXPECT(strcmp(fp4w::g_last, "") == 0);
  EXPECT(fp4w_matmul_w4a4_noalloc(A, 4, 520, B, 300, S, 33, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) ==
         FP4W_ERR_SHAPE);
  EXPECT(fp4w_matmul_w4a4_noalloc(nullptr, 4, 512, B, 300, S, 32, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) ==
         FP4W_ERR_NULL);
  EXPECT(fp4w_matmul_w4a4_noalloc(A, 0, 512, B, 300, S, 32, 16, ws2, nullptr, Y, FP4W_BF16, nullptr) == FP4W_OK);
  // select_path over a sweep of sizes, including ones near the int64 limits
  const int64_t dims[] = {0, 1, 7, 8, 9, 64, 65, 128, 480, 5120, 17408, int64_t(1) << 22, int64_t(1) << 31,
                          int64_t(1) << 40, int64_t(1) << 62};
  const int64_t blocks[] = {1, 15, 16, 64, 128};
  for (int op = 0; op <= 5; ++op)
    for (int64_t M : dims)
      for (int64_t N : dims)
        for (int64_t K : dims)
          for (int64_t bs : blocks) {
            const int64_t cols = K == 0 ? 0 : K / bs + (K % bs != 0);
            const int r = fp4w_select_path(op, M, N, K, bs, cols);
            EXPECT(r >= FP4W_ERR_ALIAS && r <= FP4W_PATH_NVFP4_GENERIC);
          }
  for (int s = -8; s <= 1; ++s) EXPECT(fp4w_status_string(s) != nullptr);
  for (int p = -1; p <= 18; ++p) EXPECT(fp4w_path_name(p) != nullptr);
  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
