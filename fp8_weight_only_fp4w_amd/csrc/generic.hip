// Generic weight-only FP4 / FP8 matmul: correct for every legal shape
// (odd block_size, K not a multiple of 32 / 64 / 128, partial final block,
// K == 0, unaligned pointers).  Not tuned: the shapes that matter take the
// GEMV / GEMM kernels.
//
// FP4 ([FP4 doc] §2):  Y[m,n] = ws2 * sum_k A[m,k] * (e2m1 * e4m3) + bias[n]
// FP8 ([FP8 doc] §2):  Y[m,n] = sum_k A[m,k] * (e4m3 * b_scale) + bias[n]
//
// One wave64 per output column n and group of up to 8 rows; lanes stride over
// K, each decoding one weight element with its own scale column
// min(k / block_size, scale_cols - 1), and the partial sums are reduced across
// the wave with DPP/permute shuffles.  Products are formed exactly where the
// formats allow (E2M1 x E4M3 x T for FP4, E4M3 x T for FP8) and accumulated
// in FP32.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
// [FP8 doc] = "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"

#include <hip/hip_runtime.h>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

constexpr int kRowsPerWave = 8;
constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <typename T, bool FP4>
__global__ __launch_bounds__(64 * kWavesPerBlock) void matmul_generic_kernel(
    const T* __restrict__ A, const uint8_t* __restrict__ B, const void* __restrict__ scales,
    const float* __restrict__ ws2p, const T* __restrict__ bias, T* __restrict__ Y, int64_t M,
    int64_t N, int64_t K, int64_t bs, int64_t cols) {
  const int lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (n >= N) return;  // whole wave leaves; no barrier in this kernel
  const int64_t groups = (M + kRowsPerWave - 1) / kRowsPerWave;
  const float b = bias ? static_cast<float>(bias[n]) : 0.0f;
  const float ws2 = (FP4 && K > 0) ? *ws2p : 1.0f;
  for (int64_t grp = blockIdx.y; grp < groups; grp += gridDim.y) {
    const int64_t m0 = grp * kRowsPerWave;
    const int mcount = static_cast<int>(min<int64_t>(kRowsPerWave, M - m0));
    float acc[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) acc[r] = 0.0f;
    for (int64_t k = lane; k < K; k += 64) {
      const int64_t col = min(k / bs, cols - 1);
      float w, s;
      if (FP4) {
        const uint32_t byte = B[n * (K / 2) + (k >> 1)];
        const f32x2 q2 = e2m1x2_to_f32<0>(byte);
        // E2M1 x E4M3 is exact in FP32; A x (that) is exact too (<= 17 bits)
        w = ((k & 1) ? q2.y : q2.x) *
            e4m3_to_f32<0>(static_cast<const uint8_t*>(scales)[n * cols + col]);
        s = 1.0f;
      } else {
        w = e4m3_to_f32<0>(B[n * K + k]);  // A x E4M3 is exact (<= 15 bits)
        s = static_cast<const float*>(scales)[n * cols + col];
      }
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        if (r < mcount) {
          const float a = static_cast<float>(A[(m0 + r) * K + k]);
          acc[r] = fmaf(a * w, s, acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const float tot = wave_sum(acc[r]);
      if (lane == r && r < mcount) {
        const float y = FP4 ? (K > 0 ? fmaf(tot, ws2, b) : b) : tot + b;
        Y[(m0 + r) * N + n] = round_to<T>(y);
      }
    }
  }
}

template <typename T, bool FP4>
int launch(const MatmulArgs& a) {
  const int64_t gx = (a.N + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t groups = (a.M + kRowsPerWave - 1) / kRowsPerWave;
  if (gx > 0x7fffffff) return -1;
  const int gy = static_cast<int>(groups < 65535 ? groups : 65535);
  hipLaunchKernelGGL((matmul_generic_kernel<T, FP4>), dim3(static_cast<unsigned>(gx), gy),
                     dim3(64 * kWavesPerBlock), 0, static_cast<hipStream_t>(a.stream),
                     static_cast<const T*>(a.A), a.B, a.scales, a.ws2,
                     static_cast<const T*>(a.bias), static_cast<T*>(a.Y), a.M, a.N, a.K,
                     a.block_size, a.scale_cols);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_fp4_generic(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch<__bf16, true>(a) : launch<_Float16, true>(a);
}

int launch_fp8_generic(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch<__bf16, false>(a) : launch<_Float16, false>(a);
}

}  // namespace fp4w
