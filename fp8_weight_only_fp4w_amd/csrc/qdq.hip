// Activation quantize/dequantize for the optional W8A8 mode of the FP8
// operator ([FP8 doc] §6, Optional W8A8 Activation Path):
//
//   out[i] = RNE_T( RNE_f32( e4m3( sat448( RNE_f32(A[i] / a_scale) ) ) * a_scale ) )
//
// The pages write fp8_e4m3(.) without a rounding or overflow rule.  Taken
// here: round to nearest even (the conversion instruction's mode) and
// saturation of magnitudes above 448, the largest finite E4M3 "fn" value,
// done before the conversion so that the instruction never sees an
// out-of-range input.  NaN stays NaN.
//
// gfx950 mapping: the division is IEEE (correctly rounded) FP32 division;
// v_cvt_pk_fp8_f32 encodes two FP32 values to OCP E4M3, v_cvt_pk_f32_fp8
// decodes them back exactly; the multiply by a_scale is the single FP32
// rounding of the product (an E4M3 value has 4 significand bits).  HBM-bound
// elementwise work: 16-byte loads and stores, 8 elements per chunk, a flat
// grid-stride loop.
//
// [FP8 doc] = "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"

#include <hip/hip_runtime.h>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

constexpr float kE4M3Max = 448.0f;

// Saturate to +-448, NaN passing through (the comparisons are false for it).
__device__ __forceinline__ float sat448(float q) {
  q = q > kE4M3Max ? kE4M3Max : q;
  return q < -kE4M3Max ? -kE4M3Max : q;
}

// Two values through the E4M3 grid: encode (RNE) and decode back.
__device__ __forceinline__ f32x2 e4m3_round_pair(float a, float b) {
  const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  return __builtin_amdgcn_cvt_pk_f32_fp8(packed, false);
}

template <typename T>
__device__ __forceinline__ u32x4 qdq8(u32x4 in, float s) {
  typedef typename ActTraits<T>::vec8 V;
  const V x = __builtin_bit_cast(V, in);
  V r;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const float q0 = static_cast<float>(x[i]) / s;
    const float q1 = static_cast<float>(x[i + 1]) / s;
    const f32x2 d = e4m3_round_pair(q0, q1);
    r[i] = round_to<T>(d.x * s);
    r[i + 1] = round_to<T>(d.y * s);
  }
  return __builtin_bit_cast(u32x4, r);
}

constexpr int kQThreads = 256;
constexpr int kQUnroll = 4;

template <typename T>
__global__ __launch_bounds__(kQThreads) void qdq_vec_kernel(const u32x4* A, const float* a_scale,
                                                            u32x4* out, uint64_t chunks) {
  const float s = *a_scale;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kQThreads * kQUnroll;
  for (uint64_t base = static_cast<uint64_t>(blockIdx.x) * kQThreads * kQUnroll + threadIdx.x;
       base < chunks; base += stride) {
    u32x4 v[kQUnroll];
#pragma unroll
    for (int u = 0; u < kQUnroll; ++u) {
      const uint64_t c = base + u * kQThreads;
      if (c < chunks) v[u] = A[c];
    }
#pragma unroll
    for (int u = 0; u < kQUnroll; ++u) {
      const uint64_t c = base + u * kQThreads;
      if (c < chunks) out[c] = qdq8<T>(v[u], s);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void qdq_generic_kernel(const T* A, const float* a_scale, T* out,
                                                          int64_t count) {
  const float s = *a_scale;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < count;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float q = static_cast<float>(A[e]) / s;
    const f32x2 d = e4m3_round_pair(q, 0.0f);
    out[e] = round_to<T>(d.x * s);
  }
}

int grid_for(int64_t items, int per_block) {
  int64_t g = (items + per_block - 1) / per_block;
  const int64_t cap = 256 * 16;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

}  // namespace

// In-place use (out == A) is safe: every chunk is read and written by the
// same thread, the read before the write (hence no __restrict__ above).
int launch_qdq_vec(const QdqArgs& a) {
  const uint64_t chunks = static_cast<uint64_t>(a.count / 8);
  const int grid = grid_for(static_cast<int64_t>(chunks), kQThreads * kQUnroll);
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  if (a.act == Act::BF16)
    hipLaunchKernelGGL(qdq_vec_kernel<__bf16>, dim3(grid), dim3(kQThreads), 0, st,
                       static_cast<const u32x4*>(a.A), a.a_scale, static_cast<u32x4*>(a.out), chunks);
  else
    hipLaunchKernelGGL(qdq_vec_kernel<_Float16>, dim3(grid), dim3(kQThreads), 0, st,
                       static_cast<const u32x4*>(a.A), a.a_scale, static_cast<u32x4*>(a.out), chunks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_qdq_generic(const QdqArgs& a) {
  const int grid = grid_for(a.count, 256);
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  if (a.act == Act::BF16)
    hipLaunchKernelGGL(qdq_generic_kernel<__bf16>, dim3(grid), dim3(256), 0, st,
                       static_cast<const __bf16*>(a.A), a.a_scale, static_cast<__bf16*>(a.out),
                       a.count);
  else
    hipLaunchKernelGGL(qdq_generic_kernel<_Float16>, dim3(grid), dim3(256), 0, st,
                       static_cast<const _Float16*>(a.A), a.a_scale, static_cast<_Float16*>(a.out),
                       a.count);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace fp4w
