// NVFP4 activation quantization, step 1 of the FP4 operator's native
// FP4 x FP4 path ([FP4 doc] §6 Native SM120 FP4 x FP4 Path): each block of 16
// consecutive elements of a row of A becomes 16 E2M1 codes and one E4M3
// scale, by the block rules in nvfp4_block.h.  The QDQ form writes e2m1 x
// e4m3 back in T, which is exact: a W4A4 matmul is that activation times the
// dequantized weights, run by the FP4 kernels.
//
// gfx950 mapping: one thread per block (32 bytes of T in, 9 bytes or 32 bytes
// out, contiguous across the wave), a flat grid-stride loop; v_cvt_pk_fp8_f32
// encodes the scale (round to nearest even), v_cvt_f32_fp8 decodes it,
// v_cvt_scalef32_pk_fp4_f32 / _pk_f32_fp4 encode and decode the codes.  The
// decode GEMV's W4A4 form runs the same block QDQ on its LDS copy of A.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"

#include <hip/hip_runtime.h>

#include "device.h"
#include "launch.h"
#include "nvfp4_block.h"

namespace fp4w {
namespace {

constexpr int kThreads = 256;

template <typename T, bool VEC>
__device__ __forceinline__ void load_block(const T* A, int64_t b, float (&v)[16]) {
  if constexpr (VEC) {
    typedef typename ActTraits<T>::vec8 V;
    const u32x4* p = reinterpret_cast<const u32x4*>(A + 16 * b);
    const V x0 = __builtin_bit_cast(V, p[0]);
    const V x1 = __builtin_bit_cast(V, p[1]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = static_cast<float>(x0[i]);
      v[8 + i] = static_cast<float>(x1[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = static_cast<float>(A[16 * b + i]);
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void nvfp4_quantize_kernel(const T* A, uint8_t* codes, uint8_t* scales,
                                                                  int64_t blocks) {
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < blocks;
       b += static_cast<int64_t>(gridDim.x) * kThreads) {
    float v[16];
    load_block<T, VEC>(A, b, v);
    uint32_t sbyte, w[2];
    float s;
    nvfp4_quant_block(v, sbyte, s, w);
    if constexpr (VEC) {
      *reinterpret_cast<u32x2*>(codes + 8 * b) = u32x2{w[0], w[1]};
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) codes[8 * b + i] = static_cast<uint8_t>(w[i >> 2] >> (8 * (i & 3)));
    }
    scales[b] = static_cast<uint8_t>(sbyte);
  }
}

// In-place use (out == A) is safe: every block is read and written by the
// same thread, the read first (hence no __restrict__).
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void nvfp4_qdq_kernel(const T* A, T* out, int64_t blocks) {
  typedef typename ActTraits<T>::vec8 V;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < blocks;
       b += static_cast<int64_t>(gridDim.x) * kThreads) {
    float v[16];
    load_block<T, VEC>(A, b, v);
    V r[2];
    nvfp4_qdq_block<T>(v, r);
    if constexpr (VEC) {
      u32x4* q = reinterpret_cast<u32x4*>(out + 16 * b);
      q[0] = __builtin_bit_cast(u32x4, r[0]);
      q[1] = __builtin_bit_cast(u32x4, r[1]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) out[16 * b + i] = r[i >> 3][i & 7];
    }
  }
}

int grid_for(int64_t blocks) {
  int64_t g = (blocks + kThreads - 1) / kThreads;
  const int64_t cap = 256 * 16;
  return static_cast<int>(g > cap ? cap : (g < 1 ? 1 : g));
}

template <typename T>
int quantize_t(const Nvfp4Args& a, bool vec) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const T* A = static_cast<const T*>(a.A);
  if (vec)
    hipLaunchKernelGGL((nvfp4_quantize_kernel<T, true>), dim3(grid_for(a.blocks)), dim3(kThreads), 0, st, A,
                       a.codes, a.scales, a.blocks);
  else
    hipLaunchKernelGGL((nvfp4_quantize_kernel<T, false>), dim3(grid_for(a.blocks)), dim3(kThreads), 0, st, A,
                       a.codes, a.scales, a.blocks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T>
int qdq_t(const Nvfp4Args& a, bool vec) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const T* A = static_cast<const T*>(a.A);
  T* out = static_cast<T*>(a.out);
  if (vec)
    hipLaunchKernelGGL((nvfp4_qdq_kernel<T, true>), dim3(grid_for(a.blocks)), dim3(kThreads), 0, st, A, out,
                       a.blocks);
  else
    hipLaunchKernelGGL((nvfp4_qdq_kernel<T, false>), dim3(grid_for(a.blocks)), dim3(kThreads), 0, st, A, out,
                       a.blocks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_nvfp4_quantize(const Nvfp4Args& a, bool vec) {
  return a.act == Act::BF16 ? quantize_t<__bf16>(a, vec) : quantize_t<_Float16>(a, vec);
}

int launch_nvfp4_qdq(const Nvfp4Args& a, bool vec) {
  return a.act == Act::BF16 ? qdq_t<__bf16>(a, vec) : qdq_t<_Float16>(a, vec);
}

}  // namespace fp4w
